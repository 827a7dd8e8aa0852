// Block attention over [injected context ; block] for one draft layer.
//
// Per (sequence b, kv head h) the queries are the g*gamma rows (g q-heads of
// the group x gamma block positions), row R = hq*gamma + j.  Keys/values are
// the len[b] cached context rows followed by the gamma block rows; there is no
// mask inside the block and the whole context is visible (bidirectional).
//
// Work split ("split-K" over keys): chunk 0 of each (b,h) holds the block
// rows, chunks 1.. hold CH context rows each.  A workgroup of 4 wavefronts
// takes one chunk:
//  * prologue: the query rows get the per-head q RMSNorm and RoPE once per
//    workgroup (wave w builds query tiles w, w+4, ...) and are kept as MFMA
//    fragments in LDS; chunk 0 also builds the block's keys (k RMSNorm + RoPE)
//    and values (rounded, transposed to [d][key]) in LDS;
//  * the waves split the chunk's keys (and, for g*gamma > 64, the query rows)
//    and stream keys in sub-blocks of 32, loading the next sub-block while the
//    current one is computed:
//      S^T = K . Q^T   (A = key rows, B = queries)
//    with the key rows permuted so that every lane ends up holding 8
//    consecutive keys of one query - exactly the A-operand layout of
//      O  += P . V     (B = V^T rows, read straight from the transposed V cache);
//  * online softmax in base 2 (log2(e)/sqrt(D) folded into the scale); for
//    bf16 the PV product takes P as a hi + lo pair of bf16 values;
//  * the waves merge through LDS; the workgroup writes (m, l, O) for its chunk
//    and attn_merge combines the chunks with log-sum-exp weights in fixed
//    chunk order.
#pragma once

#include "common.hpp"

namespace dflash {

constexpr int ATT_THREADS = 256;

struct AttnArgs {
    const void* kcache;     // this layer: T [Bmax][n_kv][cap][D]
    const void* vcache;     // this layer: T [Bmax][n_kv][D][cap]
    const float* qkv;       // raw projections fp32 [B*gamma][qkv_ld]: q heads, then k heads, then v heads
    int qkv_ld;
    const void* q_norm;     // T [D]
    const void* k_norm;     // T [D]
    const float* rope_cos;  // [rope_rows][D/2]
    const float* rope_sin;
    int rope_rows;
    float eps;
    const int* len;         // [B]
    float* opart;           // [B][n_kv][nch_max][rpad][D]
    float* mlpart;          // [B][n_kv][nch_max][rpad][2]  (m in log2 units, l)
    int n_q, n_kv, cap, rpad, nch_max, chunk;   // chunk = CH context keys per chunk
    int gamma, group;       // rows = group * gamma
    int qg, kg;             // waves = qg query groups x kg key groups (qg*kg <= 4)
    float scale_log2;       // log2(e) / sqrt(D)
};

// Per-wave attention state for up to 4 query tiles (the query fragments
// themselves stay in LDS).
template <typename T>
struct WaveAttn {
    static constexpr int D = 256 / (int)sizeof(T);   // head_dim (one k-step)
    static constexpr int DT = D / 16;                 // d tiles
    float m[4], l[4];     // per query column r of tile qi (replicated over g)
    f32x4_t o[4][DT];     // O[q = qi*16 + g*4 + v][d = dt*16 + r]
};

// 8 consecutive keys of one V^T row (d fixed): the MFMA B operand of O += P.V.
template <typename T> struct VFrag;
template <> struct VFrag<bf16_t> { u32x4_t q; };        // 8 bf16
template <> struct VFrag<float> { u32x4_t q[2]; };      // 8 f32

// Keys [kb + g*8, +8) of V^T row p (p points at key kb + g*8).  The load is
// unconditional (no per-lane branch, so that loads of a sub-block stay in
// flight together); keys beyond the real ones are cleared by vfrag_mask.
template <typename T>
__device__ __forceinline__ void vfrag_load(VFrag<T>& v, const T* p);

template <>
__device__ __forceinline__ void vfrag_load<bf16_t>(VFrag<bf16_t>& v, const bf16_t* p) {
    v.q = *reinterpret_cast<const u32x4_t*>(p);
}

template <>
__device__ __forceinline__ void vfrag_load<float>(VFrag<float>& v, const float* p) {
    v.q[0] = *reinterpret_cast<const u32x4_t*>(p);
    v.q[1] = *reinterpret_cast<const u32x4_t*>(p + 4);
}

// Zero keys >= valid of the fragment (valid may be <= 0 or >= 8).  Stale cache
// rows may hold any bits, and 0 * NaN would poison O, so they are cleared.
__device__ __forceinline__ void vfrag_mask(VFrag<bf16_t>& v, int valid) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t keep = ((2 * j < valid) ? 0x0000FFFFu : 0u) | ((2 * j + 1 < valid) ? 0xFFFF0000u : 0u);
        v.q[j] &= keep;
    }
}

__device__ __forceinline__ void vfrag_mask(VFrag<float>& v, int valid) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        v.q[0][j] = (j < valid) ? v.q[0][j] : 0u;
        v.q[1][j] = (j + 4 < valid) ? v.q[1][j] : 0u;
    }
}

// P of one lane (8 consecutive keys of one query) as the MFMA A operand.
template <typename T> struct PFrag;
// bf16: P = hi + lo with both parts bf16 (|P - hi - lo| <= 2^-17 |P|), so the
// bf16 MFMA does not add the rounding of P to the result; V is bf16-exact.
template <> struct PFrag<bf16_t> { u32x4_t hi, lo; };
template <> struct PFrag<float> { float p[8]; };

__device__ __forceinline__ void make_pfrag(PFrag<bf16_t>& f, const float (&p)[8]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t h = pack2_bf16(p[2 * j], p[2 * j + 1]);
        f.hi[j] = h;
        f.lo[j] = pack2_bf16(p[2 * j] - __uint_as_float(h << 16), p[2 * j + 1] - __uint_as_float(h & 0xFFFF0000u));
    }
}

__device__ __forceinline__ void make_pfrag(PFrag<float>& f, const float (&p)[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) f.p[j] = p[j];
}

// acc[q][d] += P(q, 8 keys of this lane group) . V(8 keys, 16 d)
__device__ __forceinline__ void pv_mfma(f32x4_t& acc, const PFrag<bf16_t>& p, const VFrag<bf16_t>& v) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(p.hi), as_bf16x8(v.q), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(p.lo), as_bf16x8(v.q), acc, 0, 0, 0);
}

__device__ __forceinline__ void pv_mfma(f32x4_t& acc, const PFrag<float>& p, const VFrag<float>& v) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(p.p[j], __uint_as_float(v.q[j >> 2][j & 3]), acc, 0, 0, 0);
}

// A head row as held by one lane in the fragment layout: piece i (0..3) holds
// elements d = 4*PER*i + PER*g + j (j < PER, PER = 16 bytes / element size).
// Rotate-half RoPE pairs d with d + D/2, i.e. piece i with piece i + 2 of the
// same lane; the four lanes of a row (g = 0..3) are 16 lanes apart.
template <typename T>
__device__ __forceinline__ void load_row_raw(float (&x)[4][Elem<T>::PER16], const float* row, bool valid) {
    constexpr int PER = Elem<T>::PER16;
    const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int h = 0; h < PER / 4; ++h) {
            const float4 v = valid ? *reinterpret_cast<const float4*>(row + i * 4 * PER + g * PER + h * 4)
                                   : make_float4(0.f, 0.f, 0.f, 0.f);
            x[i][h * 4 + 0] = v.x; x[i][h * 4 + 1] = v.y; x[i][h * 4 + 2] = v.z; x[i][h * 4 + 3] = v.w;
        }
}

// Per-head RMSNorm (over the D elements spread over the row's four lanes) then
// rotate-half RoPE, rounded to the storage type, into an MFMA fragment.
template <typename T>
__device__ __forceinline__ void norm_rope_frag(Frag64& out, const float (&x)[4][Elem<T>::PER16], const T* wn,
                                               float eps, const float* cosr, const float* sinr) {
    constexpr int PER = Elem<T>::PER16;
    constexpr int D = 16 * PER;
    const int g = (threadIdx.x & 63) >> 4;
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < PER; ++j) ss += x[i][j] * x[i][j];
    ss += __shfl_xor(ss, 16, WAVE);
    ss += __shfl_xor(ss, 32, WAVE);
    const float rs = 1.0f / sqrtf(ss / (float)D + eps);
    Frag64 wf;
    load_frag64(wf, wn + g * PER);
    float y[4][PER];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const T* wp = reinterpret_cast<const T*>(&wf.q[i]);
#pragma unroll
        for (int j = 0; j < PER; ++j) y[i][j] = x[i][j] * rs * Elem<T>::to_f(wp[j]);
    }
    float o[4][PER];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        float c[PER], sn[PER];
#pragma unroll
        for (int h = 0; h < PER / 4; ++h) {
            const float4 c4 = *reinterpret_cast<const float4*>(cosr + i * 4 * PER + g * PER + h * 4);
            const float4 s4 = *reinterpret_cast<const float4*>(sinr + i * 4 * PER + g * PER + h * 4);
            c[h * 4 + 0] = c4.x; c[h * 4 + 1] = c4.y; c[h * 4 + 2] = c4.z; c[h * 4 + 3] = c4.w;
            sn[h * 4 + 0] = s4.x; sn[h * 4 + 1] = s4.y; sn[h * 4 + 2] = s4.z; sn[h * 4 + 3] = s4.w;
        }
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            o[i][j] = y[i][j] * c[j] - y[i + 2][j] * sn[j];
            o[i + 2][j] = y[i + 2][j] * c[j] + y[i][j] * sn[j];
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if constexpr (sizeof(T) == 2) {
            out.q[i] = u32x4_t{pack2_bf16(o[i][0], o[i][1]), pack2_bf16(o[i][2], o[i][3]),
                               pack2_bf16(o[i][4], o[i][5]), pack2_bf16(o[i][6], o[i][7])};
        } else {
            out.q[i] = u32x4_t{__float_as_uint(o[i][0]), __float_as_uint(o[i][1]), __float_as_uint(o[i][2]),
                               __float_as_uint(o[i][3])};
        }
    }
}

// LDS operand tiles: rows of 256 bytes; the 16-byte chunk c of row R sits at
// position c ^ (R & 15), so that the fragment reads of 16 rows hit distinct banks.
__device__ __forceinline__ int lds_swz(int R, int c) { return R * 256 + ((c ^ (R & 15)) * 16); }

__device__ __forceinline__ void store_frag_lds(unsigned char* base, int R, const Frag64& f) {
    const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4_t*>(base + lds_swz(R, 4 * i + g)) = f.q[i];
}

__device__ __forceinline__ void load_frag_lds(Frag64& f, const unsigned char* base, int R) {
    const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) f.q[i] = *reinterpret_cast<const u32x4_t*>(base + lds_swz(R, 4 * i + g));
}

// Key of lane row r in S^T tile t of a 32-key sub-block: (r/4)*8 + t*4 + r%4,
// so that lane group g of the result holds keys g*8 .. g*8+7.
__device__ __forceinline__ int subblock_key(int t, int r) { return (r >> 2) * 8 + t * 4 + (r & 3); }

// One 32-key sub-block of which the first `nvalid` keys are real.
// qlds holds the query fragments of this wave's tiles (rows qt0*16 ..).
template <typename T>
__device__ __forceinline__ void attn_subblock(WaveAttn<T>& w, const unsigned char* qlds, int qt0, int nqt, int nvalid,
                                              float scale_log2, const Frag64 (&kf)[2],
                                              VFrag<T> (&vf)[WaveAttn<T>::DT]) {
    constexpr int DT = WaveAttn<T>::DT;
    const int lane = threadIdx.x & 63, g = lane >> 4, r = lane & 15;
    if (nvalid < 32) {   // wave-uniform: only the last sub-block of a sequence
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) vfrag_mask(vf[dt], nvalid - g * 8);
    }
#pragma unroll
    for (int qi = 0; qi < 4; ++qi) {
        if (qi < nqt) {
            Frag64 qf;
            load_frag_lds(qf, qlds, (qt0 + qi) * 16 + r);
            f32x4_t st[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                st[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                mfma_kstep<T>(st[t], kf[t], qf);
            }
            // lane holds S[q = qi*16 + r][key = g*8 + t*4 + v]
            float s[8];
            float mx = -INFINITY;
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int key = g * 8 + t * 4 + v;
                    const float x = key < nvalid ? st[t][v] * scale_log2 : -INFINITY;
                    s[t * 4 + v] = x;
                    mx = fmaxf(mx, x);
                }
            mx = fmaxf(mx, __shfl_xor(mx, 16, WAVE));
            mx = fmaxf(mx, __shfl_xor(mx, 32, WAVE));
            const float mnew = fmaxf(w.m[qi], mx);
            const bool dead = (mnew == -INFINITY);
            const float alpha = dead ? 1.f : exp2f(w.m[qi] - mnew);
            float p[8];
            float psum = 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                p[j] = dead ? 0.f : exp2f(s[j] - mnew);
                psum += p[j];
            }
            w.l[qi] = w.l[qi] * alpha + psum;
            w.m[qi] = mnew;
            // rescale O rows q = g*4 + v by alpha of that query (held by lane g*4+v)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const float av = __shfl(alpha, g * 4 + v, WAVE);
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) w.o[qi][dt][v] *= av;
            }
            PFrag<T> pf;
            make_pfrag(pf, p);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) pv_mfma(w.o[qi][dt], pf, vf[dt]);
        }
    }
}

// Context keys [kb, kb+32) of one (b,h): K rows clamped to the last real key
// (their scores are masked); V is read whole (kb + 32 <= cap) and masked at use.
template <typename T>
__device__ __forceinline__ void fetch_ctx(Frag64 (&kf)[2], VFrag<T> (&vf)[WaveAttn<T>::DT], const T* kc, const T* vc,
                                          int cap, int kb, int nvalid) {
    constexpr int D = WaveAttn<T>::D, DT = WaveAttn<T>::DT, PER = Elem<T>::PER16;
    const int lane = threadIdx.x & 63, g = lane >> 4, r = lane & 15;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        int key = subblock_key(t, r);
        key = key < nvalid ? key : (nvalid - 1);
        load_frag64(kf[t], kc + (long long)(kb + key) * D + g * PER);
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
        vfrag_load<T>(vf[dt], vc + (long long)(dt * 16 + r) * cap + kb + g * 8);
}

// LDS of a workgroup: query fragments [16 * qtiles rows][256 B], block keys
// [32][256 B], block V^T [D][32 keys]; the wave merge later reuses the space.
__host__ __device__ inline size_t attn_q_lds_bytes(int qtiles) { return (size_t)qtiles * 16 * 256; }
static inline size_t attn_slot_floats(int elem_bytes) {
    const int DT = 256 / elem_bytes / 16;
    return (size_t)4 * DT * 64 * 4 + 2 * 4 * 4 * 64;
}
static inline size_t attn_lds_bytes_host(int elem_bytes, int qtiles, int kg) {
    const size_t prologue = attn_q_lds_bytes(qtiles) + 32 * 256 + (size_t)(256 / elem_bytes) * 32 * elem_bytes;
    const size_t slot = kg >= 2 ? attn_slot_floats(elem_bytes) * sizeof(float) : 0;
    return prologue > slot ? prologue : slot;
}

template <typename T>
__global__ __launch_bounds__(ATT_THREADS) void attn_partial_kernel(const AttnArgs a) {
    constexpr int D = WaveAttn<T>::D, DT = WaveAttn<T>::DT, PER = Elem<T>::PER16;
    extern __shared__ __align__(16) unsigned char smem[];
    const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    int len = a.len[b];
    len = len < 0 ? 0 : (len > a.cap ? a.cap : len);
    const int nch = 1 + (len + a.chunk - 1) / a.chunk;
    if (c >= nch) return;

    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, g = lane >> 4, r = lane & 15;
    const int qgi = wv / a.kg, kgi = wv % a.kg;
    const bool active_wave = wv < a.qg * a.kg;
    const int G = a.gamma;
    const int rows = a.group * G;
    const int nqt_all = (rows + 15) >> 4;
    const int qt0 = qgi * 4;
    const int nqt = active_wave ? max(0, min(4, nqt_all - qt0)) : 0;
    unsigned char* qlds = smem;
    unsigned char* klds = qlds + attn_q_lds_bytes(nqt_all);
    T* vlds = reinterpret_cast<T*>(klds + 32 * 256);   // [D][32]

    // ---- prologue: query fragments, normalised and rotated once per workgroup
    for (int qt = wv; qt < nqt_all; qt += 4) {
        const int R = qt * 16 + r;
        const bool valid = R < rows;
        const int hq = valid ? R / G : 0, j = valid ? R % G : 0;
        float x[4][PER];
        load_row_raw<T>(x, a.qkv + (long long)(b * G + j) * a.qkv_ld + (h * a.group + hq) * D, valid);
        int pos = len + j;
        pos = pos < a.rope_rows ? pos : a.rope_rows - 1;
        Frag64 f;
        norm_rope_frag<T>(f, x, reinterpret_cast<const T*>(a.q_norm), a.eps, a.rope_cos + (long long)pos * (D / 2),
                          a.rope_sin + (long long)pos * (D / 2));
        if (!valid) zero_frag64(f);
        store_frag_lds(qlds, R, f);
    }
    if (c == 0) {
        // the block's own keys (waves 0,1: keys 0..31, k RMSNorm + RoPE) and values (rounded)
        if (wv < 2) {
            const int key = wv * 16 + r;
            const bool valid = key < G;
            float x[4][PER];
            load_row_raw<T>(x, a.qkv + (long long)(b * G + (valid ? key : 0)) * a.qkv_ld + (a.n_q + h) * D, valid);
            int pos = len + (valid ? key : 0);
            pos = pos < a.rope_rows ? pos : a.rope_rows - 1;
            Frag64 f;
            norm_rope_frag<T>(f, x, reinterpret_cast<const T*>(a.k_norm), a.eps,
                              a.rope_cos + (long long)pos * (D / 2), a.rope_sin + (long long)pos * (D / 2));
            if (!valid) zero_frag64(f);
            store_frag_lds(klds, key, f);
        }
        // V^T of the block: all float4 loads of a thread are independent (one latency)
        constexpr int NV4 = 32 * D / 4;
        static_assert(NV4 % ATT_THREADS == 0, "block V tile split");
        float4 vv[NV4 / ATT_THREADS];
#pragma unroll
        for (int it = 0; it < NV4 / ATT_THREADS; ++it) {
            const int e4 = it * ATT_THREADS + threadIdx.x;
            const int key = e4 / (D / 4), d4 = e4 % (D / 4);
            vv[it] = key < G ? *reinterpret_cast<const float4*>(a.qkv + (long long)(b * G + key) * a.qkv_ld +
                                                                (a.n_q + a.n_kv + h) * D + d4 * 4)
                             : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int it = 0; it < NV4 / ATT_THREADS; ++it) {
            const int e4 = it * ATT_THREADS + threadIdx.x;
            const int key = e4 / (D / 4), d = (e4 % (D / 4)) * 4;
            vlds[(d + 0) * 32 + key] = Elem<T>::from_f(vv[it].x);
            vlds[(d + 1) * 32 + key] = Elem<T>::from_f(vv[it].y);
            vlds[(d + 2) * 32 + key] = Elem<T>::from_f(vv[it].z);
            vlds[(d + 3) * 32 + key] = Elem<T>::from_f(vv[it].w);
        }
    }
    __syncthreads();

    WaveAttn<T> w;
#pragma unroll
    for (int qi = 0; qi < 4; ++qi) {
        w.m[qi] = -INFINITY;
        w.l[qi] = 0.f;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) w.o[qi][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    if (c == 0) {
        if (nqt > 0 && kgi == 0) {
            Frag64 kf[2];
            VFrag<T> vf[DT];
#pragma unroll
            for (int t = 0; t < 2; ++t) load_frag_lds(kf[t], klds, subblock_key(t, r));
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) vfrag_load<T>(vf[dt], vlds + (dt * 16 + r) * 32 + g * 8);
            attn_subblock<T>(w, qlds, qt0, nqt, G, a.scale_log2, kf, vf);
        }
    } else if (nqt > 0) {
        const int per_wave = a.chunk / a.kg;
        const int k_lo = (c - 1) * a.chunk + kgi * per_wave;
        const int k_hi = min(k_lo + per_wave, len);
        const T* kc = reinterpret_cast<const T*>(a.kcache) + ((long long)b * a.n_kv + h) * (long long)a.cap * D;
        const T* vc = reinterpret_cast<const T*>(a.vcache) + ((long long)b * a.n_kv + h) * (long long)D * a.cap;
        // two register buffers: sub-block kb+32 loads while kb is computed
        Frag64 kfa[2], kfb[2];
        VFrag<T> vfa[DT], vfb[DT];
        if (k_lo < k_hi) fetch_ctx<T>(kfa, vfa, kc, vc, a.cap, k_lo, min(32, k_hi - k_lo));
        for (int kb = k_lo; kb < k_hi; kb += 64) {
            const int kb1 = kb + 32, kb2 = kb + 64;
            if (kb1 < k_hi) fetch_ctx<T>(kfb, vfb, kc, vc, a.cap, kb1, min(32, k_hi - kb1));
            attn_subblock<T>(w, qlds, qt0, nqt, min(32, k_hi - kb), a.scale_log2, kfa, vfa);
            if (kb1 >= k_hi) break;
            if (kb2 < k_hi) fetch_ctx<T>(kfa, vfa, kc, vc, a.cap, kb2, min(32, k_hi - kb2));
            attn_subblock<T>(w, qlds, qt0, nqt, min(32, k_hi - kb1), a.scale_log2, kfb, vfb);
        }
    }

    // ---- per-element (C-layout) statistics: l summed over the 4 lane groups
    float mq[4][4], lq[4][4];
#pragma unroll
    for (int qi = 0; qi < 4; ++qi) {
        float lt = w.l[qi];
        lt += __shfl_xor(lt, 16, WAVE);
        lt += __shfl_xor(lt, 32, WAVE);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            mq[qi][v] = __shfl(w.m[qi], g * 4 + v, WAVE);
            lq[qi][v] = __shfl(lt, g * 4 + v, WAVE);
        }
    }

    // ---- merge the key-group waves of each query group through one LDS slot
    // (pairwise rounds; the exchanges of a round run one after another)
    __syncthreads();   // the prologue tiles are dead: the slot reuses their space
    float* s = reinterpret_cast<float*>(smem);
    float* sm = s + 4 * DT * 64 * 4;
    for (int span = a.kg >> 1; span >= 1; span >>= 1) {
        for (int x = 0; x < a.qg * span; ++x) {
            const int xq = x / span, xp = x % span;
            const bool sender = active_wave && qgi == xq && kgi == span + xp;
            const bool receiver = active_wave && qgi == xq && kgi == xp;
            if (sender) {
#pragma unroll
                for (int qi = 0; qi < 4; ++qi)
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                        for (int v = 0; v < 4; ++v) s[((qi * DT + dt) * 4 + v) * 64 + lane] = w.o[qi][dt][v];
#pragma unroll
                for (int qi = 0; qi < 4; ++qi)
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        sm[(qi * 4 + v) * 64 + lane] = mq[qi][v];
                        sm[(16 + qi * 4 + v) * 64 + lane] = lq[qi][v];
                    }
            }
            __syncthreads();
            if (receiver) {
#pragma unroll
                for (int qi = 0; qi < 4; ++qi)
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const float m2 = sm[(qi * 4 + v) * 64 + lane];
                        const float l2 = sm[(16 + qi * 4 + v) * 64 + lane];
                        const float m1 = mq[qi][v];
                        const float mm = fmaxf(m1, m2);
                        const float f1 = (mm == -INFINITY) ? 0.f : exp2f(m1 - mm);
                        const float f2 = (mm == -INFINITY) ? 0.f : exp2f(m2 - mm);
#pragma unroll
                        for (int dt = 0; dt < DT; ++dt)
                            w.o[qi][dt][v] = w.o[qi][dt][v] * f1 + s[((qi * DT + dt) * 4 + v) * 64 + lane] * f2;
                        mq[qi][v] = mm;
                        lq[qi][v] = lq[qi][v] * f1 + l2 * f2;
                    }
            }
            __syncthreads();
        }
    }

    // ---- key-group 0 of every query group writes the chunk's partial
    if (active_wave && kgi == 0 && nqt > 0) {
        const long long base = (((long long)b * a.n_kv + h) * a.nch_max + c) * a.rpad;
        float* op = a.opart + base * D;
        float* mp = a.mlpart + base * 2;
#pragma unroll
        for (int qi = 0; qi < 4; ++qi)
            if (qi < nqt)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int R = (qt0 + qi) * 16 + g * 4 + v;
                    if (R < rows) {
#pragma unroll
                        for (int dt = 0; dt < DT; ++dt) op[(long long)R * D + dt * 16 + r] = w.o[qi][dt][v];
                        if (r == 0) {
                            mp[R * 2 + 0] = mq[qi][v];
                            mp[R * 2 + 1] = lq[qi][v];
                        }
                    }
                }
    }
}

// o[b*gamma + j][(h*g + hq)*D + d] = rho( sum_c w_c O_c / sum_c w_c l_c ),  w_c = 2^(m_c - max m)
struct MergeArgs {
    const float* opart;
    const float* mlpart;
    const int* len;
    void* out;              // T [B*gamma][n_q*D]
    int n_kv, group, gamma, rpad, nch_max, chunk, cap, head_dim;
};

constexpr int MERGE_MAX_CHUNKS = 1024;
constexpr int MERGE_BATCH = 16;   // chunk partials loaded together per lane

template <typename T>
__global__ __launch_bounds__(64) void attn_merge_kernel(const MergeArgs a) {
    // blockIdx.x = row (b*gamma + j), blockIdx.y = q head; one wavefront, lane
    // owns d = lane*DPL .. +DPL.  Chunks are summed in ascending order.
    constexpr int D = 256 / (int)sizeof(T), DPL = D / 64;
    __shared__ float wts[MERGE_MAX_CHUNKS];
    const int m = blockIdx.x, hq_all = blockIdx.y;
    const int b = m / a.gamma, j = m % a.gamma;
    const int h = hq_all / a.group, hq = hq_all % a.group;
    const int R = hq * a.gamma + j;
    const int lane = threadIdx.x;
    int len = a.len[b];
    len = len < 0 ? 0 : (len > a.cap ? a.cap : len);
    const int nch = 1 + (len + a.chunk - 1) / a.chunk;
    const long long base = ((long long)b * a.n_kv + h) * a.nch_max;
    float mmax = -INFINITY;
    for (int c = lane; c < nch; c += 64) mmax = fmaxf(mmax, a.mlpart[((base + c) * a.rpad + R) * 2]);
    mmax = wave_max(mmax);
    float den = 0.f;
    for (int c = lane; c < nch; c += 64) {
        const long long row = (base + c) * a.rpad + R;
        const float mc = a.mlpart[row * 2];
        const float wc = (mc == -INFINITY) ? 0.f : exp2f(mc - mmax);
        wts[c] = wc;
        den += wc * a.mlpart[row * 2 + 1];
    }
    den = wave_sum(den);
    __syncthreads();
    const float* op = a.opart + (base * a.rpad + R) * (long long)D + lane * DPL;
    const long long cstride = (long long)a.rpad * D;
    float num[DPL];
#pragma unroll
    for (int k = 0; k < DPL; ++k) num[k] = 0.f;
    for (int c0 = 0; c0 < nch; c0 += MERGE_BATCH) {
        float ov[MERGE_BATCH][DPL];
#pragma unroll
        for (int u = 0; u < MERGE_BATCH; ++u) {
            const int c = min(c0 + u, nch - 1);
#pragma unroll
            for (int k = 0; k < DPL; ++k) ov[u][k] = op[c * cstride + k];
        }
#pragma unroll
        for (int u = 0; u < MERGE_BATCH; ++u) {
            if (c0 + u < nch) {
                const float wc = wts[c0 + u];
#pragma unroll
                for (int k = 0; k < DPL; ++k) num[k] += wc * ov[u][k];
            }
        }
    }
    T* out = reinterpret_cast<T*>(a.out) + (long long)m * (gridDim.y * D) + (long long)hq_all * D + lane * DPL;
#pragma unroll
    for (int k = 0; k < DPL; ++k) out[k] = Elem<T>::from_f(num[k] / den);
}

}  // namespace dflash
