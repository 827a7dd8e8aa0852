// Block attention over [injected context ; block] for one draft layer.
//
// Per (sequence b, kv head h) the queries are the g*gamma rows (g q-heads of
// the group x gamma block positions), row R = hq*gamma + j.  Keys/values are
// the len[b] cached context rows followed by the gamma block rows; there is no
// mask inside the block and the whole context is visible (bidirectional).
//
// Work split ("split-K" over keys): chunk 0 of each (b,h) holds the block
// rows, chunks 1.. hold CH context rows each.  A workgroup of 4 wavefronts
// takes one chunk; its waves split the chunk's keys (and, for g*gamma > 64,
// the query rows).  Each wave streams keys in sub-blocks of 32:
//   S^T = K . Q^T   (A = key rows read straight from the cache, B = queries)
// with the key rows permuted so that every lane ends up holding 8 consecutive
// keys of one query - exactly the A-operand layout of the following
//   O  += P . V     (B = V^T rows, read straight from the transposed V cache).
// Online softmax in base 2 (log2(e)/sqrt(D) folded into the scale); for bf16
// the PV product takes P as a hi + lo pair of bf16 values.  The waves of a workgroup
// merge through LDS; the workgroup writes (m, l, O) for its chunk, and
// attn_merge combines the chunks of a (b,h) with log-sum-exp weights in fixed
// chunk order.
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

// Per-wave attention state for up to 4 query tiles.
template <typename T>
struct WaveAttn {
    static constexpr int D = 256 / (int)sizeof(T);   // head_dim (one k-step)
    static constexpr int DT = D / 16;                 // d tiles
    Frag64 qf[4];
    float m[4], l[4];     // per query column r of tile qi (replicated over g)
    f32x4_t o[4][DT];     // O[q = qi*16 + g*4 + v][d = dt*16 + r]
};

template <typename T>
__device__ __forceinline__ void vfrag_load(float (&v)[8], const T* p, int valid);   // 8 consecutive keys

template <>
__device__ __forceinline__ void vfrag_load<bf16_t>(float (&v)[8], const bf16_t* p, int valid) {
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        v[2 * j] = (2 * j < valid) ? __uint_as_float(w[j] << 16) : 0.f;
        v[2 * j + 1] = (2 * j + 1 < valid) ? __uint_as_float(w[j] & 0xFFFF0000u) : 0.f;
    }
}

template <>
__device__ __forceinline__ void vfrag_load<float>(float (&v)[8], const float* p, int valid) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    const float t[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = (j < valid) ? t[j] : 0.f;
}

// O[qi][dt] += P(8 keys of this lane's group) . V(8 keys x 16 d)
template <typename T>
__device__ __forceinline__ void pv_mfma(f32x4_t& acc, const float (&p)[8], const float (&v)[8]);

// P is split into hi + lo bf16 parts (|P - hi - lo| <= 2^-17 |P|), so the bf16
// MFMA does not add the rounding of P to the result; V is bf16-exact already.
template <>
__device__ __forceinline__ void pv_mfma<bf16_t>(f32x4_t& acc, const float (&p)[8], const float (&v)[8]) {
    bf16x8_t hi, lo, b;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const bf16_t h = f32_to_bf16(p[j]);
        hi[j] = (short)h;
        lo[j] = (short)f32_to_bf16(p[j] - bf16_to_f32(h));
        b[j] = (short)f32_to_bf16(v[j]);
    }
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi, b, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo, b, acc, 0, 0, 0);
}

template <>
__device__ __forceinline__ void pv_mfma<float>(f32x4_t& acc, const float (&p)[8], const float (&v)[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(p[j], v[j], acc, 0, 0, 0);
}

// Load the K fragments (two S^T tiles) and V^T fragments of keys [kb, kb+32) from
// the cache; keys at or beyond `nvalid` are clamped on load and masked later.
template <typename T>
__device__ __forceinline__ void load_ctx_frags(Frag64 (&kf)[2], float (&vf)[WaveAttn<T>::DT][8], const T* kc,
                                               const T* vc, int cap, int kb, int nvalid) {
    constexpr int D = WaveAttn<T>::D, DT = WaveAttn<T>::DT, STEP = Elem<T>::STEP;
    const int lane = threadIdx.x & 63, g = lane >> 4, r = lane & 15;
    // key rows of the two S^T tiles: lane row r -> key (r/4)*8 + t*4 + r%4
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        int key = (r >> 2) * 8 + t * 4 + (r & 3);
        key = key < nvalid ? key : (nvalid - 1);
        load_frag64(kf[t], kc + (long long)(kb + key) * D + g * Elem<T>::PER16);
    }
    // V^T fragments: lane (g,r), d = dt*16 + r, keys kb + g*8 .. +8
    const int vvalid = nvalid - g * 8;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) vfrag_load<T>(vf[dt], vc + (long long)(dt * 16 + r) * cap + kb + g * 8, vvalid);
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
            uint32_t w4[4];
#pragma unroll
            for (int k = 0; k < 4; ++k)
                w4[k] = (uint32_t)f32_to_bf16(o[i][2 * k]) | ((uint32_t)f32_to_bf16(o[i][2 * k + 1]) << 16);
            out.q[i] = u32x4_t{w4[0], w4[1], w4[2], w4[3]};
        } else {
            out.q[i] = u32x4_t{__float_as_uint(o[i][0]), __float_as_uint(o[i][1]), __float_as_uint(o[i][2]),
                               __float_as_uint(o[i][3])};
        }
    }
}

// Process keys [kb, kb+32) of which the first `nvalid` are real.
template <typename T>
__device__ __forceinline__ void attn_subblock(WaveAttn<T>& w, int nqt, int nvalid, float scale_log2,
                                              const Frag64 (&kf)[2], const float (&vf)[WaveAttn<T>::DT][8]) {
    constexpr int DT = WaveAttn<T>::DT;
    const int lane = threadIdx.x & 63, g = lane >> 4;
#pragma unroll
    for (int qi = 0; qi < 4; ++qi) {
        if (qi < nqt) {
            f32x4_t st[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                st[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                mfma_kstep<T>(st[t], kf[t], w.qf[qi]);
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
            float pv[8];
            float psum = 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                pv[j] = dead ? 0.f : exp2f(s[j] - mnew);
                psum += pv[j];
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
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) pv_mfma<T>(w.o[qi][dt], pv, vf[dt]);
        }
    }
}

template <typename T>
__global__ __launch_bounds__(ATT_THREADS) void attn_partial_kernel(const AttnArgs a) {
    constexpr int D = WaveAttn<T>::D, DT = WaveAttn<T>::DT, STEP = Elem<T>::STEP;
    extern __shared__ __align__(16) unsigned char smem[];
    const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    int len = a.len[b];
    len = len < 0 ? 0 : (len > a.cap ? a.cap : len);
    const int nch = 1 + (len + a.chunk - 1) / a.chunk;
    if (c >= nch) return;

    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, g = lane >> 4, r = lane & 15;
    const int qgi = wv / a.kg, kgi = wv % a.kg;
    const bool active_wave = wv < a.qg * a.kg;
    const int rows = a.group * a.gamma;
    const int nqt_all = (rows + 15) >> 4;
    const int qt0 = qgi * 4;
    const int nqt = active_wave ? max(0, min(4, nqt_all - qt0)) : 0;

    WaveAttn<T> w;
    constexpr int PER = Elem<T>::PER16;
    const T* qn = reinterpret_cast<const T*>(a.q_norm);
    const T* kn = reinterpret_cast<const T*>(a.k_norm);
    const int G = a.gamma;
#pragma unroll
    for (int qi = 0; qi < 4; ++qi) {
        // query row R = hq*gamma + j of q head (h*group + hq) at block position j
        const int R = (qt0 + qi) * 16 + r;
        const bool valid = qi < nqt && R < rows;
        const int hq = valid ? R / G : 0, j = valid ? R % G : 0;
        float x[4][PER];
        load_row_raw<T>(x, a.qkv + (long long)(b * G + j) * a.qkv_ld + (h * a.group + hq) * D, valid);
        int pos = len + j;
        pos = pos < a.rope_rows ? pos : a.rope_rows - 1;
        norm_rope_frag<T>(w.qf[qi], x, qn, a.eps, a.rope_cos + (long long)pos * (D / 2),
                          a.rope_sin + (long long)pos * (D / 2));
        if (!valid) zero_frag64(w.qf[qi]);
        w.m[qi] = -INFINITY;
        w.l[qi] = 0.f;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) w.o[qi][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    if (c == 0) {
        // the block's own keys/values, from the raw projections (k: norm + RoPE; v: rounded)
        if (nqt > 0 && kgi == 0) {
            Frag64 kf[2];
            float vf[DT][8];
            const float* kraw = a.qkv + (long long)(b * G) * a.qkv_ld + (a.n_q + h) * D;
            const float* vraw = a.qkv + (long long)(b * G) * a.qkv_ld + (a.n_q + a.n_kv + h) * D;
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int key = (r >> 2) * 8 + t * 4 + (r & 3);
                const bool valid = key < G;
                float x[4][PER];
                load_row_raw<T>(x, kraw + (long long)(valid ? key : 0) * a.qkv_ld, valid);
                int pos = len + (valid ? key : 0);
                pos = pos < a.rope_rows ? pos : a.rope_rows - 1;
                norm_rope_frag<T>(kf[t], x, kn, a.eps, a.rope_cos + (long long)pos * (D / 2),
                                  a.rope_sin + (long long)pos * (D / 2));
            }
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int jj = 0; jj < 8; ++jj) {
                    const int key = g * 8 + jj;
                    const float v = vraw[(long long)(key < G ? key : 0) * a.qkv_ld + dt * 16 + r];
                    vf[dt][jj] = key < G ? Elem<T>::rho(v) : 0.f;
                }
            attn_subblock<T>(w, nqt, G, a.scale_log2, kf, vf);
        }
    } else if (nqt > 0) {
        const int per_wave = a.chunk / a.kg;
        const int k_lo = (c - 1) * a.chunk + kgi * per_wave;
        const int k_hi = min(k_lo + per_wave, len);
        const T* kc = reinterpret_cast<const T*>(a.kcache) + ((long long)b * a.n_kv + h) * (long long)a.cap * D;
        const T* vc = reinterpret_cast<const T*>(a.vcache) + ((long long)b * a.n_kv + h) * (long long)D * a.cap;
        for (int kb = k_lo; kb < k_hi; kb += 32) {
            const int nvalid = min(32, k_hi - kb);
            Frag64 kf[2];
            float vf[DT][8];
            load_ctx_frags<T>(kf, vf, kc, vc, a.cap, kb, nvalid);
            attn_subblock<T>(w, nqt, nvalid, a.scale_log2, kf, vf);
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

static inline size_t attn_lds_bytes_host(int elem_bytes, int qg, int kg) {
    (void)qg;
    const int D = 256 / elem_bytes, DT = D / 16;
    const int slot_floats = 4 * DT * 64 * 4 + 2 * 4 * 4 * 64;
    return kg >= 2 ? (size_t)slot_floats * sizeof(float) : 0;
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

template <typename T>
__global__ __launch_bounds__(64) void attn_merge_kernel(const MergeArgs a) {
    // blockIdx.x = row (b*gamma + j), blockIdx.y = q head; one wavefront
    __shared__ float wts[MERGE_MAX_CHUNKS];
    const int m = blockIdx.x, hq_all = blockIdx.y;
    const int b = m / a.gamma, j = m % a.gamma;
    const int h = hq_all / a.group, hq = hq_all % a.group;
    const int R = hq * a.gamma + j;
    const int D = a.head_dim;
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
    for (int d = lane; d < D; d += 64) {
        float num = 0.f;
        int c = 0;
        for (; c + 4 <= nch; c += 4) {
            const float o0 = a.opart[((base + c) * a.rpad + R) * D + d];
            const float o1 = a.opart[((base + c + 1) * a.rpad + R) * D + d];
            const float o2 = a.opart[((base + c + 2) * a.rpad + R) * D + d];
            const float o3 = a.opart[((base + c + 3) * a.rpad + R) * D + d];
            num += wts[c] * o0;
            num += wts[c + 1] * o1;
            num += wts[c + 2] * o2;
            num += wts[c + 3] * o3;
        }
        for (; c < nch; ++c) num += wts[c] * a.opart[((base + c) * a.rpad + R) * D + d];
        reinterpret_cast<T*>(a.out)[(long long)m * (gridDim.y * D) + (long long)hq_all * D + d] =
            Elem<T>::from_f(num / den);
    }
}

}  // namespace dflash
