// Block attention over [injected context ; block] for one draft layer.
//
// Per (sequence b, kv head h) the queries are the g*gamma rows (g q-heads of
// the group x gamma block positions), row R = hq*gamma + j.  Keys/values are
// the len[b] cached context rows followed by the gamma block rows; there is no
// mask inside the block and the whole context is visible (bidirectional).
//
// Work split ("split-K" over keys): chunk 0 of each (b,h) holds the block
// rows, chunks 1.. hold CH context rows each.  A workgroup takes one chunk and
// up to 8 query tiles of 16 rows; it has KG waves per query tile, which split
// the chunk's keys.  A wave owns one query tile:
//  * it builds the tile's q fragments itself (per-head RMSNorm + RoPE);
//  * the waves of a key group stream their keys through an LDS ring of 32-key
//    sub-blocks (direct-to-LDS loads of whole 1 KB spans, each byte fetched
//    once per workgroup; the ring holds a whole 256-key chunk, so the chunk is
//    requested at once) and every wave computes from LDS:
//      S^T = K . Q^T    (A = key rows, B = queries)
//    with the key rows permuted so that every lane ends up holding 8
//    consecutive keys of one query - exactly the B-operand layout of
//      O^T += V^T . P^T (A = V^T rows of the V cache, stored as 32-key blocks of V^T),
//    whose result leaves every lane with output columns of the same query as its
//    scores, so the online-softmax rescaling needs no data exchange;
//  * online softmax in base 2 (log2(e)/sqrt(D) folded into the scale); for
//    bf16 the PV product takes P rounded to bf16.
// Chunk 0's workgroup first builds the block's keys (k RMSNorm + RoPE) and
// values (rounded, transposed) in LDS; for a verifying target it also copies
// them into the cache at positions len .. len + gamma - 1 (len is not changed).  The KG waves of a tile merge through
// LDS (all tiles at once); the workgroup writes (m, l, O) per chunk and
// attn_merge combines the chunks with log-sum-exp weights in fixed chunk order.
#pragma once

#include "common.hpp"

namespace dflash {

// V cache in blocks of 32 keys: the values of keys 32 i .. 32 i + 31 are stored transposed
// and contiguous, [D][32], so one 32-key sub-block of V^T is one 8 KB span (bf16).
constexpr int VBLK = 32;
__host__ __device__ __forceinline__ long long vblk_offset(int pos, int d, int D) {
    return (long long)(pos / VBLK) * (D * VBLK) + d * VBLK + pos % VBLK;
}

struct AttnArgs {
    const void* kcache;     // this layer: T [Bmax][n_kv][cap][D]
    const void* vcache;     // this layer: T [Bmax][n_kv][cap / 32][D][32] (32-key blocks of V^T)
    const float* qkv;       // raw projections fp32 [B*gamma][qkv_ld]: q heads, then k heads, then v heads
    int qkv_ld;
    const void* q_norm;     // T [D]
    const void* k_norm;     // T [D]
    const float* rope_cos;  // [rope_rows][D/2]
    const float* rope_sin;
    int rope_rows;
    float eps;
    const int* len;         // [B]
    void* opart;            // T [B][n_kv][nch_max][rpad][D]: unnormalised O of each chunk, storage type
    float* mlpart;          // [B][n_kv][nch_max][rpad][2]  (m in log2 units, l)
    int n_q, n_kv, cap, rpad, nch_max, chunk;   // chunk = CH context keys per chunk
    int gamma, group;       // rows = group * gamma
    int nqs;                // workgroups per (b, h, chunk): query tiles split in groups of QTW
    float scale_log2;       // log2(e) / sqrt(D)
    int causal;             // block keys after a query's own position are masked (a verifying target)
    void* kwrite;           // nullable: this layer's K cache, where the block's keys are kept at len ..
    void* vwrite;           // ... and its V^T cache (a verifying target); nothing is written when null
    unsigned* status;       // sticky error bits (with kwrite: len < 0, len + gamma beyond the cache)
    int kv_nt;              // load the context K/V with the non-temporal hint
};

// Per-wave attention state for one query tile.
template <typename T>
struct WaveAttn {
    static constexpr int D = 256 / (int)sizeof(T);   // head_dim (one k-step)
    static constexpr int DT = D / 16;                 // d tiles
    Frag64 qf;            // B operand: lane (g,r) holds query r
    float m, l;           // running max (log2 units) of query r; this lane's share of its sum
    f32x4_t o[DT];        // O^T[d = dt*16 + g*4 + v][q = r]
};

// 8 consecutive keys of one V^T row (d fixed): the MFMA B operand of O += P.V.
template <typename T> struct VFrag;
template <> struct VFrag<bf16_t> { u32x4_t q; };        // 8 bf16
template <> struct VFrag<float> { u32x4_t q[2]; };      // 8 f32

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

// P of one lane (8 consecutive keys of one query) as the MFMA B operand: bf16 (the
// rounding of P the precision contract allows in the attention product; V is bf16-exact
// already), or fp32 for fp32 storage.  Splitting P into two bf16 parts (hi + lo, two
// MFMAs) keeps ~16 bits but measured a third slower in the sub-block loop, which the
// matrix core bounds at the Qwen3-8B shape, and does not change how far the bf16
// forward can agree with an fp64 one (the roundings of the later stages dominate).
template <typename T> struct PFrag;
template <> struct PFrag<bf16_t> { u32x4_t q; };
template <> struct PFrag<float> { float p[8]; };

__device__ __forceinline__ void make_pfrag(PFrag<bf16_t>& f, const float (&p)[8]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) f.q[j] = pack2_bf16(p[2 * j], p[2 * j + 1]);
}

__device__ __forceinline__ void make_pfrag(PFrag<float>& f, const float (&p)[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) f.p[j] = p[j];
}

// acc[d][q] += V^T(16 d, 8 keys of this lane group) . P^T(8 keys, q)
__device__ __forceinline__ void pv_mfma(f32x4_t& acc, const PFrag<bf16_t>& p, const VFrag<bf16_t>& v) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(v.q), as_bf16x8(p.q), acc, 0, 0, 0);
}

__device__ __forceinline__ void pv_mfma(f32x4_t& acc, const PFrag<float>& p, const VFrag<float>& v) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(v.q[j >> 2][j & 3]), p.p[j], acc, 0, 0, 0);
}

// A head row as held by one lane in the fragment layout: piece i (0..3) holds
// elements d = 4*PER*i + PER*g + j (j < PER, PER = 16 bytes / element size).
// Rotate-half RoPE pairs d with d + D/2, i.e. piece i with piece i + 2 of the
// same lane; the four lanes of a row (g = 0..3) are 16 lanes apart.
//
// RowIn holds what one lane needs to build its pieces of a normalised, rotated
// row: the raw fp32 values, the norm scale and the cos/sin of its position.  A query
// row's raw values are issued as opaque loads (row_in_issue_x) and waited for
// explicitly, so that they can be in flight together with the K/V stream; its norm
// scale and cos/sin come from rows staged once per workgroup (row_in_aux).
template <typename T>
struct RowIn {
    static constexpr int PER = Elem<T>::PER16, F4 = PER / 4;
    u32x4_t x[4 * F4];               // piece i, vector h -> x[i * F4 + h]
    Frag64 w;                        // norm scale
    u32x4_t c[2 * F4], s[2 * F4];    // cos / sin for pieces 0, 1 (paired with 2, 3)
};

template <typename T>
__device__ __forceinline__ void row_in_issue_x(RowIn<T>& in, const float* row) {
    constexpr int PER = RowIn<T>::PER, F4 = RowIn<T>::F4;
    const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int h = 0; h < F4; ++h) vload_b128(in.x[i * F4 + h], row + i * 4 * PER + g * PER + h * 4);
}

template <typename T>
__device__ __forceinline__ void row_in_tie_x(RowIn<T>& in) {
#pragma unroll
    for (int k = 0; k < 4 * RowIn<T>::F4; ++k) tie(in.x[k]);
}

// The same inputs read from rows staged in LDS (raw fp32 row, norm weight, cos and
// sin rows), with the lane layout of row_in_issue_x.
template <typename T>
__device__ __forceinline__ void row_in_lds(RowIn<T>& in, const unsigned char* row, const unsigned char* wn,
                                           const unsigned char* cosr, const unsigned char* sinr) {
    constexpr int PER = RowIn<T>::PER, F4 = RowIn<T>::F4;
    const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int h = 0; h < F4; ++h)
            in.x[i * F4 + h] = *reinterpret_cast<const u32x4_t*>(row + (i * 4 * PER + g * PER + h * 4) * 4);
#pragma unroll
    for (int i = 0; i < 4; ++i)
        in.w.q[i] = *reinterpret_cast<const u32x4_t*>(wn + (i * 4 * PER + g * PER) * (int)sizeof(T));
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int h = 0; h < F4; ++h) {
            in.c[i * F4 + h] = *reinterpret_cast<const u32x4_t*>(cosr + (i * 4 * PER + g * PER + h * 4) * 4);
            in.s[i * F4 + h] = *reinterpret_cast<const u32x4_t*>(sinr + (i * 4 * PER + g * PER + h * 4) * 4);
        }
}

// Per-head RMSNorm (over the D elements spread over the row's four lanes) then
// rotate-half RoPE, rounded to the storage type, into an MFMA fragment.
template <typename T>
__device__ __forceinline__ void norm_rope_frag(Frag64& out, const RowIn<T>& in, float eps) {
    constexpr int PER = RowIn<T>::PER, F4 = RowIn<T>::F4;
    constexpr int D = 16 * PER;
    float x[4][PER];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < PER; ++j) x[i][j] = __uint_as_float(in.x[i * F4 + j / 4][j % 4]);
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < PER; ++j) ss += x[i][j] * x[i][j];
    ss += __shfl_xor(ss, 16, WAVE);
    ss += __shfl_xor(ss, 32, WAVE);
    const float rs = 1.0f / sqrtf(ss / (float)D + eps);
    float y[4][PER];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const T* wp = reinterpret_cast<const T*>(&in.w.q[i]);
#pragma unroll
        for (int j = 0; j < PER; ++j) y[i][j] = x[i][j] * rs * Elem<T>::to_f(wp[j]);
    }
    float o[4][PER];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const float c = __uint_as_float(in.c[i * F4 + j / 4][j % 4]);
            const float sn = __uint_as_float(in.s[i * F4 + j / 4][j % 4]);
            o[i][j] = y[i][j] * c - y[i + 2][j] * sn;
            o[i + 2][j] = y[i + 2][j] * c + y[i][j] * sn;
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

// K tile of a sub-block in LDS: key row at key*256 B, 16-byte chunk c at
// position c ^ kswz(key); the 16 rows read by one fragment load hit 16
// different bank groups.
__device__ __forceinline__ int kswz(int key) { return ((key >> 1) & 12) | (key & 3); }
__device__ __forceinline__ int k_lds_off(int key, int c) { return key * 256 + ((c ^ kswz(key)) << 4); }

// V^T tile of a sub-block in LDS: row d holds the 32 keys (32 * element bytes);
// bf16 rows (64 B) put chunk c at position c ^ ((d >> 2) & 3), f32 rows are plain.
template <typename T> __device__ __forceinline__ int v_lds_off(int d, int c);
template <> __device__ __forceinline__ int v_lds_off<bf16_t>(int d, int c) { return d * 64 + ((c ^ ((d >> 2) & 3)) << 4); }
template <> __device__ __forceinline__ int v_lds_off<float>(int d, int c) { return d * 128 + (c << 4); }

// A chunk's unnormalised O in the storage type: four consecutive columns per store (8 bytes
// in bf16, each value rounded to nearest even by the packed hardware conversion, which keeps
// the kernel's register peak where it was), DPL consecutive columns per lane when merged.
typedef __bf16 bf16x2_hw __attribute__((ext_vector_type(2)));
typedef float f32x2_hw __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void store_o4(bf16_t* p, const f32x4_t& v) {
    const f32x2_hw a = {v[0], v[1]}, b = {v[2], v[3]};
    *reinterpret_cast<uint2*>(p) = make_uint2(__builtin_bit_cast(uint32_t, __builtin_convertvector(a, bf16x2_hw)),
                                              __builtin_bit_cast(uint32_t, __builtin_convertvector(b, bf16x2_hw)));
}
__device__ __forceinline__ void store_o4(float* p, const f32x4_t& v) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}
template <typename T, int DPL> __device__ __forceinline__ void load_o(float (&o)[DPL], const T* p);
template <> __device__ __forceinline__ void load_o<bf16_t, 2>(float (&o)[2], const bf16_t* p) {
    const uint32_t u = *reinterpret_cast<const uint32_t*>(p);
    o[0] = __uint_as_float(u << 16);
    o[1] = __uint_as_float(u & 0xFFFF0000u);
}
template <> __device__ __forceinline__ void load_o<float, 1>(float (&o)[1], const float* p) { o[0] = *p; }

constexpr int ATT_STAGE_BYTES = 16384;   // K (32 x 256 B) then V^T (8 KB)
constexpr int ATT_V_OFF = 8192;
// chunk 0 only (it streams no context): raw inputs of the block's keys and values
// staged behind stage 0
constexpr int ATT_RAW_K = 16384;         // 16 fp32 rows of D (at most 512 B each)
constexpr int ATT_RAW_V = 24576;
constexpr int ATT_RAW_COS = 32768;       // 16 rows of D / 2 fp32 (at most 256 B each)
constexpr int ATT_RAW_SIN = 36864;
constexpr int ATT_RAW_KN = 40960;        // k-norm weight (1 KB slot)

__device__ __forceinline__ void store_frag_lds(unsigned char* kt, int key, const Frag64& f) {
    const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4_t*>(kt + k_lds_off(key, 4 * i + g)) = f.q[i];
}

__device__ __forceinline__ void load_frag_lds(Frag64& f, const unsigned char* kt, int key) {
    const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) f.q[i] = *reinterpret_cast<const u32x4_t*>(kt + k_lds_off(key, 4 * i + g));
}

// Keys g*8 .. g*8+7 of V^T row d of a staged sub-block.
__device__ __forceinline__ void vfrag_lds(VFrag<bf16_t>& v, const unsigned char* vt, int d) {
    const int g = (threadIdx.x & 63) >> 4;
    v.q = *reinterpret_cast<const u32x4_t*>(vt + v_lds_off<bf16_t>(d, g));
}
__device__ __forceinline__ void vfrag_lds(VFrag<float>& v, const unsigned char* vt, int d) {
    const int g = (threadIdx.x & 63) >> 4;
    v.q[0] = *reinterpret_cast<const u32x4_t*>(vt + v_lds_off<float>(d, 2 * g));
    v.q[1] = *reinterpret_cast<const u32x4_t*>(vt + v_lds_off<float>(d, 2 * g + 1));
}

// Key of lane row r in S^T tile t of a 32-key sub-block: (r/4)*8 + t*4 + r%4,
// so that lane group g of the result holds keys g*8 .. g*8+7.
__device__ __forceinline__ int subblock_key(int t, int r) { return (r >> 2) * 8 + t * 4 + (r & 3); }

// One 32-key sub-block.  MASKED: only the first `nvalid` (>= 1) keys are real
// (the last sub-block of a sequence, and the block itself); their V entries are
// cleared (stale cache rows may hold any bits), and scores of keys at or past
// this lane's `klim` (<= nvalid, >= 1; = nvalid except for causal block rows) are -inf.
// Softmax in base 2 with the raw hardware exp2 (arguments are <= 0; results
// below the fp32 normal range flush to 0).  O is rescaled only when the running
// max of some query in the wave moved.
template <typename T, bool MASKED>
__device__ __forceinline__ void attn_subblock(WaveAttn<T>& w, int nvalid, int klim, float scale_log2,
                                              const Frag64 (&kf)[2], VFrag<T> (&vf)[WaveAttn<T>::DT]) {
    constexpr int DT = WaveAttn<T>::DT;
    const int g = (threadIdx.x & 63) >> 4;
    if constexpr (MASKED) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) vfrag_mask(vf[dt], nvalid - g * 8);
    }
    f32x4_t st[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        st[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        mfma_kstep<T>(st[t], kf[t], w.qf);
    }
    // lane holds S[q = r][key = g*8 + t*4 + v]
    float s[8];
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            float x = st[t][v] * scale_log2;
            if constexpr (MASKED) x = (g * 8 + t * 4 + v) < klim ? x : -INFINITY;
            s[t * 4 + v] = x;
            mx = fmaxf(mx, x);
        }
    mx = fmaxf(mx, __shfl_xor(mx, 16, WAVE));
    mx = fmaxf(mx, __shfl_xor(mx, 32, WAVE));
    const float mnew = fmaxf(w.m, mx);            // finite: some key of the sub-block is real
    const float alpha = __builtin_amdgcn_exp2f(w.m - mnew);
    float p[8];
    float psum = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        p[j] = __builtin_amdgcn_exp2f(s[j] - mnew);
        psum += p[j];
    }
    w.l = w.l * alpha + psum;
    if (__ballot(mnew != w.m)) {                  // wave-uniform
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) w.o[dt] *= alpha;
    }
    w.m = mnew;
    PFrag<T> pf;
    make_pfrag(pf, p);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) pv_mfma(w.o[dt], pf, vf[dt]);
}

// Direct-to-LDS loads of context keys [kb, kb+32) of one (b,h) into a stage:
// 8 instructions of 1 KB for K (rows beyond the real keys repeat the last real
// one; their scores are masked) and 8 for V^T (the 32-key block, one contiguous 8 KB span
// of the blocked V cache: kb + 32 <= cap; keys
// beyond the real ones are cleared at use).  Instruction j goes to the wave
// iw = j % NW of the key group: every wave issues exactly 16 / NW of them (with the
// non-temporal hint when nt).
template <typename T, int NW>
__device__ __forceinline__ void stage_issue(uint32_t stage, const T* kc, const T* vc, int cap, int kb, int nvalid,
                                            int iw, int nt) {
    constexpr int D = 256 / (int)sizeof(T), KPC = 16 / (int)sizeof(T);   // elements per 16 bytes
    constexpr int RB = 32 * (int)sizeof(T), CPR = RB / 16, RPI = 1024 / RB;
    const int lane = threadIdx.x & 63;
    static_assert(16 % NW == 0, "whole instructions per wave");
#pragma unroll
    for (int jj0 = 0; jj0 < 16 / NW; ++jj0) {
        const int j = jj0 * NW + iw;
        if (j < 8) {
            const int key = 4 * j + (lane >> 4);
            const int src = key < nvalid ? key : nvalid - 1;
            const int c = (lane & 15) ^ kswz(key);
            if (nt) dma_b128_nt(kc + (long long)(kb + src) * D + c * KPC, stage + j * 1024);
            else dma_b128(kc + (long long)(kb + src) * D + c * KPC, stage + j * 1024);
        } else {
            const int jj = j - 8;
            const int d = jj * RPI + lane / CPR, p = lane % CPR;
            const int c = sizeof(T) == 2 ? (p ^ ((d >> 2) & 3)) : p;
            if (nt) dma_b128_nt(vc + (long long)kb * D + d * VBLK + c * KPC, stage + ATT_V_OFF + jj * 1024);
            else dma_b128(vc + (long long)kb * D + d * VBLK + c * KPC, stage + ATT_V_OFF + jj * 1024);
        }
    }
}

// Geometry, by the number QTW of query tiles per workgroup (1, 2, 4 or 8), the ring
// size RING (stages of 16 KB per workgroup) and the number KG of waves per tile that
// split the chunk's keys (8 waves in all, 4 for QTW 1 and for the four-wave layout
// QTW 4 / KG 1); every key group owns a ring of RING / KG stages in LDS.  RING 8
// (128 KB) holds a whole 256-key chunk, for launches with fewer workgroups than CUs;
// RING 4 (64 KB) for launches with many (measured 2-4% faster there) and for the
// four-wave layout with 128-key chunks, where the ring holds the whole chunk and two
// workgroups share a CU.  Chunk 0 builds the block's keys and values in the first
// stage; afterwards the key-group merge reuses the space with one slot (O^T, m, l of
// a wave) per sending wave.
constexpr int ATT_MAX_TILES = 8;
constexpr int ATT_MAX_WAVES = 8;
__host__ __device__ constexpr int att_default_kg(int qtw) { return qtw >= 8 ? 1 : (qtw == 4 ? 2 : 4); }
template <int QTW, int RING, int KG_ = att_default_kg(QTW)> struct AttGeom {
    static constexpr int KG = KG_;
    static constexpr int WAVES = QTW * KG;
    static constexpr int R = RING / KG;         // ring stages per key group
    static constexpr int NPW = 16 / QTW;        // loads per wave per stage
    static_assert(R >= 1 && RING % KG == 0, "whole stages per key group");
    static_assert((R - 1) * NPW <= 63, "vmcnt range");
};
// Rows every workgroup of a launch shares, staged once per workgroup after the ring: the
// cos and sin rows of the block positions (row j = position len + j, D / 2 fp32; the
// 16-byte chunk c of row j sits at position c ^ (j mod chunks per row), so the 16 rows of
// one read hit different banks) and the q-norm weight (D elements).  Every wave of a
// workgroup loading them itself costs 12 more loads per lane of a query tile (~13 MB of L2
// reads per layer at the Qwen3-8B shape for 8.3 KB of distinct data).
constexpr int ATT_AUX_COS = 0, ATT_AUX_SIN = 4096, ATT_AUX_QN = 8192, ATT_AUX_BYTES = 9216;
__host__ __device__ constexpr int attn_aux_offset(int ring) {
    return ring * ATT_STAGE_BYTES > ATT_RAW_KN + 1024 ? ring * ATT_STAGE_BYTES : ATT_RAW_KN + 1024;
}

// LDS of a workgroup: the ring, which also holds chunk 0's staged inputs (up to
// ATT_RAW_KN + 1 KB) and the key-group merge slots (at most 4 of 8.5 KB), then the
// shared rows
static inline size_t attn_lds_bytes_host(int ring) { return (size_t)attn_aux_offset(ring) + ATT_AUX_BYTES; }

// Direct-to-LDS loads of the shared rows, round-robin over the waves: the 16 cos rows, the
// 16 sin rows (rows past the block repeat row 0's position; positions past the RoPE table
// read its last row), the q-norm weight (the lanes past its 16 chunks repeat them into the
// rest of its 1 KB slot).
template <typename T>
__device__ __forceinline__ void aux_stage_issue(uint32_t aux_lds, const float* cos_tab, const float* sin_tab,
                                                const void* qn, int len, int G, int rope_rows, int wv, int nw) {
    constexpr int D = 256 / (int)sizeof(T), CPR = D / 8;       // 16-byte chunks per cos row
    constexpr int RPI = 64 / CPR, NT = 16 / RPI;                // rows per 1 KB load, loads per table
    const int lane = threadIdx.x & 63;
    for (int ins = wv; ins < 2 * NT + 1; ins += nw) {
        const void* src;
        uint32_t dst;
        if (ins < 2 * NT) {
            const int k = ins % NT, j = k * RPI + lane / CPR, pp = lane % CPR;
            int pos = len + (j < G ? j : 0);
            pos = pos < rope_rows ? pos : rope_rows - 1;
            const int c = pp ^ (j & (CPR - 1));
            src = (ins < NT ? cos_tab : sin_tab) + (long long)pos * (D / 2) + c * 4;
            dst = aux_lds + (ins < NT ? ATT_AUX_COS : ATT_AUX_SIN) + k * 1024;
        } else {
            src = reinterpret_cast<const unsigned char*>(qn) + (lane & 15) * 16;
            dst = aux_lds + ATT_AUX_QN;
        }
        dma_b128(src, dst);
    }
}

// The norm weight and the cos / sin rows of block position j from the staged rows, with
// the lane layout of row_in_issue_x.
template <typename T>
__device__ __forceinline__ void row_in_aux(RowIn<T>& in, const unsigned char* aux, int j) {
    constexpr int PER = RowIn<T>::PER, F4 = RowIn<T>::F4, D = 16 * PER, CPR = D / 8;
    const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) in.w.q[i] = *reinterpret_cast<const u32x4_t*>(aux + ATT_AUX_QN + (i * 4 + g) * 16);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int h = 0; h < F4; ++h) {
            const int c = i * PER + g * (PER / 4) + h, pp = c ^ (j & (CPR - 1));
            in.c[i * F4 + h] = *reinterpret_cast<const u32x4_t*>(aux + ATT_AUX_COS + (j * CPR + pp) * 16);
            in.s[i * F4 + h] = *reinterpret_cast<const u32x4_t*>(aux + ATT_AUX_SIN + (j * CPR + pp) * 16);
        }
}

// Wait until at most `later` (<= MAXL) stages of NPW loads each, issued after the
// awaited loads, are still in flight.
template <int NPW, int MAXL>
__device__ __forceinline__ void wait_stage(int later) {
    static_assert(MAXL * NPW <= 63, "vmcnt range");
    switch (later) {
        case 0: vm_wait<0>(); break;
        case 1: vm_wait<(MAXL >= 1 ? NPW : 0)>(); break;
        case 2: vm_wait<(MAXL >= 2 ? 2 * NPW : 0)>(); break;
        case 3: vm_wait<(MAXL >= 3 ? 3 * NPW : 0)>(); break;
        case 4: vm_wait<(MAXL >= 4 ? 4 * NPW : 0)>(); break;
        case 5: vm_wait<(MAXL >= 5 ? 5 * NPW : 0)>(); break;
        case 6: vm_wait<(MAXL >= 6 ? 6 * NPW : 0)>(); break;
        case 7: vm_wait<(MAXL >= 7 ? 7 * NPW : 0)>(); break;
        default: vm_wait<(MAXL >= 8 ? 8 * NPW : 0)>(); break;
    }
}

template <typename T, int QTW, int RING, int KG_>
__global__ __launch_bounds__(64 * (RING == 8 ? QTW * KG_ : ATT_MAX_WAVES)) void attn_partial_kernel(const AttnArgs a) {
    constexpr int D = WaveAttn<T>::D, DT = WaveAttn<T>::DT, PER = Elem<T>::PER16;
    using Geo = AttGeom<QTW, RING, KG_>;
    constexpr int KG = Geo::KG, R = Geo::R, NPW = Geo::NPW;
    extern __shared__ __align__(16) unsigned char smem[];
    // workgroup -> (chunk c, kv head h, query group qs, sequence b).  With several query
    // groups per chunk the launch is taken chunk-major (context chunk 1 of every (b, h, qs),
    // then chunk 2, ..., the block chunk 0 last), so the workgroups that read one chunk run
    // side by side and the second finds it in the last-level cache: Coder-30B drafter shape,
    // batch 8, gamma 16, attention 958 -> 897 us per cycle.  Otherwise chunk-fastest (with
    // ragged contexts at batch 32 the chunk-major order measured 21 us per cycle slower).
    int c = blockIdx.x, y = blockIdx.y, b = blockIdx.z;
    if (a.nqs > 1) {
        const int nyz = gridDim.y * gridDim.z;
        const int lin = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
        const int cc = lin / nyz, yz = lin % nyz;
        c = cc + 1 < (int)gridDim.x ? cc + 1 : 0;
        y = yz % gridDim.y;
        b = yz / gridDim.y;
    }
    const int h = y / a.nqs, qs = y % a.nqs;
    int len = a.len[b];
    // a length outside the cache, or a block past the RoPE table, is reported (the reads
    // below are clamped into bounds; the drafts of that sequence are then meaningless)
    if (c == 0 && y == 0 && threadIdx.x == 0 && a.kwrite == nullptr) {
        if (len < 0) atomicOr(a.status, STATUS_BAD_COUNT);
        else if (len > a.cap || len + a.gamma > a.rope_rows) atomicOr(a.status, STATUS_KV_OVERFLOW);
    }
    len = len < 0 ? 0 : (len > a.cap ? a.cap : len);
    const int nch = 1 + (len + a.chunk - 1) / a.chunk;
    if (c >= nch) return;

    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, g = lane >> 4, r = lane & 15;
    const int G = a.gamma;
    const int rows = a.group * G;
    const int qt = qs * QTW + wv / KG;              // this wave's query tile
    const int kgi = wv % KG;
    const bool active = qt * 16 < rows;

    WaveAttn<T> w;
    w.m = -INFINITY;
    w.l = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) w.o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const T* kc = reinterpret_cast<const T*>(a.kcache) + ((long long)b * a.n_kv + h) * (long long)a.cap * D;
    const T* vc = reinterpret_cast<const T*>(a.vcache) + ((long long)b * a.n_kv + h) * (long long)D * a.cap;
    // this wave's context keys [k_lo, k_hi); empty for chunk 0 (the block).  Every
    // wave runs n_iter sub-block steps (the count of key group 0) for the barriers.
    const int per_wave = a.chunk / KG;
    const int c0 = (c - 1) * a.chunk;
    const int k_lo = c == 0 ? 0 : c0 + kgi * per_wave;
    const int k_hi = c == 0 ? 0 : min(k_lo + per_wave, len);
    const int n_iter = c == 0 ? 0 : (min(per_wave, len - c0) + 31) / 32;
    const int tl = __builtin_amdgcn_readfirstlane(wv / KG);     // tile within the workgroup (wave-uniform)
    const int kgi_u = __builtin_amdgcn_readfirstlane(kgi);
    unsigned char* kgbuf = smem + kgi_u * R * ATT_STAGE_BYTES;
    const uint32_t kgbuf_lds = lds_offset(smem) + (uint32_t)kgi_u * (R * ATT_STAGE_BYTES);

    // The tile's query inputs first; then, in chunk 0, the block's own raw key and
    // value rows, their RoPE rows and the k-norm weight straight into free LDS,
    // else the first R sub-blocks of K/V (the whole chunk at 256 keys): all a
    // workgroup reads before its first sub-block is in flight at once, and one wait
    // covers it.
    const int Rq = qt * 16 + r;
    const bool qvalid = Rq < rows;
    RowIn<T> qin;
    const int qj = qvalid ? Rq % G : 0;                 // the query row's block position
    if (active) {
        const int hq = qvalid ? Rq / G : 0;
        row_in_issue_x<T>(qin, a.qkv + (long long)(b * G + qj) * a.qkv_ld + (h * a.group + hq) * D);
    }
    const unsigned char* aux = smem + attn_aux_offset(RING);
    aux_stage_issue<T>(lds_offset(smem) + (uint32_t)attn_aux_offset(RING), a.rope_cos, a.rope_sin, a.q_norm, len, G,
                       a.rope_rows, __builtin_amdgcn_readfirstlane(wv), (int)(blockDim.x >> 6));
    if (c == 0) {
        // direct-to-LDS loads of 1 KB, round-robin over the waves: raw k rows, raw
        // v rows (fp32, D * 4 bytes each), cos and sin rows of the block positions
        // (D * 2 bytes each), the k-norm weight.  Rows beyond the block repeat row 0;
        // their keys are cleared below.
        constexpr int KRB = D * 4, KLPR = KRB / 16, KRPI = 64 / KLPR, KNI = 16 / KRPI;
        constexpr int CRB = D * 2, CLPR = CRB / 16, CRPI = 64 / CLPR, CNI = 16 / CRPI;
        constexpr int NI = 2 * KNI + 2 * CNI + 1;
        const int nw = blockDim.x >> 6;
        const int wv_u = __builtin_amdgcn_readfirstlane(wv);
        const uint32_t base = lds_offset(smem);
        for (int ins = wv_u; ins < NI; ins += nw) {
            const void* src;
            uint32_t dst;
            if (ins < 2 * KNI) {
                const int jj = ins % KNI, key = KRPI * jj + lane / KLPR;
                const int kk = key < G ? key : 0;
                const int col = ins < KNI ? (a.n_q + h) * D : (a.n_q + a.n_kv + h) * D;
                src = a.qkv + (long long)(b * G + kk) * a.qkv_ld + col + (lane % KLPR) * 4;
                dst = base + (ins < KNI ? ATT_RAW_K : ATT_RAW_V) + jj * 1024;
            } else if (ins < 2 * KNI + 2 * CNI) {
                const int ic = ins - 2 * KNI;
                const int jj = ic % CNI, key = CRPI * jj + lane / CLPR;
                int pos = len + (key < G ? key : 0);
                pos = pos < a.rope_rows ? pos : a.rope_rows - 1;
                src = (ic < CNI ? a.rope_cos : a.rope_sin) + (long long)pos * (D / 2) + (lane % CLPR) * 4;
                dst = base + (ic < CNI ? ATT_RAW_COS : ATT_RAW_SIN) + jj * 1024;
            } else {
                constexpr int WCH = D * (int)sizeof(T) / 16;      // 16-byte pieces of the weight
                src = reinterpret_cast<const unsigned char*>(a.k_norm) + (lane % WCH) * 16;
                dst = base + ATT_RAW_KN;
            }
            dma_b128(src, dst);
        }
    }
    int n_issued = 0;
#pragma unroll
    for (int st = 0; st < R; ++st) {
        const int kb = k_lo + 32 * st;
        if (kb < k_hi) {
            stage_issue<T, QTW>(kgbuf_lds + st * ATT_STAGE_BYTES, kc, vc, a.cap, kb, min(32, k_hi - kb), tl, a.kv_nt);
            ++n_issued;
        }
    }
    if (c == 0) {
        vm_wait<0>();                       // one latency for every input of chunk 0
        __syncthreads();                    // ... of every wave
        if (active) {
            row_in_tie_x(qin);
            row_in_aux<T>(qin, aux, qj);
            norm_rope_frag<T>(w.qf, qin, a.eps);
            if (!qvalid) zero_frag64(w.qf);
        }
        // the block's keys (wave 0: keys 0..15, k RMSNorm + RoPE; wave 1: keys 16..31,
        // never real since a block has at most 16 tokens) and values (rounded) into
        // stage 0 of key group 0
        if (wv < 2) {
            Frag64 f;
            zero_frag64(f);
            if (wv == 0) {
                RowIn<T> kin;
                row_in_lds<T>(kin, smem + ATT_RAW_K + r * (D * 4), smem + ATT_RAW_KN,
                              smem + ATT_RAW_COS + r * (D * 2), smem + ATT_RAW_SIN + r * (D * 2));
                norm_rope_frag<T>(f, kin, a.eps);
                if (r >= G) zero_frag64(f);
            }
            store_frag_lds(smem, wv * 16 + r, f);
        }
        constexpr int NV4 = 32 * D / 4, KPC = 16 / (int)sizeof(T);
        static_assert(NV4 % 256 == 0, "block V tile split");
        if (threadIdx.x < 256) {
#pragma unroll
            for (int it = 0; it < NV4 / 256; ++it) {
                const int e4 = it * 256 + threadIdx.x;
                const int key = e4 / (D / 4), d = (e4 % (D / 4)) * 4;
                const float4 vv = key < G ? *reinterpret_cast<const float4*>(smem + ATT_RAW_V + key * (D * 4) + d * 4)
                                          : make_float4(0.f, 0.f, 0.f, 0.f);
                const float vals[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    *reinterpret_cast<T*>(smem + ATT_V_OFF + v_lds_off<T>(d + u, key / KPC) +
                                          (key % KPC) * (int)sizeof(T)) = Elem<T>::from_f(vals[u]);
            }
        }
        __syncthreads();
        if (active && kgi == 0) {
            Frag64 kf[2];
            VFrag<T> vf[DT];
#pragma unroll
            for (int t = 0; t < 2; ++t) load_frag_lds(kf[t], smem, subblock_key(t, r));
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) vfrag_lds(vf[dt], smem + ATT_V_OFF, dt * 16 + r);
            // causal block rows: query row Rq is position Rq % G of the block and sees keys 0 .. Rq % G
            const int klim = (a.causal && qvalid) ? Rq % G + 1 : G;
            attn_subblock<T, true>(w, G, klim, a.scale_log2, kf, vf);
        }
        if (a.kwrite != nullptr && qs == 0) {
            // the block's keys and values as used above, into the cache (one workgroup per (b, h))
            const int raw = a.len[b];
            const bool bad = raw < 0;
            const bool over = !bad && (raw + G > a.cap || raw + G > a.rope_rows);
            if (h == 0 && threadIdx.x == 0) {
                if (bad) atomicOr(a.status, STATUS_BAD_COUNT);
                else if (over) atomicOr(a.status, STATUS_KV_OVERFLOW);
            }
            if (!bad && !over) {
                constexpr int KPC = 16 / (int)sizeof(T), CPR = D / KPC;     // 16-byte chunks per key row
                T* kw = reinterpret_cast<T*>(a.kwrite) + ((long long)b * a.n_kv + h) * (long long)a.cap * D;
                T* vw = reinterpret_cast<T*>(a.vwrite) + ((long long)b * a.n_kv + h) * (long long)D * a.cap;
                for (int e = threadIdx.x; e < G * CPR; e += blockDim.x) {
                    const int key = e / CPR, cc = e % CPR;
                    *reinterpret_cast<u32x4_t*>(kw + (long long)(raw + key) * D + cc * KPC) =
                        *reinterpret_cast<const u32x4_t*>(smem + k_lds_off(key, cc));
                }
                for (int e = threadIdx.x; e < D * G; e += blockDim.x) {
                    const int d = e / G, key = e % G;
                    vw[vblk_offset(raw + key, d, D)] = *reinterpret_cast<const T*>(
                        smem + ATT_V_OFF + v_lds_off<T>(d, key / KPC) + (key % KPC) * (int)sizeof(T));
                }
            }
        }
    } else {
        wait_stage<NPW, R>(n_issued);      // this wave's query row and shared-row loads came first
        __syncthreads();                   // ... and every wave's share of the shared rows
        if (active) {
            row_in_tie_x(qin);
            row_in_aux<T>(qin, aux, qj);
            norm_rope_frag<T>(w.qf, qin, a.eps);
            if (!qvalid) zero_frag64(w.qf);
        }
    }
    for (int it = 0; it < n_iter; ++it) {
        const int kb = k_lo + 32 * it;
        // this wave's loads of stage `it` have landed (loads complete in issue order;
        // the stages issued after it by this wave may still be in flight) ...
        const int later_kb_end = min(k_hi, k_lo + 32 * min(n_iter, it + R));
        wait_stage<NPW, R - 1>(max(0, (later_kb_end - kb - 1) / 32));
        __syncthreads();    // ... and every wave's
        if (active && kb < k_hi) {
            const unsigned char* st = kgbuf + (it % R) * ATT_STAGE_BYTES;
            Frag64 kf[2];
            VFrag<T> vf[DT];
#pragma unroll
            for (int t = 0; t < 2; ++t) load_frag_lds(kf[t], st, subblock_key(t, r));
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) vfrag_lds(vf[dt], st + ATT_V_OFF, dt * 16 + r);
            const int nvalid = __builtin_amdgcn_readfirstlane(min(32, k_hi - kb));
            if (nvalid < 32) attn_subblock<T, true>(w, nvalid, nvalid, a.scale_log2, kf, vf);
            else attn_subblock<T, false>(w, 32, 32, a.scale_log2, kf, vf);
        }
        if (it + R < n_iter) {          // refill this stage once every wave has read it
            __syncthreads();
            const int kbn = kb + 32 * R;
            if (kbn < k_hi)
                stage_issue<T, QTW>(kgbuf_lds + (it % R) * ATT_STAGE_BYTES, kc, vc, a.cap, kbn, min(32, k_hi - kbn), tl,
                                    a.kv_nt);
        }
    }

    // ---- l of query r summed over the 4 lane groups
    float lt = w.l;
    lt += __shfl_xor(lt, 16, WAVE);
    lt += __shfl_xor(lt, 32, WAVE);
    float mt = w.m;

    // ---- merge the KG waves of each tile (all tiles at once; pairwise rounds)
    constexpr int slot_bytes = DT * 4 * 64 * 4 + 2 * 64 * 4;
    static_assert(QTW * (KG / 2) * slot_bytes <= ATT_RAW_KN + 1024, "merge slots fit the smallest LDS size");
    for (int span = KG >> 1; span >= 1; span >>= 1) {
        __syncthreads();   // previous users of the LDS space are done
        if (kgi >= span && kgi < 2 * span) {
            float* sl = reinterpret_cast<float*>(smem + (tl * span + (kgi - span)) * slot_bytes);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int v = 0; v < 4; ++v) sl[(dt * 4 + v) * 64 + lane] = w.o[dt][v];
            sl[DT * 4 * 64 + lane] = mt;
            sl[DT * 4 * 64 + 64 + lane] = lt;
        }
        __syncthreads();
        if (kgi < span) {
            const float* sl = reinterpret_cast<const float*>(smem + (tl * span + kgi) * slot_bytes);
            const float m2 = sl[DT * 4 * 64 + lane];
            const float l2 = sl[DT * 4 * 64 + 64 + lane];
            const float mm = fmaxf(mt, m2);
            const float f1 = (mm == -INFINITY) ? 0.f : exp2f(mt - mm);
            const float f2 = (mm == -INFINITY) ? 0.f : exp2f(m2 - mm);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int v = 0; v < 4; ++v) w.o[dt][v] = w.o[dt][v] * f1 + sl[(dt * 4 + v) * 64 + lane] * f2;
            mt = mm;
            lt = lt * f1 + l2 * f2;
        }
    }

    // ---- key-group 0 of every tile writes the chunk's partial for its 16 rows
    if (active && kgi == 0) {
        const int R = qt * 16 + r;
        if (R < rows) {
            const long long row = (((long long)b * a.n_kv + h) * a.nch_max + c) * a.rpad + R;
            T* op = reinterpret_cast<T*>(a.opart) + row * D;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) store_o4(op + dt * 16 + g * 4, w.o[dt]);
            if (g == 0) *reinterpret_cast<float2*>(a.mlpart + row * 2) = make_float2(mt, lt);
        }
    }
}

// o[b*gamma + j][(h*g + hq)*D + d] = rho( sum_c w_c O_c / sum_c w_c l_c ),  w_c = 2^(m_c - max m)
struct MergeArgs {
    const void* opart;      // T, as AttnArgs::opart
    const float* mlpart;
    const int* len;
    void* out;              // T [B*gamma][n_q*D], or in fragment order (out_frag)
    int n_kv, group, gamma, rpad, nch_max, chunk, cap, head_dim;
    int out_frag;
};

constexpr int MERGE_MAX_CHUNKS = 1024;
constexpr int MERGE_BATCH = 16;   // chunk partials loaded together per lane
constexpr int MERGE_WAVES = 4;    // waves per output row and q head, each over a range of chunks

// Workgroup (row m = b*gamma + j, q head) of nw waves (1, or 4 when rows have more chunks
// than one batch): wave w folds the contiguous chunk range [w*per, (w+1)*per) (per =
// ceil(nch / nw)), loading every chunk's (m, l) and its lane's
// DPL columns of O in one batch, so one memory latency covers a range of up to
// MERGE_BATCH chunks; wave 0 then combines the (max, sum, O) triples in wave order.
// Every sum runs in a fixed order: the result is deterministic.
template <typename T>
__global__ __launch_bounds__(64 * MERGE_WAVES) void attn_merge_kernel(const MergeArgs a) {
    constexpr int D = 256 / (int)sizeof(T), DPL = D / 64;
    __shared__ float red_ml[MERGE_WAVES][2];
    __shared__ float red_o[MERGE_WAVES][DPL][64];
    const int m = blockIdx.x, hq_all = blockIdx.y;
    const int b = m / a.gamma, j = m % a.gamma;
    const int h = hq_all / a.group, hq = hq_all % a.group;
    const int R = hq * a.gamma + j;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;   // nw <= MERGE_WAVES
    int len = a.len[b];
    len = len < 0 ? 0 : (len > a.cap ? a.cap : len);
    const int nch = 1 + (len + a.chunk - 1) / a.chunk;
    const int per = (nch + nw - 1) / nw;
    const int c_lo = w * per, c_hi = min(nch, c_lo + per);
    const long long base = ((long long)b * a.n_kv + h) * a.nch_max;
    float mw = -INFINITY, lw = 0.f, ow[DPL];
#pragma unroll
    for (int k = 0; k < DPL; ++k) ow[k] = 0.f;
    for (int cb = c_lo; cb < c_hi; cb += MERGE_BATCH) {
        float mc[MERGE_BATCH], lc[MERGE_BATCH], oc[MERGE_BATCH][DPL];
#pragma unroll
        for (int u = 0; u < MERGE_BATCH; ++u) {
            const int c = min(cb + u, c_hi - 1);       // past the range: re-read the last chunk, unused
            const long long row = (base + c) * a.rpad + R;
            mc[u] = a.mlpart[row * 2];
            lc[u] = a.mlpart[row * 2 + 1];
            load_o<T, DPL>(oc[u], reinterpret_cast<const T*>(a.opart) + row * D + lane * DPL);
        }
        float mb = mw;
#pragma unroll
        for (int u = 0; u < MERGE_BATCH; ++u)
            if (cb + u < c_hi) mb = fmaxf(mb, mc[u]);
        const float sc = (mw == -INFINITY) ? 0.f : exp2f(mw - mb);
        lw *= sc;
#pragma unroll
        for (int k = 0; k < DPL; ++k) ow[k] *= sc;
#pragma unroll
        for (int u = 0; u < MERGE_BATCH; ++u) {
            if (cb + u < c_hi) {
                const float wc = (mc[u] == -INFINITY) ? 0.f : exp2f(mc[u] - mb);
                lw += wc * lc[u];
#pragma unroll
                for (int k = 0; k < DPL; ++k) ow[k] += wc * oc[u][k];
            }
        }
        mw = mb;
    }
    if (lane == 0) {
        red_ml[w][0] = mw;
        red_ml[w][1] = lw;
    }
#pragma unroll
    for (int k = 0; k < DPL; ++k) red_o[w][k][lane] = ow[k];
    __syncthreads();
    if (w != 0) return;
    float mx = -INFINITY;
    for (int v = 0; v < nw; ++v) mx = fmaxf(mx, red_ml[v][0]);
    float den = 0.f, num[DPL];
#pragma unroll
    for (int k = 0; k < DPL; ++k) num[k] = 0.f;
    for (int v = 0; v < nw; ++v) {
        const float mv = red_ml[v][0];
        const float f = (mv == -INFINITY) ? 0.f : exp2f(mv - mx);
        den += f * red_ml[v][1];
#pragma unroll
        for (int k = 0; k < DPL; ++k) num[k] += f * red_o[v][k][lane];
    }
    T* out = reinterpret_cast<T*>(a.out);
    const int ncol = gridDim.y * D, col = hq_all * D + lane * DPL;
#pragma unroll
    for (int k = 0; k < DPL; ++k)
        out[a.out_frag ? afrag_offset<T>(m, col + k, ncol) : (long long)m * ncol + col + k] = Elem<T>::from_f(num[k] / den);
}

}  // namespace dflash
