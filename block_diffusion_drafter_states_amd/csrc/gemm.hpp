// Weight-streaming GEMM for few rows (M <= 64 per workgroup): out = A . W^T.
//
// Used for every projection of the drafter (W_fuse, W_k|W_v injection,
// W_q|W_k|W_v, W_o, W_gate|W_up, W_down, LM head).  The weights are the
// dominant HBM traffic; each weight byte is read exactly once per launch.
//
// Workgroup = 4 wavefronts, output tile = 128 weight rows (columns of out) x
// up to 64 rows of A, over a K range [k0, k0 + kw) ("split").
//  * W: each wave owns 32 weight rows (2 MFMA n-tiles) and streams them from
//    HBM straight into registers with 16-byte loads, 4 k-steps in flight.
//  * A: staged through LDS one k-step at a time, double-buffered.  The
//    optional prologue applies RMSNorm on load (x * rstd * w, rounded to the
//    storage type), with rstd taken from per-tile partial sums of squares
//    written by the kernel that produced x.
//  * Split-K partials go to a workspace; the last workgroup of a tile (atomic
//    counter, self-resetting) sums them in split order (deterministic) and
//    runs the fused epilogue.
#pragma once

#include "common.hpp"

namespace dflash {

enum { A_PLAIN = 0, A_NORM = 1 };
enum { EPI_STORE = 0, EPI_QKV = 1, EPI_SWIGLU = 2, EPI_ARGMAX = 3, EPI_KV_INJECT = 4 };

constexpr int GEMM_THREADS = 256;
constexpr int GEMM_TILE_N = 128;   // weight rows per workgroup
constexpr int GEMM_MAX_M = 64;     // A rows per workgroup
constexpr int GEMM_NT = 2;         // MFMA n-tiles per wave
constexpr int GEMM_RING = 4;       // k-steps of W in flight per wave
constexpr int MAX_LAYERS = 16;

struct GemmLayer {
    const void* w[3];       // weight segments (concatenated along N)
    const void* norm_w;     // A_NORM scale [K]
    const void* head_norm;  // EPI_QKV / EPI_KV_INJECT: per-head RMSNorm scale [D] (q for seg 0, k for seg 1)
    const void* head_norm2; // EPI_QKV: k_norm (segment 1)
    void* kcache;           // EPI_KV_INJECT: this layer's K cache [Bmax][n_kv][cap][D]
    void* vcache;           // EPI_KV_INJECT: this layer's V cache [Bmax][n_kv][D][cap]
};

struct GemmArgs {
    // ---- A operand
    int a_mode;
    const void* a;          // T [M][lda] (A_PLAIN) or float [M][lda] (A_NORM)
    long long lda;
    const float* ssq;       // A_NORM: [n_ssq][ssq_ld] partial sums of squares of each row
    int n_ssq;
    int ssq_ld;
    float eps;
    int M;
    int K;
    // ---- W operand
    int seg_n[3];           // rows per segment (each a multiple of GEMM_TILE_N, except the last may be ragged)
    int n_seg;
    int N;                  // total weight rows (sum of seg_n)
    int n_tiles;            // tiles along N
    int n_mgroups;          // ceil(M / 64)
    int n_layers;           // grid layers (EPI_KV_INJECT), else 1
    GemmLayer layer[MAX_LAYERS];
    // ---- split-K
    int S;                  // splits
    int kw;                 // K per split (multiple of the A chunk)
    float* partial;         // [layers][S][M][N] fp32
    unsigned* counters;     // [layers][mgroups][tiles] + 1 global (self-resetting)
    // ---- epilogue
    float* out;             // EPI_STORE: [M][ldo] fp32 (residual added when `residual`)
    int ldo;
    int residual;
    float* ssq_out;         // EPI_STORE: [n_tiles][ssq_out_ld]
    int ssq_out_ld;
    void* out_t;            // EPI_SWIGLU: T [M][ldo]
    // attention inputs (EPI_QKV)
    void* qbuf;             // T [B][n_kv][rpad][D]
    void* kblk;             // T [B][n_kv][32][D]
    void* vblk;             // T [B][n_kv][D][32]
    int rpad;
    int gamma;              // rows per sequence in A (block size, or rows_stride for injection)
    int n_q, n_kv, head_dim, cap;
    const int* len;         // [B]
    const int* n_new;       // EPI_KV_INJECT: [B]
    const float* rope_cos;
    const float* rope_sin;
    int rope_rows;
    unsigned* status;
    // EPI_ARGMAX
    unsigned long long* slots;  // [B][gamma-1]
    int* draft;                 // [B][gamma-1]
    float* dbg_logits;          // nullable [B][gamma-1][N]
    int batch;
};

// Threads per A chunk unit: one unit = 8 elements of one row.
template <typename T>
struct AChunk {
    static constexpr int STEP = Elem<T>::STEP;
    static constexpr int KC = STEP;                     // elements per chunk (one k-step)
    static constexpr int PADE = 16 / (int)sizeof(T);    // row padding (16 bytes)
    static constexpr int LDS_LD = KC + PADE;            // LDS row stride (elements)
    static constexpr int UNITS_PER_ROW = KC / 8;
    static constexpr int MAX_UNITS = GEMM_MAX_M * UNITS_PER_ROW / GEMM_THREADS;  // per thread
};

static inline size_t gemm_lds_bytes_host(int elem_bytes, int mpad) {
    const int step = elem_bytes == 2 ? 128 : 64;
    const int kc = step;
    const int ld = kc + 16 / elem_bytes;
    size_t a = 2ull * mpad * ld * elem_bytes;
    size_t c = (size_t)mpad * GEMM_TILE_N * sizeof(float);
    return a > c ? a : c;
}

// Load (and optionally normalise) one A chunk into registers.
template <typename T>
struct AStage {
    float v[AChunk<T>::MAX_UNITS][8];
};

template <typename T>
__device__ __forceinline__ void load8(float (&v)[8], const T* p);
template <>
__device__ __forceinline__ void load8<bf16_t>(float (&v)[8], const bf16_t* p) {
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        v[2 * j] = __uint_as_float(w[j] << 16);
        v[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
    }
}
template <>
__device__ __forceinline__ void load8<float>(float (&v)[8], const float* p) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

template <typename T>
__device__ __forceinline__ void store8(T* p, const float (&v)[8]);
template <>
__device__ __forceinline__ void store8<bf16_t>(bf16_t* p, const float (&v)[8]) {
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = (uint32_t)f32_to_bf16(v[2 * j]) | ((uint32_t)f32_to_bf16(v[2 * j + 1]) << 16);
    *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
}
template <>
__device__ __forceinline__ void store8<float>(float* p, const float (&v)[8]) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}

template <typename T>
__device__ __forceinline__ void a_fetch(AStage<T>& st, const GemmArgs& p, const GemmLayer& L, int m0,
                                        int mpad, int kbase, const float* rstd_s) {
    constexpr int UPR = AChunk<T>::UNITS_PER_ROW;
    const int units = mpad * UPR;
#pragma unroll
    for (int i = 0; i < AChunk<T>::MAX_UNITS; ++i) {
        const int u = threadIdx.x + i * GEMM_THREADS;
        if (u < units) {
            const int row = u / UPR, c8 = u % UPR;
            const int m = m0 + row;
            const int k = kbase + c8 * 8;
            if (m < p.M) {
                if (p.a_mode == A_NORM) {
                    float xv[8], wv[8];
                    load8<float>(xv, reinterpret_cast<const float*>(p.a) + (long long)m * p.lda + k);
                    load8<T>(wv, reinterpret_cast<const T*>(L.norm_w) + k);
                    const float rs = rstd_s[row];
#pragma unroll
                    for (int j = 0; j < 8; ++j) st.v[i][j] = Elem<T>::rho(xv[j] * rs * wv[j]);
                } else {
                    load8<T>(st.v[i], reinterpret_cast<const T*>(p.a) + (long long)m * p.lda + k);
                }
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j) st.v[i][j] = 0.f;
            }
        }
    }
}

template <typename T>
__device__ __forceinline__ void a_store(const AStage<T>& st, T* buf, int mpad) {
    constexpr int UPR = AChunk<T>::UNITS_PER_ROW;
    const int units = mpad * UPR;
#pragma unroll
    for (int i = 0; i < AChunk<T>::MAX_UNITS; ++i) {
        const int u = threadIdx.x + i * GEMM_THREADS;
        if (u < units) {
            const int row = u / UPR, c8 = u % UPR;
            store8<T>(buf + row * AChunk<T>::LDS_LD + c8 * 8, st.v[i]);
        }
    }
}

// Weight-row mapping of lane (wave wv, n-tile t, lane row r) inside a tile.
template <int EPI>
__device__ __forceinline__ int tile_row(int wv, int t, int r) {
    if (EPI == EPI_SWIGLU) {
        // waves 0,1 -> gate rows [0,64), waves 2,3 -> up rows [0,64) of the output tile
        return (wv & 1) * 32 + t * 16 + r;
    }
    return wv * 32 + t * 16 + r;
}

template <typename T, int EPI>
__device__ void gemm_epilogue(const GemmArgs& p, const GemmLayer& L, int layer, int tile, int m0,
                              int mrows, const float* Ct);

// --------------------------------------------------------------------------------------------
template <typename T, int EPI>
__global__ __launch_bounds__(GEMM_THREADS) void gemm_kernel(const GemmArgs p) {
    constexpr int STEP = Elem<T>::STEP;
    constexpr int LDA = AChunk<T>::LDS_LD;
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ float rstd_s[GEMM_MAX_M];
    __shared__ int last_flag;

    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, g = lane >> 4, r = lane & 15;

    // ---- work decode: blockIdx.x = 8*j + xcd; the S splits of one tile share an XCD.
    const int S = p.S;
    const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
    const int tile = (j / S) * 8 + xcd, split = j % S;
    if (tile >= p.n_tiles) return;
    const int mg = blockIdx.y;
    const int layer = blockIdx.z;
    const GemmLayer& L = p.layer[layer];
    const int m0 = mg * GEMM_MAX_M;
    const int mrows = min(GEMM_MAX_M, p.M - m0);
    const int mt_n = (mrows + 15) >> 4;
    const int mpad = mt_n * 16;

    const int K = p.K;
    const int k0 = split * p.kw;
    const int k1 = min(K, k0 + p.kw);
    const int nsteps = (k1 - k0) / STEP;

    // ---- segment of this tile (tiles never straddle segments)
    int seg = 0, seg_row0 = 0;
    {
        int n_out0 = (EPI == EPI_SWIGLU) ? tile * 64 : tile * GEMM_TILE_N;
        int acc = 0;
        for (int s = 0; s < p.n_seg; ++s) {
            const int span = p.seg_n[s];
            if (n_out0 < acc + span || s == p.n_seg - 1) { seg = s; seg_row0 = n_out0 - acc; break; }
            acc += span;
        }
    }

    // ---- weight row pointers
    const T* wrow[GEMM_NT];
#pragma unroll
    for (int t = 0; t < GEMM_NT; ++t) {
        int row;
        const T* base;
        int seg_rows;
        if (EPI == EPI_SWIGLU) {
            const int s = (wv < 2) ? 0 : 1;    // gate, up
            base = reinterpret_cast<const T*>(L.w[s]);
            seg_rows = p.seg_n[0];
            row = tile * 64 + tile_row<EPI>(wv, t, r);
        } else {
            base = reinterpret_cast<const T*>(L.w[seg]);
            seg_rows = p.seg_n[seg];
            row = seg_row0 + tile_row<EPI>(wv, t, r);
        }
        row = min(row, seg_rows - 1);   // ragged last tile: re-read a valid row, result discarded
        wrow[t] = base + (long long)row * K + k0 + g * (STEP / 4);
    }

    // ---- rstd for the normalised prologue (fixed summation order over the partial tiles)
    if (p.a_mode == A_NORM) {
        for (int row = threadIdx.x; row < mpad; row += GEMM_THREADS) {
            const int m = m0 + row;
            float s = 0.f;
            if (m < p.M)
                for (int t = 0; t < p.n_ssq; ++t) s += p.ssq[(long long)t * p.ssq_ld + m];
            rstd_s[row] = 1.0f / sqrtf(s / (float)K + p.eps);
        }
        __syncthreads();
    }

    // ---- prologue: W ring, A chunk 0
    Frag64 wreg[GEMM_RING][GEMM_NT];
#pragma unroll
    for (int q = 0; q < GEMM_RING; ++q)
        if (q < nsteps)
#pragma unroll
            for (int t = 0; t < GEMM_NT; ++t) load_frag64(wreg[q][t], wrow[t] + q * STEP);

    T* As = reinterpret_cast<T*>(smem);
    AStage<T> st;
    a_fetch<T>(st, p, L, m0, mpad, k0, rstd_s);
    a_store<T>(st, As, mpad);
    __syncthreads();

    f32x4_t acc[4][GEMM_NT];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int t = 0; t < GEMM_NT; ++t) acc[mt][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    for (int s0 = 0; s0 < nsteps; s0 += GEMM_RING) {
#pragma unroll
        for (int q = 0; q < GEMM_RING; ++q) {
            const int step = s0 + q;
            if (step < nsteps) {
                const bool more = step + 1 < nsteps;
                if (more) a_fetch<T>(st, p, L, m0, mpad, k0 + (step + 1) * STEP, rstd_s);
                const T* Ab = As + (step & 1) * mpad * LDA;
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    if (mt < mt_n) {
                        Frag64 af;
                        const T* ap = Ab + (mt * 16 + r) * LDA + g * (STEP / 4);
#pragma unroll
                        for (int i = 0; i < 4; ++i) af.q[i] = *reinterpret_cast<const uint4*>(ap + i * (STEP / 16));
#pragma unroll
                        for (int t = 0; t < GEMM_NT; ++t) mfma_kstep<T>(acc[mt][t], af, wreg[q][t]);
                    }
                }
                if (step + GEMM_RING < nsteps)
#pragma unroll
                    for (int t = 0; t < GEMM_NT; ++t)
                        load_frag64(wreg[q][t], wrow[t] + (step + GEMM_RING) * STEP);
                if (more) a_store<T>(st, As + ((step + 1) & 1) * mpad * LDA, mpad);
                __syncthreads();
            }
        }
    }

    // ---- combine splits
    float* Ct = reinterpret_cast<float*>(smem);   // [mpad][128]
    const int N = p.N;
    if (S == 1) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
            if (mt < mt_n)
#pragma unroll
                for (int t = 0; t < GEMM_NT; ++t)
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        Ct[(mt * 16 + g * 4 + v) * GEMM_TILE_N + wv * 32 + t * 16 + r] = acc[mt][t][v];
        __syncthreads();
    } else {
        // partial[layer][split][m][n_tile_col]: tile-major so one tile's slab is contiguous
        const long long slab = (long long)p.M * GEMM_TILE_N;
        float* part = p.partial + ((long long)layer * p.n_tiles + (long long)tile) * S * slab;
        float* mine = part + (long long)split * slab;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
            if (mt < mt_n)
#pragma unroll
                for (int t = 0; t < GEMM_NT; ++t)
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const int row = mt * 16 + g * 4 + v;
                        if (m0 + row < p.M)
                            mine[(long long)(m0 + row) * GEMM_TILE_N + wv * 32 + t * 16 + r] = acc[mt][t][v];
                    }
        __threadfence();
        __syncthreads();
        unsigned* ctr = p.counters + ((long long)layer * p.n_mgroups + mg) * p.n_tiles + tile;
        if (threadIdx.x == 0) {
            const unsigned prev = atomicAdd(ctr, 1u);
            last_flag = (prev == (unsigned)(S - 1));
        }
        __syncthreads();
        if (!last_flag) return;
        __threadfence();
        for (int e = threadIdx.x; e < mpad * GEMM_TILE_N; e += GEMM_THREADS) {
            const int row = e / GEMM_TILE_N, col = e % GEMM_TILE_N;
            float s = 0.f;
            if (m0 + row < p.M) {
                const float* src = part + (long long)(m0 + row) * GEMM_TILE_N + col;
                for (int sp = 0; sp < S; ++sp) s += __builtin_nontemporal_load(src + (long long)sp * slab);
            }
            Ct[e] = s;
        }
        if (threadIdx.x == 0) *ctr = 0u;   // self-reset for the next launch
        __syncthreads();
    }

    gemm_epilogue<T, EPI>(p, L, layer, tile, m0, mrows, Ct);
}

// --------------------------------------------------------------------------------------------
// Epilogues.  One wavefront per output row (rows strided over the 4 waves).

template <typename T>
__device__ __forceinline__ void head_norm_rope_store(const float* src, int D, const T* wnorm, float eps,
                                                     const float* cosr, const float* sinr, bool rope,
                                                     T* dst, long long dst_stride) {
    // lane i < D/2 owns the rotate-half pair (i, i + D/2) of one head
    const int lane = threadIdx.x & 63;
    const int half = D >> 1;
    float x1 = 0.f, x2 = 0.f;
    if (lane < half) { x1 = src[lane]; x2 = src[lane + half]; }
    const float ss = wave_sum(x1 * x1 + x2 * x2);
    const float rs = 1.0f / sqrtf(ss / (float)D + eps);
    if (lane < half) {
        float y1 = x1 * rs * Elem<T>::to_f(wnorm[lane]);
        float y2 = x2 * rs * Elem<T>::to_f(wnorm[lane + half]);
        if (rope) {
            const float c = cosr[lane], s = sinr[lane];
            const float o1 = y1 * c - y2 * s;
            const float o2 = y2 * c + y1 * s;
            y1 = o1; y2 = o2;
        }
        dst[(long long)lane * dst_stride] = Elem<T>::from_f(y1);
        dst[(long long)(lane + half) * dst_stride] = Elem<T>::from_f(y2);
    }
}

template <typename T, int EPI>
__device__ void gemm_epilogue(const GemmArgs& p, const GemmLayer& L, int layer, int tile, int m0,
                              int mrows, const float* Ct) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;

    if (EPI == EPI_STORE) {
        const int n0 = tile * GEMM_TILE_N;
        for (int row = wv; row < mrows; row += 4) {
            const int m = m0 + row;
            float ss = 0.f;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int col = lane + h * 64;
                const int n = n0 + col;
                if (n < p.N) {
                    float v = Ct[row * GEMM_TILE_N + col];
                    float* o = p.out + (long long)m * p.ldo + n;
                    if (p.residual) v += *o;
                    *o = v;
                    ss += v * v;
                }
            }
            ss = wave_sum(ss);
            if (lane == 0 && p.ssq_out) p.ssq_out[(long long)tile * p.ssq_out_ld + m] = ss;
        }
    } else if (EPI == EPI_SWIGLU) {
        const int n0 = tile * 64;
        for (int row = wv; row < mrows; row += 4) {
            const int m = m0 + row;
            const float gt = Ct[row * GEMM_TILE_N + lane];
            const float up = Ct[row * GEMM_TILE_N + 64 + lane];
            const float h = gt / (1.0f + __expf(-gt)) * up;
            reinterpret_cast<T*>(p.out_t)[(long long)m * p.ldo + n0 + lane] = Elem<T>::from_f(h);
        }
    } else if (EPI == EPI_QKV) {
        // tile covers 128 columns = 128/D heads of one segment (q, k or v)
        const int D = p.head_dim;
        const int heads_per_tile = GEMM_TILE_N / D;
        const int nq_cols = p.n_q * D, nk_cols = p.n_kv * D;
        const int n0 = tile * GEMM_TILE_N;
        const int g = p.n_q / p.n_kv;
        const int G = p.gamma;
        for (int task = wv; task < mrows * heads_per_tile; task += 4) {
            const int row = task / heads_per_tile, hh = task % heads_per_tile;
            const int m = m0 + row;
            const int b = m / G, jj = m % G;
            const int col0 = n0 + hh * D;
            const float* src = Ct + row * GEMM_TILE_N + hh * D;
            int pos = p.len[b] + jj;
            if (pos < 0) pos = 0;
            if (pos >= p.rope_rows) {
                if (lane == 0) atomicOr(p.status, STATUS_KV_OVERFLOW);
                pos = p.rope_rows - 1;
            }
            const float* cr = p.rope_cos + (long long)pos * (D / 2);
            const float* sr = p.rope_sin + (long long)pos * (D / 2);
            if (col0 < nq_cols) {
                const int h = col0 / D;
                const int hk = h / g, hq = h % g;
                T* dst = reinterpret_cast<T*>(p.qbuf) +
                         (((long long)b * p.n_kv + hk) * p.rpad + (hq * G + jj)) * D;
                head_norm_rope_store<T>(src, D, reinterpret_cast<const T*>(L.head_norm), p.eps, cr, sr, true, dst, 1);
            } else if (col0 < nq_cols + nk_cols) {
                const int h = (col0 - nq_cols) / D;
                T* dst = reinterpret_cast<T*>(p.kblk) + (((long long)b * p.n_kv + h) * 32 + jj) * D;
                head_norm_rope_store<T>(src, D, reinterpret_cast<const T*>(L.head_norm2), p.eps, cr, sr, true, dst, 1);
            } else {
                const int h = (col0 - nq_cols - nk_cols) / D;
                T* dst = reinterpret_cast<T*>(p.vblk) + ((long long)b * p.n_kv + h) * D * 32 + jj;
                for (int d = lane; d < D; d += 64) dst[(long long)d * 32] = Elem<T>::from_f(src[d]);
            }
        }
    } else if (EPI == EPI_KV_INJECT) {
        const int D = p.head_dim;
        const int heads_per_tile = GEMM_TILE_N / D;
        const int nk_cols = p.n_kv * D;
        const int n0 = tile * GEMM_TILE_N;
        const int RS = p.gamma;    // rows_stride
        const int cap = p.cap;
        for (int task = wv; task < mrows * heads_per_tile; task += 4) {
            const int row = task / heads_per_tile, hh = task % heads_per_tile;
            const int m = m0 + row;
            const int b = m / RS, i = m % RS;
            const int len = p.len[b], nn = p.n_new[b];
            if (nn < 0 || nn > RS || len < 0) continue;      // flagged by the length update
            if (i >= nn) continue;
            if (len + nn > cap || len + nn > p.rope_rows) continue;   // flagged by the length update
            const int pos = len + i;
            const int col0 = n0 + hh * D;
            const float* src = Ct + row * GEMM_TILE_N + hh * D;
            if (col0 < nk_cols) {
                const int h = col0 / D;
                const float* cr = p.rope_cos + (long long)pos * (D / 2);
                const float* sr = p.rope_sin + (long long)pos * (D / 2);
                T* dst = reinterpret_cast<T*>(L.kcache) + (((long long)b * p.n_kv + h) * cap + pos) * D;
                head_norm_rope_store<T>(src, D, reinterpret_cast<const T*>(L.head_norm), p.eps, cr, sr, true, dst, 1);
            } else {
                const int h = (col0 - nk_cols) / D;
                T* dst = reinterpret_cast<T*>(L.vcache) + ((long long)b * p.n_kv + h) * D * (long long)cap + pos;
                for (int d = lane; d < D; d += 64) dst[(long long)d * cap] = Elem<T>::from_f(src[d]);
            }
        }
        // the last tile-workgroup of the whole launch advances the lengths
        __threadfence();
        __syncthreads();
        __shared__ int fin;
        unsigned* gctr = p.counters + (long long)p.n_layers * p.n_mgroups * p.n_tiles;
        if (threadIdx.x == 0) {
            const unsigned total = (unsigned)(p.n_layers * p.n_mgroups * p.n_tiles);
            fin = (atomicAdd(gctr, 1u) == total - 1u);
        }
        __syncthreads();
        if (fin) {
            __threadfence();
            for (int b = threadIdx.x; b < p.batch; b += GEMM_THREADS) {
                const int len = p.len[b], nn = p.n_new[b];
                if (nn < 0 || nn > RS || len < 0) { atomicOr(p.status, STATUS_BAD_COUNT); continue; }
                if (len + nn > cap || len + nn > p.rope_rows) { atomicOr(p.status, STATUS_KV_OVERFLOW); continue; }
                const_cast<int*>(p.len)[b] = len + nn;
            }
            if (threadIdx.x == 0) *gctr = 0u;
        }
    } else if (EPI == EPI_ARGMAX) {
        const int n0 = tile * GEMM_TILE_N;
        const int G = p.gamma;
        for (int row = wv; row < mrows; row += 4) {
            const int m = m0 + row;
            const int b = m / G, jj = m % G;
            if (jj == 0) continue;     // anchor row: no draft
            unsigned long long best = 0ull;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int col = lane + h * 64;
                const int n = n0 + col;
                if (n < p.N) {
                    const float v = Ct[row * GEMM_TILE_N + col];
                    const unsigned long long key = pack_argmax(v, (uint32_t)n);
                    best = key > best ? key : best;
                    if (p.dbg_logits) p.dbg_logits[((long long)b * (G - 1) + (jj - 1)) * p.N + n] = v;
                }
            }
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) {
                const unsigned long long other = __shfl_xor(best, o, WAVE);
                best = other > best ? other : best;
            }
            if (lane == 0) atomicMax(p.slots + (long long)b * (G - 1) + (jj - 1), best);
        }
        __threadfence();
        __syncthreads();
        __shared__ int fin;
        unsigned* gctr = p.counters + (long long)p.n_layers * p.n_mgroups * p.n_tiles;
        if (threadIdx.x == 0) {
            const unsigned total = (unsigned)(p.n_layers * p.n_mgroups * p.n_tiles);
            fin = (atomicAdd(gctr, 1u) == total - 1u);
        }
        __syncthreads();
        if (fin) {
            __threadfence();
            const int nslots = p.batch * (G - 1);
            for (int i = threadIdx.x; i < nslots; i += GEMM_THREADS) {
                const unsigned long long v = atomicExch(p.slots + i, 0ull);
                p.draft[i] = (int)unpack_argmax_index(v);
            }
            if (threadIdx.x == 0) *gctr = 0u;
        }
    }
}

}  // namespace dflash
