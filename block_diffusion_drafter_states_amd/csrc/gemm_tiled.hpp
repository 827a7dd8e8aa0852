// Tiled GEMM for many rows (M >= 128: batch x block rows at larger batches, a whole
// prompt's injection): out = A . W^T with the same epilogues as the weight-streaming
// GEMM (store + residual + per-tile sums of squares, SwiGLU, argmax).
//
// At these sizes the product is a dense contraction: each workgroup computes a BM x BN
// block (BM = 128 or 256 rows of A against BN = 128 or 64 weight rows; SwiGLU: 64 gate +
// 64 up rows of the same 64 output columns), its BM / 32 waves arranged BM / 64 x 2, each
// wave 64 x BN/2 (4 x BN/32 MFMA tiles of 16 x 16).  Both operands go HBM -> LDS with
// direct-to-LDS loads, KB bytes of every row per stage, two stages.  KB = 256 (128 KB of
// LDS at 128 x 128: one workgroup per CU) for launches with few workgroups, KB = 128 (64 KB:
// several workgroups per CU hide each other's barriers and load latency) for launches
// with many; 256 x 128 blocks (96 KB, eight waves) for some of those.  Inside a 16-row tile the 16-byte chunk c of row rho sits at c ^ swz(rho)
// (rho for 256-byte rows, (rho >> 1) & 7 for 128-byte rows), so the fragment reads of
// 16 lanes (one row each) hit 16 different bank groups.
//
// The M-blocks of one weight block are dispatched on the same XCD (workgroup w runs on
// XCD w % 8), one after the other, so the weight block comes from HBM once and from
// that XCD's L2 for the other M-blocks.
#pragma once

#include "common.hpp"
#include "gemm.hpp"

namespace dflash {

constexpr int TG_BM = 128;                               // rows of A per workgroup (or 2 x TG_BM)
// threads of a workgroup over BM rows of A: BM / 32 waves, 2 along the weight rows
__host__ __device__ constexpr int tg_threads(int bm) { return 2 * bm; }
// bytes per stage and of the two stages, for BM rows of A, BN weight rows and KB bytes per row
__host__ __device__ constexpr int tg_stage_bytes(int bm, int bn, int kb) { return (bm + bn) * kb; }
__host__ __device__ constexpr int tg_lds_bytes(int bm, int bn, int kb) { return 2 * tg_stage_bytes(bm, bn, kb); }

template <int KB> __device__ __forceinline__ int tg_swz(int rho) { return KB == 256 ? rho : ((rho >> 1) & 7); }

// LDS fragment of 16 rows (one per lane r) x KB bytes, lane group g: KB / 64 pieces of 16 bytes
template <int KB>
__device__ __forceinline__ void tg_frag(u32x4_t (&f)[KB / 64], const unsigned char* tile, int r, int g) {
#pragma unroll
    for (int i = 0; i < KB / 64; ++i)
        f[i] = *reinterpret_cast<const u32x4_t*>(tile + r * KB + (((i * 4 + g) ^ tg_swz<KB>(r)) << 4));
}

// acc += A . B^T over the KB bytes of a stage (lane pieces of 8 bf16 or 4 fp32 elements)
template <typename T, int CH>
__device__ __forceinline__ void tg_mfma(f32x4_t& acc, const u32x4_t (&a)[CH], const u32x4_t (&b)[CH]) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
        if constexpr (sizeof(T) == 2) {
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[i]), as_bf16x8(b[i]), acc, 0, 0, 0);
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c)
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[i][c]), __uint_as_float(b[i][c]), acc, 0,
                                                          0, 0);
        }
    }
}

// Output columns per workgroup (SwiGLU: 64 outputs from 64 gate + 64 up rows).
__host__ __device__ constexpr int tg_cols(int epi, int bn) { return epi == EPI_SWIGLU ? bn / 2 : bn; }

// Epilogues of a workgroup's BM x BN block (the stages are no longer read).  Lane (g, r)
// of tile (a, b) holds C[m][n] for m = m0 + wm*64 + a*16 + 4g + v, column wn*BN/2 + b*16 + r
// of the workgroup.
template <typename T, int EPI, int BN, int BM>
__device__ __forceinline__ void tg_epilogue(const GemmArgs& p, const GemmLayer& L, f32x4_t (&acc)[4][BN / 32],
                                            int tile, int m0, int wm, int wn, unsigned char* smem) {
    constexpr int WN = BN / 32;
    const int lane = threadIdx.x & 63, g = lane >> 4, r = lane & 15;
    float* red = reinterpret_cast<float*>(smem);            // the stages are no longer read
    if constexpr (EPI == EPI_STORE) {
        float* const outp = L.out ? L.out : p.out;
        const int ncol0 = tile * BN + wn * (BN / 2);
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int mr = wm * 64 + a * 16 + 4 * g + v;    // row within the workgroup
                const int m = m0 + mr;
                float ss = 0.f;
#pragma unroll
                for (int b = 0; b < WN; ++b) {
                    const int n = ncol0 + b * 16 + r;
                    float x = acc[a][b][v];
                    if (m < p.M && n < p.N) {
                        float* o = outp + (long long)m * p.ldo + n;
                        if (p.residual) x += *o;
                        *o = x;
                    } else {
                        x = 0.f;
                    }
                    ss += x * x;
                }
                // sum over the 16 lanes of the row (fixed order), then over the two wn waves
                ss += __shfl_xor(ss, 1, WAVE);
                ss += __shfl_xor(ss, 2, WAVE);
                ss += __shfl_xor(ss, 4, WAVE);
                ss += __shfl_xor(ss, 8, WAVE);
                if (r == 0) red[wn * BM + mr] = ss;
            }
        __syncthreads();
        if (p.ssq_out && threadIdx.x < BM && m0 + (int)threadIdx.x < p.M)
            p.ssq_out[(long long)tile * p.ssq_out_ld + m0 + threadIdx.x] = red[threadIdx.x] + red[BM + threadIdx.x];
    } else if constexpr (EPI == EPI_SWIGLU) {
        // tiles b = 0, 2: gate of output tiles 0, 1 of this wave; b = 1, 3: up
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int m = m0 + wm * 64 + a * 16 + 4 * g + v;
                    const int n = tile * 64 + wn * 32 + c * 16 + r;
                    if (m < p.M && n < p.N) {
                        const float gt = acc[a][2 * c][v], up = acc[a][2 * c + 1][v];
                        const float h = gt / (1.0f + __expf(-gt)) * up;
                        reinterpret_cast<T*>(p.out_t)[(long long)m * p.ldo + n] = Elem<T>::from_f(h);
                    }
                }
    } else if constexpr (EPI == EPI_LSE) {
        // per row: largest logit and sum of exp(logit - max) over this wave's columns (16
        // lanes: xor shuffles), then over the two wn waves through LDS; the lane holding
        // the row's label column stores its logit
        float2* redl = reinterpret_cast<float2*>(smem);
        const int G = p.gamma;
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int mr = wm * 64 + a * 16 + 4 * g + v;
                const int m = m0 + mr;
                const int bb = m / G, jj = m % G;
                const int lab = (m < p.M && jj >= 1) ? p.labels[bb * (G - 1) + jj - 1] : -1;
                float mx = -INFINITY;
#pragma unroll
                for (int b = 0; b < WN; ++b) {
                    const int n = tile * BN + wn * (BN / 2) + b * 16 + r;
                    if (m < p.M && n < p.N) {
                        const float x = acc[a][b][v];
                        mx = fmaxf(mx, x);
                        if (n == lab) p.lab_logit[m] = x;
                        if (p.dbg_logits && jj >= p.dbg_first)
                            p.dbg_logits[((long long)bb * (G - p.dbg_first) + (jj - p.dbg_first)) * p.N + n] = x;
                    }
                }
#pragma unroll
                for (int o = 1; o < 16; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, WAVE));
                float se = 0.f;
#pragma unroll
                for (int b = 0; b < WN; ++b) {
                    const int n = tile * BN + wn * (BN / 2) + b * 16 + r;
                    if (m < p.M && n < p.N) se += __expf(acc[a][b][v] - mx);
                }
#pragma unroll
                for (int o = 1; o < 16; o <<= 1) se += __shfl_xor(se, o, WAVE);
                if (r == 0) redl[wn * BM + mr] = make_float2(mx, se);
            }
        __syncthreads();
        if (threadIdx.x < BM && m0 + (int)threadIdx.x < p.M) {
            const float2 x0 = redl[threadIdx.x], x1 = redl[BM + threadIdx.x];
            const float mx = fmaxf(x0.x, x1.x);
            const float se = (x0.x == -INFINITY ? 0.f : x0.y * __expf(x0.x - mx)) +
                             (x1.x == -INFINITY ? 0.f : x1.y * __expf(x1.x - mx));
            p.lse[(long long)tile * p.M + m0 + threadIdx.x] = make_float2(mx, se);
        }
    } else {    // EPI_ARGMAX
        unsigned long long* redu = reinterpret_cast<unsigned long long*>(smem);
        const int G = p.gamma;
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int mr = wm * 64 + a * 16 + 4 * g + v;
                const int m = m0 + mr;
                unsigned long long best = 0ull;
#pragma unroll
                for (int b = 0; b < WN; ++b) {
                    const int n = tile * BN + wn * (BN / 2) + b * 16 + r;
                    if (m < p.M && n < p.N) {
                        const float x = acc[a][b][v];
                        const unsigned long long key = pack_argmax(x, (uint32_t)n);
                        best = key > best ? key : best;
                        const int bb = m / G, jj = m % G;
                        if (p.dbg_logits && jj >= p.dbg_first)
                            p.dbg_logits[((long long)bb * (G - p.dbg_first) + (jj - p.dbg_first)) * p.N + n] = x;
                    }
                }
#pragma unroll
                for (int o = 1; o < 16; o <<= 1) {
                    const unsigned long long other = __shfl_xor(best, o, WAVE);
                    best = other > best ? other : best;
                }
                if (r == 0) redu[wn * BM + mr] = best;
            }
        __syncthreads();
        if (threadIdx.x < BM && m0 + (int)threadIdx.x < p.M) {
            const unsigned long long x0 = redu[threadIdx.x], x1 = redu[BM + threadIdx.x];
            p.amax[amax_slot(m0 + (int)threadIdx.x, tile, p.n_tiles)] = x0 > x1 ? x0 : x1;
        }
    }
}

// BN = 128 or 64 weight rows per workgroup (64: twice the workgroups for narrow weights;
// SwiGLU always 128), BM = 128 or 256 rows of A (BM / 32 waves).  Wave (wm, wn) computes A
// rows wm*64 .. +63 against W rows wn*BN/2 .. +BN/2-1: 4 x WN MFMA tiles.
template <typename T, int EPI, int BN, int KB, int BM>
__global__ __launch_bounds__(tg_threads(BM)) void gemm_tiled_kernel(const GemmArgs p) {
    static_assert(BN == 128 || (BN == 64 && EPI != EPI_SWIGLU), "tile width");
    static_assert(KB == 256 || KB == 128, "stage row bytes");
    static_assert(BM == TG_BM || (BM == 2 * TG_BM && KB == 128), "rows of A per workgroup");
    constexpr int STEP = Elem<T>::STEP * KB / 256;          // elements of a row per stage
    constexpr int WN = BN / 32;                             // n-tiles per wave
    constexpr int LPR = KB / 16;                            // lanes per row in a 1 KB instruction
    constexpr int RPI = 64 / LPR;                           // rows per instruction
    constexpr int IPT = 16 / RPI;                           // instructions per 16-row tile
    constexpr int TILEB = 16 * KB;                          // bytes of a 16-row tile
    constexpr int CH = KB / 64;                             // 16-byte pieces per lane and tile
    constexpr int NW = BM / 32;                             // waves
    constexpr int AT = BM / 16;                             // 16-row A tiles per stage
    constexpr int NI = (BM + BN) / 16 * IPT;                // direct-to-LDS instructions per stage
    static_assert(NI % NW == 0, "whole instructions per wave");
    constexpr int NIW = NI / NW;                            // ... per wave
    constexpr int STAGE = tg_stage_bytes(BM, BN, KB);
    extern __shared__ __align__(16) unsigned char smem[];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, g = lane >> 4, r = lane & 15;
    const int wm = wv >> 1, wn = wv & 1;

    // ---- workgroup -> (weight block, M-block): the M-blocks of a weight block share an XCD
    const int mgroups = gridDim.y;
    const int wlin = blockIdx.x + blockIdx.y * gridDim.x;
    const int xcd = wlin & 7, wslot = wlin >> 3;
    const int tile = (wslot / mgroups) * 8 + xcd;           // gridDim.x = n_tiles rounded up to 8
    const int m0 = (wslot % mgroups) * BM;
    if (tile >= p.n_tiles) return;                          // whole workgroup, before any barrier
    const int layer = blockIdx.z;
    const GemmLayer& L = p.layer[layer];
    const int K = p.K;
    const int nsteps = K / STEP;

    // ---- load plan: NI direct-to-LDS instructions per stage (AT A tiles, BN / 16 W tiles,
    // IPT per tile), instruction j by wave j % NW; each fetches RPI rows x KB bytes
    const int lq = lane / LPR, lc = lane % LPR;
    const void* abase = L.a ? L.a : p.a;
    const char* src[NIW];
    uint32_t dst[NIW];
    const uint32_t lds0 = lds_offset(smem);
    const int wv_u = __builtin_amdgcn_readfirstlane(wv);
#pragma unroll
    for (int u = 0; u < NIW; ++u) {
        const int j = u * NW + wv_u;                // 0..NI-1, wave-uniform
        const int t = j / IPT, i = j % IPT;         // tile (0..AT-1 A, AT.. W), rows RPI*i ..
        const int rho = i * RPI + lq;
        const T* rowp;
        if (t < AT) {
            int m = m0 + t * 16 + rho;
            m = m < p.M ? m : p.M - 1;              // rows past M: re-read a valid row, result discarded
            rowp = reinterpret_cast<const T*>(abase) + (long long)m * p.lda;
        } else {
            const int nt = t - AT;
            const T* base;
            int row, rows;
            if (EPI == EPI_SWIGLU) {                // n-tile 2c: gate tile c, 2c + 1: up tile c
                row = tile * 64 + (nt >> 1) * 16 + rho;
                base = reinterpret_cast<const T*>((nt & 1) ? L.w[1] : L.w[0]);
                rows = p.N;
            } else {                                // segment of a 16-row tile: wave-uniform
                const int n0 = min(tile * BN + nt * 16, p.N - 1);
                const int sg = n0 < p.seg_end[0] ? 0 : (n0 < p.seg_end[1] ? 1 : 2);
                const int lo = sg == 0 ? 0 : (sg == 1 ? p.seg_end[0] : p.seg_end[1]);
                base = reinterpret_cast<const T*>(sg == 0 ? L.w[0] : (sg == 1 ? L.w[1] : L.w[2]));
                row = n0 - lo + rho;
                rows = (sg == 0 ? p.seg_end[0] : (sg == 1 ? p.seg_end[1] : p.seg_end[2])) - lo;
            }
            row = min(row, rows - 1);
            rowp = base + (long long)row * K;
        }
        src[u] = reinterpret_cast<const char*>(rowp) + ((lc ^ tg_swz<KB>(rho)) * 16);
        dst[u] = (uint32_t)(t * TILEB + i * 1024);
    }
    auto issue = [&](int stage, int step) {
#pragma unroll
        for (int u = 0; u < NIW; ++u) dma_b128(src[u] + (size_t)step * KB, lds0 + stage * STAGE + dst[u]);
    };

    f32x4_t acc[4][WN];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < WN; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    issue(0, 0);
    if (nsteps > 1) issue(1, 1);
    for (int s = 0; s < nsteps; ++s) {
        // this wave's loads of stage s have landed (at most one later stage is in flight) ...
        if (s + 1 < nsteps) vm_wait<NIW>();
        else vm_wait<0>();
        __syncthreads();    // ... and every wave's
        const unsigned char* st = smem + (s & 1) * STAGE;
        u32x4_t af[4][CH], bf[WN][CH];
#pragma unroll
        for (int a = 0; a < 4; ++a) tg_frag<KB>(af[a], st + (wm * 4 + a) * TILEB, r, g);
#pragma unroll
        for (int b = 0; b < WN; ++b) tg_frag<KB>(bf[b], st + (AT + wn * WN + b) * TILEB, r, g);
        __syncthreads();    // every wave holds the stage in registers: it can be refilled
        // the refill (step s + 2) is issued a quarter at a time between the MFMA groups: issuing
        // a direct-to-LDS load holds the wave, so the matrix core works through it
        const bool refill = s + 2 < nsteps;
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            if (refill) {
#pragma unroll
                for (int u = a * NIW / 4; u < (a + 1) * NIW / 4; ++u)
                    dma_b128(src[u] + (size_t)(s + 2) * KB, lds0 + (s & 1) * STAGE + dst[u]);
            }
#pragma unroll
            for (int b = 0; b < WN; ++b) tg_mfma<T, CH>(acc[a][b], af[a], bf[b]);
        }
    }

    tg_epilogue<T, EPI, BN, BM>(p, L, acc, tile, m0, wm, wn, smem);
}


}  // namespace dflash
