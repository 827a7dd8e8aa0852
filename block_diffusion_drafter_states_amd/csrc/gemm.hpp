// Weight-streaming GEMM for few rows (up to 16*MT rows per workgroup): out = A . W^T.
//
// Used for every projection of the drafter (W_fuse, W_k|W_v of every layer for
// injection, W_q|W_k|W_v, W_o, W_gate|W_up, W_down, LM head).  At batch 1 the weights are
// the whole HBM traffic and each weight byte is read exactly once.
//
// Geometry.  A workgroup owns WCOLS = NS * NTW * 16 complete weight rows
// (output columns) and is made of NS x KS wavefronts: NS groups of waves own
// different rows (NTW MFMA n-tiles of 16 rows per wave), the KS waves of a
// group split the K range.  No workgroup
// ever waits for another one: the KS partial sums are reduced through LDS in
// a fixed order (deterministic) and the workgroup runs the fused epilogue.
//
// Streaming.  Weights go from HBM straight into a per-wave LDS ring with
// direct-to-LDS loads (global_load_lds, 16 bytes per lane): one instruction
// fetches 4 weight rows x 256 contiguous bytes, P k-steps ahead, without
// passing through registers, with the non-temporal hint (a launch reads each weight
// byte once per 16*MT-row group).  Inside a 16-row x 256-byte ring tile, the
// 16-byte chunk c of row rho sits at position c ^ rho, so the MFMA fragment
// reads (lane r <- row r) hit 16 distinct bank groups.  The few activation
// rows (storage type, already normalised where the model normalises them;
// L2-resident) are loaded into registers in the same ring slot; explicit vmcnt
// waits (loads complete in issue order) make a slot's LDS data visible.
//
// RMSNorm carried across a GEMM pair.  RMSNorm(x; w) = f_m * (x ⊙ w) with one factor
// f_m = 1 / sqrt(mean(x_m^2) + eps) per row, and a GEMM is linear in each row, so the
// norm before a GEMM needs no launch of its own: the GEMM that produces x also stores
// x ⊙ w (rounded, in the next GEMM's fragment order), and the next GEMM multiplies its
// output rows by f_m, summed from the producer's per-tile sums of squares.  Only the
// rounding point moves (x ⊙ w is rounded instead of f_m * x ⊙ w).
#pragma once

#include "common.hpp"

namespace dflash {

enum { EPI_STORE = 0, EPI_SWIGLU = 1, EPI_ARGMAX = 2, EPI_LSE = 3 };

constexpr int MAX_LAYERS = 16;
constexpr int GEMM_ZMAX = 8;    // norm-weighted copies a producer can write (one per consumer layer)
constexpr int GEMM_RSQ = 4;     // 16-byte loads of sums of squares per thread (a consumer's row factors)

struct GemmLayer {
    const void* a;          // nullable: this layer's A operand (overrides GemmArgs::a)
    const void* w[3];       // weight segments: rows [seg_end[i-1], seg_end[i]) come from w[i]
    float* out;             // nullable, EPI_STORE: this layer's output (overrides GemmArgs::out)
};

struct GemmArgs {
    // ---- A operand
    const void* a;          // T [M][lda], or in fragment order (a_frag, weight-streaming kernel only)
    long long lda;
    int a_frag;             // A in fragment order (afrag_offset, K columns, whole 16-row tiles)
    int M;
    int K;
    // ---- W operand and geometry
    int N;                  // weight rows (EPI_SWIGLU: rows of each of gate / up)
    int seg_end[3];         // cumulative rows of the segments (EPI_SWIGLU: gate = w[0], up = w[1])
    int ns, ks;             // wave groups along N, waves along K
    int kw;                 // K per wave (multiple of the k-step)
    int n_tiles;            // workgroups along N
    int n_layers;           // grid z: independent problems (one per layer), each with its own GemmLayer
    GemmLayer layer[MAX_LAYERS];
    // ---- epilogue
    float* out;             // EPI_STORE: fp32 [M][ldo] (+= when residual)
    int ldo;
    int residual;
    float* ssq_out;         // EPI_STORE: [n_tiles][ssq_out_ld] sums of squares of the new rows (nullable)
    int ssq_out_ld;
    void* out_t;            // EPI_SWIGLU: T [M][ldo], or in fragment order with N columns (out_frag)
    int out_frag;
    unsigned long long* amax;   // EPI_ARGMAX: packed (value, index) maxima per (row, tile), at amax_slot
    float* dbg_logits;      // EPI_ARGMAX: nullable [B][gamma-dbg_first][N] logits of rows j >= dbg_first
    int gamma;              // EPI_ARGMAX / EPI_LSE: rows per sequence in A (block size)
    int dbg_first;
    float2* lse;            // EPI_LSE: [n_tiles][M] per tile (max logit, sum of exp(logit - max))
    const int* labels;      // EPI_LSE: [B][gamma-1] label ids of rows j >= 1
    float* lab_logit;       // EPI_LSE: [M] logit of row m's label (written by the tile holding it)
    // ---- RMSNorm carried across a GEMM (weight-streaming kernel, one M-tile; see below)
    // Consumer: the A rows are x * w_norm without their RMSNorm row factor, which is applied
    // to the output instead: row m is multiplied by 1 / sqrt(sum_t rs_ssq[t][m] / rs_k + rs_eps)
    // (EPI_STORE before the residual is added, EPI_SWIGLU before the activation).
    const float* rs_ssq;    // nullable: [rs_n][rs_ld] per-tile sums of squares of x (a producer's ssq_out)
    int rs_n, rs_ld;
    float rs_k, rs_eps;
    // Producer (EPI_STORE, at most one output element per thread): for z < n_z also store
    // the new value times zw[z][column], in the storage type and in fragment order (K = N),
    // at zout + z * zstride elements: the next GEMM's A operand for norm weight zw[z].
    int n_z;
    const void* zw[GEMM_ZMAX];
    void* zout;
    long long zstride;
    // nullable: workgroup (0, 0, 0) copies snap_src[0 .. snap_n) to snap_dst at its end
    const int* snap_src;
    int* snap_dst;
    int snap_n;
};

// Ring depth (k-steps in flight): the weights live in LDS; the registers of a
// slot hold only the A fragments (~160 VGPRs budget), and the loads of P-1
// steps must fit the 6-bit vmcnt.
__host__ __device__ constexpr int gemm_ring_depth(int mt, int ntw) {
    const int slot = mt * 16;
    const int lps = ntw * 4 + mt * 4;
    int p = 160 / slot;
    p = p > 4 ? 4 : (p < 1 ? 1 : p);
    while (p > 1 && (p - 1) * lps > 63) --p;
    return p;
}

static inline size_t gemm_lds_bytes_host(int ns, int ks, int mt, int ntw, int ring_depth) {
    const size_t slots = (size_t)ns * ks * mt * ntw * 4 * 64 * sizeof(float);
    const size_t ct = (size_t)mt * 16 * ns * ntw * 16 * sizeof(float);
    const size_t ring = (size_t)ns * ks * ring_depth * ntw * 4096;
    return ring > slots + ct ? ring : slots + ct;
}

template <typename T, int EPI>
__device__ void gemm_epilogue(const GemmArgs& p, const GemmLayer& L, int tile, int m0, int mrows, int wcols,
                              const float* Ct);

// --------------------------------------------------------------------------------------------
template <typename T, int EPI, int MT, int NTW, int P>
__global__ __launch_bounds__(512) void gemm_kernel(const GemmArgs p) {
    constexpr int STEP = Elem<T>::STEP;
    // NTW = weight tiles per ring slot (EPI_SWIGLU: one gate tile + one up tile)
    static_assert(EPI != EPI_SWIGLU || NTW == 2, "SwiGLU pairs one gate and one up tile");
    extern __shared__ __align__(16) unsigned char smem[];

    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, g = lane >> 4, r = lane & 15;
    const int tile = blockIdx.x;
    const int m0 = blockIdx.y * (16 * MT);
    const int layer = blockIdx.z;
    const GemmLayer& L = p.layer[layer];
    const int mrows = min(16 * MT, p.M - m0);
    const int ns_i = wv / p.ks, ks_i = wv % p.ks;
    const int K = p.K;
    const int k0 = ks_i * p.kw;
    const int k1 = min(K, k0 + p.kw);
    const int nsteps = k1 > k0 ? (k1 - k0) / STEP : 0;

    // ---- weight rows of this wave: ring loads fetch rows 4*i + (lane>>4) of each n-tile
    // vector-memory instructions per ring step, all issued by this loop in a fixed order:
    // 4 direct-to-LDS loads per weight tile, then 4 per M-tile for the A fragments
    constexpr int LPS = NTW * 4 + MT * 4;
    static_assert((P - 1) * LPS <= 63, "vmcnt range");
    const int lq = lane >> 4, lc = lane & 15;
    // The segment of a 16-row tile is wave-uniform (segment boundaries are
    // multiples of 16 rows), so the base pointer is picked in scalar registers and
    // no lane waits for a load before the first weight request.
    const int ns_u = __builtin_amdgcn_readfirstlane(ns_i);
    const char* wsrc[NTW][4];
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
        const T* base;
        int r0, rows;                                    // first row of the tile in its segment; segment rows
        if (EPI == EPI_SWIGLU) {
            r0 = tile * (p.ns * 16) + ns_u * 16;
            base = reinterpret_cast<const T*>(L.w[t]);    // t = 0 gate, t = 1 up
            rows = p.N;
        } else {
            const int n0 = min(tile * (p.ns * NTW * 16) + ns_u * (NTW * 16) + t * 16, p.N - 1);
            const int sg = n0 < p.seg_end[0] ? 0 : (n0 < p.seg_end[1] ? 1 : 2);
            const int lo = sg == 0 ? 0 : (sg == 1 ? p.seg_end[0] : p.seg_end[1]);
            base = reinterpret_cast<const T*>(sg == 0 ? L.w[0] : (sg == 1 ? L.w[1] : L.w[2]));
            r0 = n0 - lo;
            rows = (sg == 0 ? p.seg_end[0] : (sg == 1 ? p.seg_end[1] : p.seg_end[2])) - lo;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int rho = i * 4 + lq;                  // row within the 16-row tile
            // ragged last tile: re-read a valid row; its result is discarded
            const int row = min(r0 + rho, rows - 1);
            wsrc[t][i] = reinterpret_cast<const char*>(base + (long long)row * K + k0) + ((lc ^ rho) * 16);
        }
    }
    const int wv_u = __builtin_amdgcn_readfirstlane(wv);
    const uint32_t ring_lds = lds_offset(smem) + (uint32_t)wv_u * (P * NTW * 4096);
    const char* ring = reinterpret_cast<const char*>(smem) + (size_t)wv_u * P * NTW * 4096;

    // ---- A row pointers (one row per lane and M-tile) and the byte strides of a k-step
    // and of a piece: plain rows, or fragment order (one contiguous 1 KB per piece)
    const char* arow[MT];
    bool avalid[MT];
    const void* abase = L.a ? L.a : p.a;
    const int a_step = p.a_frag ? 4096 : 256, a_piece = p.a_frag ? 1024 : 64;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int m = m0 + mt * 16 + r;
        avalid[mt] = m < p.M;
        if (p.a_frag) {         // tiles past the last one re-read it; their MFMA input is zeroed
            const int tl = min((m0 >> 4) + mt, (p.M - 1) >> 4);
            arow[mt] = reinterpret_cast<const char*>(abase) +
                       ((((long long)tl * (K / STEP) + k0 / STEP) * 4) * 64 + lane) * 16;
        } else {
            const int mm = avalid[mt] ? m : 0;   // padding rows read row 0; their MFMA input is zeroed
            arow[mt] = reinterpret_cast<const char*>(reinterpret_cast<const T*>(abase) + (long long)mm * p.lda + k0 +
                                                     g * Elem<T>::PER16);
        }
    }

    // EPI_STORE with a residual, one M-tile: the old output values do not depend
    // on this kernel, so they are requested now, ahead of the weight stream (ns ==
    // 1: at most 4 * NTW elements per thread), and read after the stream's last
    // wait: the epilogue does not wait for a second memory latency.  Issued before
    // every ring load, they complete first, so the ring's waits stay valid.
    constexpr bool RES_EARLY = EPI == EPI_STORE && MT == 1;
    constexpr int RPT = RES_EARLY ? 4 * NTW : 1;
    const int wcols = p.ns * NTW * 16;
    float* const outp = L.out ? L.out : p.out;
    uint32_t resid_u[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) resid_u[i] = 0u;
    if constexpr (RES_EARLY) {
        if (p.residual) {
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const int e = threadIdx.x + i * blockDim.x;
                const int row = e / wcols, n = tile * wcols + e % wcols;
                const bool ok = e < mrows * wcols && n < p.N;     // else: a valid address, value unused
                vload_b32(resid_u[i], outp + (ok ? (long long)(m0 + row) * p.ldo + n : 0));
            }
        }
    }

    Frag64 areg[P][MT];
    auto issue = [&](int q, int step) {
#pragma unroll
        for (int t = 0; t < NTW; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                dma_b128_nt(wsrc[t][i] + (size_t)step * 256, ring_lds + (uint32_t)((q * NTW + t) * 4096 + i * 1024));
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const char* a = arow[mt] + (size_t)step * a_step;
#pragma unroll
            for (int i = 0; i < 4; ++i) vload_b128(areg[q][mt].q[i], a + i * a_piece);
        }
    };
    // all loads of ring slot q are complete once at most `later` later steps are outstanding
    // The wait counts only the ring loads issued after the slot.  Other loads issued after
    // it (the RMSNorm row sums and norm weights below) only make the wait stricter: with
    // them in flight, "at most N outstanding" still implies the slot's loads have landed.
    auto wait_slot = [&](int q, int later) {
        if (later <= 0) vm_wait<0>();
        else if (P > 1 && later == 1) vm_wait<(P > 1 ? LPS : 0)>();
        else if (P > 2 && later == 2) vm_wait<(P > 2 ? 2 * LPS : 0)>();
        else vm_wait<(P > 3 ? 3 * LPS : 0)>();
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) tie(areg[q][mt]);
    };

#pragma unroll
    for (int q = 0; q < P; ++q)
        if (q < nsteps) issue(q, q);

    // RMSNorm carried across the GEMM: requested right after the first ring stages (so
    // they do not delay the first weights) and read after the stream's last wait.
    // Consumer (one M-tile): this thread's share of the producer's per-tile sums of squares,
    // rows 4q .. 4q+3 of tiles j0, j0 + step, ... (out-of-range slots re-read tile 0 and
    // are skipped when summed).  Producer: the norm weights of this thread's output element.
    constexpr bool FOLD_RS = MT == 1 && (EPI == EPI_STORE || EPI == EPI_SWIGLU);
    const bool rs_on = FOLD_RS && p.rs_ssq != nullptr;
    u32x4_t rsv[GEMM_RSQ];
#pragma unroll
    for (int i = 0; i < GEMM_RSQ; ++i) rsv[i] = u32x4_t{0u, 0u, 0u, 0u};
    if constexpr (FOLD_RS) {
        if (rs_on) {
            const int q = threadIdx.x & 3, j0 = threadIdx.x >> 2, step = blockDim.x >> 2;
#pragma unroll
            for (int i = 0; i < GEMM_RSQ; ++i) {
                const int j = j0 + i * step;
                const bool ok = j < p.rs_n && 4 * q < mrows;
                vload_b128(rsv[i], p.rs_ssq + (ok ? (long long)j * p.rs_ld + m0 + 4 * q : 0));
            }
        }
    }
    uint32_t zg[GEMM_ZMAX];
#pragma unroll
    for (int z = 0; z < GEMM_ZMAX; ++z) zg[z] = 0u;
    if constexpr (RES_EARLY) {
        if (p.n_z > 0) {
            const int e = threadIdx.x, n = tile * wcols + e % wcols;
            const long long off = e < mrows * wcols && n < p.N ? n : 0;
#pragma unroll
            for (int z = 0; z < GEMM_ZMAX; ++z) {
                if (z < p.n_z) {
                    if constexpr (sizeof(T) == 2) vload_u16(zg[z], reinterpret_cast<const T*>(p.zw[z]) + off);
                    else vload_b32(zg[z], reinterpret_cast<const T*>(p.zw[z]) + off);
                }
            }
        }
    }


    f32x4_t acc[MT][NTW];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int t = 0; t < NTW; ++t) acc[mt][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    for (int s0 = 0; s0 < nsteps; s0 += P) {
#pragma unroll
        for (int q = 0; q < P; ++q) {
            const int step = s0 + q;
            if (step < nsteps) {
                wait_slot(q, min(P - 1, nsteps - 1 - step));
                const char* slotp = ring + (size_t)q * NTW * 4096;
                Frag64 bf[NTW];
#pragma unroll
                for (int t = 0; t < NTW; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        bf[t].q[i] = *reinterpret_cast<const u32x4_t*>(slotp + t * 4096 + r * 256 + (((i * 4 + g) ^ r) * 16));
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    if (mt * 16 < mrows) {
                        Frag64 af = areg[q][mt];
                        if (!avalid[mt]) zero_frag64(af);
#pragma unroll
                        for (int t = 0; t < NTW; ++t) mfma_kstep<T>(acc[mt][t], af, bf[t]);
                    }
                }
                // the slot's LDS tiles are in registers before the slot is refilled
                asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
                if (step + P < nsteps) issue(q, step + P);
            }
        }
    }
    vm_wait<0>();
    __syncthreads();   // every wave is done with its ring: the LDS is reused below
    float resid[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        tie(resid_u[i]);
        resid[i] = __uint_as_float(resid_u[i]);
    }
#pragma unroll
    for (int i = 0; i < GEMM_RSQ; ++i) tie(rsv[i]);
#pragma unroll
    for (int z = 0; z < GEMM_ZMAX; ++z) tie(zg[z]);

    // ---- reduce the KS partial sums (fixed order) into Ct[mrows][wcols]
    float* slot = reinterpret_cast<float*>(smem);
    float* Ct = slot + (size_t)p.ns * p.ks * MT * NTW * 4 * 64;
    __shared__ float rs_wave[16][16];                            // [wave][row] sums of squares
    {
        float* mine = slot + (size_t)wv * MT * NTW * 4 * 64;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int t = 0; t < NTW; ++t)
#pragma unroll
                for (int v = 0; v < 4; ++v) mine[((mt * NTW + t) * 4 + v) * 64 + lane] = acc[mt][t][v];
    }
    if constexpr (FOLD_RS) {
        if (rs_on) {
            // this thread's sums for rows 4q .. 4q+3 (its tiles in order), then the 16 lanes
            // of the wave with the same q (lane bits 2..5, xor shuffles in a fixed order):
            // lane q of every wave holds the wave's sums of rows 4q .. 4q+3
            const int q = threadIdx.x & 3, j0 = threadIdx.x >> 2, step = blockDim.x >> 2;
            float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < GEMM_RSQ; ++i) {
                if (j0 + i * step < p.rs_n && 4 * q < mrows) {
#pragma unroll
                    for (int c = 0; c < 4; ++c) s4[c] += __uint_as_float(rsv[i][c]);
                }
            }
#pragma unroll
            for (int o = 4; o < 64; o <<= 1)
#pragma unroll
                for (int c = 0; c < 4; ++c) s4[c] += __shfl_xor(s4[c], o, WAVE);
            if (lane < 4) {
#pragma unroll
                for (int c = 0; c < 4; ++c) rs_wave[wv][4 * lane + c] = s4[c];
            }
        }
    }
    __syncthreads();
    // the row factor of row r: the waves' sums in wave order
    auto row_factor = [&](int r) {
        float s = 0.f;
        for (int w = 0; w < (int)(blockDim.x >> 6); ++w) s += rs_wave[w][r];
        return 1.0f / sqrtf(s / p.rs_k + p.rs_eps);
    };
    const int nthreads = blockDim.x;
    // sum of the KS partials of output element e (row-major over [mrows][wcols]), fixed order
    auto ksum = [&](int e) {
        const int row = e / wcols, c = e % wcols;
        const int mt = row >> 4, gg = (row & 15) >> 2, v = row & 3;
        const int gi = c / (NTW * 16), t = (c % (NTW * 16)) >> 4, rr = c & 15;
        const int ln = gg * 16 + rr;
        float s = 0.f;
        for (int k = 0; k < p.ks; ++k)
            s += slot[((size_t)(gi * p.ks + k) * MT * NTW * 4 * 64) + ((mt * NTW + t) * 4 + v) * 64 + ln];
        return s;
    };
    if constexpr (EPI == EPI_STORE) {
        // element-parallel store (+ residual); a row's wcols elements sit in wcols
        // consecutive lanes of one wave (wcols divides 64), so its sum of squares is
        // reduced with xor shuffles in a fixed order
        auto store = [&](int e, float res) {
            const int row = e / wcols, n = tile * wcols + e % wcols;
            float v = 0.f;
            if (e < mrows * wcols && n < p.N) {
                float* o = outp + (long long)(m0 + row) * p.ldo + n;
                v = ksum(e);
                if (rs_on) v *= row_factor(row);
                if (p.residual) v += RES_EARLY ? res : *o;
                *o = v;
                if constexpr (RES_EARLY) {
                    // the next GEMM's A operand(s): v * w_norm[n], rounded, in fragment order
                    if (p.n_z > 0 && e == (int)threadIdx.x) {
                        T* zo = reinterpret_cast<T*>(p.zout) + afrag_offset<T>(m0 + row, n, p.N);
#pragma unroll
                        for (int z = 0; z < GEMM_ZMAX; ++z) {
                            if (z < p.n_z) {
                                float wz;
                                if constexpr (sizeof(T) == 2) wz = bf16_to_f32((bf16_t)zg[z]);
                                else wz = __uint_as_float(zg[z]);
                                zo[z * p.zstride] = Elem<T>::from_f(v * wz);
                            }
                        }
                    }
                }
            }
            float ss = v * v;
            for (int w = 1; w < wcols; w <<= 1) ss += __shfl_xor(ss, w, WAVE);
            if (p.ssq_out && e < mrows * wcols && e % wcols == 0)
                p.ssq_out[(long long)tile * p.ssq_out_ld + m0 + row] = ss;
        };
        if constexpr (RES_EARLY) {
#pragma unroll
            for (int i = 0; i < RPT; ++i)
                if (i * nthreads < 16 * MT * wcols) store(threadIdx.x + i * nthreads, resid[i]);
        } else {
            for (int e0 = 0; e0 < 16 * MT * wcols; e0 += nthreads) store(e0 + threadIdx.x, 0.f);
        }
        if (p.snap_n > 0 && tile == 0 && blockIdx.y == 0 && blockIdx.z == 0)
            for (int i = threadIdx.x; i < p.snap_n; i += nthreads) p.snap_dst[i] = p.snap_src[i];
        return;
    }
    for (int e = threadIdx.x; e < mrows * wcols; e += nthreads) Ct[e] = rs_on ? ksum(e) * row_factor(e / wcols) : ksum(e);
    __syncthreads();
    gemm_epilogue<T, EPI>(p, L, tile, m0, mrows, wcols, Ct);
}

// --------------------------------------------------------------------------------------------
// SwiGLU, argmax and log-sum-exp epilogues: one wavefront per output row (rows strided
// over the waves).
// (The store epilogue is element-parallel, in the kernel.)

__device__ __forceinline__ int nthreads_epi(int threads, int lpr) { return threads / lpr; }

template <typename T, int EPI>
__device__ void gemm_epilogue(const GemmArgs& p, const GemmLayer& L, int tile, int m0, int mrows, int wcols,
                              const float* Ct) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int nwaves = blockDim.x >> 6;

    if (EPI == EPI_SWIGLU) {
        // Ct column c = gi*32 + t*16 + rr: t = 0 gate, t = 1 up (same output column gi*16 + rr)
        const int ocols = wcols / 2;
        const int n0 = tile * ocols;
        for (int row = wv; row < mrows; row += nwaves) {
            const int m = m0 + row;
            for (int co = lane; co < ocols; co += 64) {
                const int cg = (co >> 4) * 32 + (co & 15);
                const float gt = Ct[row * wcols + cg];
                const float up = Ct[row * wcols + cg + 16];
                const float h = gt / (1.0f + __expf(-gt)) * up;
                if (n0 + co < p.N)
                    reinterpret_cast<T*>(p.out_t)[p.out_frag ? afrag_offset<T>(m, n0 + co, p.N)
                                                             : (long long)m * p.ldo + n0 + co] = Elem<T>::from_f(h);
            }
        }
    } else if (EPI == EPI_ARGMAX || EPI == EPI_LSE) {
        // element-parallel: a row's wcols columns are spread over LPR consecutive lanes
        // (EPT consecutive columns each), all rows of the tile at once; the lanes of a row
        // combine with xor shuffles (a fixed order)
        constexpr int LPR = 8;
        const int ept = wcols / LPR;
        const int n0 = tile * wcols;
        const int G = p.gamma;
        const int sub = threadIdx.x % LPR;
        for (int row = threadIdx.x / LPR; row < ((mrows + 15) & ~15); row += nthreads_epi(blockDim.x, LPR)) {
            const int m = m0 + row;
            const bool live = row < mrows;
            const int b = m / G, jj = m % G;
            const bool dbg = live && p.dbg_logits && jj >= p.dbg_first;
            if (EPI == EPI_ARGMAX) {
                unsigned long long best = 0ull;
                for (int e = 0; e < ept; ++e) {
                    const int c = sub * ept + e, n = n0 + c;
                    if (live && n < p.N) {
                        const float v = Ct[row * wcols + c];
                        const unsigned long long key = pack_argmax(v, (uint32_t)n);
                        best = key > best ? key : best;
                        if (dbg) p.dbg_logits[((long long)b * (G - p.dbg_first) + (jj - p.dbg_first)) * p.N + n] = v;
                    }
                }
#pragma unroll
                for (int o = 1; o < LPR; o <<= 1) {
                    const unsigned long long other = __shfl_xor(best, o, WAVE);
                    best = other > best ? other : best;
                }
                if (live && sub == 0) p.amax[amax_slot(m, tile, p.n_tiles)] = best;
            } else {
                // the tile's largest logit mx and sum of exp(logit - mx); the lane holding
                // the row's label column stores its logit
                const int lab = (live && jj >= 1) ? p.labels[b * (G - 1) + jj - 1] : -1;
                float mx = -INFINITY;
                for (int e = 0; e < ept; ++e) {
                    const int c = sub * ept + e, n = n0 + c;
                    if (live && n < p.N) {
                        const float v = Ct[row * wcols + c];
                        mx = fmaxf(mx, v);
                        if (n == lab) p.lab_logit[m] = v;
                        if (dbg) p.dbg_logits[((long long)b * (G - p.dbg_first) + (jj - p.dbg_first)) * p.N + n] = v;
                    }
                }
#pragma unroll
                for (int o = 1; o < LPR; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, WAVE));
                float se = 0.f;
                for (int e = 0; e < ept; ++e) {
                    const int c = sub * ept + e;
                    if (live && n0 + c < p.N) se += __expf(Ct[row * wcols + c] - mx);
                }
#pragma unroll
                for (int o = 1; o < LPR; o <<= 1) se += __shfl_xor(se, o, WAVE);
                if (live && sub == 0) p.lse[(long long)tile * p.M + m] = make_float2(mx, se);
            }
        }
    }
}

// draft[i] = the vocabulary argmax of draft row i: row m = b*gamma + j with
// i = b*(gamma - first) + j - first, j >= first (first = 1: the drafts, rows after the
// anchor; 0: every row, a target's verification).  One workgroup per draft row reads the
// row's tile maxima (amax_slot layout): lane l of a round takes tile u*256 + l, so a wave's
// 64 loads fall in 8 cache lines (one per XCD run); tiles past the last one re-read the
// last tile (a repeated value leaves a maximum unchanged), so every load is unconditional
// and all of a lane's loads are in flight at once.  The maxima fold with the packed
// (value, index) order — the larger value, and the lower index among equal values, so the
// result does not depend on the order — in registers, across the wave with xor shuffles and
// across the waves in LDS.  No atomics and no second pass: one memory round trip after the
// launch.
constexpr int ARGMAX_FIN_LOADS = 24;       // tiles per thread per round (6144 per workgroup)
__global__ __launch_bounds__(256) void argmax_finish_kernel(const unsigned long long* __restrict__ amax, int n_tiles,
                                                            int gamma, int first, int* __restrict__ draft) {
    __shared__ unsigned long long red[4];
    const int i = blockIdx.x, per_seq = gamma - first;
    const int m = (i / per_seq) * gamma + first + i % per_seq;
    const int per = amax_per(n_tiles);
    const unsigned long long* row = amax + (long long)m * amax_ld(n_tiles);
    unsigned long long best = 0ull;
    for (int t0 = 0; t0 < n_tiles; t0 += 256 * ARGMAX_FIN_LOADS) {
        unsigned long long v[ARGMAX_FIN_LOADS];
#pragma unroll
        for (int u = 0; u < ARGMAX_FIN_LOADS; ++u) {
            const int t = min(t0 + u * 256 + (int)threadIdx.x, n_tiles - 1);
            v[u] = row[(t & 7) * per + (t >> 3)];
        }
#pragma unroll
        for (int u = 0; u < ARGMAX_FIN_LOADS; ++u) best = v[u] > best ? v[u] : best;
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const unsigned long long other = __shfl_xor(best, o, WAVE);
        best = other > best ? other : best;
    }
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = best;
    __syncthreads();
    if (threadIdx.x == 0) {
        unsigned long long x = red[0];
        for (int w = 1; w < 4; ++w) x = red[w] > x ? red[w] : x;
        draft[i] = (int)unpack_argmax_index(x);
    }
}

}  // namespace dflash
