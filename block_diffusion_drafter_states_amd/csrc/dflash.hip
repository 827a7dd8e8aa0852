// Host side of the DFlash C ABI: argument validation, workspace carving,
// launch planning and the kernel sequence of each entry point.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/dflash.h"
#include "attention.hpp"
#include "gemm.hpp"
#include "gemm_tiled.hpp"
#include "loss.hpp"
#include "small_kernels.hpp"

using namespace dflash;

// Fixed scratch of dflash_draft_block_noalloc (see below): file scope, one copy per GPU.
constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

namespace {

constexpr size_t ALIGN = 256;
constexpr int TARGET_MAX_LAYERS = 128;   // a verifying target model; the drafter's injection needs L <= MAX_LAYERS
constexpr size_t GEMM_MAX_LDS = 160 * 1024 - 4096;   // dynamic LDS per workgroup (static LDS needs the rest)

inline size_t align_up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

// Host-only audit of a call's workspace writes (dflash_audit_workspace).  Nothing is launched:
// each launch site reports, for every workspace buffer its kernel writes, the byte range that
// the kernel's indexing reaches with the launch's arguments and grid, and each range must lie
// inside the one region of the layout it starts in.
struct Audit {
    struct Region {
        size_t off, bytes;
    };
    uintptr_t base = 0;             // stand-in address of the workspace (never dereferenced)
    std::vector<Region> regions;
    int launches = 0, writes = 0, violations = 0;
    void write(const void* p, size_t bytes) {
        ++writes;
        const uintptr_t a = reinterpret_cast<uintptr_t>(p);
        if (bytes == 0) return;
        if (a < base) {
            ++violations;
            return;
        }
        const size_t off = a - base;
        for (const Region& r : regions)
            if (off >= r.off && off < r.off + r.bytes) {
                if (off + bytes > r.off + r.bytes) ++violations;
                return;
            }
        ++violations;   // starts in no region (padding, or past the workspace)
    }
};

// Records caller-provided events around each launch (see dflash_trace); with `au` set the
// launches are only audited, not made.
struct Tracer {
    dflash_trace* t;
    hipStream_t st;
    int i = 0;
    Audit* au = nullptr;
    void begin(const char* name) {
        if (au) ++au->launches;
        if (t && i < t->capacity) {
            if (t->names) t->names[i] = name;
            if (t->events && t->events[2 * i]) (void)hipEventRecord(static_cast<hipEvent_t>(t->events[2 * i]), st);
        }
    }
    void end() {
        if (t && i < t->capacity && t->events && t->events[2 * i + 1])
            (void)hipEventRecord(static_cast<hipEvent_t>(t->events[2 * i + 1]), st);
        ++i;
        if (t) t->count = i;
    }
};
inline int cdiv(int a, int b) { return (a + b - 1) / b; }
inline int pad16(int m) { return cdiv(m, 16) * 16; }

// A launch through the tracer: made, or (audit) only counted.
#define DFL_LAUNCH(tr, ...)                                  \
    do {                                                     \
        if (!(tr).au) hipLaunchKernelGGL(__VA_ARGS__);       \
    } while (0)
inline bool launched(const Tracer& tr) { return tr.au || hipGetLastError() == hipSuccess; }

// Write extents (bytes from the buffer's start) of the two activation layouts: plain rows
// (rows x cols elements, ld apart) and the weight-streaming GEMM's fragment order
// (afrag_offset over M rows x K columns; the largest offset lies in the last 16-row tile
// and the last 256-byte step, which are searched exhaustively).
inline size_t span_rows(long long rows, long long ld, long long cols, int esize) {
    return rows > 0 && cols > 0 ? (size_t)(((rows - 1) * ld + cols) * esize) : 0;
}
template <typename T>
size_t span_afrag(int M, int K) {
    constexpr int S = 256 / (int)sizeof(T);
    long long mx = -1;
    for (int m = std::max(0, M - 16); m < M; ++m)
        for (int k = std::max(0, K - S); k < K; ++k) mx = std::max(mx, afrag_offset<T>(m, k, K));
    return (size_t)(mx + 1) * sizeof(T);
}
template <typename T>
size_t span_act(int frag, int M, int cols, long long ld) {
    return frag ? span_afrag<T>(M, cols) : span_rows(M, ld, cols, (int)sizeof(T));
}

constexpr int MAX_GAMMA = 16;     // block rows: one 16-row MFMA tile per (sequence, q head)
constexpr int LSE_MAX_SLICES = 256; // block loss: slices of the LM-head tiles folded per row in stage 1

struct Shape {
    int H, nq, nkv, D, I, L, F, V, gmax, mask, Bmax, cap, esize, step, group, rpad, chunk, nch_max;
    float eps;
    bool bf16;
    bool att_narrow;    // 128-key chunks for four-wave attention workgroups (two per CU)
};

int make_shape(const dflash_config* c, Shape& s) {
    if (!c) return DFLASH_EINVAL;
    if (c->dtype != DFLASH_F32 && c->dtype != DFLASH_BF16) return DFLASH_EUNSUPPORTED;
    s.bf16 = c->dtype == DFLASH_BF16;
    s.esize = s.bf16 ? 2 : 4;
    s.step = s.bf16 ? 128 : 64;
    s.H = c->hidden; s.nq = c->n_q_heads; s.nkv = c->n_kv_heads; s.D = c->head_dim; s.I = c->inter;
    s.L = c->n_layers; s.F = c->n_feat; s.V = c->vocab; s.gmax = c->gamma_max; s.mask = c->mask_token_id;
    s.Bmax = c->max_batch; s.cap = c->kv_capacity; s.eps = c->rms_eps;
    if (s.H <= 0 || s.nq <= 0 || s.nkv <= 0 || s.D <= 0 || s.I <= 0 || s.L <= 0 || s.F <= 0 || s.V < 2 ||
        s.Bmax <= 0 || s.cap <= 0 || !(s.eps > 0.f) || !std::isfinite(s.eps))
        return DFLASH_EINVAL;
    if (s.gmax < 2 || s.gmax > MAX_GAMMA) return DFLASH_EINVAL;
    if (s.mask < 0 || s.mask >= s.V) return DFLASH_EINVAL;
    if (s.nq % s.nkv) return DFLASH_EUNSUPPORTED;
    if (s.D * s.esize != 256) return DFLASH_EUNSUPPORTED;
    if (s.L > TARGET_MAX_LAYERS) return DFLASH_EUNSUPPORTED;   // the injection needs L <= MAX_LAYERS
    if (s.cap % 64) return DFLASH_EUNSUPPORTED;
    if (s.H % s.step || s.I % s.step || (s.nq * s.D) % s.step || ((long long)s.F * s.H) % s.step)
        return DFLASH_EUNSUPPORTED;
    if (s.H % 128 || (s.nq * s.D) % 128 || (s.nkv * s.D) % 128 || s.I % 64) return DFLASH_EUNSUPPORTED;
    if (cdiv(s.H, 16) > NORM_MAX_PARTIALS) return DFLASH_EUNSUPPORTED;   // per-tile sums of squares of a row
    if (s.H > EMBED_MAX_HIDDEN) return DFLASH_EUNSUPPORTED;
    s.group = s.nq / s.nkv;
    if (s.group * s.gmax > 256) return DFLASH_EUNSUPPORTED;
    s.rpad = cdiv(s.group * s.gmax, 16) * 16;
    // context keys per attention chunk: the largest power of two in 256 .. 1024 that
    // still gives >= 1024 workgroups (four per CU) when the cache is full.  A workgroup
    // streams its chunk through the LDS ring, so longer chunks amortise its start (query
    // build, first loads) and its partial write; below four per CU the GPU idles.  2048-key
    // chunks leave too few, too long workgroups for the slots of a ragged batch
    // (LLaMA-3.1-8B shape, batch 32, contexts 512..8192: 888 workgroups with keys for 512
    // slots; 1024-key chunks: attention 795 -> 683 us per cycle)
    int ch = 1024;
    while (ch > 256 && (long long)s.Bmax * s.nkv * cdiv(s.cap, ch) < 1024) ch >>= 1;
    // 128-key chunks when even those fit one round of workgroups (one per CU): shorter
    // chunks shorten every workgroup (measured: Qwen3-4B shape, context 1024, batch 1:
    // attention 88 -> 70 us per cycle; at context 4096 the 272 workgroups of 128-key
    // chunks would need two rounds, 91 -> 119 us)
    const long long nqs_max = cdiv(cdiv(s.group * s.gmax, 16), ATT_MAX_TILES);
    s.att_narrow = false;
    if (ch == 256 && (1 + cdiv(s.cap, 128)) * (long long)s.nkv * nqs_max * s.Bmax <= 256) {
        ch = 128;
    } else if (ch == 256 && cdiv(s.group * s.gmax, 16) == 4 &&
               (1 + cdiv(s.cap, 256)) * (long long)s.nkv * s.Bmax < 256 &&
               (1 + cdiv(s.cap, 128)) * (long long)s.nkv * s.Bmax <= 512) {
        // four query tiles (group 4 at block size 16) whose 256-key chunks leave CUs idle
        // (the Qwen3-8B shape at context 4096: 144 workgroups for 256 CUs): 128-key chunks
        // in four-wave workgroups, one wave per tile over the whole chunk, 64 KB of LDS and
        // so two workgroups per CU - one round of 272 workgroups
        ch = 128;
        s.att_narrow = true;
    }
    s.chunk = ch;
    s.nch_max = 1 + cdiv(s.cap, ch);
    if (s.nch_max > MERGE_MAX_CHUNKS) return DFLASH_EUNSUPPORTED;
    return DFLASH_OK;
}

struct GemmPlan {
    int ns, ks, kw, n_tiles, mt, mgroups, layers, ntw, epi;
    int ring;       // weight-streaming kernel: ring depth (k-steps in flight per wave); 0 = the default
    bool tiled;     // gemm_tiled_kernel (many rows) instead of the weight-streaming kernel
    int bn;         // tiled: weight rows per workgroup (128, or 64 when that leaves CUs idle)
    int kb;         // tiled: bytes of every row per LDS stage (256; 128 for launches with many workgroups)
    int bm;         // tiled: rows of A per workgroup (TG_BM, or 2 x TG_BM with 128-byte stages)
    size_t lds;
};

constexpr int TILED_MIN_ROWS = 128;   // from this many rows on, A is reused from LDS across 128 weight rows
// ... except where the tiled launch would have fewer than TILED_MIN_WGS workgroups
// while the weight-streaming one (K split inside the workgroup, each weight read once
// per 64-row group) fits one round of STREAM_ROUND_WGS (one per CU).  Measured on
// MI355X at 128 rows: 2048-wide projections (32 tiled blocks against 256 streaming
// workgroups) 40 -> 24 us for W_o and 49 -> 31 us for W_down; 2560-wide ones (40
// blocks against 320 workgroups, two rounds) stay faster tiled (38 against 41 us).
constexpr int TILED_MIN_WGS = 128;
constexpr int STREAM_ROUND_WGS = 256;

// Geometry of one projection.  wrows = weight rows (EPI_SWIGLU: rows of each of
// gate/up).  Every workgroup owns complete output columns (no cross-workgroup
// reduction); its waves split K (ks) and rows (ns).  The A operand is always a
// storage-type matrix (rows normalised by rmsnorm_rows_kernel, or x * w_norm stored by the
// producing GEMM where the norm is carried across).
// Choices follow sweeps on MI355X at 16 rows: store projections in 16-column tiles
// (ntw 1) with 8 waves along K (128 KB of ring, one workgroup per CU) when the launch
// has at most one workgroup per CU, else 4 waves (64 KB, two per CU, so that every
// workgroup is resident at once: q|k|v at the Qwen3-8B shape, 384 workgroups, 88.6 ->
// 87.4 us per cycle, at the Coder-30B drafter shape (320) 76.0 -> 59.1 us, against
// 32-column tiles with 4 waves, 192 workgroups, one per CU); 4 waves per 16 gate + 16 up
// rows for SwiGLU; 4 waves per 32 vocabulary rows for the LM head over one 16-row tile, 2
// over more; one workgroup's LDS ring must fit the 160 KB of a CU.
GemmPlan plan_streaming(const Shape& s, int epi, int wrows, int K, int M, int layers) {
    GemmPlan p;
    p.bn = 0;
    p.kb = 0;
    p.bm = 0;
    p.epi = epi;
    p.layers = layers;
    p.tiled = false;
    p.mt = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
    p.mgroups = cdiv(M, 16 * p.mt);
    p.ns = 1;
    p.ntw = 2;
    int ks;
    if (epi == EPI_ARGMAX || epi == EPI_LSE) {
        // the LM head over one 16-row tile: four waves on a 2-stage ring (64 KB, two workgroups
        // per CU), measured at the Qwen3-8B shape with the non-temporal weight stream: argmax
        // 199.2 -> 179.5 us per launch (6.9 TB/s) against two waves on a 4-stage ring
        ks = p.mt == 1 ? 4 : 2;
    } else if (epi == EPI_SWIGLU) {
        // measured at 16 rows: four waves (128 KB of ring, three rounds of one workgroup per CU)
        // 40.8 us per Qwen3-8B gate|up launch; two waves (64 KB, two per CU, 1.5 rounds) 45 us
        ks = 4;
    } else {
        p.ntw = 1;
        ks = cdiv(wrows, 16) * layers > STREAM_ROUND_WGS ? 4 : 8;
    }
    if (epi == EPI_SWIGLU) p.n_tiles = cdiv(wrows, 16);   // 16 gate + 16 up rows per workgroup
    else p.n_tiles = cdiv(wrows, p.ns * p.ntw * 16);
    // gate|up over one 16-row tile: a 2-stage ring (64 KB) so that two workgroups share a CU
    // and one streams while the other starts or runs its epilogue (measured at the Qwen3-8B
    // shape, 768 workgroups: 47 -> 39.6 us per launch; a 4-stage ring, one workgroup per
    // CU, idles each CU between its three workgroups; HIP-event times)
    p.ring = ((epi == EPI_SWIGLU || epi == EPI_ARGMAX || epi == EPI_LSE) && p.mt == 1) ? 2 : 0;
    const int ring = p.ring ? p.ring : gemm_ring_depth(p.mt, p.ntw);
    while (ks > 1 && K / s.step < 2 * ks) ks /= 2;        // at least two k-steps per wave
    while (ks > 1 && gemm_lds_bytes_host(p.ns, ks, p.mt, p.ntw, ring) > GEMM_MAX_LDS) ks /= 2;
    p.ks = ks;
    p.kw = cdiv(cdiv(K, ks), s.step) * s.step;
    p.lds = gemm_lds_bytes_host(p.ns, p.ks, p.mt, p.ntw, ring);
    return p;
}

GemmPlan plan_gemm(const Shape& s, int epi, int wrows, int K, int M, int layers) {
    const GemmPlan ps = plan_streaming(s, epi, wrows, K, M, layers);
    if (M < TILED_MIN_ROWS) return ps;
    GemmPlan p = ps;
    p.tiled = true;
    p.ns = 1;
    p.ks = 4;
    p.kw = K;
    p.mt = 8;
    p.ntw = 0;
    p.bm = TG_BM;
    p.mgroups = cdiv(M, p.bm);
    p.bn = 128;
    // 64-wide blocks when 128-wide ones would leave half the CUs idle (measured at 512 rows:
    // down 4096 x 14336 138 -> 90 us; q|k|v 6144 x 4096, 192 blocks, 47 -> 58 us the other way)
    if (epi != EPI_SWIGLU && cdiv(wrows, 128) * p.mgroups * layers <= 128) p.bn = 64;
    p.n_tiles = cdiv(wrows, tg_cols(epi, p.bn));
    const long long tiled_wgs = (long long)p.n_tiles * p.mgroups * layers;
    if (tiled_wgs < TILED_MIN_WGS && (long long)ps.n_tiles * ps.mgroups * layers <= STREAM_ROUND_WGS) return ps;
    // 128-byte stages (64 KB at BN 128: several workgroups per CU) pay off from ~2
    // workgroups per CU on (measured at 512 rows: LM head 857 -> 636 us, gate|up
    // 182 -> 143 us; with 256 workgroups they pack onto fewer CUs and lose)
    p.kb = tiled_wgs >= 512 ? 128 : 256;
    // 256-row blocks (eight waves, 96 KB of LDS, one workgroup per CU) for those launches:
    // a quarter fewer bytes staged per flop and fewer loads issued per wave per k-step.
    // Measured at 512 rows: gate|up 660.7 -> 624.5 us per cycle; the 4096-row prefill 1535.6
    // -> 1442.6 us; not for the LM-head epilogues (argmax 540.1 -> 561.6 us)
    if (p.kb == 128 && p.bn == 128 && M >= 2 * TG_BM && epi != EPI_ARGMAX && epi != EPI_LSE) {
        p.bm = 2 * TG_BM;
        p.mgroups = cdiv(M, p.bm);
    }
    p.lds = tg_lds_bytes(p.bm, p.bn, p.kb);
    return p;
}

// Attention launch shape: a workgroup takes QTW query tiles (the next power of
// two >= the tiles of one (b, h), at most ATT_MAX_TILES) of one (b, h, chunk).
// The ring is 8 stages unless the launch has at least ATT_SMALL_RING_WGS
// workgroups, when 4-stage rings are used.
constexpr long long ATT_SMALL_RING_WGS = 512;

struct AttnPlan {
    int qtw, nqs, ring, kg;
};

AttnPlan plan_attn(const Shape& s, int gamma, int batch) {
    AttnPlan a;
    const int qt = cdiv(s.group * gamma, 16);
    a.qtw = 1;
    while (a.qtw < qt && a.qtw < ATT_MAX_TILES) a.qtw *= 2;
    a.nqs = cdiv(qt, a.qtw);
    a.ring = (long long)s.nch_max * s.nkv * a.nqs * batch >= ATT_SMALL_RING_WGS ? 4 : 8;
    a.kg = att_default_kg(a.qtw);
    // eight tiles in a launch of many workgroups: two four-wave workgroups of four tiles each
    // (the same eight waves per CU as one eight-wave workgroup, finer-grained balance; the
    // second workgroup of a chunk finds its K/V in the last-level cache).  Coder-30B-drafter
    // shape, batch 8, gamma 16: attention 952 -> 924 us per cycle
    if (a.qtw == 8 && a.ring == 4) {
        a.qtw = 4;
        a.nqs = cdiv(qt, 4);
    }
    // four waves, one per tile, 64 KB ring: the kernel's 209 VGPRs allow two such workgroups
    // per CU (eight-wave ones: one), which doubles the K/V bytes each CU keeps in flight - for
    // the 128-key chunks of the Qwen3-8B shape, and for launches with many workgroups
    if (a.qtw == 4 && (s.att_narrow || a.ring == 4)) {
        a.kg = 1;
        a.ring = 4;
    }
    return a;
}

template <typename T, int QTW, int RING, int KG>
void launch_attention_k(const AttnArgs& a, dim3 grid, hipStream_t st) {
    hipLaunchKernelGGL((attn_partial_kernel<T, QTW, RING, KG>), grid, dim3(64 * AttGeom<QTW, RING, KG>::WAVES),
                       attn_lds_bytes_host(RING), st, a);
}

template <typename T, int QTW>
void launch_attention_q(const AttnArgs& a, const AttnPlan& ap, dim3 grid, hipStream_t st) {
    constexpr int KG = att_default_kg(QTW);
    if constexpr (QTW == 4) {
        if (ap.kg == 1) {
            launch_attention_k<T, QTW, 4, 1>(a, grid, st);
            return;
        }
    }
    if (ap.ring == 4) launch_attention_k<T, QTW, 4, KG>(a, grid, st);
    else launch_attention_k<T, QTW, 8, KG>(a, grid, st);
}

template <typename T>
int launch_attention(const AttnArgs& a, const AttnPlan& ap, int nch_max, int nkv, int batch, hipStream_t st,
                     Tracer& tr) {
    const dim3 grid(nch_max, nkv * ap.nqs, batch);
    if (ap.ring != 4 && ap.ring != 8) return DFLASH_EINVAL;
    if (ap.qtw != 1 && ap.qtw != 2 && ap.qtw != 4 && ap.qtw != 8) return DFLASH_EINVAL;
    if (tr.au) {    // partial (m, l, O) of every (b, h, chunk) and query row R < group * gamma <= rpad
        const long long rows = (long long)a.group * a.gamma;
        const long long last = (((long long)(batch - 1) * nkv + nkv - 1) * nch_max + nch_max - 1) * a.rpad + rows;
        tr.au->write(a.opart, (size_t)(last * (256 / sizeof(T)) * sizeof(T)));
        tr.au->write(a.mlpart, (size_t)(last * 2 * 4));
        return rows <= a.rpad ? DFLASH_OK : DFLASH_EUNSUPPORTED;
    }
    switch (ap.qtw) {
        case 1: launch_attention_q<T, 1>(a, ap, grid, st); break;
        case 2: launch_attention_q<T, 2>(a, ap, grid, st); break;
        case 4: launch_attention_q<T, 4>(a, ap, grid, st); break;
        case 8: launch_attention_q<T, 8>(a, ap, grid, st); break;
        default: return DFLASH_EINVAL;
    }
    return hipGetLastError() == hipSuccess ? DFLASH_OK : DFLASH_ELAUNCH;
}

struct InjectPlans {
    GemmPlan fuse, kv;
};

InjectPlans inject_plans(const Shape& s, int batch, int rows) {
    const int M = batch * rows;
    return {plan_gemm(s, EPI_STORE, s.H, s.F * s.H, M, 1), plan_gemm(s, EPI_STORE, 2 * s.nkv * s.D, s.H, M, s.L)};
}

struct DraftPlans {
    GemmPlan qkv, o, gateup, down, lm;
};

DraftPlans draft_plans(const Shape& s, int M) {
    return {plan_gemm(s, EPI_STORE, (s.nq + 2 * s.nkv) * s.D, s.H, M, 1), plan_gemm(s, EPI_STORE, s.H, s.nq * s.D, M, 1),
            plan_gemm(s, EPI_SWIGLU, s.I, s.H, M, 1), plan_gemm(s, EPI_STORE, s.H, s.I, M, 1),
            plan_gemm(s, EPI_ARGMAX, s.V, s.H, M, 1)};
}

// Workspace carving, sized from the same plans that the launches use.  Everything
// is per-call scratch: no state survives a call.
struct Layout {
    // draft
    size_t x, ssq_x, qkv, opart, mlpart, obuf, hbuf, amax, nbuf, lse_part, lab, lse_row,
        draft_end;
    int ssq_x_tiles, amax_tiles;
    // inject
    size_t c, ssq_c, cnorm, kvraw, lensnap, inject_end;
    int ssq_c_tiles;
    std::vector<Audit::Region> regions;     // every carved buffer: offset and requested bytes
};

// Row stride of the per-tile sums of squares a store GEMM writes for the next RMSNorm: the rows
// rounded up to 4, so that a consumer's 16-byte loads of four rows stay aligned (the padding rows
// are loaded and never used).
constexpr int ssq_ld(long long rows) { return (int)((rows + 3) & ~3LL); }

Layout make_layout(const Shape& s, int batch, int rows) {
    Layout l;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        l.regions.push_back({o, bytes});
        off = align_up(off + bytes);
        return o;
    };
    const size_t M = (size_t)batch * s.gmax;
    // tile counts from the weight-streaming plans, which have the most tiles (the tiled
    // plans of a call with many rows use fewer), so any call's plans fit
    const DraftPlans dp = draft_plans(s, std::min((int)M, TILED_MIN_ROWS - 1));
    l.ssq_x_tiles = std::max(1, std::max(dp.o.n_tiles, dp.down.n_tiles));
    l.amax_tiles = dp.lm.n_tiles;
    l.x = take(M * s.H * 4);
    l.ssq_x = take((size_t)l.ssq_x_tiles * ssq_ld(M) * 4);
    l.qkv = take(M * (size_t)(s.nq + 2 * s.nkv) * s.D * 4);
    l.opart = take((size_t)batch * s.nkv * s.nch_max * s.rpad * s.D * s.esize);
    l.mlpart = take((size_t)batch * s.nkv * s.nch_max * s.rpad * 2 * 4);
    const size_t Mp = pad16((int)M);                          // GEMM A operands: whole 16-row tiles
    l.obuf = take(Mp * s.nq * s.D * s.esize);
    l.hbuf = take(Mp * s.I * s.esize);
    l.amax = take((size_t)amax_ld(l.amax_tiles) * M * 8);     // per-tile maxima (amax_slot), or [tile][M] float2
    l.nbuf = take(Mp * s.H * s.esize);                        // RMSNorm-ed rows (GEMM A operand)
    l.lse_part = take((size_t)LSE_MAX_SLICES * M * 8);        // block loss: per-slice (max, sum exp)
    l.lab = take(M * 4);                                      // block loss: the label's logit per row
    l.lse_row = take(M * 4);                                  // block loss: log-sum-exp per row (gradient)
    l.draft_end = off;
    l.c = l.ssq_c = l.cnorm = l.kvraw = l.lensnap = 0;
    l.ssq_c_tiles = 0;
    if (rows > 0) {
        const size_t Mi = (size_t)batch * rows;
        l.ssq_c_tiles = plan_gemm(s, EPI_STORE, s.H, s.F * s.H, std::min((int)Mi, TILED_MIN_ROWS - 1), 1).n_tiles;
        l.c = take(Mi * s.H * 4);
        l.ssq_c = take((size_t)l.ssq_c_tiles * ssq_ld(Mi) * 4);
        l.cnorm = take((size_t)s.L * pad16((int)Mi) * s.H * s.esize);   // per-layer RMSNorm-ed rows
        l.kvraw = take((size_t)s.L * Mi * 2 * s.nkv * s.D * 4); // per-layer k | v projections
        l.lensnap = take((size_t)batch * 4);                     // len before this injection
    }
    l.inject_end = off;
    return l;
}

template <typename T, int EPI, int MT, int NTW>
int launch_gemm(const GemmArgs& a, const GemmPlan& p, hipStream_t st, Tracer& tr, const char* name) {
    constexpr int P = gemm_ring_depth(MT, NTW);
    // the one non-default ring: gate|up and the LM head over one 16-row tile, 2 stages
    constexpr bool RING2 = (EPI == EPI_SWIGLU || EPI == EPI_ARGMAX || EPI == EPI_LSE) && MT == 1;
    if (p.ring && p.ring != P && !(RING2 && p.ring == 2)) return DFLASH_EINVAL;
    dim3 grid(p.n_tiles, p.mgroups, p.layers);
    tr.begin(name);
    if (p.ring && p.ring != P) {
        if constexpr (RING2)
            DFL_LAUNCH(tr, (gemm_kernel<T, EPI, MT, NTW, 2>), grid, dim3(64 * p.ns * p.ks), p.lds, st, a);
    } else {
        DFL_LAUNCH(tr, (gemm_kernel<T, EPI, MT, NTW, P>), grid, dim3(64 * p.ns * p.ks), p.lds, st, a);
    }
    const bool ok = launched(tr);
    tr.end();
    return ok ? DFLASH_OK : DFLASH_ELAUNCH;
}

template <typename T, int EPI, int NTW>
int launch_gemm_mt(const GemmArgs& a, const GemmPlan& p, hipStream_t st, Tracer& tr, const char* name) {
    switch (p.mt) {
        case 1: return launch_gemm<T, EPI, 1, NTW>(a, p, st, tr, name);
        case 2: return launch_gemm<T, EPI, 2, NTW>(a, p, st, tr, name);
        case 4: return launch_gemm<T, EPI, 4, NTW>(a, p, st, tr, name);
    }
    return DFLASH_EINVAL;
}

template <typename T, int EPI, int BN>
int launch_gemm_tiled(const GemmArgs& a, const GemmPlan& p, hipStream_t st, Tracer& tr, const char* name) {
    dim3 grid(cdiv(p.n_tiles, 8) * 8, p.mgroups, p.layers);   // the kernel maps blocks XCD-aware
    if (p.bm != TG_BM && (p.bm != 2 * TG_BM || p.kb != 128 || BN != 128)) return DFLASH_EINVAL;
    if (p.kb != 128 && p.kb != 256) return DFLASH_EINVAL;
    tr.begin(name);
    if (p.bm == 2 * TG_BM) {
        if constexpr (BN == 128)
            DFL_LAUNCH(tr, (gemm_tiled_kernel<T, EPI, BN, 128, 2 * TG_BM>), grid, dim3(tg_threads(2 * TG_BM)), p.lds,
                       st, a);
    } else if (p.kb == 128) {
        DFL_LAUNCH(tr, (gemm_tiled_kernel<T, EPI, BN, 128, TG_BM>), grid, dim3(tg_threads(TG_BM)), p.lds, st, a);
    } else {
        DFL_LAUNCH(tr, (gemm_tiled_kernel<T, EPI, BN, 256, TG_BM>), grid, dim3(tg_threads(TG_BM)), p.lds, st, a);
    }
    const bool ok = launched(tr);
    tr.end();
    return ok ? DFLASH_OK : DFLASH_ELAUNCH;
}

// Workspace writes of a GEMM launch (both kernels): per layer the store output (rows < M,
// columns < N), the per-tile sums of squares [tile < n_tiles][m < M], the SwiGLU output,
// the per-tile argmax / log-sum-exp slots [tile < n_tiles][m < M] and the label logits.
template <typename T>
void audit_gemm(const GemmArgs& a, const GemmPlan& p, Audit& au) {
    for (int z = 0; z < p.layers; ++z) {
        const GemmLayer& L = a.layer[z];
        if (p.epi == EPI_STORE) au.write(L.out ? L.out : a.out, span_rows(a.M, a.ldo, a.N, 4));
    }
    if (p.epi == EPI_STORE && a.ssq_out) au.write(a.ssq_out, span_rows(p.n_tiles, a.ssq_out_ld, a.M, 4));
    if (p.epi == EPI_SWIGLU) au.write(a.out_t, span_act<T>(a.out_frag, a.M, a.N, a.ldo));
    if (p.epi == EPI_ARGMAX) au.write(a.amax, span_rows(a.M, amax_ld(p.n_tiles), amax_ld(p.n_tiles), 8));
    if (p.epi == EPI_LSE) {
        au.write(a.lse, span_rows(p.n_tiles, a.M, a.M, 8));
        au.write(a.lab_logit, (size_t)a.M * 4);
    }
    if (a.n_z > 0) au.write(a.zout, (size_t)(a.n_z - 1) * a.zstride * sizeof(T) + span_act<T>(1, a.M, a.N, a.N));
    if (a.snap_n > 0) au.write(a.snap_dst, (size_t)a.snap_n * 4);
}

// An RMSNorm can be carried across a GEMM pair (the producer's store epilogue writes x * w_norm
// in fragment order, the consumer multiplies its output rows by the norm's row factor) when
// both are weight-streaming launches over one tile of at most 16 rows (a multiple of 4: the
// consumer reads the sums of squares of 4 rows in one 16-byte load), the producer's store
// epilogue has one output element per thread and the consumer's threads can hold the
// producer's per-tile sums of squares in GEMM_RSQ loads each.
bool fold_producer_ok(const GemmPlan& p, int M) {
    return !p.tiled && p.mt == 1 && p.epi == EPI_STORE && M <= 16 &&
           16 * p.ns * p.ntw * 16 <= 64 * p.ns * p.ks;
}
bool fold_consumer_ok(const GemmPlan& c, int rs_n, int M) {
    return !c.tiled && c.mt == 1 && (c.epi == EPI_STORE || c.epi == EPI_SWIGLU) && M <= 16 &&
           rs_n >= 1 && rs_n <= GEMM_RSQ * 64 * c.ns * c.ks / 4;
}

template <typename T>
int gemm_dispatch(const GemmArgs& a, const GemmPlan& p, hipStream_t st, Tracer& tr, const char* name) {
    if (p.layers < 1 || p.layers > MAX_LAYERS || a.M < 1) return DFLASH_EINVAL;
    if (a.rs_ssq && (!fold_consumer_ok(p, a.rs_n, a.M) || a.rs_ld % 4 || a.rs_ld < a.M || !a.a_frag))
        return DFLASH_EINVAL;
    if (a.n_z && (a.n_z < 0 || a.n_z > GEMM_ZMAX || !fold_producer_ok(p, a.M) || !a.zout)) return DFLASH_EINVAL;
    if (a.snap_n && (p.tiled || p.epi != EPI_STORE || !a.snap_src || !a.snap_dst)) return DFLASH_EINVAL;
    if (tr.au) audit_gemm<T>(a, p, *tr.au);
    if (p.tiled) {
        if (a.a_frag || a.out_frag) return DFLASH_EINVAL;     // the tiled kernel reads and writes plain rows
        for (int k = 0; k < 2; ++k)     // a 16-row weight tile never straddles two segments
            if (a.seg_end[k] < a.N && a.seg_end[k] % 16) return DFLASH_EINVAL;
        const bool wide = p.bn == 128;
        switch (p.epi) {
            case EPI_STORE:
                return wide ? launch_gemm_tiled<T, EPI_STORE, 128>(a, p, st, tr, name)
                            : launch_gemm_tiled<T, EPI_STORE, 64>(a, p, st, tr, name);
            case EPI_SWIGLU: return wide ? launch_gemm_tiled<T, EPI_SWIGLU, 128>(a, p, st, tr, name) : DFLASH_EINVAL;
            case EPI_ARGMAX:
                return wide ? launch_gemm_tiled<T, EPI_ARGMAX, 128>(a, p, st, tr, name)
                            : launch_gemm_tiled<T, EPI_ARGMAX, 64>(a, p, st, tr, name);
            case EPI_LSE:
                return wide ? launch_gemm_tiled<T, EPI_LSE, 128>(a, p, st, tr, name)
                            : launch_gemm_tiled<T, EPI_LSE, 64>(a, p, st, tr, name);
        }
        return DFLASH_EINVAL;
    }
    if (p.epi == EPI_STORE && (p.ns != 1 || 64 % (p.ntw * 16))) return DFLASH_EINVAL;   // store epilogue layout
    for (int k = 0; k < 2; ++k)     // a 16-row weight tile never straddles two segments
        if (a.seg_end[k] < a.N && a.seg_end[k] % 16) return DFLASH_EINVAL;
    switch (p.epi) {
        case EPI_STORE: return p.ntw == 1 ? launch_gemm_mt<T, EPI_STORE, 1>(a, p, st, tr, name) : DFLASH_EINVAL;
        case EPI_SWIGLU: return launch_gemm_mt<T, EPI_SWIGLU, 2>(a, p, st, tr, name);
        case EPI_ARGMAX: return launch_gemm_mt<T, EPI_ARGMAX, 2>(a, p, st, tr, name);
        case EPI_LSE: return launch_gemm_mt<T, EPI_LSE, 2>(a, p, st, tr, name);
    }
    return DFLASH_EINVAL;
}

GemmArgs gemm_base(const Shape& s, const GemmPlan& p, int M, int K) {
    GemmArgs a;
    std::memset(&a, 0, sizeof(a));
    a.M = M;
    a.K = K;
    a.ns = p.ns;
    a.ks = p.ks;
    a.kw = p.kw;
    a.n_tiles = p.n_tiles;
    a.n_layers = p.layers;
    return a;
}

bool weights_ok(const Shape& s, const dflash_weights* w, bool need_fuse = true) {
    if (!w || (need_fuse && !w->w_fuse) || !w->embed || !w->final_norm || !w->lm_head || !w->rope_cos ||
        !w->rope_sin || !w->layers)
        return false;
    for (int l = 0; l < s.L; ++l) {
        const dflash_layer_weights& x = w->layers[l];
        if (!x.in_norm || !x.wq || !x.wk || !x.wv || !x.q_norm || !x.k_norm || !x.wo || !x.post_norm ||
            !x.w_gate || !x.w_up || !x.w_down)
            return false;
    }
    return true;
}

// A operand = RMSNorm(x; w) in the storage type: rows normalised into nbuf by
// rmsnorm_rows_kernel (rstd from the producers' per-tile sums of squares), in fragment
// order when the consumer is the weight-streaming GEMM (afrag).
template <typename T>
int set_norm_a(GemmArgs& a, const Shape& s, const float* x, int M, const float* ssq, int n_ssq, const void* w,
               void* nbuf, int afrag, hipStream_t st, Tracer& tr, bool row_factor = true) {
    NormWeights nw{};
    nw.w[0] = w;
    tr.begin("rmsnorm");
    if (tr.au) tr.au->write(nbuf, span_act<T>(afrag, M, s.H, s.H));
    DFL_LAUNCH(tr, (rmsnorm_rows_kernel<T>), dim3(M, cdiv(s.H, 1024), 1), dim3(256), 0, st, x, s.H, ssq, n_ssq, ssq_ld(M),
               nw, s.H, s.eps, static_cast<T*>(nbuf), s.H, 0LL, nullptr, nullptr, 0, afrag, row_factor ? 1 : 0);
    tr.end();
    a.a = nbuf;
    a.lda = s.H;
    a.a_frag = afrag;
    return launched(tr) ? DFLASH_OK : DFLASH_ELAUNCH;
}

// A operand = the rows x * w_norm that the producing GEMM wrote into nbuf (fragment order);
// this GEMM multiplies its output rows by the norm's row factor, from the producer's
// per-tile sums of squares of x.
void set_carried_norm_a(GemmArgs& a, const Shape& s, void* nbuf, const float* ssq, int n_ssq, int M) {
    a.a = nbuf;
    a.lda = s.H;
    a.a_frag = 1;
    a.rs_ssq = ssq;
    a.rs_n = n_ssq;
    a.rs_ld = ssq_ld(M);
    a.rs_k = (float)s.H;
    a.rs_eps = s.eps;
}

template <typename T>
int run_inject(const Shape& s, const dflash_weights* w, const dflash_kv* kv, int batch, const void* feat,
               int rows, const int* n_new, void* ws, const Layout& lay, hipStream_t st, Tracer& tr) {
    char* wsb = static_cast<char*>(ws);
    const InjectPlans pl = inject_plans(s, batch, rows);
    const int M = batch * rows;
    if ((long long)batch * cdiv(rows, KV_ROWS) > 65535) return DFLASH_EUNSUPPORTED;   // kv_finish grid
    float* c = reinterpret_cast<float*>(wsb + lay.c);
    float* ssq_c = reinterpret_cast<float*>(wsb + lay.ssq_c);
    float* kvraw = reinterpret_cast<float*>(wsb + lay.kvraw);
    int* lensnap = reinterpret_cast<int*>(wsb + lay.lensnap);
    int rc;
    // the layout was carved from these plans' tile counts; checked before anything is launched
    if (pl.fuse.n_tiles > lay.ssq_c_tiles) return DFLASH_EUNSUPPORTED;
    T* cn = reinterpret_cast<T*>(wsb + lay.cnorm);
    const size_t cn_layer = (size_t)pad16(M) * s.H;    // whole 16-row tiles per layer
    // every layer's RMSNorm carried across the GEMMs where the plans allow it: the fusion
    // GEMM writes c * w_in,l for each layer (and the len snapshot), W_k|W_v scales its rows
    const bool carry = s.L <= GEMM_ZMAX && fold_producer_ok(pl.fuse, M) && fold_consumer_ok(pl.kv, pl.fuse.n_tiles, M);
    {   // stage 1: c = W_fuse . concat(feat)
        GemmArgs a = gemm_base(s, pl.fuse, M, s.F * s.H);
        a.a = feat;
        a.lda = (long long)s.F * s.H;
        a.N = s.H;
        a.seg_end[0] = a.seg_end[1] = a.seg_end[2] = s.H;
        a.layer[0].w[0] = w->w_fuse;
        a.out = c;
        a.ldo = s.H;
        a.residual = 0;
        a.ssq_out = ssq_c;
        a.ssq_out_ld = ssq_ld(M);
        if (carry) {
            a.n_z = s.L;
            for (int l = 0; l < s.L; ++l) a.zw[l] = w->layers[l].in_norm;
            a.zout = cn;
            a.zstride = (long long)cn_layer;
            a.snap_src = kv->len;
            a.snap_dst = lensnap;
            a.snap_n = batch;
        }
        if ((rc = gemm_dispatch<T>(a, pl.fuse, st, tr, "fuse"))) return rc;
    }
    {   // stage 2: every layer's RMSNorm -> W_k | W_v (one launch for all layers)
        GemmArgs a = gemm_base(s, pl.kv, M, s.H);
        const int afrag = M < TILED_MIN_ROWS ? 1 : 0;       // fragment order for the weight-streaming GEMM
        if (carry) {
            set_carried_norm_a(a, s, cn, ssq_c, pl.fuse.n_tiles, M);
        } else {
            NormWeights nw{};   // one normalised copy of c per layer (each layer has its own scale)
            for (int l = 0; l < s.L; ++l) nw.w[l] = w->layers[l].in_norm;
            tr.begin("rmsnorm");
            if (tr.au) {
                tr.au->write(cn, (size_t)(s.L - 1) * cn_layer * sizeof(T) + span_act<T>(afrag, M, s.H, s.H));
                tr.au->write(lensnap, (size_t)batch * 4);
            }
            DFL_LAUNCH(tr, (rmsnorm_rows_kernel<T>), dim3(M, cdiv(s.H, 1024), s.L), dim3(256), 0, st, c, s.H, ssq_c,
                       pl.fuse.n_tiles, ssq_ld(M), nw, s.H, s.eps, cn, s.H, (long long)cn_layer, kv->len, lensnap, batch,
                       afrag, 1);
            tr.end();
            if (!launched(tr)) return DFLASH_ELAUNCH;
        }
        const int ld = 2 * s.nkv * s.D;
        a.lda = s.H;
        a.N = ld;
        a.seg_end[0] = s.nkv * s.D;
        a.seg_end[1] = a.seg_end[2] = ld;
        a.ldo = ld;
        a.a_frag = afrag;
        for (int l = 0; l < s.L; ++l) {
            a.layer[l].a = cn + (size_t)l * cn_layer;
            a.layer[l].w[0] = w->layers[l].wk;
            a.layer[l].w[1] = w->layers[l].wv;
            a.layer[l].out = kvraw + (size_t)l * M * ld;
        }
        if ((rc = gemm_dispatch<T>(a, pl.kv, st, tr, "inject_kv"))) return rc;
    }
    {   // stage 3: k-norm + RoPE -> K cache, v -> V cache (32-key blocks of V^T)
        KvFinishArgs a;
        std::memset(&a, 0, sizeof(a));
        a.kv = kvraw;
        a.layer_stride = (long long)M * 2 * s.nkv * s.D;
        a.row_ld = 2 * s.nkv * s.D;
        a.layer0 = 0;
        a.update_len = 1;
        a.rows_stride = rows;
        a.n_kv = s.nkv;
        a.head_dim = s.D;
        a.cap = s.cap;
        a.rope_rows = w->rope_rows;
        a.cache_layer = (long long)s.Bmax * s.nkv * s.cap * s.D;
        a.kcache = kv->k;
        a.vcache = kv->v;
        for (int l = 0; l < s.L; ++l) a.k_norm[l] = w->layers[l].k_norm;
        a.eps = s.eps;
        a.len_snap = lensnap;
        a.len = kv->len;
        a.n_new = n_new;
        a.rope_cos = w->rope_cos;
        a.rope_sin = w->rope_sin;
        a.status = kv->status;
        tr.begin("kv_finish");
        const int rb_n = cdiv(rows, KV_ROWS);
        DFL_LAUNCH(tr, (kv_finish_kernel<T>), dim3(2 * s.nkv, s.L, batch * rb_n), dim3(256), 0, st, a, rb_n);
        tr.end();
        if (!launched(tr)) return DFLASH_ELAUNCH;
    }
    return DFLASH_OK;
}

// What differs between the drafter's block pass and a verifying target's forward over the
// same rows: the target reads its own tokens, masks later block positions (causal), keeps
// the block's K/V in its cache, taps hidden states and takes the argmax of every row.
struct PassMode {
    const int* tokens;      // nullable: [batch][gamma] ids (else anchor + mask tokens)
    int causal;
    int write_kv;           // K / V^T rows of the block at len .. len + gamma - 1 (len unchanged)
    const int* taps;        // [host] n_taps 1-based decoder layers; feat [batch][gamma][n_taps][H]
    int n_taps;
    void* feat;
    int first_row;          // argmax rows: 1 (drafts) or 0 (every row)
    const int* labels;      // nullable: [batch][gamma-1] labels of the mask rows -> block loss instead of drafts
    float* loss;            // with labels: [1] weighted mean cross-entropy
    float* row_loss;        // with labels: nullable [batch][gamma-1] cross-entropy per mask row
    float* dlogits;         // with labels: nullable [batch][gamma-1][V] gradient of the loss w.r.t. the logits
    const float* x_in;      // nullable: fp32 [batch*gamma][H] input rows instead of token embeddings
    const float* ssq_in;    // with x_in: [n_ssq_in][ssq_ld(batch*gamma)] per-tile sums of squares of x_in
    int n_ssq_in;
    int no_head;            // stop after the last decoder layer (no final norm, LM head or argmax)
};

constexpr PassMode DRAFT_PASS = {nullptr, 0, 0, nullptr, 0, nullptr, 1};

template <typename T>
int run_draft(const Shape& s, const dflash_weights* w, const dflash_kv* kv, int batch, int gamma,
              const int* anchor, int* draft, float* dbg_hidden, float* dbg_logits, void* ws, const Layout& lay,
              hipStream_t st, Tracer& tr, const PassMode& md = DRAFT_PASS) {
    char* wsb = static_cast<char*>(ws);
    const int M = batch * gamma;
    const DraftPlans pl = draft_plans(s, M);
    // the workspace was carved for other plans: checked before anything is launched
    if (pl.lm.n_tiles > lay.amax_tiles || std::max(pl.o.n_tiles, pl.down.n_tiles) > lay.ssq_x_tiles)
        return DFLASH_EUNSUPPORTED;
    if (md.labels && plan_gemm(s, EPI_LSE, s.V, s.H, M, 1).n_tiles != pl.lm.n_tiles) return DFLASH_EUNSUPPORTED;
    float* x = reinterpret_cast<float*>(wsb + lay.x);
    float* ssq_x = reinterpret_cast<float*>(wsb + lay.ssq_x);
    float* qkv = reinterpret_cast<float*>(wsb + lay.qkv);
    void* opart = wsb + lay.opart;
    float* mlpart = reinterpret_cast<float*>(wsb + lay.mlpart);
    void* obuf = wsb + lay.obuf;
    void* hbuf = wsb + lay.hbuf;
    unsigned long long* amax = reinterpret_cast<unsigned long long*>(wsb + lay.amax);
    void* nbuf = wsb + lay.nbuf;
    const int n_draft = batch * (gamma - md.first_row);
    // the weight-streaming GEMM (fewer than TILED_MIN_ROWS rows) reads A in fragment order
    const int afrag = M < TILED_MIN_ROWS ? 1 : 0;
    const int qkv_ld = (s.nq + 2 * s.nkv) * s.D;
    int rc;

    if (md.x_in) {      // input rows given (fp32): they start the residual stream
        const long long n = (long long)M * s.H;
        const unsigned blocks = (unsigned)std::min<long long>(1024, (n + 255) / 256);
        tr.begin("copy_input");
        if (tr.au) tr.au->write(x, (size_t)n * 4);
        DFL_LAUNCH(tr, copy_f32_kernel, dim3(blocks), dim3(256), 0, st, md.x_in, x, n);
        tr.end();
    } else {
        tr.begin("embed_norm");
        if (tr.au) {
            tr.au->write(x, span_rows(M, s.H, s.H, 4));
            tr.au->write(nbuf, span_act<T>(afrag, M, s.H, s.H));
        }
        DFL_LAUNCH(tr, (embed_norm_kernel<T>), dim3(M), dim3(256), 0, st, static_cast<const T*>(w->embed),
                           anchor, md.tokens, s.mask, s.V, gamma, s.H, static_cast<const T*>(w->layers[0].in_norm),
                           s.eps, x, static_cast<T*>(nbuf), kv->status, afrag);
        tr.end();
    }
    if (!launched(tr)) return DFLASH_ELAUNCH;
    int n_ssq = 0;      // per-tile partial sums of squares of x (written by o / down)
    // RMSNorm carried across the GEMMs where both plans allow it: o writes x * w_post for
    // gate|up, down writes x * w_in of the next layer for its q|k|v, and those two scale their
    // output rows; the final norm before the LM head keeps its own launch
    const bool carry_mlp = fold_producer_ok(pl.o, M) && fold_consumer_ok(pl.gateup, pl.o.n_tiles, M);
    const bool carry_attn = fold_producer_ok(pl.down, M) && fold_consumer_ok(pl.qkv, pl.down.n_tiles, M);
    // The argmax LM head reads rho(x * w_final) and leaves out the final RMSNorm's row factor,
    // which is positive and so leaves every row's argmax where it is: the last down GEMM stores
    // that operand where its plan allows, else the norm launch writes it without the factor.
    // The loss head needs the true logits and keeps the whole RMSNorm.
    const bool head_argmax = md.labels == nullptr && !md.no_head;
    const bool carry_head = head_argmax && fold_producer_ok(pl.down, M);

    const AttnPlan ap = plan_attn(s, gamma, batch);
    const size_t layer_elems = (size_t)s.Bmax * s.nkv * s.cap * s.D;

    for (int l = 0; l < s.L; ++l) {
        const dflash_layer_weights& lw = w->layers[l];
        {   // raw q | k | v of the block (three weight tensors, one launch)
            GemmArgs a = gemm_base(s, pl.qkv, M, s.H);
            if (l == 0 && md.x_in) {
                if ((rc = set_norm_a<T>(a, s, x, M, md.ssq_in, md.n_ssq_in, lw.in_norm, nbuf, afrag, st, tr)))
                    return rc;
            } else if (l == 0) {       // the embedding kernel normalised the rows already
                a.a = nbuf;
                a.lda = s.H;
                a.a_frag = afrag;
            } else if (carry_attn) {   // the previous layer's down wrote x * w_in into nbuf
                set_carried_norm_a(a, s, nbuf, ssq_x, n_ssq, M);
            } else if ((rc = set_norm_a<T>(a, s, x, M, ssq_x, n_ssq, lw.in_norm, nbuf, afrag, st, tr))) {
                return rc;
            }
            a.N = qkv_ld;
            a.seg_end[0] = s.nq * s.D;
            a.seg_end[1] = (s.nq + s.nkv) * s.D;
            a.seg_end[2] = qkv_ld;
            a.layer[0].w[0] = lw.wq;
            a.layer[0].w[1] = lw.wk;
            a.layer[0].w[2] = lw.wv;
            a.out = qkv;
            a.ldo = qkv_ld;
            if ((rc = gemm_dispatch<T>(a, pl.qkv, st, tr, "qkv_proj"))) return rc;
        }
        {   // attention over [context ; block]
            AttnArgs a;
            std::memset(&a, 0, sizeof(a));
            a.kcache = static_cast<const T*>(kv->k) + l * layer_elems;
            a.vcache = static_cast<const T*>(kv->v) + l * layer_elems;
            a.qkv = qkv;
            a.qkv_ld = qkv_ld;
            a.q_norm = lw.q_norm;
            a.k_norm = lw.k_norm;
            a.rope_cos = w->rope_cos;
            a.rope_sin = w->rope_sin;
            a.rope_rows = w->rope_rows;
            a.eps = s.eps;
            a.len = kv->len;
            a.opart = opart;
            a.mlpart = mlpart;
            a.n_q = s.nq;
            a.n_kv = s.nkv;
            a.cap = s.cap;
            a.rpad = s.rpad;
            a.nch_max = s.nch_max;
            a.chunk = s.chunk;
            a.gamma = gamma;
            a.group = s.group;
            a.nqs = ap.nqs;
            // the context K/V with the non-temporal hint when one workgroup reads each chunk and
            // the cache (all layers) does not fit the 256 MB last-level cache, so that nothing of
            // it would be found there by the next cycle anyway (LLaMA-3.1-8B shape at batch 32:
            // 3139 -> 3097 us per cycle; at the Qwen3-8B shape, batch 1, the 85 MB cache is read
            // from that cache every cycle and the hint cost 5 us)
            a.kv_nt = ap.nqs == 1 && (double)batch * s.nkv * s.cap * s.D * 2 * s.esize * s.L > 256.0 * (1 << 20);
            a.causal = md.causal;
            if (md.write_kv) {  // the block's keys and values are kept in this layer's cache
                a.kwrite = static_cast<T*>(kv->k) + l * layer_elems;
                a.vwrite = static_cast<T*>(kv->v) + l * layer_elems;
            }
            a.status = kv->status;
            a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)s.D));
            tr.begin("attention");
            rc = launch_attention<T>(a, ap, s.nch_max, s.nkv, batch, st, tr);
            tr.end();
            if (rc) return rc;
            MergeArgs mgr;
            mgr.opart = opart;
            mgr.mlpart = mlpart;
            mgr.len = kv->len;
            mgr.out = obuf;
            mgr.n_kv = s.nkv;
            mgr.group = s.group;
            mgr.gamma = gamma;
            mgr.rpad = s.rpad;
            mgr.nch_max = s.nch_max;
            mgr.chunk = s.chunk;
            mgr.cap = s.cap;
            mgr.head_dim = s.D;
            mgr.out_frag = afrag;
            tr.begin("attn_merge");
            if (tr.au) tr.au->write(obuf, span_act<T>(afrag, M, s.nq * s.D, s.nq * s.D));
            // four waves per (row, head) when a row has more chunks than one batch of loads
            const int merge_waves = s.nch_max > MERGE_BATCH ? MERGE_WAVES : 1;
            DFL_LAUNCH(tr, (attn_merge_kernel<T>), dim3(M, s.nq), dim3(64 * merge_waves), 0, st, mgr);
            tr.end();
            if (!launched(tr)) return DFLASH_ELAUNCH;
        }
        {   // x += W_o o
            GemmArgs a = gemm_base(s, pl.o, M, s.nq * s.D);
            a.a = obuf;
            a.lda = s.nq * s.D;
            a.a_frag = afrag;
            a.N = s.H;
            a.seg_end[0] = a.seg_end[1] = a.seg_end[2] = s.H;
            a.layer[0].w[0] = lw.wo;
            a.out = x;
            a.ldo = s.H;
            a.residual = 1;
            a.ssq_out = ssq_x;
            a.ssq_out_ld = ssq_ld(M);
            if (carry_mlp) {        // gate|up's A operand: x * w_post
                a.n_z = 1;
                a.zw[0] = lw.post_norm;
                a.zout = nbuf;
            }
            if ((rc = gemm_dispatch<T>(a, pl.o, st, tr, "o_proj"))) return rc;
            n_ssq = pl.o.n_tiles;
        }
        {   // h = silu(W_gate a2) * (W_up a2)
            GemmArgs a = gemm_base(s, pl.gateup, M, s.H);
            if (carry_mlp) set_carried_norm_a(a, s, nbuf, ssq_x, n_ssq, M);
            else if ((rc = set_norm_a<T>(a, s, x, M, ssq_x, n_ssq, lw.post_norm, nbuf, afrag, st, tr))) return rc;
            a.N = s.I;
            a.seg_end[0] = a.seg_end[1] = a.seg_end[2] = s.I;
            a.layer[0].w[0] = lw.w_gate;
            a.layer[0].w[1] = lw.w_up;
            a.out_t = hbuf;
            a.ldo = s.I;
            a.out_frag = afrag;
            if ((rc = gemm_dispatch<T>(a, pl.gateup, st, tr, "gate_up"))) return rc;
        }
        {   // x += W_down h
            GemmArgs a = gemm_base(s, pl.down, M, s.I);
            a.a = hbuf;
            a.lda = s.I;
            a.a_frag = afrag;
            a.N = s.H;
            a.seg_end[0] = a.seg_end[1] = a.seg_end[2] = s.H;
            a.layer[0].w[0] = lw.w_down;
            a.out = x;
            a.ldo = s.H;
            a.residual = 1;
            a.ssq_out = ssq_x;
            a.ssq_out_ld = ssq_ld(M);
            if (carry_attn && l + 1 < s.L) {     // the next layer's q|k|v A operand: x * w_in
                a.n_z = 1;
                a.zw[0] = w->layers[l + 1].in_norm;
                a.zout = nbuf;
            } else if (carry_head && l + 1 == s.L) {     // the LM head's A operand: x * w_final
                a.n_z = 1;
                a.zw[0] = w->final_norm;
                a.zout = nbuf;
            }
            if ((rc = gemm_dispatch<T>(a, pl.down, st, tr, "down_proj"))) return rc;
            n_ssq = pl.down.n_tiles;
        }
        for (int f = 0; f < md.n_taps; ++f) {   // hidden state after decoder layer l + 1
            if (md.taps[f] != l + 1) continue;
            const long long n = (long long)M * s.H;
            const unsigned blocks = (unsigned)std::min<long long>(2048, (n + 255) / 256);
            tr.begin("tap");
            DFL_LAUNCH(tr, (tap_kernel<T>), dim3(blocks), dim3(256), 0, st, x, n, s.H, md.n_taps, f,
                       static_cast<T*>(md.feat));
            tr.end();
            if (!launched(tr)) return DFLASH_ELAUNCH;
        }
    }
    if (dbg_hidden) {
        const long long n = (long long)M * s.H;
        const unsigned blocks = (unsigned)std::min<long long>(1024, (n + 255) / 256);
        tr.begin("copy_hidden");
        DFL_LAUNCH(tr, copy_f32_kernel, dim3(blocks), dim3(256), 0, st, x, dbg_hidden, n);
        tr.end();
        if (!launched(tr)) return DFLASH_ELAUNCH;
    }
    if (md.no_head) return DFLASH_OK;
    {   // final norm -> LM head -> per-tile argmax (or log-sum-exp and label logits)
        const bool loss = md.labels != nullptr;
        const GemmPlan plm = loss ? plan_gemm(s, EPI_LSE, s.V, s.H, M, 1) : pl.lm;   // same tiles (checked above)
        GemmArgs a = gemm_base(s, plm, M, s.H);
        if (carry_head) {           // the last down GEMM wrote x * w_final into nbuf
            a.a = nbuf;
            a.lda = s.H;
            a.a_frag = afrag;
        } else if ((rc = set_norm_a<T>(a, s, x, M, ssq_x, n_ssq, w->final_norm, nbuf, afrag, st, tr, !head_argmax))) {
            return rc;
        }
        a.N = s.V;
        a.seg_end[0] = a.seg_end[1] = a.seg_end[2] = s.V;
        a.layer[0].w[0] = w->lm_head;
        a.gamma = gamma;
        a.amax = amax;
        a.dbg_logits = (loss && !dbg_logits) ? md.dlogits : dbg_logits;   // the gradient needs the logits
        a.dbg_first = md.first_row;
        if (loss) {
            a.lse = reinterpret_cast<float2*>(amax);     // the same [n_tiles][M] 8-byte slots
            a.labels = md.labels;
            a.lab_logit = reinterpret_cast<float*>(wsb + lay.lab);
        }
        if ((rc = gemm_dispatch<T>(a, plm, st, tr, loss ? "lm_head_lse" : "lm_head_argmax"))) return rc;
    }
    if (head_argmax && dbg_logits && n_draft > 0) {   // the returned logits, with the row factor
        tr.begin("scale_logits");
        DFL_LAUNCH(tr, scale_logit_rows_kernel, dim3((unsigned)std::min(64, cdiv(s.V, 256)), (unsigned)n_draft),
                   dim3(256), 0, st, dbg_logits, s.V, ssq_x, n_ssq, ssq_ld(M), gamma, md.first_row, s.H, s.eps);
        tr.end();
        if (!launched(tr)) return DFLASH_ELAUNCH;
    }
    const int row_blocks = cdiv(M, 64);
    if (md.labels) {
        const int n_slices = std::max(1, std::min({pl.lm.n_tiles, 256 / row_blocks, LSE_MAX_SLICES}));
        float2* part = reinterpret_cast<float2*>(wsb + lay.lse_part);
        tr.begin("lse_slices");
        if (tr.au) tr.au->write(part, span_rows(n_slices, M, M, 8));
        DFL_LAUNCH(tr, lse_slices_kernel, dim3(n_slices, row_blocks), dim3(256), 0, st,
                   reinterpret_cast<const float2*>(amax), pl.lm.n_tiles, n_slices, M, part);
        tr.end();
        if (!launched(tr)) return DFLASH_ELAUNCH;
        tr.begin("block_loss");
        float* lse_row = reinterpret_cast<float*>(wsb + lay.lse_row);
        if (tr.au && md.dlogits) tr.au->write(lse_row, (size_t)M * 4);
        DFL_LAUNCH(tr, block_loss_kernel, dim3(1), dim3(BLOCK_LOSS_THREADS), 0, st, part, n_slices, M, gamma,
                           md.labels, reinterpret_cast<const float*>(wsb + lay.lab), s.V, md.loss, md.row_loss,
                           md.dlogits ? lse_row : nullptr, kv->status);
        tr.end();
        if (!launched(tr)) return DFLASH_ELAUNCH;
        if (md.dlogits) {
            // rows x vocabulary slices of 256 ids, at most 64 slices per row (strided beyond)
            const dim3 grid((unsigned)std::min(64, cdiv(s.V, 256)), (unsigned)(batch * (gamma - 1)));
            tr.begin("block_loss_grad");
            DFL_LAUNCH(tr, block_loss_grad_kernel, grid, dim3(256), 0, st,
                               dbg_logits ? dbg_logits : md.dlogits, md.dlogits, lse_row, md.labels, batch, gamma, s.V);
            tr.end();
        }
        return launched(tr) ? DFLASH_OK : DFLASH_ELAUNCH;
    }
    if (n_draft < 1) return DFLASH_OK;
    tr.begin("argmax_finish");      // one workgroup per draft row; writes only the ids
    DFL_LAUNCH(tr, argmax_finish_kernel, dim3(n_draft), dim3(256), 0, st, amax, pl.lm.n_tiles, gamma, md.first_row,
               draft);
    tr.end();
    return launched(tr) ? DFLASH_OK : DFLASH_ELAUNCH;
}

// Input-fusion conditioning (the alternative the summary's KV injection is compared with,
// section 2.2 and the ablations of section 4): the fused feature of each new context row is
// the drafter's input at that position; every draft layer runs over the rows (causal among
// them, attending to the cached context) and keeps its own K/V rows.  All rows_stride rows
// of a sequence are computed and written at len .. len + rows_stride - 1; len then advances
// by n_new[b], so rows past n_new[b] are overwritten by later ones.
template <typename T>
int run_inject_input_fusion(const Shape& s, const dflash_weights* w, const dflash_kv* kv, int batch,
                            const void* feat, int rows, const int* n_new, void* ws, const Layout& lay,
                            hipStream_t st, Tracer& tr) {
    char* wsb = static_cast<char*>(ws);
    const InjectPlans pl = inject_plans(s, batch, rows);
    const int M = batch * rows;
    float* c = reinterpret_cast<float*>(wsb + lay.c);
    float* ssq_c = reinterpret_cast<float*>(wsb + lay.ssq_c);
    int rc;
    if (pl.fuse.n_tiles > lay.ssq_c_tiles) return DFLASH_EUNSUPPORTED;   // before anything is launched
    {   // c = W_fuse . concat(feat), with per-tile sums of squares for the first layer's norm
        GemmArgs a = gemm_base(s, pl.fuse, M, s.F * s.H);
        a.a = feat;
        a.lda = (long long)s.F * s.H;
        a.N = s.H;
        a.seg_end[0] = a.seg_end[1] = a.seg_end[2] = s.H;
        a.layer[0].w[0] = w->w_fuse;
        a.out = c;
        a.ldo = s.H;
        a.residual = 0;
        a.ssq_out = ssq_c;
        a.ssq_out_ld = ssq_ld(M);
        if ((rc = gemm_dispatch<T>(a, pl.fuse, st, tr, "fuse"))) return rc;
    }
    PassMode md = DRAFT_PASS;
    md.causal = 1;
    md.write_kv = 1;
    md.first_row = 0;
    md.x_in = c;
    md.ssq_in = ssq_c;
    md.n_ssq_in = pl.fuse.n_tiles;
    md.no_head = 1;
    if ((rc = run_draft<T>(s, w, kv, batch, rows, nullptr, nullptr, nullptr, nullptr, ws, lay, st, tr, md)))
        return rc;
    tr.begin("advance_len");
    DFL_LAUNCH(tr, advance_len_kernel, dim3(1), dim3(64), 0, st, kv->len, n_new, batch, s.cap, rows, rows, kv->status);
    tr.end();
    return launched(tr) ? DFLASH_OK : DFLASH_ELAUNCH;
}

// ---- fixed scratch for dflash_draft_block_noalloc (callers that cannot allocate) -------------
// One array per GPU, in the library's code object: the loader places it in each device's
// memory, where it stays until the process ends.  In host code `scratch` only names the
// symbol; its device address is looked up once per device (hipGetSymbolAddress, with that
// device current) and that address is what the kernels receive.
constexpr int NOALLOC_MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[NOALLOC_MAX_DEVICES] = {};

// Device address of the current device's scratch array (looked up on the first call there).
int scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return DFLASH_ELAUNCH;
    if (dev < 0 || dev >= NOALLOC_MAX_DEVICES) return DFLASH_EUNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_addr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return DFLASH_ELAUNCH;
        g_scratch_addr[dev] = p;
    }
    *out = g_scratch_addr[dev];
    return DFLASH_OK;
}

}  // namespace

extern "C" {

size_t dflash_workspace_bytes(const dflash_config* cfg, int32_t batch, int32_t max_rows_per_seq) {
    Shape s;
    if (make_shape(cfg, s) != DFLASH_OK) return 0;
    if (batch < 1 || batch > s.Bmax || max_rows_per_seq < 0) return 0;
    if (max_rows_per_seq > 0 && s.L > MAX_LAYERS) return 0;   // injection: one launch serves every layer
    const Layout l = make_layout(s, batch, max_rows_per_seq);
    return l.inject_end;
}

int dflash_inject_kv_traced(const dflash_config* cfg, const dflash_weights* w, const dflash_kv* kv, int32_t batch,
                            const void* feat, int32_t rows_stride, const int32_t* n_new, void* workspace,
                            size_t workspace_bytes, void* stream, dflash_trace* trace) {
    Shape s;
    int rc = make_shape(cfg, s);
    if (rc) return rc;
    if (!w || !kv || !feat || !n_new || !kv->k || !kv->v || !kv->len || !kv->status) return DFLASH_EINVAL;
    if (!weights_ok(s, w)) return DFLASH_EINVAL;
    if (s.L > MAX_LAYERS) return DFLASH_EUNSUPPORTED;      // one launch serves every layer
    if (batch < 1 || batch > s.Bmax || rows_stride < 1) return DFLASH_EINVAL;
    if (w->rope_rows < s.cap + s.gmax) return DFLASH_EINVAL;
    if (trace && trace->capacity < 0) return DFLASH_EINVAL;
    if (!workspace) return DFLASH_EWORKSPACE;
    const Layout lay = make_layout(s, batch, rows_stride);
    if (workspace_bytes < lay.inject_end) return DFLASH_EWORKSPACE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    Tracer tr{trace, st};
    if (trace) trace->count = 0;
    return s.bf16 ? run_inject<bf16_t>(s, w, kv, batch, feat, rows_stride, n_new, workspace, lay, st, tr)
                  : run_inject<float>(s, w, kv, batch, feat, rows_stride, n_new, workspace, lay, st, tr);
}

int dflash_inject_kv(const dflash_config* cfg, const dflash_weights* w, const dflash_kv* kv, int32_t batch,
                     const void* feat, int32_t rows_stride, const int32_t* n_new, void* workspace,
                     size_t workspace_bytes, void* stream) {
    return dflash_inject_kv_traced(cfg, w, kv, batch, feat, rows_stride, n_new, workspace, workspace_bytes, stream,
                                   nullptr);
}

int dflash_draft_block_traced(const dflash_config* cfg, const dflash_weights* w, const dflash_kv* kv, int32_t batch,
                              int32_t gamma, const int32_t* anchor, int32_t* draft, float* dbg_hidden,
                              float* dbg_logits, void* workspace, size_t workspace_bytes, void* stream,
                              dflash_trace* trace) {
    Shape s;
    int rc = make_shape(cfg, s);
    if (rc) return rc;
    if (!w || !kv || !anchor || !draft || !kv->k || !kv->v || !kv->len || !kv->status) return DFLASH_EINVAL;
    if (!weights_ok(s, w)) return DFLASH_EINVAL;
    if (batch < 1 || batch > s.Bmax || gamma < 2 || gamma > s.gmax) return DFLASH_EINVAL;
    if (w->rope_rows < s.cap + s.gmax) return DFLASH_EINVAL;
    if (trace && trace->capacity < 0) return DFLASH_EINVAL;
    if (!workspace) return DFLASH_EWORKSPACE;
    const Layout lay = make_layout(s, batch, 0);
    if (workspace_bytes < lay.draft_end) return DFLASH_EWORKSPACE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    Tracer tr{trace, st};
    if (trace) trace->count = 0;
    return s.bf16 ? run_draft<bf16_t>(s, w, kv, batch, gamma, anchor, draft, dbg_hidden, dbg_logits, workspace, lay,
                                      st, tr)
                  : run_draft<float>(s, w, kv, batch, gamma, anchor, draft, dbg_hidden, dbg_logits, workspace, lay,
                                     st, tr);
}

int dflash_draft_block(const dflash_config* cfg, const dflash_weights* w, const dflash_kv* kv, int32_t batch,
                       int32_t gamma, const int32_t* anchor, int32_t* draft, float* dbg_hidden, float* dbg_logits,
                       void* workspace, size_t workspace_bytes, void* stream) {
    return dflash_draft_block_traced(cfg, w, kv, batch, gamma, anchor, draft, dbg_hidden, dbg_logits, workspace,
                                     workspace_bytes, stream, nullptr);
}

size_t dflash_noalloc_scratch_bytes(void) { return NOALLOC_SCRATCH_BYTES; }

int dflash_draft_block_noalloc(const dflash_config* cfg, const dflash_weights* w, const dflash_kv* kv, int32_t batch,
                               int32_t gamma, const int32_t* anchor, int32_t* draft, float* dbg_hidden,
                               float* dbg_logits, void* stream) {
    Shape s;
    int rc = make_shape(cfg, s);
    if (rc) return rc;
    if (!w || !kv || !anchor || !draft || !kv->k || !kv->v || !kv->len || !kv->status) return DFLASH_EINVAL;
    if (!weights_ok(s, w)) return DFLASH_EINVAL;
    if (batch < 1 || batch > s.Bmax || gamma < 2 || gamma > s.gmax) return DFLASH_EINVAL;
    if (w->rope_rows < s.cap + s.gmax) return DFLASH_EINVAL;
    // the layout of this call (batch sequences), not of max_batch: it must fit the array
    const Layout lay = make_layout(s, batch, 0);
    if (lay.draft_end > NOALLOC_SCRATCH_BYTES) return DFLASH_ESCRATCH;
    void* ws = nullptr;
    if ((rc = scratch_address(&ws))) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    Tracer tr{nullptr, st};
    return s.bf16 ? run_draft<bf16_t>(s, w, kv, batch, gamma, anchor, draft, dbg_hidden, dbg_logits, ws, lay, st, tr)
                  : run_draft<float>(s, w, kv, batch, gamma, anchor, draft, dbg_hidden, dbg_logits, ws, lay, st, tr);
}

int dflash_inject_kv_input_fusion(const dflash_config* cfg, const dflash_weights* w, const dflash_kv* kv,
                                  int32_t batch, const void* feat, int32_t rows_stride, const int32_t* n_new,
                                  void* workspace, size_t workspace_bytes, void* stream) {
    Shape s;
    int rc = make_shape(cfg, s);
    if (rc) return rc;
    if (!w || !kv || !feat || !n_new || !kv->k || !kv->v || !kv->len || !kv->status) return DFLASH_EINVAL;
    if (!weights_ok(s, w)) return DFLASH_EINVAL;
    if (batch < 1 || batch > s.Bmax || rows_stride < 1 || rows_stride > s.gmax) return DFLASH_EINVAL;
    if (w->rope_rows < s.cap + s.gmax) return DFLASH_EINVAL;
    if (!workspace) return DFLASH_EWORKSPACE;
    const Layout lay = make_layout(s, batch, rows_stride);
    if (workspace_bytes < lay.inject_end) return DFLASH_EWORKSPACE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    Tracer tr{nullptr, st};
    return s.bf16 ? run_inject_input_fusion<bf16_t>(s, w, kv, batch, feat, rows_stride, n_new, workspace, lay, st, tr)
                  : run_inject_input_fusion<float>(s, w, kv, batch, feat, rows_stride, n_new, workspace, lay, st, tr);
}

int dflash_block_loss(const dflash_config* cfg, const dflash_weights* w, const dflash_kv* kv, int32_t batch,
                      int32_t gamma, const int32_t* anchor, const int32_t* labels, float* loss, float* row_loss,
                      float* dlogits, float* dbg_logits, void* workspace, size_t workspace_bytes, void* stream) {
    Shape s;
    int rc = make_shape(cfg, s);
    if (rc) return rc;
    if (!w || !kv || !anchor || !labels || !loss || !kv->k || !kv->v || !kv->len || !kv->status) return DFLASH_EINVAL;
    if (!weights_ok(s, w, false)) return DFLASH_EINVAL;
    if (batch < 1 || batch > s.Bmax || gamma < 2 || gamma > s.gmax) return DFLASH_EINVAL;
    if (w->rope_rows < s.cap + s.gmax) return DFLASH_EINVAL;
    if (!workspace) return DFLASH_EWORKSPACE;
    const Layout lay = make_layout(s, batch, 0);
    if (workspace_bytes < lay.draft_end) return DFLASH_EWORKSPACE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    Tracer tr{nullptr, st};
    PassMode md = DRAFT_PASS;
    md.labels = labels;
    md.loss = loss;
    md.row_loss = row_loss;
    md.dlogits = dlogits;
    return s.bf16 ? run_draft<bf16_t>(s, w, kv, batch, gamma, anchor, nullptr, nullptr, dbg_logits, workspace, lay,
                                      st, tr, md)
                  : run_draft<float>(s, w, kv, batch, gamma, anchor, nullptr, nullptr, dbg_logits, workspace, lay,
                                     st, tr, md);
}

int dflash_verify(int32_t batch, int32_t gamma, const int32_t* draft, const int32_t* target, int32_t* accept_len,
                  int32_t* committed, int32_t* next_anchor, void* stream) {
    if (batch < 1 || gamma < 2 || gamma > 1024) return DFLASH_EINVAL;
    if (!draft || !target || !accept_len || !committed || !next_anchor) return DFLASH_EINVAL;
    hipLaunchKernelGGL(verify_kernel, dim3(batch), dim3(64), 0, static_cast<hipStream_t>(stream), batch, gamma, draft,
                       target, accept_len, committed, next_anchor);
    return hipGetLastError() == hipSuccess ? DFLASH_OK : DFLASH_ELAUNCH;
}

int dflash_target_forward(const dflash_config* cfg, const dflash_weights* w, const dflash_kv* kv, int32_t batch,
                          int32_t rows, const int32_t* tokens, int32_t* y, void* feat, const int32_t* taps,
                          int32_t n_taps, float* dbg_logits, void* workspace, size_t workspace_bytes, void* stream) {
    Shape s;
    int rc = make_shape(cfg, s);
    if (rc) return rc;
    if (!w || !kv || !tokens || !y || !kv->k || !kv->v || !kv->len || !kv->status) return DFLASH_EINVAL;
    if (!weights_ok(s, w, false)) return DFLASH_EINVAL;
    if (batch < 1 || batch > s.Bmax || rows < 1 || rows > s.gmax) return DFLASH_EINVAL;
    if (n_taps < 0 || n_taps > MAX_LAYERS || (n_taps > 0 && (!taps || !feat))) return DFLASH_EINVAL;
    for (int f = 0; f < n_taps; ++f)
        if (taps[f] < 1 || taps[f] > s.L) return DFLASH_EINVAL;
    if (w->rope_rows < s.cap + s.gmax) return DFLASH_EINVAL;
    if (!workspace) return DFLASH_EWORKSPACE;
    const Layout lay = make_layout(s, batch, 0);
    if (workspace_bytes < lay.draft_end) return DFLASH_EWORKSPACE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    Tracer tr{nullptr, st};
    const PassMode md = {tokens, 1, 1, taps, n_taps, feat, 0};
    return s.bf16 ? run_draft<bf16_t>(s, w, kv, batch, rows, nullptr, y, nullptr, dbg_logits, workspace, lay, st, tr,
                                      md)
                  : run_draft<float>(s, w, kv, batch, rows, nullptr, y, nullptr, dbg_logits, workspace, lay, st, tr,
                                     md);
}

int dflash_advance_len(const dflash_config* cfg, const dflash_kv* kv, int32_t batch, const int32_t* n, void* stream) {
    Shape s;
    const int rc = make_shape(cfg, s);
    if (rc) return rc;
    if (!kv || !kv->len || !kv->status || !n || batch < 1 || batch > s.Bmax) return DFLASH_EINVAL;
    hipLaunchKernelGGL(advance_len_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream), kv->len, n, batch,
                       s.cap, s.cap, 0, kv->status);
    return hipGetLastError() == hipSuccess ? DFLASH_OK : DFLASH_ELAUNCH;
}

int dflash_choose_gamma(const int32_t* tau, const int32_t* gamma_used, int32_t n, const float* cost_us,
                        int32_t gamma_min, int32_t gamma_max, double prior_p, double prior_weight,
                        int32_t* gamma_out, double* p_out) {
    if (n < 0 || (n > 0 && (!tau || !gamma_used)) || !cost_us || !gamma_out) return DFLASH_EINVAL;
    if (gamma_min < 2 || gamma_max > MAX_GAMMA || gamma_min > gamma_max) return DFLASH_EINVAL;
    if (!(prior_p >= 0.0 && prior_p <= 1.0) || !(prior_weight >= 0.0)) return DFLASH_EINVAL;
    // maximum-likelihood estimate of the per-position acceptance with pseudo-counts
    double acc = 0.0, rej = 0.0;
    for (int i = 0; i < n; ++i) {
        if (gamma_used[i] < 2 || gamma_used[i] > MAX_GAMMA || tau[i] < 1 || tau[i] > gamma_used[i])
            return DFLASH_EINVAL;
        acc += tau[i] - 1;
        if (tau[i] < gamma_used[i]) rej += 1.0;
    }
    const double den = acc + rej + prior_weight;
    const double p = den > 0.0 ? (acc + prior_weight * prior_p) / den : prior_p;
    // expected tokens per cycle over cycle time; E(g) summed term by term
    int best = 0;
    double best_rate = -1.0;
    for (int g = gamma_min; g <= gamma_max; ++g) {
        if (!(cost_us[g] > 0.0f)) continue;
        double e = 0.0, pj = 1.0;
        for (int j = 0; j < g; ++j) {
            e += pj;
            pj *= p;
        }
        const double rate = e / (double)cost_us[g];
        if (rate > best_rate) {
            best_rate = rate;
            best = g;
        }
    }
    if (best == 0) return DFLASH_EINVAL;
    *gamma_out = best;
    if (p_out) *p_out = p;
    return DFLASH_OK;
}

int dflash_audit_workspace(const dflash_config* cfg, int32_t batch, int32_t gamma, int32_t rows_stride,
                           int32_t* launches, int32_t* writes, int32_t* violations) {
    Shape s;
    int rc = make_shape(cfg, s);
    if (rc) return rc;
    if (!launches || !writes || !violations) return DFLASH_EINVAL;
    if (batch < 1 || batch > s.Bmax || gamma < 2 || gamma > s.gmax || rows_stride < 1) return DFLASH_EINVAL;
    if (s.L > MAX_LAYERS) return DFLASH_EUNSUPPORTED;
    // stand-in device addresses: the audit never dereferences them and launches nothing
    const void* fake = reinterpret_cast<const void*>(uintptr_t(1) << 40);
    int32_t* ifake = reinterpret_cast<int32_t*>(uintptr_t(1) << 41);
    float* ffake = reinterpret_cast<float*>(uintptr_t(1) << 42);
    std::vector<dflash_layer_weights> lw(s.L);
    for (dflash_layer_weights& x : lw) x = {fake, fake, fake, fake, fake, fake, fake, fake, fake, fake, fake};
    const dflash_weights w = {fake, fake, fake, fake, ffake, ffake, s.cap + s.gmax, lw.data()};
    const dflash_kv kv = {const_cast<void*>(fake), const_cast<void*>(fake), ifake,
                          reinterpret_cast<uint32_t*>(ifake)};
    Audit au;
    au.base = uintptr_t(1) << 44;
    void* ws = reinterpret_cast<void*>(au.base);
    auto run = [&](int rows, auto&& body) {
        const Layout lay = make_layout(s, batch, rows);
        au.regions = lay.regions;
        Tracer tr{nullptr, nullptr};
        tr.au = &au;
        return body(lay, tr);
    };
    const int taps[1] = {1};
    const int if_rows = std::min<int>(rows_stride, s.gmax);
    PassMode loss = DRAFT_PASS;
    loss.labels = ifake;
    loss.loss = ffake;
    loss.row_loss = ffake;
    loss.dlogits = ffake;
    const PassMode target = {ifake, 1, 1, taps, 1, const_cast<void*>(fake), 0};
    rc = run(rows_stride, [&](const Layout& lay, Tracer& tr) {
        return s.bf16 ? run_inject<bf16_t>(s, &w, &kv, batch, fake, rows_stride, ifake, ws, lay, nullptr, tr)
                      : run_inject<float>(s, &w, &kv, batch, fake, rows_stride, ifake, ws, lay, nullptr, tr);
    });
    if (!rc) rc = run(if_rows, [&](const Layout& lay, Tracer& tr) {
        return s.bf16 ? run_inject_input_fusion<bf16_t>(s, &w, &kv, batch, fake, if_rows, ifake, ws, lay, nullptr, tr)
                      : run_inject_input_fusion<float>(s, &w, &kv, batch, fake, if_rows, ifake, ws, lay, nullptr, tr);
    });
    for (const PassMode* md : {&DRAFT_PASS, (const PassMode*)&loss, &target}) {
        if (rc) break;
        rc = run(0, [&](const Layout& lay, Tracer& tr) {
            return s.bf16 ? run_draft<bf16_t>(s, &w, &kv, batch, gamma, ifake, ifake, ffake, ffake, ws, lay, nullptr,
                                              tr, *md)
                          : run_draft<float>(s, &w, &kv, batch, gamma, ifake, ifake, ffake, ffake, ws, lay, nullptr,
                                             tr, *md);
        });
    }
    *launches = au.launches;
    *writes = au.writes;
    *violations = au.violations;
    return rc;
}

const char* dflash_status_str(int status) {
    switch (status) {
        case DFLASH_OK: return "DFLASH_OK";
        case DFLASH_EINVAL: return "DFLASH_EINVAL: null pointer or size out of range";
        case DFLASH_EUNSUPPORTED: return "DFLASH_EUNSUPPORTED: shape or dtype not supported";
        case DFLASH_EWORKSPACE: return "DFLASH_EWORKSPACE: workspace missing or too small";
        case DFLASH_ELAUNCH: return "DFLASH_ELAUNCH: kernel launch failed";
        case DFLASH_ESCRATCH:
            return "DFLASH_ESCRATCH: the call needs more scratch than the library's fixed array "
                   "(dflash_noalloc_scratch_bytes); use the workspace entry point";
    }
    return "unknown dflash status";
}

}  // extern "C"
