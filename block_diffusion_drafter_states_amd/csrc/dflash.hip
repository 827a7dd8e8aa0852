// Host side of the DFlash C ABI: argument validation, workspace carving,
// launch planning and the kernel sequence of each entry point.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>

#include "../../include/dflash.h"
#include "attention.hpp"
#include "gemm.hpp"
#include "small_kernels.hpp"

using namespace dflash;

namespace {

constexpr size_t ALIGN = 256;
constexpr size_t COUNTER_SLOTS = 65536;   // fixed-size, self-resetting counters at workspace offset 0

inline size_t align_up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

// Records caller-provided events around each launch (see dflash_trace).
struct Tracer {
    dflash_trace* t;
    hipStream_t st;
    int i = 0;
    void begin(const char* name) {
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

struct Shape {
    int H, nq, nkv, D, I, L, F, V, gmax, mask, Bmax, cap, esize, step, group, rpad, chunk, nch_max;
    float eps;
    bool bf16;
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
    if (s.gmax < 2 || s.gmax > 16) return DFLASH_EINVAL;
    if (s.mask < 0 || s.mask >= s.V) return DFLASH_EINVAL;
    if (s.nq % s.nkv) return DFLASH_EUNSUPPORTED;
    if (s.D * s.esize != 256) return DFLASH_EUNSUPPORTED;
    if (s.L > MAX_LAYERS) return DFLASH_EUNSUPPORTED;
    if (s.cap % 64) return DFLASH_EUNSUPPORTED;
    if (s.H % s.step || s.I % s.step || (s.nq * s.D) % s.step || ((long long)s.F * s.H) % s.step)
        return DFLASH_EUNSUPPORTED;
    if (s.H % GEMM_TILE_N || (s.nq * s.D) % GEMM_TILE_N || (s.nkv * s.D) % GEMM_TILE_N || s.I % 64)
        return DFLASH_EUNSUPPORTED;
    s.group = s.nq / s.nkv;
    if (s.group * s.gmax > 256) return DFLASH_EUNSUPPORTED;
    s.rpad = cdiv(s.group * s.gmax, 16) * 16;
    // context keys per attention chunk: large enough that the per-chunk partial
    // (rpad x D fp32) is <= 1/8 of the chunk's K+V bytes, small enough to give
    // >= 512 workgroups when the cache is full
    int ch = 16 * s.rpad / s.esize;
    ch = std::max(256, std::min(2048, ch));
    int p2 = 256;
    while (p2 < ch) p2 <<= 1;
    ch = p2;
    while (ch > 256 && (long long)s.Bmax * s.nkv * cdiv(s.cap, ch) < 512) ch >>= 1;
    s.chunk = ch;
    s.nch_max = 1 + cdiv(s.cap, ch);
    return DFLASH_OK;
}

struct GemmPlan {
    int n_tiles, n_mgroups, S, kw, layers;
    size_t partial_floats;
    size_t counters;
    int mpad;
};

GemmPlan plan_gemm(const Shape& s, int n_tiles, int M, int K, int layers) {
    GemmPlan p;
    p.n_tiles = n_tiles;
    p.n_mgroups = cdiv(M, GEMM_MAX_M);
    p.layers = layers;
    const int base = n_tiles * p.n_mgroups * layers;
    const int maxS = K / s.step;
    const int mrows = std::min(M, GEMM_MAX_M);
    const int capS = std::max(1, (int)((long long)K * s.esize / (32LL * std::max(16, mrows))));
    int S = 1;
    while ((long long)base * S < 512 && S < maxS && S < capS) ++S;
    int kw = cdiv(cdiv(K, S), s.step) * s.step;
    S = cdiv(K, kw);
    p.S = S;
    p.kw = kw;
    p.partial_floats = S > 1 ? (size_t)layers * n_tiles * S * (size_t)M * GEMM_TILE_N : 0;
    p.counters = (size_t)layers * p.n_mgroups * n_tiles + 1;
    p.mpad = std::min(GEMM_MAX_M, cdiv(M, 16) * 16);
    return p;
}

struct AttnPlan {
    int qg, kg;
};

AttnPlan plan_attn(const Shape& s, int gamma) {
    AttnPlan a;
    const int qt = cdiv(s.group * gamma, 16);
    a.qg = cdiv(qt, 4);
    a.kg = a.qg == 1 ? 4 : (a.qg == 2 ? 2 : 1);
    return a;
}

// Workspace carving.  Offsets of the counters and argmax slots are fixed (they
// persist between calls); everything after them is per-call scratch.
struct Layout {
    size_t counters, slots;
    // draft
    size_t x, ssq_x, qbuf, kblk, vblk, opart, mlpart, obuf, hbuf, dpartial, draft_end;
    // inject
    size_t c, ssq_c, ipartial, inject_end;
    size_t dpartial_floats, ipartial_floats;
};

void draft_plans(const Shape& s, int batch, GemmPlan* g) {
    const int M = batch * s.gmax;
    g[0] = plan_gemm(s, (s.nq * s.D + 2 * s.nkv * s.D) / GEMM_TILE_N, M, s.H, 1);   // qkv
    g[1] = plan_gemm(s, s.H / GEMM_TILE_N, M, s.nq * s.D, 1);                      // o
    g[2] = plan_gemm(s, s.I / 64, M, s.H, 1);                                       // gate/up
    g[3] = plan_gemm(s, s.H / GEMM_TILE_N, M, s.I, 1);                              // down
    g[4] = plan_gemm(s, cdiv(s.V, GEMM_TILE_N), M, s.H, 1);                         // lm head
}

void inject_plans(const Shape& s, int batch, int rows, GemmPlan* g) {
    const int M = batch * rows;
    g[0] = plan_gemm(s, s.H / GEMM_TILE_N, M, s.F * s.H, 1);                     // fuse
    g[1] = plan_gemm(s, 2 * s.nkv * s.D / GEMM_TILE_N, M, s.H, s.L);            // kv (all layers)
}

Layout make_layout(const Shape& s, int batch, int rows) {
    Layout l;
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes); return o; };
    l.counters = take(COUNTER_SLOTS * sizeof(unsigned));
    l.slots = take((size_t)s.Bmax * (s.gmax - 1) * sizeof(unsigned long long));
    const size_t M = (size_t)batch * s.gmax;
    l.x = take(M * s.H * 4);
    l.ssq_x = take((size_t)(s.H / GEMM_TILE_N) * M * 4);
    l.qbuf = take((size_t)batch * s.nkv * s.rpad * s.D * s.esize);
    l.kblk = take((size_t)batch * s.nkv * 32 * s.D * s.esize);
    l.vblk = take((size_t)batch * s.nkv * 32 * s.D * s.esize);
    l.opart = take((size_t)batch * s.nkv * s.nch_max * s.rpad * s.D * 4);
    l.mlpart = take((size_t)batch * s.nkv * s.nch_max * s.rpad * 2 * 4);
    l.obuf = take(M * s.nq * s.D * s.esize);
    l.hbuf = take(M * s.I * s.esize);
    GemmPlan dp[5];
    draft_plans(s, batch, dp);
    l.dpartial_floats = 0;
    for (auto& p : dp) l.dpartial_floats = std::max(l.dpartial_floats, p.partial_floats);
    l.dpartial = take(l.dpartial_floats * 4);
    l.draft_end = off;
    l.c = l.ssq_c = l.ipartial = 0;
    l.ipartial_floats = 0;
    if (rows > 0) {
        const size_t Mi = (size_t)batch * rows;
        l.c = take(Mi * s.H * 4);
        l.ssq_c = take((size_t)(s.H / GEMM_TILE_N) * Mi * 4);
        GemmPlan ip[2];
        inject_plans(s, batch, rows, ip);
        l.ipartial_floats = std::max(ip[0].partial_floats, ip[1].partial_floats);
        l.ipartial = take(l.ipartial_floats * 4);
    }
    l.inject_end = off;
    return l;
}

template <typename T, int EPI>
int launch_gemm(const GemmArgs& a, const GemmPlan& p, size_t lds, hipStream_t st, Tracer& tr, const char* name) {
    dim3 grid(8 * cdiv(p.n_tiles, 8) * p.S, p.n_mgroups, p.layers);
    tr.begin(name);
    hipLaunchKernelGGL((gemm_kernel<T, EPI>), grid, dim3(GEMM_THREADS), lds, st, a);
    const bool ok = hipGetLastError() == hipSuccess;
    tr.end();
    return ok ? DFLASH_OK : DFLASH_ELAUNCH;
}

template <typename T>
int gemm_dispatch(int epi, const GemmArgs& a, const GemmPlan& p, const Shape& s, hipStream_t st, Tracer& tr,
                  const char* name) {
    const size_t lds = gemm_lds_bytes_host(s.esize, p.mpad);
    switch (epi) {
        case EPI_STORE: return launch_gemm<T, EPI_STORE>(a, p, lds, st, tr, name);
        case EPI_QKV: return launch_gemm<T, EPI_QKV>(a, p, lds, st, tr, name);
        case EPI_SWIGLU: return launch_gemm<T, EPI_SWIGLU>(a, p, lds, st, tr, name);
        case EPI_ARGMAX: return launch_gemm<T, EPI_ARGMAX>(a, p, lds, st, tr, name);
        case EPI_KV_INJECT: return launch_gemm<T, EPI_KV_INJECT>(a, p, lds, st, tr, name);
    }
    return DFLASH_EINVAL;
}

GemmArgs gemm_base(const Shape& s, const GemmPlan& p, int M, int K, void* ws, const Layout& lay, float* partial) {
    GemmArgs a;
    std::memset(&a, 0, sizeof(a));
    a.M = M;
    a.K = K;
    a.eps = s.eps;
    a.S = p.S;
    a.kw = p.kw;
    a.n_tiles = p.n_tiles;
    a.n_mgroups = p.n_mgroups;
    a.n_layers = p.layers;
    a.partial = partial;
    a.counters = reinterpret_cast<unsigned*>(static_cast<char*>(ws) + lay.counters);
    a.n_q = s.nq;
    a.n_kv = s.nkv;
    a.head_dim = s.D;
    a.cap = s.cap;
    return a;
}

bool weights_ok(const Shape& s, const dflash_weights* w) {
    if (!w || !w->w_fuse || !w->embed || !w->final_norm || !w->lm_head || !w->rope_cos || !w->rope_sin ||
        !w->layers)
        return false;
    for (int l = 0; l < s.L; ++l) {
        const dflash_layer_weights& x = w->layers[l];
        if (!x.in_norm || !x.wq || !x.wk || !x.wv || !x.q_norm || !x.k_norm || !x.wo || !x.post_norm ||
            !x.w_gate || !x.w_up || !x.w_down)
            return false;
    }
    return true;
}

template <typename T>
int run_inject(const Shape& s, const dflash_weights* w, const dflash_kv* kv, int batch, const void* feat,
               int rows, const int* n_new, void* ws, const Layout& lay, hipStream_t st, Tracer& tr) {
    char* wsb = static_cast<char*>(ws);
    GemmPlan pl[2];
    inject_plans(s, batch, rows, pl);
    const int M = batch * rows;
    float* c = reinterpret_cast<float*>(wsb + lay.c);
    float* ssq_c = reinterpret_cast<float*>(wsb + lay.ssq_c);
    float* part = reinterpret_cast<float*>(wsb + lay.ipartial);
    int rc;
    {   // stage 1: c = W_fuse . concat(feat)
        GemmArgs a = gemm_base(s, pl[0], M, s.F * s.H, ws, lay, part);
        a.a_mode = A_PLAIN;
        a.a = feat;
        a.lda = (long long)s.F * s.H;
        a.n_seg = 1;
        a.seg_n[0] = s.H;
        a.N = s.H;
        a.layer[0].w[0] = w->w_fuse;
        a.out = c;
        a.ldo = s.H;
        a.residual = 0;
        a.ssq_out = ssq_c;
        a.ssq_out_ld = M;
        if ((rc = gemm_dispatch<T>(EPI_STORE, a, pl[0], s, st, tr, "fuse"))) return rc;
    }
    {   // stage 2: every layer's RMSNorm -> W_k | W_v -> k-norm + RoPE -> cache
        GemmArgs a = gemm_base(s, pl[1], M, s.H, ws, lay, part);
        a.a_mode = A_NORM;
        a.a = c;
        a.lda = s.H;
        a.ssq = ssq_c;
        a.n_ssq = s.H / GEMM_TILE_N;
        a.ssq_ld = M;
        a.n_seg = 2;
        a.seg_n[0] = s.nkv * s.D;
        a.seg_n[1] = s.nkv * s.D;
        a.N = 2 * s.nkv * s.D;
        const size_t layer_elems = (size_t)s.Bmax * s.nkv * s.cap * s.D;
        for (int l = 0; l < s.L; ++l) {
            const dflash_layer_weights& lw = w->layers[l];
            a.layer[l].w[0] = lw.wk;
            a.layer[l].w[1] = lw.wv;
            a.layer[l].norm_w = lw.in_norm;
            a.layer[l].head_norm = lw.k_norm;
            a.layer[l].kcache = static_cast<T*>(kv->k) + l * layer_elems;
            a.layer[l].vcache = static_cast<T*>(kv->v) + l * layer_elems;
        }
        a.gamma = rows;
        a.len = kv->len;
        a.n_new = n_new;
        a.rope_cos = w->rope_cos;
        a.rope_sin = w->rope_sin;
        a.rope_rows = w->rope_rows;
        a.status = kv->status;
        a.batch = batch;
        if ((rc = gemm_dispatch<T>(EPI_KV_INJECT, a, pl[1], s, st, tr, "inject_kv"))) return rc;
    }
    return DFLASH_OK;
}

template <typename T>
int run_draft(const Shape& s, const dflash_weights* w, const dflash_kv* kv, int batch, int gamma,
              const int* anchor, int* draft, float* dbg_hidden, float* dbg_logits, void* ws, const Layout& lay,
              hipStream_t st, Tracer& tr) {
    char* wsb = static_cast<char*>(ws);
    const int M = batch * gamma;
    GemmPlan pl[5];
    {
        // plans for the call's gamma (workspace was sized for gamma_max)
        const int Mg = M;
        pl[0] = plan_gemm(s, (s.nq * s.D + 2 * s.nkv * s.D) / GEMM_TILE_N, Mg, s.H, 1);
        pl[1] = plan_gemm(s, s.H / GEMM_TILE_N, Mg, s.nq * s.D, 1);
        pl[2] = plan_gemm(s, s.I / 64, Mg, s.H, 1);
        pl[3] = plan_gemm(s, s.H / GEMM_TILE_N, Mg, s.I, 1);
        pl[4] = plan_gemm(s, cdiv(s.V, GEMM_TILE_N), Mg, s.H, 1);
        for (auto& p : pl)
            if (p.partial_floats > lay.dpartial_floats || p.counters > COUNTER_SLOTS) return DFLASH_EUNSUPPORTED;
    }
    float* x = reinterpret_cast<float*>(wsb + lay.x);
    float* ssq_x = reinterpret_cast<float*>(wsb + lay.ssq_x);
    float* part = reinterpret_cast<float*>(wsb + lay.dpartial);
    void* qbuf = wsb + lay.qbuf;
    void* kblk = wsb + lay.kblk;
    void* vblk = wsb + lay.vblk;
    float* opart = reinterpret_cast<float*>(wsb + lay.opart);
    float* mlpart = reinterpret_cast<float*>(wsb + lay.mlpart);
    void* obuf = wsb + lay.obuf;
    void* hbuf = wsb + lay.hbuf;
    const int ntH = s.H / GEMM_TILE_N;
    int rc;

    tr.begin("embed");
    hipLaunchKernelGGL((embed_block_kernel<T>), dim3(M), dim3(256), 0, st, static_cast<const T*>(w->embed), anchor,
                       s.mask, s.V, gamma, s.H, x, ssq_x, kv->status);
    tr.end();
    if (hipGetLastError() != hipSuccess) return DFLASH_ELAUNCH;
    int n_ssq = 1;

    const AttnPlan ap = plan_attn(s, gamma);
    const size_t attn_lds = attn_lds_bytes_host(s.esize, ap.qg, ap.kg);
    const size_t layer_elems = (size_t)s.Bmax * s.nkv * s.cap * s.D;

    for (int l = 0; l < s.L; ++l) {
        const dflash_layer_weights& lw = w->layers[l];
        {   // q, k, v of the block (+ per-head norm, RoPE)
            GemmArgs a = gemm_base(s, pl[0], M, s.H, ws, lay, part);
            a.a_mode = A_NORM;
            a.a = x;
            a.lda = s.H;
            a.ssq = ssq_x;
            a.n_ssq = n_ssq;
            a.ssq_ld = M;
            a.n_seg = 3;
            a.seg_n[0] = s.nq * s.D;
            a.seg_n[1] = s.nkv * s.D;
            a.seg_n[2] = s.nkv * s.D;
            a.N = (s.nq + 2 * s.nkv) * s.D;
            a.layer[0].w[0] = lw.wq;
            a.layer[0].w[1] = lw.wk;
            a.layer[0].w[2] = lw.wv;
            a.layer[0].norm_w = lw.in_norm;
            a.layer[0].head_norm = lw.q_norm;
            a.layer[0].head_norm2 = lw.k_norm;
            a.qbuf = qbuf;
            a.kblk = kblk;
            a.vblk = vblk;
            a.rpad = s.rpad;
            a.gamma = gamma;
            a.len = kv->len;
            a.rope_cos = w->rope_cos;
            a.rope_sin = w->rope_sin;
            a.rope_rows = w->rope_rows;
            a.status = kv->status;
            a.batch = batch;
            if ((rc = gemm_dispatch<T>(EPI_QKV, a, pl[0], s, st, tr, "qkv"))) return rc;
        }
        {   // attention over [context ; block]
            AttnArgs a;
            std::memset(&a, 0, sizeof(a));
            a.kcache = static_cast<const T*>(kv->k) + l * layer_elems;
            a.vcache = static_cast<const T*>(kv->v) + l * layer_elems;
            a.qbuf = qbuf;
            a.kblk = kblk;
            a.vblk = vblk;
            a.len = kv->len;
            a.opart = opart;
            a.mlpart = mlpart;
            a.n_kv = s.nkv;
            a.cap = s.cap;
            a.rpad = s.rpad;
            a.nch_max = s.nch_max;
            a.chunk = s.chunk;
            a.gamma = gamma;
            a.group = s.group;
            a.qg = ap.qg;
            a.kg = ap.kg;
            a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)s.D));
            tr.begin("attention");
            hipLaunchKernelGGL((attn_partial_kernel<T>), dim3(s.nch_max, s.nkv, batch), dim3(ATT_THREADS), attn_lds,
                               st, a);
            tr.end();
            if (hipGetLastError() != hipSuccess) return DFLASH_ELAUNCH;
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
            tr.begin("attn_merge");
            hipLaunchKernelGGL((attn_merge_kernel<T>), dim3(M, s.nq), dim3(128), 0, st, mgr);
            tr.end();
            if (hipGetLastError() != hipSuccess) return DFLASH_ELAUNCH;
        }
        {   // x += W_o o
            GemmArgs a = gemm_base(s, pl[1], M, s.nq * s.D, ws, lay, part);
            a.a_mode = A_PLAIN;
            a.a = obuf;
            a.lda = s.nq * s.D;
            a.n_seg = 1;
            a.seg_n[0] = s.H;
            a.N = s.H;
            a.layer[0].w[0] = lw.wo;
            a.out = x;
            a.ldo = s.H;
            a.residual = 1;
            a.ssq_out = ssq_x;
            a.ssq_out_ld = M;
            if ((rc = gemm_dispatch<T>(EPI_STORE, a, pl[1], s, st, tr, "o_proj"))) return rc;
            n_ssq = ntH;
        }
        {   // h = silu(W_gate a2) * (W_up a2)
            GemmArgs a = gemm_base(s, pl[2], M, s.H, ws, lay, part);
            a.a_mode = A_NORM;
            a.a = x;
            a.lda = s.H;
            a.ssq = ssq_x;
            a.n_ssq = n_ssq;
            a.ssq_ld = M;
            a.n_seg = 2;
            a.seg_n[0] = s.I;
            a.seg_n[1] = s.I;
            a.N = 2 * s.I;
            a.layer[0].w[0] = lw.w_gate;
            a.layer[0].w[1] = lw.w_up;
            a.layer[0].norm_w = lw.post_norm;
            a.out_t = hbuf;
            a.ldo = s.I;
            if ((rc = gemm_dispatch<T>(EPI_SWIGLU, a, pl[2], s, st, tr, "gate_up"))) return rc;
        }
        {   // x += W_down h
            GemmArgs a = gemm_base(s, pl[3], M, s.I, ws, lay, part);
            a.a_mode = A_PLAIN;
            a.a = hbuf;
            a.lda = s.I;
            a.n_seg = 1;
            a.seg_n[0] = s.H;
            a.N = s.H;
            a.layer[0].w[0] = lw.w_down;
            a.out = x;
            a.ldo = s.H;
            a.residual = 1;
            a.ssq_out = ssq_x;
            a.ssq_out_ld = M;
            if ((rc = gemm_dispatch<T>(EPI_STORE, a, pl[3], s, st, tr, "down_proj"))) return rc;
        }
    }
    if (dbg_hidden) {
        const long long n = (long long)M * s.H;
        const unsigned blocks = (unsigned)std::min<long long>(1024, (n + 255) / 256);
        tr.begin("copy_hidden");
        hipLaunchKernelGGL(copy_f32_kernel, dim3(blocks), dim3(256), 0, st, x, dbg_hidden, n);
        tr.end();
        if (hipGetLastError() != hipSuccess) return DFLASH_ELAUNCH;
    }
    {   // final norm -> LM head -> argmax over the vocabulary
        GemmArgs a = gemm_base(s, pl[4], M, s.H, ws, lay, part);
        a.a_mode = A_NORM;
        a.a = x;
        a.lda = s.H;
        a.ssq = ssq_x;
        a.n_ssq = n_ssq;
        a.ssq_ld = M;
        a.n_seg = 1;
        a.seg_n[0] = s.V;
        a.N = s.V;
        a.layer[0].w[0] = w->lm_head;
        a.layer[0].norm_w = w->final_norm;
        a.gamma = gamma;
        a.batch = batch;
        a.slots = reinterpret_cast<unsigned long long*>(wsb + lay.slots);
        a.draft = draft;
        a.dbg_logits = dbg_logits;
        if ((rc = gemm_dispatch<T>(EPI_ARGMAX, a, pl[4], s, st, tr, "lm_head_argmax"))) return rc;
    }
    return DFLASH_OK;
}

}  // namespace

extern "C" {

size_t dflash_workspace_bytes(const dflash_config* cfg, int32_t batch, int32_t max_rows_per_seq) {
    Shape s;
    if (make_shape(cfg, s) != DFLASH_OK) return 0;
    if (batch < 1 || batch > s.Bmax || max_rows_per_seq < 0) return 0;
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
    if (batch < 1 || batch > s.Bmax || rows_stride < 1) return DFLASH_EINVAL;
    if (w->rope_rows < s.cap + s.gmax) return DFLASH_EINVAL;
    if (trace && trace->capacity < 0) return DFLASH_EINVAL;
    if (!workspace) return DFLASH_EWORKSPACE;
    const Layout lay = make_layout(s, batch, rows_stride);
    if (workspace_bytes < lay.inject_end) return DFLASH_EWORKSPACE;
    GemmPlan ip[2];
    inject_plans(s, batch, rows_stride, ip);
    if (ip[0].counters > COUNTER_SLOTS || ip[1].counters > COUNTER_SLOTS) return DFLASH_EUNSUPPORTED;
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

int dflash_verify(int32_t batch, int32_t gamma, const int32_t* draft, const int32_t* target, int32_t* accept_len,
                  int32_t* committed, int32_t* next_anchor, void* stream) {
    if (batch < 1 || gamma < 2 || gamma > 1024) return DFLASH_EINVAL;
    if (!draft || !target || !accept_len || !committed || !next_anchor) return DFLASH_EINVAL;
    hipLaunchKernelGGL(verify_kernel, dim3(batch), dim3(64), 0, static_cast<hipStream_t>(stream), batch, gamma, draft,
                       target, accept_len, committed, next_anchor);
    return hipGetLastError() == hipSuccess ? DFLASH_OK : DFLASH_ELAUNCH;
}

const char* dflash_status_str(int status) {
    switch (status) {
        case DFLASH_OK: return "DFLASH_OK";
        case DFLASH_EINVAL: return "DFLASH_EINVAL: null pointer or size out of range";
        case DFLASH_EUNSUPPORTED: return "DFLASH_EUNSUPPORTED: shape or dtype not supported";
        case DFLASH_EWORKSPACE: return "DFLASH_EWORKSPACE: workspace missing or too small";
        case DFLASH_ELAUNCH: return "DFLASH_ELAUNCH: kernel launch failed";
    }
    return "unknown dflash status";
}

}  // extern "C"
