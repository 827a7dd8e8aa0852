// Small kernels of the cycle: block embedding, greedy verification, copies.
#pragma once

#include "common.hpp"

namespace dflash {

// x[b*gamma + j][:] = E[id] with id = anchor[b] (j == 0) or the mask id, and the
// first layer's input RMSNorm of that row, rho(x * rstd * w), into xn (one
// workgroup owns the whole row, so its sum of squares needs no partial tiles).
// Token ids outside [0, vocab) set STATUS_BAD_TOKEN and read row 0.
constexpr int EMBED_MAX_HIDDEN = 8192;

template <typename T>
__global__ __launch_bounds__(256) void embed_norm_kernel(const T* __restrict__ embed, const int* __restrict__ anchor,
                                                         const int* __restrict__ tokens, int mask_id, int vocab,
                                                         int gamma, int H,
                                                         const T* __restrict__ w_norm, float eps,
                                                         float* __restrict__ x, T* __restrict__ xn,
                                                         unsigned* status, int xn_frag) {
    constexpr int EPC = 16 / (int)sizeof(T);                    // elements per 16-byte chunk
    constexpr int MAXC = EMBED_MAX_HIDDEN / EPC / 256;           // chunks per thread
    __shared__ float red[4];
    const int m = blockIdx.x;
    const int b = m / gamma, j = m % gamma;
    int id = tokens ? tokens[m] : ((j == 0) ? anchor[b] : mask_id);
    if (id < 0 || id >= vocab) {
        if (threadIdx.x == 0) atomicOr(status, STATUS_BAD_TOKEN);
        id = 0;
    }
    const T* e = embed + (long long)id * H;
    u32x4_t ev[MAXC], wv[MAXC];
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
        const int k = (c * 256 + threadIdx.x) * EPC;
        if (k < H) {
            ev[c] = *reinterpret_cast<const u32x4_t*>(e + k);
            wv[c] = *reinterpret_cast<const u32x4_t*>(w_norm + k);
        }
    }
    float ss = 0.f;
    float xv[MAXC][EPC];
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
        const int k = (c * 256 + threadIdx.x) * EPC;
        if (k < H) {
            const T* ep = reinterpret_cast<const T*>(&ev[c]);
#pragma unroll
            for (int u = 0; u < EPC; ++u) {
                xv[c][u] = Elem<T>::to_f(ep[u]);
                ss += xv[c][u] * xv[c][u];
            }
            float* xr = x + (long long)m * H + k;
#pragma unroll
            for (int u = 0; u < EPC; u += 4)
                *reinterpret_cast<float4*>(xr + u) = make_float4(xv[c][u], xv[c][u + 1], xv[c][u + 2], xv[c][u + 3]);
        }
    }
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float rs = 1.0f / sqrtf(((red[0] + red[1]) + (red[2] + red[3])) / (float)H + eps);
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
        const int k = (c * 256 + threadIdx.x) * EPC;
        if (k < H) {
            const T* wp = reinterpret_cast<const T*>(&wv[c]);
            T* o = xn + (xn_frag ? afrag_offset<T>(m, k, H) : (long long)m * H + k);   // one 16-byte chunk
#pragma unroll
            for (int u = 0; u < EPC; ++u) o[u] = Elem<T>::from_f(xv[c][u] * rs * Elem<T>::to_f(wp[u]));
        }
    }
}

// One wavefront per sequence: k = leading matches of draft[j] == target[j].
__global__ __launch_bounds__(64) void verify_kernel(int batch, int gamma, const int* __restrict__ draft,
                                                    const int* __restrict__ target, int* __restrict__ accept_len,
                                                    int* __restrict__ committed, int* __restrict__ next_anchor) {
    const int b = blockIdx.x;
    const int lane = threadIdx.x;
    const int* d = draft + (long long)b * (gamma - 1);
    const int* y = target + (long long)b * gamma;
    int k = gamma - 1;
    for (int base = 0; base < gamma - 1; base += 64) {
        const int j = base + lane;
        const bool mism = (j < gamma - 1) && (d[j] != y[j]);
        const unsigned long long ball = __ballot(mism);
        if (ball) {
            k = base + __ffsll((long long)ball) - 1;
            break;
        }
    }
    for (int j = lane; j < gamma; j += 64) committed[(long long)b * gamma + j] = (j <= k) ? y[j] : -1;
    if (lane == 0) {
        accept_len[b] = k + 1;
        next_anchor[b] = y[k];
    }
}

// out[z][m][k] = rho(x[m][k] * rstd_m * w_z[k]); rstd_m from the per-tile sums of
// squares of row m.  blockIdx.x = row, blockIdx.y = 1024-column chunk,
// blockIdx.z = weight set (one per layer when the same rows feed every layer).
// Every load of a thread is issued before the first reduction (one memory
// latency); the partial sums are added in a fixed order (deterministic).
struct NormWeights {
    const void* w[16];
};

constexpr int NORM_MAX_PARTIALS = 512;

// When len_snap is given, block 0 also copies len[0 .. n_len) there (the K/V
// cache writes that follow read positions from the copy while len itself is
// advanced).  row_factor = 0 writes rho(x * w) without the row's factor (the input of an
// argmax LM head: a positive factor per row leaves each row's argmax where it is).
template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_rows_kernel(const float* __restrict__ x, int ldx,
                                                           const float* __restrict__ ssq, int n_ssq, int ssq_ld,
                                                           const NormWeights wz, int K, float eps,
                                                           T* __restrict__ out, int ldo, long long out_z,
                                                           const int* __restrict__ len, int* __restrict__ len_snap,
                                                           int n_len, int out_frag, int row_factor) {
    __shared__ float red[4];
    if (len_snap && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0)
        for (int b = threadIdx.x; b < n_len; b += 256) len_snap[b] = len[b];
    const int m = blockIdx.x;
    const int k = blockIdx.y * 1024 + threadIdx.x * 4;   // K % 4 == 0
    const bool has = k < K;
    const T* w = reinterpret_cast<const T*>(wz.w[blockIdx.z]);
    const float4 xv = has ? *reinterpret_cast<const float4*>(x + (long long)m * ldx + k) : make_float4(0.f, 0.f, 0.f, 0.f);
    float wv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) wv[u] = has ? Elem<T>::to_f(w[k + u]) : 0.f;
    const int t0 = threadIdx.x, t1 = threadIdx.x + 256;
    const float s0 = t0 < n_ssq ? ssq[(long long)t0 * ssq_ld + m] : 0.f;
    const float s1 = t1 < n_ssq ? ssq[(long long)t1 * ssq_ld + m] : 0.f;
    float s = wave_sum(s0 + s1);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
    __syncthreads();
    const float rs = row_factor ? 1.0f / sqrtf(((red[0] + red[1]) + (red[2] + red[3])) / (float)K + eps) : 1.0f;
    if (has) {
        // four consecutive columns stay contiguous in fragment order (k % 4 == 0)
        T* o = out + (long long)blockIdx.z * out_z + (out_frag ? afrag_offset<T>(m, k, K) : (long long)m * ldo + k);
        o[0] = Elem<T>::from_f(xv.x * rs * wv[0]);
        o[1] = Elem<T>::from_f(xv.y * rs * wv[1]);
        o[2] = Elem<T>::from_f(xv.z * rs * wv[2]);
        o[3] = Elem<T>::from_f(xv.w * rs * wv[3]);
    }
}

// Returned logits of an argmax LM head whose input rows were rho(x * w) without the final
// RMSNorm's row factor: logits[i][n] *= f_m, f_m = 1 / sqrt(sum_t ssq[t][m] / K + eps), for the
// draft rows i = b*(gamma - first) + j - first (row m = b*gamma + j, j >= first).  Workgroup
// (s, i) takes vocabulary slice s of row i; every workgroup of a row sums the row's partial
// sums of squares in the same order.  Only runs when the caller asks for the logits.
__global__ __launch_bounds__(256) void scale_logit_rows_kernel(float* __restrict__ logits, int V,
                                                               const float* __restrict__ ssq, int n_ssq, int ssq_ld,
                                                               int gamma, int first, int K, float eps) {
    __shared__ float red[4];
    const int i = blockIdx.y, per_seq = gamma - first;
    const int m = (i / per_seq) * gamma + first + i % per_seq;
    const int t0 = threadIdx.x, t1 = threadIdx.x + 256;
    const float s0 = t0 < n_ssq ? ssq[(long long)t0 * ssq_ld + m] : 0.f;
    const float s1 = t1 < n_ssq ? ssq[(long long)t1 * ssq_ld + m] : 0.f;
    const float s = wave_sum(s0 + s1);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
    __syncthreads();
    const float f = 1.0f / sqrtf(((red[0] + red[1]) + (red[2] + red[3])) / (float)K + eps);
    float* row = logits + (long long)i * V;
    for (int n = blockIdx.x * 256 + threadIdx.x; n < V; n += gridDim.x * 256) row[n] *= f;
}

// Per-head RMSNorm then rotate-half RoPE of one row of D values, rounded into
// dst; one wavefront, lane i < D/2 owns the pair (i, i + D/2).
template <typename T>
__device__ __forceinline__ void head_norm_rope_store(const float* src, int D, const T* wnorm, float eps,
                                                     const float* cosr, const float* sinr, T* dst) {
    const int lane = threadIdx.x & 63;
    const int half = D >> 1;
    float x1 = 0.f, x2 = 0.f;
    if (lane < half) { x1 = src[lane]; x2 = src[lane + half]; }
    const float ss = wave_sum(x1 * x1 + x2 * x2);
    const float rs = 1.0f / sqrtf(ss / (float)D + eps);
    if (lane < half) {
        const float y1 = x1 * rs * Elem<T>::to_f(wnorm[lane]);
        const float y2 = x2 * rs * Elem<T>::to_f(wnorm[lane + half]);
        const float c = cosr[lane], s = sinr[lane];
        dst[lane] = Elem<T>::from_f(y1 * c - y2 * s);
        dst[lane + half] = Elem<T>::from_f(y2 * c + y1 * s);
    }
}

// Injected rows -> cache.  kv holds the fp32 projections [L][Mi][2 * n_kv * D]
// (k heads, then v heads) of row m = b * rows_stride + i.  Row i < n_new[b] of
// sequence b lands at position len[b] + i: k heads get the layer's k RMSNorm and
// RoPE (K cache [L][Bmax][n_kv][cap][D]), v heads are rounded into the
// V cache in 32-key blocks of V^T, [L][Bmax][n_kv][cap / 32][D][32].  Positions come from len_snap, a
// copy of len taken before this kernel; workgroup (0, 0, b) then advances
// len[b] += n_new[b], or sets STATUS_BAD_COUNT / STATUS_KV_OVERFLOW and writes
// nothing for that sequence.  blockIdx = (head of 2 n_kv, layer, sequence);
// 256 threads.
struct KvFinishArgs {
    const float* kv;            // [layers][rows][row_ld]; k heads then v heads at the row start
    long long layer_stride;     // between layers of kv
    int row_ld;                 // floats between rows of kv (2 * n_kv * D for injection)
    int rows_stride, n_kv, head_dim, cap, rope_rows;
    int layer0;                 // cache layer of grid layer 0
    int update_len;             // advance len by n_new (injection) or leave it (target block rows)
    int n_const;
    long long cache_layer;      // Bmax * n_kv * cap * D
    void* kcache;
    void* vcache;
    const void* k_norm[16];     // per grid layer [D]
    float eps;
    const int* len_snap;
    int* len;
    const int* n_new;           // nullable: then every sequence writes n_const rows
    const float* rope_cos;
    const float* rope_sin;
    unsigned* status;
};

// Grid (2 n_kv, L, batch * row blocks): workgroup (hh, l, b * rb_n + rb) writes rows
// rb * KV_ROWS .. of sequence b for head hh (k heads first, then v heads) of layer l,
// so a whole prompt's injection spreads over many workgroups.  Workgroup (0, 0, b * rb_n)
// checks the counts and advances len[b]; every workgroup reads the position from the
// snapshot taken before this injection.
constexpr int KV_ROWS = 64;

template <typename T>
__global__ __launch_bounds__(256) void kv_finish_kernel(const KvFinishArgs a, int rb_n) {
    const int hh = blockIdx.x, gl = blockIdx.y, l = a.layer0 + gl, b = blockIdx.z / rb_n, rb = blockIdx.z % rb_n;
    const int D = a.head_dim, RS = a.rows_stride, cap = a.cap;
    const int len = a.len_snap[b], nn = a.n_new ? a.n_new[b] : a.n_const;
    const bool bad_count = nn < 0 || nn > RS || len < 0;
    const bool overflow = !bad_count && (len + nn > cap || len + nn > a.rope_rows);
    if (hh == 0 && gl == 0 && rb == 0 && threadIdx.x == 0) {
        if (bad_count) atomicOr(a.status, STATUS_BAD_COUNT);
        else if (overflow) atomicOr(a.status, STATUS_KV_OVERFLOW);
        else if (a.update_len) a.len[b] = len + nn;
    }
    if (bad_count || overflow) return;
    const int i0 = rb * KV_ROWS, nr = min(KV_ROWS, nn - i0);
    if (nr <= 0) return;
    const bool is_k = hh < a.n_kv;
    const int h = is_k ? hh : hh - a.n_kv;
    const int ld = a.row_ld;
    const float* src = a.kv + gl * a.layer_stride + ((long long)b * RS + i0) * ld + (long long)hh * D;
    if (is_k) {
        T* kc = reinterpret_cast<T*>(a.kcache) + l * a.cache_layer + ((long long)b * a.n_kv + h) * cap * (long long)D;
        const int wv = threadIdx.x >> 6;
        for (int i = wv; i < nr; i += 4) {
            const int pos = len + i0 + i;
            head_norm_rope_store<T>(src + (long long)i * ld, D, reinterpret_cast<const T*>(a.k_norm[gl]), a.eps,
                                    a.rope_cos + (long long)pos * (D / 2), a.rope_sin + (long long)pos * (D / 2),
                                    kc + (long long)pos * D);
        }
    } else {
        // V^T rows: consecutive threads write consecutive positions of one d
        T* vc = reinterpret_cast<T*>(a.vcache) + l * a.cache_layer + ((long long)b * a.n_kv + h) * (long long)D * cap;
        for (int e = threadIdx.x; e < D * nr; e += 256) {
            const int d = e / nr, i = e % nr;
            const int pos = len + i0 + i;      // 32-key blocks of V^T ([cap / 32][D][32])
            vc[(long long)(pos / 32) * (D * 32) + d * 32 + pos % 32] = Elem<T>::from_f(src[(long long)i * ld + d]);
        }
    }
}

// feat[b][j][f][:] = x[b * rows + j][:] in the storage type: the hidden state after a
// tapped decoder layer, as the drafter's injection reads it ([B][rows][F][H]).
template <typename T>
__global__ __launch_bounds__(256) void tap_kernel(const float* __restrict__ x, long long n, int H, int F, int f,
                                                  T* __restrict__ feat) {
    for (long long e = blockIdx.x * 256ll + threadIdx.x; e < n; e += (long long)gridDim.x * 256) {
        const long long m = e / H;
        const int k = (int)(e % H);
        feat[(m * F + f) * H + k] = Elem<T>::from_f(x[e]);
    }
}

// len[b] += n[b] after a verification (n = accepted length) or a chunk of a prompt;
// a count outside 0 .. cap - len sets a status bit and leaves len.
// len[b] += n[b] when 0 <= n[b] <= max_n and len[b] + max(n[b], need) <= cap (need: rows
// the same call wrote from len[b] on, which must all have fitted); else a status bit.
__global__ __launch_bounds__(64) void advance_len_kernel(int* __restrict__ len, const int* __restrict__ n, int batch,
                                                         int cap, int max_n, int need, unsigned* status) {
    for (int b = threadIdx.x; b < batch; b += 64) {
        const int l = len[b], k = n[b];
        if (k < 0 || k > max_n || l < 0) atomicOr(status, STATUS_BAD_COUNT);
        else if (l + (k > need ? k : need) > cap) atomicOr(status, STATUS_KV_OVERFLOW);
        else len[b] = l + k;
    }
}

__global__ __launch_bounds__(256) void copy_f32_kernel(const float* __restrict__ src, float* __restrict__ dst,
                                                       long long n) {
    for (long long i = blockIdx.x * 256ll + threadIdx.x; i < n; i += (long long)gridDim.x * 256) dst[i] = src[i];
}

}  // namespace dflash
