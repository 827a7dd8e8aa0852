// Block loss finishes: the position-weighted block cross-entropy over the per-tile
// (max logit, sum of exp) pairs that the LM head's log-sum-exp epilogue writes, and its
// gradient with respect to the logits.
#pragma once

#include "common.hpp"

namespace dflash {

// ---- block loss: cross-entropy of the mask rows against their labels, weighted per
// block position ("DFlash" technical summary, section 2.3, loss weighting: the weight of
// block position k is exp(-(k - 1) / gamma), early positions count more).
//
// Stage 1.  lse is [n_tiles][M] (max logit, sum of exp(logit - max)) per LM-head tile.
// Workgroup (s, rb) folds slice s of n_slices of the tiles for the 64 rows rb*64 ..
// +63 (one row per lane; wave w takes tiles s0 + w, s0 + w + 4, ... in ascending
// order, so every read is 64 consecutive pairs) and writes part[s][m]: the four waves
// are combined through LDS in wave order.  Deterministic: fixed orders throughout.
__device__ __forceinline__ float2 lse_fold(float2 acc, float2 t) {
    if (t.x == -INFINITY) return acc;
    if (acc.x == -INFINITY) return t;
    const float mx = fmaxf(acc.x, t.x);
    return make_float2(mx, acc.y * __expf(acc.x - mx) + t.y * __expf(t.x - mx));
}

__global__ __launch_bounds__(256) void lse_slices_kernel(const float2* __restrict__ lse, int n_tiles, int n_slices,
                                                         int M, float2* __restrict__ part) {
    __shared__ float2 red[4][64];
    const int s = blockIdx.x;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int m = blockIdx.y * 64 + lane;
    const int per = (n_tiles + n_slices - 1) / n_slices;
    const int t0 = s * per, t1 = min(n_tiles, t0 + per);
    float2 acc = make_float2(-INFINITY, 0.f);
    if (m < M)
        for (int t = t0 + w; t < t1; t += 4) acc = lse_fold(acc, lse[(long long)t * M + m]);
    red[w][lane] = acc;
    __syncthreads();
    if (threadIdx.x < 64 && m < M) {
        float2 x = red[0][lane];
        for (int k = 1; k < 4; ++k) x = lse_fold(x, red[k][lane]);
        part[(long long)s * M + m] = x;
    }
}

// Stage 2 (one workgroup of BLOCK_LOSS_THREADS threads, one wavefront per row at a
// time; lse_out [M], nullable, receives each mask row's log-sum-exp).  Row m = b*gamma + j with j >= 1: the lanes fold the slices s = lane, lane +
// 64, ... in ascending order and an xor-shuffle tree combines the lanes; LSE - logit
// of the label is the row's CE; row_loss[b][j-1] = CE (nullable); loss[0] = sum_b
// sum_j w_j CE / (batch * sum_j w_j) with w_j = exp(-(j - 1) / gamma), each wave
// summing its rows in ascending order and the waves summed in wave order.  A label
// outside [0, vocab) sets STATUS_BAD_TOKEN and makes its row (and the total) NaN.
constexpr int BLOCK_LOSS_THREADS = 1024;

__global__ __launch_bounds__(BLOCK_LOSS_THREADS) void block_loss_kernel(
    const float2* __restrict__ part, int n_slices, int M, int gamma, const int* __restrict__ labels,
    const float* __restrict__ lab_logit, int vocab, float* __restrict__ loss, float* __restrict__ row_loss,
    float* __restrict__ lse_out, unsigned* status) {
    constexpr int NW = BLOCK_LOSS_THREADS / 64;
    __shared__ float red[NW];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int G = gamma;
    float acc = 0.f;
    for (int m = wv; m < M; m += NW) {
        const int b = m / G, j = m % G;
        if (j == 0) continue;
        const int lab = labels[b * (G - 1) + j - 1];
        float ce;
        if (lab < 0 || lab >= vocab) {
            if (lane == 0) atomicOr(status, STATUS_BAD_TOKEN);
            ce = __int_as_float(0x7fc00000);
        } else {
            float2 x = make_float2(-INFINITY, 0.f);
            for (int sl = lane; sl < n_slices; sl += 64) x = lse_fold(x, part[(long long)sl * M + m]);
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const float2 y = make_float2(__shfl_xor(x.x, o, WAVE), __shfl_xor(x.y, o, WAVE));
                x = lse_fold(x, y);
            }
            const float lse = x.x + logf(x.y);
            if (lse_out && lane == 0) lse_out[m] = lse;
            ce = lse - lab_logit[m];
        }
        if (lane == 0 && row_loss) row_loss[b * (G - 1) + j - 1] = ce;
        acc += expf(-(float)(j - 1) / (float)G) * ce;
    }
    if (lane == 0) red[wv] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        float tot = 0.f, wsum = 0.f;
        for (int k = 0; k < NW; ++k) tot += red[k];
        for (int j = 1; j < G; ++j) wsum += expf(-(float)(j - 1) / (float)G);
        loss[0] = tot / ((float)(M / G) * wsum);
    }
}

// Gradient of the block loss with respect to the mask rows' logits:
//   dL/dz[b][j][v] = w_j / (batch * sum_j w_j) * (exp(z[b][j][v] - LSE[b][j]) - [v == label[b][j]])
// z and dz are fp32 [batch][gamma-1][vocab] and may be the same buffer (in place).
// blockIdx.y is the mask row (b, j); the x blocks stride over its vocabulary, consecutive
// threads on consecutive ids.  A row whose label is outside [0, vocab) gets NaN.
__global__ __launch_bounds__(256) void block_loss_grad_kernel(const float* z, float* dz, const float* __restrict__ lse,
                                                              const int* __restrict__ labels, int batch, int gamma,
                                                              int vocab) {
    const int row = blockIdx.y;                          // b * (gamma - 1) + j - 1
    const int b = row / (gamma - 1), j = row % (gamma - 1) + 1;
    float wsum = 0.f;
    for (int k = 1; k < gamma; ++k) wsum += expf(-(float)(k - 1) / (float)gamma);
    const float c = expf(-(float)(j - 1) / (float)gamma) / ((float)batch * wsum);
    const int lab = labels[row];
    const bool bad = lab < 0 || lab >= vocab;
    const float l = lse[b * gamma + j];
    const float* zr = z + (long long)row * vocab;
    float* dr = dz + (long long)row * vocab;
    for (int v = blockIdx.x * blockDim.x + threadIdx.x; v < vocab; v += gridDim.x * blockDim.x) {
        const float p = __expf(zr[v] - l);
        dr[v] = bad ? __int_as_float(0x7fc00000) : c * (p - (v == lab ? 1.f : 0.f));
    }
}

}  // namespace dflash
