// Measurement probes for the roofline: the HBM read bandwidth a plain streaming kernel
// reaches on this GPU, and the bf16 matrix-core rate of a loop of independent MFMAs.
// Built as a separate library (libdflash_probe.so): the benchmark reports the drafting
// cycle's kernels against these measured ceilings as well as against the published peaks.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

// Every thread reads 16-byte vectors in a grid-stride loop, four independent loads per
// iteration; the XOR of everything read decides a store that never happens for the data
// the caller passes (all bytes zero or any data whose XOR differs from the key), so the
// loads cannot be removed.  sink has one entry per workgroup.
__global__ __launch_bounds__(256) void read_probe_kernel(const uint4* __restrict__ src, long long n_vec,
                                                         unsigned key, unsigned* __restrict__ sink) {
    const long long stride = (long long)gridDim.x * blockDim.x;
    unsigned acc = 0u;
    long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + 3 * stride < n_vec; i += 4 * stride) {
        const uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
        acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
    }
    for (; i < n_vec; i += stride) {
        const uint4 a = src[i];
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    if (acc == key) sink[blockIdx.x] = acc;
}

// The same read with the non-temporal hint and eight independent loads per thread in
// flight: on MI355X the best of the shapes measured (one workgroup per CU, 7.1-7.2 TB/s
// over 2 GiB against ~5.5 TB/s for the plain loads above with many workgroups).
typedef unsigned u32x4v __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(256) void read_nt_probe_kernel(const u32x4v* __restrict__ src, long long n_vec,
                                                            unsigned key, unsigned* __restrict__ sink) {
    const long long stride = (long long)gridDim.x * blockDim.x;
    unsigned acc = 0u;
    long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + 7 * stride < n_vec; i += 8 * stride) {
        u32x4v v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n_vec; i += stride) {
        const u32x4v a = src[i];
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    if (acc == key) sink[blockIdx.x] = acc;
}

// Each wave runs `iters` rounds of NACC independent v_mfma_f32_16x16x32_bf16 on register
// operands (no memory traffic in the loop); lane 0 of each workgroup stores a sum of its
// accumulators so that the chain is kept.  16 x 16 x 32 x 2 flops per instruction.
constexpr int NACC = 8;

__global__ __launch_bounds__(256) void mfma_probe_kernel(int iters, float* __restrict__ sink) {
    bf16x8_t a, b;
    for (int j = 0; j < 8; ++j) {
        a[j] = (short)(0x3f80 + (threadIdx.x & 7));      // bf16 values near 1
        b[j] = (short)(0x3f80 - (threadIdx.x & 3));
    }
    f32x4_t acc[NACC];
    for (int k = 0; k < NACC; ++k) acc[k] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int k = 0; k < NACC; ++k) acc[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[k], 0, 0, 0);
    }
    float s = 0.f;
    for (int k = 0; k < NACC; ++k) s += acc[k][0] + acc[k][1] + acc[k][2] + acc[k][3];
    if (threadIdx.x == 0) sink[blockIdx.x] = s;
}

typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

// The same with v_mfma_f32_32x32x16_bf16 (32 x 32 x 16 x 2 flops per instruction), NACC32
// independent 32 x 32 accumulators per wave.
constexpr int NACC32 = 4;

__global__ __launch_bounds__(256) void mfma32_probe_kernel(int iters, float* __restrict__ sink) {
    bf16x8_t a, b;
    for (int j = 0; j < 8; ++j) {
        a[j] = (short)(0x3f80 + (threadIdx.x & 7));
        b[j] = (short)(0x3f80 - (threadIdx.x & 3));
    }
    f32x16_t acc[NACC32];
    for (int k = 0; k < NACC32; ++k)
        for (int e = 0; e < 16; ++e) acc[k][e] = 0.f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int k = 0; k < NACC32; ++k) acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[k], 0, 0, 0);
    }
    float s = 0.f;
    for (int k = 0; k < NACC32; ++k)
        for (int e = 0; e < 16; ++e) s += acc[k][e];
    if (threadIdx.x == 0) sink[blockIdx.x] = s;
}

}  // namespace

extern "C" {

// Read `bytes` (a multiple of 16) from the device buffer `buf` with `blocks` workgroups of
// 256 threads; sink: device, `blocks` entries (written only when the XOR of the data equals
// `key`).  Returns 0, or -1 for invalid arguments / a failed launch.  Asynchronous on stream.
int dflash_probe_read(const void* buf, size_t bytes, unsigned key, unsigned* sink, int blocks, void* stream) {
    if (!buf || !sink || blocks < 1 || bytes % 16) return -1;
    hipLaunchKernelGGL(read_probe_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const uint4*>(buf), (long long)(bytes / 16), key, sink);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

// As dflash_probe_read with the non-temporal eight-load kernel.
int dflash_probe_read_nt(const void* buf, size_t bytes, unsigned key, unsigned* sink, int blocks, void* stream) {
    if (!buf || !sink || blocks < 1 || bytes % 16) return -1;
    hipLaunchKernelGGL(read_nt_probe_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4v*>(buf), (long long)(bytes / 16), key, sink);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

// `blocks` workgroups of 4 waves, each wave `iters` x 8 bf16 MFMAs of 16 x 16 x 32; sink:
// device, `blocks` floats.  Flops issued: blocks * 4 * iters * 8 * 16384.
int dflash_probe_mfma(int iters, int blocks, float* sink, void* stream) {
    if (!sink || blocks < 1 || iters < 1) return -1;
    hipLaunchKernelGGL(mfma_probe_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream), iters, sink);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

// As dflash_probe_mfma with 32 x 32 x 16 MFMAs: flops issued blocks * 4 * iters * 4 * 32768.
int dflash_probe_mfma32(int iters, int blocks, float* sink, void* stream) {
    if (!sink || blocks < 1 || iters < 1) return -1;
    hipLaunchKernelGGL(mfma32_probe_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream), iters,
                       sink);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // extern "C"
