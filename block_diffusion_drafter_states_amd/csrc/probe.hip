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

// LDS read rate: each workgroup fills 32 KB of LDS, then every thread reads 16-byte
// vectors from it, four per iteration, consecutive lanes at consecutive vectors (no bank
// conflicts); the XOR of everything read decides a store into sink[blockIdx.x] that the
// key rules out in practice.  Four VALU operations per vector read: at 64 lanes over 4
// cycles per SIMD that caps the probe at 256 bytes per clock per CU, so a result near that
// figure means "at least", below it the LDS is what limits.
constexpr int LDS_VEC = 2048;

__global__ __launch_bounds__(256) void lds_probe_kernel(int iters, unsigned key, unsigned* __restrict__ sink) {
    __shared__ uint4 tile[LDS_VEC];
    for (int i = threadIdx.x; i < LDS_VEC; i += 256) tile[i] = make_uint4(i, i * 3u, i * 5u, i * 7u + blockIdx.x);
    __syncthreads();
    uint4 acc = make_uint4(0u, 0u, 0u, 0u);
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const uint4 v = tile[(threadIdx.x + (it * 4 + u) * 256) & (LDS_VEC - 1)];
            acc.x ^= v.x;
            acc.y ^= v.y;
            acc.z ^= v.z;
            acc.w ^= v.w;
        }
        // the addresses repeat every two iterations: keep the compiler from merging the
        // reads of equal addresses (which would cancel in the XOR)
        asm volatile("" ::: "memory");
    }
    const unsigned a = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if (a == key) sink[blockIdx.x] = a;
}

// Direct-to-LDS load rate: every wave streams 1 KB per instruction (global_load_lds_dwordx4,
// 16 bytes per lane) from a buffer of n_chunks 1 KB chunks (grid-stride over the waves) into a
// ring of 16 LDS slots of its own, at most DEPTH + 1 instructions in flight per wave (a slot is
// rewritten 16 instructions later, after its load has completed).  Nothing reads the LDS.
constexpr int DMA_SLOTS = 16;

template <int DEPTH>
__global__ __launch_bounds__(256) void dma_probe_kernel(const unsigned char* __restrict__ src, int n_chunks,
                                                        int iters) {
    static_assert(DEPTH + 1 < DMA_SLOTS, "a slot is rewritten only after its load has completed");
    __shared__ __align__(1024) unsigned char ring[4][DMA_SLOTS][1024];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const long long waves = (long long)gridDim.x * 4;
    const long long w0 = (long long)blockIdx.x * 4 + wave;
    const uint32_t lds0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)&ring[wave][0][0];
    for (int it = 0; it < iters; ++it) {
        const long long chunk = (w0 + (long long)it * waves) & (n_chunks - 1);   // n_chunks: a power of two
        const unsigned char* g = src + chunk * 1024 + lane * 16;
        const uint32_t lds = lds0 + (uint32_t)(it % DMA_SLOTS) * 1024u;
        asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(g), "s"(lds) : "memory", "m0");
        asm volatile("s_waitcnt vmcnt(%0)" : : "n"(DEPTH) : "memory");
    }
    asm volatile("s_waitcnt vmcnt(0)" : : : "memory");
}

// Issue cost of direct-to-LDS loads: every wave issues 16 loads of 1 KB (one GEMM stage's worth
// per wave) into its own LDS slots, reading the shader clock before and after the issue loop and
// after the loads have completed; lane 0 stores (issue cycles, issue + completion cycles) for
// its wave in out[2w], out[2w + 1].
__global__ __launch_bounds__(256) void dma_issue_probe_kernel(const unsigned char* __restrict__ src, int n_chunks,
                                                              long long* __restrict__ out) {
    __shared__ __align__(1024) unsigned char ring[4][DMA_SLOTS][1024];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const long long w0 = (long long)blockIdx.x * 4 + wave;
    const uint32_t lds0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)&ring[wave][0][0];
    const long long t0 = clock64();
#pragma unroll
    for (int it = 0; it < DMA_SLOTS; ++it) {
        const long long chunk = (w0 * DMA_SLOTS + it) & (n_chunks - 1);
        const unsigned char* g = src + chunk * 1024 + lane * 16;
        asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                     : : "v"(g), "s"(lds0 + (uint32_t)it * 1024u) : "memory", "m0");
    }
    const long long t1 = clock64();
    asm volatile("s_waitcnt vmcnt(0)" : : : "memory");
    const long long t2 = clock64();
    if (lane == 0) {
        out[w0 * 2] = t1 - t0;
        out[w0 * 2 + 1] = t2 - t0;
    }
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

// `blocks` workgroups of 256 threads, each thread `iters` x 4 LDS reads of 16 bytes: bytes
// read blocks * 256 * iters * 64; sink: device, `blocks` entries.
int dflash_probe_lds(int iters, int blocks, unsigned key, unsigned* sink, void* stream) {
    if (!sink || blocks < 1 || iters < 1) return -1;
    hipLaunchKernelGGL(lds_probe_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream), iters, key,
                       sink);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

// `blocks` workgroups of 4 waves, each wave `iters` direct-to-LDS loads of 1 KB from the first
// n_chunks KB (a power of two) of the device buffer `buf`, at most depth + 1 in flight per wave
// (depth 8 or 14): bytes loaded blocks * 4 * iters * 1024.
int dflash_probe_dma(const void* buf, int n_chunks, int iters, int blocks, int depth, void* stream) {
    if (!buf || n_chunks < 1 || (n_chunks & (n_chunks - 1)) || iters < 1 || blocks < 1) return -1;
    if (depth != 8 && depth != 14) return -1;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const unsigned char* src = static_cast<const unsigned char*>(buf);
    if (depth == 8) hipLaunchKernelGGL(dma_probe_kernel<8>, dim3(blocks), dim3(256), 0, st, src, n_chunks, iters);
    else hipLaunchKernelGGL(dma_probe_kernel<14>, dim3(blocks), dim3(256), 0, st, src, n_chunks, iters);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

// `blocks` workgroups of 4 waves, each wave 16 direct-to-LDS loads of 1 KB from the first n_chunks
// KB (a power of two) of `buf`; out: device, 8 * blocks int64 (per wave: issue cycles, issue +
// completion cycles, shader clock).
int dflash_probe_dma_issue(const void* buf, int n_chunks, long long* out, int blocks, void* stream) {
    if (!buf || !out || n_chunks < 1 || (n_chunks & (n_chunks - 1)) || blocks < 1) return -1;
    hipLaunchKernelGGL(dma_issue_probe_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const unsigned char*>(buf), n_chunks, out);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // extern "C"
