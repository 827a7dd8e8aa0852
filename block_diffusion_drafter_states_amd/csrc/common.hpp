// Device-side building blocks shared by the DFlash kernels (gfx950 / CDNA4).
//
// Conventions used everywhere:
//  * a wavefront is 64 lanes; lane = g*16 + r with g = lane/16 (0..3), r = lane%16;
//  * MFMA 16x16x32 bf16 operand layout: lane (g,r) supplies A[m=r][k=g*8+j] and
//    B[k=g*8+j][n=r] for j = 0..7 and receives C[m=g*4+v][n=r] for v = 0..3;
//  * MFMA 16x16x4 f32 layout: lane (g,r) supplies A[m=r][k=g], B[k=g][n=r] and
//    receives the same C layout.
//  A "k-step" is 256 bytes of every operand row: each lane reads 64 contiguous
//  bytes of a row (32 bf16 or 16 f32), which feed 4 (bf16) or 16 (f32) MFMAs.
//  The reduction index is permuted consistently on both operands, so any
//  assignment of k to MFMA slots gives the same dot products.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dflash {

typedef uint16_t bf16_t;  // bf16 bit pattern
typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

constexpr int WAVE = 64;

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
    return __uint_as_float(((uint32_t)b) << 16);
}

// Round to nearest even; inputs are finite.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (bf16_t)(u >> 16);
}

__device__ __forceinline__ float round_bf16(float f) { return bf16_to_f32(f32_to_bf16(f)); }

// Element storage type traits: bf16 (bit patterns) or f32.
template <typename T> struct Elem;
template <> struct Elem<bf16_t> {
    static constexpr int PER16 = 8;               // elements per 16-byte load
    static constexpr int STEP = 128;              // elements per k-step (4 groups x 64 B)
    __device__ static float load(const bf16_t* p) { return bf16_to_f32(*p); }
    __device__ static float to_f(bf16_t v) { return bf16_to_f32(v); }
    __device__ static bf16_t from_f(float v) { return f32_to_bf16(v); }
    __device__ static float rho(float v) { return round_bf16(v); }
};
template <> struct Elem<float> {
    static constexpr int PER16 = 4;
    static constexpr int STEP = 64;
    __device__ static float load(const float* p) { return *p; }
    __device__ static float to_f(float v) { return v; }
    __device__ static float from_f(float v) { return v; }
    __device__ static float rho(float v) { return v; }
};

// 64 bytes of one operand row held by one lane: 4 x 16-byte pieces.
struct Frag64 {
    uint4 q[4];
};

__device__ __forceinline__ void load_frag64(Frag64& f, const void* p) {
    const uint4* s = reinterpret_cast<const uint4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) f.q[i] = s[i];
}

__device__ __forceinline__ void zero_frag64(Frag64& f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f.q[i] = make_uint4(0, 0, 0, 0);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& v) {
    bf16x8_t r;
    __builtin_memcpy(&r, &v, 16);
    return r;
}

// acc += A_frag . B_frag over one k-step (64 bytes per lane of each operand).
template <typename T>
__device__ __forceinline__ void mfma_kstep(f32x4_t& acc, const Frag64& a, const Frag64& b);

template <>
__device__ __forceinline__ void mfma_kstep<bf16_t>(f32x4_t& acc, const Frag64& a, const Frag64& b) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a.q[i]), as_bf16x8(b.q[i]), acc, 0, 0, 0);
}

template <>
__device__ __forceinline__ void mfma_kstep<float>(f32x4_t& acc, const Frag64& a, const Frag64& b) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint4 av = a.q[i], bv = b.q[i];
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(av.x), __uint_as_float(bv.x), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(av.y), __uint_as_float(bv.y), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(av.z), __uint_as_float(bv.z), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(av.w), __uint_as_float(bv.w), acc, 0, 0, 0);
    }
}

// Deterministic wave-wide reductions (fixed butterfly order).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, WAVE);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, WAVE));
    return v;
}

// Order-preserving map of a finite float onto uint32 (larger float -> larger key).
__device__ __forceinline__ uint32_t float_order_key(float f) {
    uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// (value, index) packed so that unsigned max picks the larger value and, among
// equal values, the lower index.
__device__ __forceinline__ unsigned long long pack_argmax(float v, uint32_t idx) {
    return ((unsigned long long)float_order_key(v) << 32) | (unsigned long long)(0xFFFFFFFFu - idx);
}

__device__ __forceinline__ uint32_t unpack_argmax_index(unsigned long long p) {
    return 0xFFFFFFFFu - (uint32_t)(p & 0xFFFFFFFFull);
}

// Status bits (sticky, OR-ed into dflash_kv.status).
constexpr uint32_t STATUS_KV_OVERFLOW = 1u;   // len + rows > kv_capacity
constexpr uint32_t STATUS_BAD_TOKEN = 2u;     // token id outside [0, vocab)
constexpr uint32_t STATUS_BAD_COUNT = 4u;     // n_new outside [0, rows_stride] or len < 0

}  // namespace dflash
