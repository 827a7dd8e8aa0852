// Device-side building blocks shared by the DFlash kernels (gfx950 / CDNA4).
//
// Conventions used everywhere:
//  * a wavefront is 64 lanes; lane = g*16 + r with g = lane/16 (0..3), r = lane%16;
//  * MFMA 16x16x32 bf16 operand layout: lane (g,r) supplies A[m=r][k=g*8+j] and
//    B[k=g*8+j][n=r] for j = 0..7 and receives C[m=g*4+v][n=r] for v = 0..3;
//  * MFMA 16x16x4 f32 layout: lane (g,r) supplies A[m=r][k=g], B[k=g][n=r] and
//    receives the same C layout.
//  A "k-step" is 256 bytes of every operand row, read as four 64-byte lines:
//  in load i the four lanes of row r (g = 0..3) read bytes [64 i + 16 g, +16),
//  so every load instruction covers whole 64-byte lines.  Piece i feeds MFMA i
//  (bf16: k = 32 i + 8 g + j, the native 16x16x32 layout) or MFMAs 4i..4i+3
//  (f32).  Both operands use the same assignment of k to MFMA slots.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dflash {

typedef uint16_t bf16_t;  // bf16 bit pattern
typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(unsigned)))) unsigned u32x4_t;

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

// Two floats -> two bf16 (round to nearest even) packed low/high in one dword,
// with gfx950's packed conversion instruction.
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_hw_t;
__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
    const bf16x2_hw_t v = {(__bf16)lo, (__bf16)hi};
    uint32_t u;
    __builtin_memcpy(&u, &v, 4);
    return u;
}

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

// 64 bytes of one operand row held by one lane: 4 x 16-byte pieces, 64 bytes apart.
struct Frag64 {
    u32x4_t q[4];
};

// p = row start + 16*g bytes (the lane's first piece); pieces follow every 64 bytes.
__device__ __forceinline__ void load_frag64(Frag64& f, const void* p) {
    const u32x4_t* s = reinterpret_cast<const u32x4_t*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) f.q[i] = s[4 * i];
}

__device__ __forceinline__ void zero_frag64(Frag64& f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f.q[i] = u32x4_t{0u, 0u, 0u, 0u};
}

__device__ __forceinline__ bf16x8_t as_bf16x8(const u32x4_t& v) {
    bf16x8_t r;
    __builtin_memcpy(&r, &v, 16);
    return r;
}

// ---- A operand in fragment order ------------------------------------------------------------
// The weight-streaming GEMM reads, per 16-row tile of A and 256-byte k-step, piece i of lane
// (g, r) = row r, 16-byte chunk 4i + g of the step.  Rows laid out plainly put the 16 rows of one
// load instruction 64 bytes apart in 16 cache lines; producers feeding that GEMM write A in
// fragment order instead, where that instruction reads 1 KB of contiguous bytes:
//   A[m][k] at element ((((m / 16) * (K / S) + k / S) * 4 + i) * 64 + g * 16 + m % 16) * E + k % E
// with S elements per 256-byte step, E per 16 bytes and 4i + g = (k % S) / E.  A buffer holds
// whole 16-row tiles; K must be a multiple of S.
template <typename T>
__host__ __device__ __forceinline__ long long afrag_offset(int m, int k, int K) {
    constexpr int E = 16 / (int)sizeof(T), S = 256 / (int)sizeof(T);
    const int kk = k % S, c = kk / E;
    return ((((long long)(m >> 4) * (K / S) + k / S) * 4 + (c >> 2)) * 64 + (c & 3) * 16 + (m & 15)) * E + kk % E;
}

// ---- explicitly scheduled vector-memory operations (streaming loops) ----------------------
// These are opaque to the compiler's wait-count pass: the caller issues them in a
// fixed order and waits with vm_wait<N>() (loads complete in issue order), then
// ties the destination registers so that no use is scheduled before the wait.

// LDS byte offset of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// 16 bytes per lane from global memory straight into LDS at lds + 16 * lane
// (lds must be wave-uniform).
__device__ __forceinline__ void dma_b128(const void* g, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(g), "s"(lds)
                 : "memory", "m0");
}

// The same with the non-temporal hint, for data a launch reads once (streamed weights):
// on MI355X the LM head's weight stream (1.24 GB) took 198 us with it against 217 us
// without, whole cycle 816.5 -> 766.2 us at the Qwen3-8B shape.
__device__ __forceinline__ void dma_b128_nt(const void* g, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
                 :
                 : "v"(g), "s"(lds)
                 : "memory", "m0");
}

__device__ __forceinline__ void vload_b128(u32x4_t& d, const void* g) {
    asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(d) : "v"(g) : "memory");
}

__device__ __forceinline__ void vload_b32(uint32_t& d, const void* g) {
    asm volatile("global_load_dword %0, %1, off" : "=v"(d) : "v"(g) : "memory");
}

__device__ __forceinline__ void vload_u16(uint32_t& d, const void* g) {
    asm volatile("global_load_ushort %0, %1, off" : "=v"(d) : "v"(g) : "memory");
}

template <int N>
__device__ __forceinline__ void vm_wait() {
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

__device__ __forceinline__ void tie(u32x4_t& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void tie(uint32_t& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void tie(Frag64& f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) tie(f.q[i]);
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
        const u32x4_t av = a.q[i], bv = b.q[i];
#pragma unroll
        for (int c = 0; c < 4; ++c)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(av[c]), __uint_as_float(bv[c]), acc, 0, 0, 0);
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

// Per-tile maxima of an argmax LM-head launch: row m holds 8 runs of amax_per slots, tile t
// in slot (t mod 8) * amax_per + t / 8.  Workgroup t of the launch runs on XCD t mod 8 (the
// dispatcher deals workgroups round-robin over the eight XCDs, and the tiled kernel maps
// tiles that way), so what one XCD writes of a row is one contiguous run of whole cache
// lines in its own L2, and the finish reads a row as one contiguous span.  Slots of tiles
// >= n_tiles (at most 7 per row) are never written.
__host__ __device__ constexpr int amax_per(int n_tiles) { return (n_tiles + 7) >> 3; }
__host__ __device__ constexpr long long amax_ld(int n_tiles) { return 8LL * amax_per(n_tiles); }
__host__ __device__ constexpr long long amax_slot(int m, int tile, int n_tiles) {
    return (long long)m * amax_ld(n_tiles) + (long long)(tile & 7) * amax_per(n_tiles) + (tile >> 3);
}

// Status bits (sticky, OR-ed into dflash_kv.status).
constexpr uint32_t STATUS_KV_OVERFLOW = 1u;   // len + rows > kv_capacity
constexpr uint32_t STATUS_BAD_TOKEN = 2u;     // token id outside [0, vocab)
constexpr uint32_t STATUS_BAD_COUNT = 4u;     // n_new outside [0, rows_stride] or len < 0

}  // namespace dflash
