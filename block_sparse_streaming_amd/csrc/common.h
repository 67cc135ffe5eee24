// Device-side helpers shared by the SSA kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Raw v_exp_f32 (2^x). exp2(-inf) = 0, which the online softmax relies on.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Two floats -> two bf16 (round to nearest even), packed low/high.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// Low/high halves of a packed bf16 pair as floats.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Gather 16-bit element e (0..7) of row a and of row b into one 32-bit word
// (a in the low half). Rows are 8 bf16 held as four 32-bit words.
__device__ __forceinline__ uint32_t pick_pair(const u32x4& a, const u32x4& b, int e) {
    uint32_t wa = a[e >> 1], wb = b[e >> 1];
    return (e & 1) ? ((wa >> 16) | (wb & 0xffff0000u)) : ((wa & 0xffffu) | (wb << 16));
}

// Blocks are dispatched round-robin over the 8 XCDs, each with its own L2.
// Renumber them so that XCD x runs one contiguous range of logical ids:
// neighbouring work items then share an L2. A bijection on [0, total).
__device__ __forceinline__ int xcd_remap(int bid, int total) {
    const int x = bid & 7, idx = bid >> 3;
    const int q = total >> 3, r = total & 7;
    return x * q + (x < r ? x : r) + idx;
}

}  // namespace ssa
