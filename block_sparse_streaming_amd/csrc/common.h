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

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] + vmcnt_hi[15:14],
// expcnt[6:4], lgkmcnt[11:8]); the counters not named are left at their max.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_lgkmcnt0() {
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));
}

// Work-group barrier for pipelines that load LDS with direct global->LDS
// transfers. __syncthreads() carries a fence that waits for every outstanding
// vector-memory operation, prefetches included; here the caller waits for
// exactly the transfers it needs (wait_vmcnt) and this barrier only orders
// the waves. The empty asm statements keep the compiler from moving memory
// accesses across it.
__device__ __forceinline__ void barrier_no_fence() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Barrier after which every wave's LDS reads issued before it have completed,
// so the buffer they read may be overwritten.
__device__ __forceinline__ void barrier_lds_drained() {
    asm volatile("" ::: "memory");
    wait_lgkmcnt0();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// 16 bytes global -> LDS without passing through registers. Lane i of the wave
// writes lds_wave_base + 16*i; the base must be the same for the whole wave.
__device__ __forceinline__ void dma16(const void *src, void *lds_wave_base) {
    __builtin_amdgcn_global_load_lds(src, (lds_void *)lds_wave_base, 16, 0, 0);
}

// The same 16-byte global -> LDS transfer, issued from inline assembly so that
// the compiler does not track it: it then adds no waits of its own before LDS
// reads (its alias tracking of these transfers does not survive loops), and
// the caller alone orders the buffer with wait_vmcnt + a barrier. The
// instruction writes no VGPR. lds_wave_base is the wave-uniform LDS byte
// address of lane 0's 16 bytes.
// M0 carries the LDS address; the statement restores it, since the compiler
// reserves M0 and assumes it unchanged.
__device__ __forceinline__ void dma16_untracked(const void *src, uint32_t lds_wave_base) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(src), "s"(lds_wave_base)
        : "memory");
}

// The same untracked 16-byte transfer addressed as a wave-uniform base plus a
// 32-bit per-lane byte offset (the global instruction's scalar-base form):
// no 64-bit address arithmetic per lane and per transfer. `base` must be
// uniform; it is read from the first active lane.
__device__ __forceinline__ void dma16_sbase_untracked(const void *base, uint32_t off, uint32_t lds_wave_base) {
    const uint64_t b = (uint64_t)(uintptr_t)base;
    // readfirstlane returns a signed int: take both halves as uint32_t before
    // widening, or a low half with bit 31 set would sign-extend over the high one.
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
    const uint64_t sb = ((uint64_t)hi << 32) | lo;
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(off), "s"(sb), "s"(lds_wave_base)
        : "memory");
}

// A 4-byte untracked global -> LDS transfer: lane i's dword lands at
// lds_wave_base + 4 i. Same contract as dma16_untracked.
__device__ __forceinline__ void dma4_untracked(const void *src, uint32_t lds_wave_base) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dword %1, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(src), "s"(lds_wave_base)
        : "memory");
}

// max(x, x from lane ^ 16) and max(x, x from lane ^ 32) on the VALU (gfx950
// permlane swaps), instead of an LDS round trip through ds_bpermute.
__device__ __forceinline__ float max_xor16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)(const lds_void *)p;
}

// LDS transpose read (ds_read_b64_tr_b16). Within each group of 16 lanes,
// result lane i, element k is element (i % 4) of the 8 bytes addressed by
// lane 4k + i/4. If lane s of a group points at row s/4, columns 4(s%4)..+3 of
// a row-major 4x16 block of 16-bit values, lane i receives column i.
__device__ __forceinline__ i16x4 lds_read_tr16(const void *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p));
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
