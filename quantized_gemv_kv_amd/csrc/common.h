// common.h — internal definitions shared by the libtsd HIP sources (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace tsd {

// ---- weight formats in the kernel ("packed") layout -----------------------------------------
// Canonical blocks (18/34-byte AoS) are not 16-byte aligned, so every matrix is repacked at
// model creation into structure-of-arrays form: per row, the quantized payload is contiguous
// (one 16-byte slot = one dwordx4 load per lane), and the fp16 scales (and affine biases) sit
// in separate row-major arrays.
//   Q4_0: slot = one 32-element block's 16 nibble bytes, same nibble order as the canonical
//         block (low nibbles = elements 0..15, high = 16..31).
//   Q8_0: slot = half a block (16 elements); bytes stored as q + 128 (unsigned), so that the
//         byte-to-float conversions need no sign handling; the -128 is folded into the sum.
//   AFF8: slot = a quarter of a 64-group (16 elements); q stored as is.
//   Q5_0: slot = one block's 16 nibble bytes in Q4_0's order; the block's 32 fifth bits (bit j
//         for element j) in a separate array of 32-bit words; w = (q - 16) d.
//   AFF4_G64 / AFF4_G32: slot = 32 elements of a 64 (32) group, repacked into Q4_0's nibble
//         order (byte b: element b low, element b + 16 high); w = s q + b.
enum Fmt : int { FMT_Q4_0 = 0, FMT_Q8_0 = 1, FMT_AFF8 = 2, FMT_Q5_0 = 3, FMT_AFF4_G64 = 4, FMT_AFF4_G32 = 5 };
constexpr int FMT_COUNT = 6;

template <int F> struct FmtT;
template <> struct FmtT<FMT_Q4_0> { static constexpr int E = 32, SLOTS_PER_SCALE = 1, SCALE_GROUP = 32; };
template <> struct FmtT<FMT_Q8_0> { static constexpr int E = 16, SLOTS_PER_SCALE = 2, SCALE_GROUP = 32; };
template <> struct FmtT<FMT_AFF8> { static constexpr int E = 16, SLOTS_PER_SCALE = 4, SCALE_GROUP = 64; };
template <> struct FmtT<FMT_Q5_0> { static constexpr int E = 32, SLOTS_PER_SCALE = 1, SCALE_GROUP = 32; };
template <> struct FmtT<FMT_AFF4_G64> { static constexpr int E = 32, SLOTS_PER_SCALE = 2, SCALE_GROUP = 64; };
template <> struct FmtT<FMT_AFF4_G32> { static constexpr int E = 32, SLOTS_PER_SCALE = 1, SCALE_GROUP = 32; };

// formats whose slot holds 32 four-bit codes in Q4_0's nibble order
__host__ __device__ constexpr bool fmt_nibbles(int f) { return f == FMT_Q4_0 || f == FMT_Q5_0 || f == FMT_AFF4_G64 || f == FMT_AFF4_G32; }
// formats with a per-group bias (w = s q + b)
__host__ __device__ constexpr bool fmt_affine(int f) { return f == FMT_AFF8 || f == FMT_AFF4_G64 || f == FMT_AFF4_G32; }
__host__ __device__ inline int fmt_elems_per_slot(int f) { return fmt_nibbles(f) ? 32 : 16; }
__host__ __device__ inline int fmt_group(int f) { return f == FMT_AFF8 || f == FMT_AFF4_G64 ? 64 : 32; }
__host__ __device__ inline size_t fmt_row_bytes(int f, int K) { return fmt_nibbles(f) ? (size_t)K / 2 : (size_t)K; }

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

struct PackedMat {
    const uint8_t* q;    // [N][row_bytes]
    const __half* s;     // [N][K/group]
    const __half* b;     // [N][K/group] affine biases, else null
    const uint32_t* h;   // [N][K/32] Q5_0 fifth bits, else null
    int N, K;
};

// byte layout of one packed matrix inside a buffer
struct PackedLayout {
    size_t q_off, s_off, b_off, h_off, total;
};
inline PackedLayout packed_layout(int f, int N, int K)
{
    PackedLayout L;
    L.q_off = 0;
    L.s_off = align256((size_t)N * fmt_row_bytes(f, K));
    size_t sb = align256((size_t)N * (K / fmt_group(f)) * 2);
    L.b_off = L.s_off + sb;
    L.h_off = L.b_off + (fmt_affine(f) ? sb : 0);
    L.total = L.h_off + (f == FMT_Q5_0 ? align256((size_t)N * (K / 32) * 4) : 0);
    return L;
}
inline PackedMat packed_view(int f, void* base, int N, int K)
{
    PackedLayout L = packed_layout(f, N, K);
    uint8_t* p = (uint8_t*)base;
    PackedMat m;
    m.q = p + L.q_off;
    m.s = (const __half*)(p + L.s_off);
    m.b = fmt_affine(f) ? (const __half*)(p + L.b_off) : nullptr;
    m.h = f == FMT_Q5_0 ? (const uint32_t*)(p + L.h_off) : nullptr;
    m.N = N;
    m.K = K;
    return m;
}

// A GEMV shape is supported when the lanes of a wave map onto row slots without remainder:
// slots per row (K / elements-per-slot) is a power of two up to 64, or larger than 64.
inline bool gemv_shape_ok(int f, int K)
{
    int E = fmt_elems_per_slot(f);
    if (K <= 0 || K % fmt_group(f)) return false;
    int lpr = K / E;
    if (lpr > 64) return true;
    return (lpr & (lpr - 1)) == 0;
}

// ---- wave-level helpers --------------------------------------------------------------------
// DPP lane moves (CDNA row = 16 lanes): xor-1 and xor-2 inside quads, mirrors inside the half
// row and the row; gfx950's permlane swaps exchange rows 16 and 32 lanes apart.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float swap16_sum(float v)
{
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float swap32_sum(float v)
{
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
#ifndef TSD_PERMLANE_SWAP
#define TSD_PERMLANE_SWAP 1
#endif
// sum over aligned groups of g lanes (g a power of two <= 64); every lane gets its group's sum
__device__ __forceinline__ float group_sum(float v, int g)
{
    if (g >= 2) v += dpp_mov<0xB1>(v);    // quad_perm [1,0,3,2]
    if (g >= 4) v += dpp_mov<0x4E>(v);    // quad_perm [2,3,0,1]
    if (g >= 8) v += dpp_mov<0x141>(v);   // row_half_mirror
    if (g >= 16) v += dpp_mov<0x140>(v);  // row_mirror
#if TSD_PERMLANE_SWAP
    if (g >= 32) v = swap16_sum(v);
    if (g >= 64) v = swap32_sum(v);
#else
    if (g >= 32) v += __shfl_xor(v, 16, 64);
    if (g >= 64) v += __shfl_xor(v, 32, 64);
#endif
    return v;
}
__device__ __forceinline__ float wave_sum(float v) { return group_sum(v, 64); }
__device__ __forceinline__ float wave_max(float v)
{
    v = fmaxf(v, dpp_mov<0xB1>(v));
    v = fmaxf(v, dpp_mov<0x4E>(v));
    v = fmaxf(v, dpp_mov<0x141>(v));
    v = fmaxf(v, dpp_mov<0x140>(v));
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// maximum of a 64-bit key over the wave (both halves moved by the same lane pattern)
template <int CTRL>
__device__ __forceinline__ unsigned long long dpp_mov64(unsigned long long v)
{
    const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)v, CTRL, 0xF, 0xF, true);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, true);
    return ((unsigned long long)hi << 32) | lo;
}
__device__ __forceinline__ unsigned long long max64(unsigned long long a, unsigned long long b) { return a > b ? a : b; }
__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v)
{
    v = max64(v, dpp_mov64<0xB1>(v));
    v = max64(v, dpp_mov64<0x4E>(v));
    v = max64(v, dpp_mov64<0x141>(v));
    v = max64(v, dpp_mov64<0x140>(v));
    // the swaps return (own, partner) in a lane-dependent order, the same for both halves
    auto a = __builtin_amdgcn_permlane16_swap((uint32_t)v, (uint32_t)v, false, false);
    auto b = __builtin_amdgcn_permlane16_swap((uint32_t)(v >> 32), (uint32_t)(v >> 32), false, false);
    v = max64(((unsigned long long)b[0] << 32) | a[0], ((unsigned long long)b[1] << 32) | a[1]);
    a = __builtin_amdgcn_permlane32_swap((uint32_t)v, (uint32_t)v, false, false);
    b = __builtin_amdgcn_permlane32_swap((uint32_t)(v >> 32), (uint32_t)(v >> 32), false, false);
    return max64(((unsigned long long)b[0] << 32) | a[0], ((unsigned long long)b[1] << 32) | a[1]);
}

// global-address-space views of a pointer: loads and stores through them are global_* (vector
// memory counter only) even when the compiler cannot see where the pointer came from — flat
// accesses would also count against the LDS counter and hold up LDS-only barriers
#define TSD_GLOBAL __attribute__((address_space(1)))
template <class T>
__device__ __forceinline__ const TSD_GLOBAL T* glb(const T* p) { return (const TSD_GLOBAL T*)p; }
template <class T>
__device__ __forceinline__ TSD_GLOBAL T* glb(T* p) { return (TSD_GLOBAL T*)p; }

// uniform load through the scalar cache (read only; the value was written by an earlier kernel)
__device__ __forceinline__ int ld_uniform(const int* p)
{
    return *(const __attribute__((address_space(4))) int*)p;
}

// barrier for LDS traffic only: waits for this wave's LDS operations, not for its
// outstanding global loads (so weight loads stay in flight across the norm prologue)
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0), vmcnt/expcnt left at their maximum
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// monotone map of a float to an unsigned key (larger float -> larger key)
__device__ __forceinline__ uint32_t float_order_key(float f)
{
    uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace tsd
