// seer_device.hpp -- gfx950 device helpers shared by the library's kernels.
//
// Wave64 cross-lane primitives (DPP within 16-lane rows, permlane swaps across
// rows), bf16 unpacking and the bf16 dot2 builtin.  Nothing here is specific
// to one kernel.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace seer {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// acc + a.lo * b.lo + a.hi * b.hi with bf16 pairs (v_dot2_f32_bf16, fp32 accumulate).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), acc, false);
}

// Round-to-nearest-even fp32 -> bf16 bits (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// DPP controls (GFX9 encoding).
enum : int {
    kDppXor1 = 0xB1,        // quad_perm [1,0,3,2]
    kDppXor2 = 0x4E,        // quad_perm [2,3,0,1]
    kDppHalfMirror = 0x141, // lane i <- 7 - i within each 8-lane half row
    kDppMirror = 0x140,     // lane i <- 15 - i within each 16-lane row
    kDppRor8 = 0x128,       // lane i <- (i + 8) mod 16 within each row (= xor 8)
};

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    // bound_ctrl set: every control used here reads a valid lane, and it lets the
    // compiler fold the move into the consuming VALU op (v_add_f32_dpp).
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

// max(a, b) for non-NaN inputs in one VALU op: the median of (a, b, +inf).
__device__ __forceinline__ float fmax_fast(float a, float b) { return __builtin_amdgcn_fmed3f(a, b, __builtin_inff()); }

// gfx950 permlane swaps exchange 16-lane rows (odd rows of the first operand with
// even rows of the second) or 32-lane halves.  Fed the same value twice, the two
// results of every lane are {x, x of the partner row/half} in some order, so a
// commutative op over them is the pairwise reduction, bitwise identical in both partners.
__device__ __forceinline__ float sum_xor16(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_xor16(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmax_fast(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmax_fast(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Sum over aligned groups of N consecutive lanes (N in 8, 16), result in every lane of the group.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(N == 8 || N == 16, "group of 8 or 16 lanes");
    x += dpp<kDppXor1>(x);
    x += dpp<kDppXor2>(x);
    x += dpp<kDppHalfMirror>(x);
    if constexpr (N == 16) x += dpp<kDppMirror>(x);
    return x;
}

// Reduce across the 64/STRIDE groups of lanes that share (lane mod STRIDE), STRIDE in {8, 16, 32}.
template <int STRIDE>
__device__ __forceinline__ float cross_group_max(float x) {
    static_assert(STRIDE == 8 || STRIDE == 16 || STRIDE == 32, "stride");
    if constexpr (STRIDE == 8) x = fmax_fast(x, dpp<kDppRor8>(x));
    if constexpr (STRIDE <= 16) x = max_xor16(x);
    return max_xor32(x);
}
template <int STRIDE>
__device__ __forceinline__ float cross_group_sum(float x) {
    static_assert(STRIDE == 8 || STRIDE == 16 || STRIDE == 32, "stride");
    if constexpr (STRIDE == 8) x += dpp<kDppRor8>(x);
    if constexpr (STRIDE <= 16) x = sum_xor16(x);
    return sum_xor32(x);
}

__device__ __forceinline__ float wave_sum(float x) { return cross_group_sum<16>(group_sum<16>(x)); }

__device__ __forceinline__ float wave_max(float x) {
    x = fmax_fast(x, dpp<kDppXor1>(x));
    x = fmax_fast(x, dpp<kDppXor2>(x));
    x = fmax_fast(x, dpp<kDppHalfMirror>(x));
    x = fmax_fast(x, dpp<kDppMirror>(x));
    return cross_group_max<16>(x);
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Raw buffer descriptor word 3 for plain 32-bit dword access (gfx9 family).
constexpr int kBufferFlags = 0x00020000;

// Descriptor over [base, base + bytes); loads past its range return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, kBufferFlags);
}

// 16-byte loads at descriptor base + voff + soff (bytes): cached, and
// non-temporal (streamed past the caches' normal retention).
__device__ __forceinline__ uint4 buf_ld16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    const u32x4_t t = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
    return make_uint4(t.x, t.y, t.z, t.w);
}
__device__ __forceinline__ uint4 buf_ld16_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    const u32x4_t t = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 2));
    return make_uint4(t.x, t.y, t.z, t.w);
}
__device__ __forceinline__ float4 as_float4(uint4 u) {
    return make_float4(__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z), __uint_as_float(u.w));
}

// How the kernel bodies read and write data that another launch produced or
// consumes (launches on one stream): plain loads and stores.
struct LaunchMem {
    __device__ static int ldi(const int32_t *p) { return *p; }
    __device__ static float ldf(const float *p) { return *p; }
    __device__ static float2 ldf2(const float2 *p) { return *p; }
    __device__ static void sti(int32_t *p, int v) { *p = v; }
    __device__ static void stf(float *p, float v) { *p = v; }
    __device__ static void stf2(float2 *p, float x, float y) { *p = make_float2(x, y); }
};

}  // namespace seer
