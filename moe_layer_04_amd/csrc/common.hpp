// common.hpp -- device helpers shared by the gfx950 kernels of the fused MoE
// layer: operand vector types, bf16 / OCP-E4M3 conversions and wave64
// reductions built from DPP row permutations and ds_swizzle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef short bf16x8_t __attribute__((ext_vector_type(8)));   // 8 bf16: one MFMA K-slice
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));      // 32 fp8 codes
typedef unsigned short u16x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// number formats
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) {
    return __uint_as_float(h << 16);
}

// fp32 -> bf16 bits, round to nearest even, by the gfx950 conversion
// instruction (v_cvt_pk_bf16_f32; NaN stays a quiet NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}
// two values in one conversion instruction: lo in bits 0-15, hi in 16-31
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// fp32 -> OCP E4M3FN code: nearest value, ties to the even mantissa, after
// clamping the magnitude to 448 (the largest finite code); NaN -> 0x7F.
// Written from the format's definition: 4 exponent bits with bias 7, 3
// mantissa bits, subnormals on a 2^-9 grid below 2^-6.
__device__ __forceinline__ uint32_t f32_to_e4m3(float f) {
    uint32_t u = __float_as_uint(f);
    uint32_t sign = (u >> 24) & 0x80u;
    uint32_t a = u & 0x7fffffffu;
    if (a > 0x7f800000u) return 0x7fu;                 // NaN
    if (a > 0x43e00000u) a = 0x43e00000u;              // clamp to 448.0f
    if (a < 0x3c800000u) {                             // |f| < 2^-6: subnormal grid
        float q = __builtin_rintf(__uint_as_float(a) * 512.0f);   // exact scaling
        return sign | (uint32_t)q;                     // q == 8 is the min normal code
    }
    uint32_t ex = (a >> 23) - 127u + 7u;               // biased e4m3 exponent, 1..15
    uint32_t mant = (a & 0x7fffffu) | 0x800000u;       // 24-bit significand
    uint32_t q = mant >> 20;                           // 4 bits incl. the hidden one
    uint32_t rem = mant & 0xfffffu;
    q += (rem > 0x80000u) || (rem == 0x80000u && (q & 1u));
    if (q == 16u) { q = 8u; ++ex; }
    return sign | (ex << 3) | (q - 8u);
}

// ---------------------------------------------------------------------------
// wave64 reductions: DPP within rows of 16 lanes, ds_swizzle across the two
// rows of each half-wave, readlane across the halves.
// ---------------------------------------------------------------------------

// DPP controls (GFX9 encoding).
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;
constexpr int kSwizzleXor16 = 0x401F;   // bitmask mode: and 0x1f, xor 0x10

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, 0xF, 0xF, false);
}

__device__ __forceinline__ uint32_t swz_xor16_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, kSwizzleXor16);
}

// Generic lane exchange of a 64-bit or 32-bit value via the above.
template <int STEP>
__device__ __forceinline__ uint32_t xchg_u32(uint32_t v) {
    if constexpr (STEP == 0) return dpp_u32<kDppQuadXor1>(v);
    else if constexpr (STEP == 1) return dpp_u32<kDppQuadXor2>(v);
    else if constexpr (STEP == 2) return dpp_u32<kDppRowHalfMirror>(v);
    else if constexpr (STEP == 3) return dpp_u32<kDppRowMirror>(v);
    else return swz_xor16_u32(v);
}

template <int STEP>
__device__ __forceinline__ double xchg_f64(double v) {
    uint64_t b = __double_as_longlong(v);
    uint32_t lo = xchg_u32<STEP>((uint32_t)b);
    uint32_t hi = xchg_u32<STEP>((uint32_t)(b >> 32));
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

template <int STEP>
__device__ __forceinline__ uint64_t xchg_u64(uint64_t b) {
    uint32_t lo = xchg_u32<STEP>((uint32_t)b);
    uint32_t hi = xchg_u32<STEP>((uint32_t)(b >> 32));
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint32_t readlane_u32(uint32_t v, int lane) {
    return (uint32_t)__builtin_amdgcn_readlane((int)v, lane);
}

// Sum over all 64 lanes, result in every lane.  After the five in-half-wave
// steps each lane holds the sum of its 32-lane half.
__device__ __forceinline__ double wave_sum_f64(double v) {
    v += xchg_f64<0>(v);
    v += xchg_f64<1>(v);
    v += xchg_f64<2>(v);
    v += xchg_f64<3>(v);
    v += xchg_f64<4>(v);
    uint64_t b = __double_as_longlong(v);
    uint64_t b0 = ((uint64_t)readlane_u32((uint32_t)(b >> 32), 0) << 32) | readlane_u32((uint32_t)b, 0);
    uint64_t b1 = ((uint64_t)readlane_u32((uint32_t)(b >> 32), 32) << 32) | readlane_u32((uint32_t)b, 32);
    return __longlong_as_double((long long)b0) + __longlong_as_double((long long)b1);
}

__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// Max over all 64 lanes of a 64-bit key, result in every lane.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
    v = max_u64(v, xchg_u64<0>(v));
    v = max_u64(v, xchg_u64<1>(v));
    v = max_u64(v, xchg_u64<2>(v));
    v = max_u64(v, xchg_u64<3>(v));
    v = max_u64(v, xchg_u64<4>(v));
    uint64_t b0 = ((uint64_t)readlane_u32((uint32_t)(v >> 32), 0) << 32) | readlane_u32((uint32_t)v, 0);
    uint64_t b1 = ((uint64_t)readlane_u32((uint32_t)(v >> 32), 32) << 32) | readlane_u32((uint32_t)v, 32);
    return max_u64(b0, b1);
}

// Max over all 64 lanes of a non-negative float (as its bit pattern, whose
// unsigned order equals the float order), result in every lane.
__device__ __forceinline__ uint32_t wave_max_bits(uint32_t v) {
    v = max(v, xchg_u32<0>(v));
    v = max(v, xchg_u32<1>(v));
    v = max(v, xchg_u32<2>(v));
    v = max(v, xchg_u32<3>(v));
    v = max(v, xchg_u32<4>(v));
    return max(readlane_u32(v, 0), readlane_u32(v, 32));
}

// Max of a non-negative float over the four lanes l, l^16, l^32, l^48 (the
// lanes that share one column of a 16x16 MFMA accumulator).
__device__ __forceinline__ uint32_t col_max_bits(uint32_t v) {
    v = max(v, swz_xor16_u32(v));
    v = max(v, (uint32_t)__shfl_xor((int)v, 32));
    return v;
}

// ---------------------------------------------------------------------------
// misc
// ---------------------------------------------------------------------------

// Pin an accumulator at this point of the program.  Without it the compiler
// may sink the last MFMAs of a loop into a lane-divergent epilogue branch,
// where operands it materialises under the partial EXEC mask (such as the
// block-scale constant of the scaled FP8 MFMA) are left unset in inactive
// lanes -- while the MFMA itself still reads every lane.
template <typename T>
__device__ __forceinline__ void pin(T& v) {
    asm volatile("" : "+v"(v));
}

__device__ __forceinline__ int lane_id() { return (int)__lane_id(); }

// Token of sorted slot p (p = t*topk + j, non-negative).  The divisor is
// clamped to 1 so that the compiler may compute the quotient for every lane
// (a division by a value that might be zero stays behind a lane-divergent
// branch, which also serialises the loads feeding it).
__device__ __forceinline__ int slot_token(int p, int topk) {
    return (int)((uint32_t)p / (uint32_t)max(topk, 1));
}

// z / (1 + e^-z) with the hardware reciprocal (1 ulp) in place of the IEEE
// division sequence; e^-z = inf gives z * 0 = -0, as the division would.
__device__ __forceinline__ float silu(float z) {
    return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

}  // namespace moe
