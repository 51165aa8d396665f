// Device-side helpers shared by the gfx950 kernels of the kvq library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

constexpr int kD = 128;        // head dimension
constexpr int kGroup = 32;     // channels per scale/zero group
constexpr int kNGroups = kD / kGroup;
constexpr int kCodeBytes = kD / 4;   // packed bytes per row
constexpr float kMinNormalHalf = 6.103515625e-05f;   // 2^-14, least normal fp16

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bits_as_float(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t float_as_bits(float f) { return __builtin_bit_cast(uint32_t, f); }

__device__ __forceinline__ float half_bits_to_float(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}
// fp32 -> fp16 with round-to-nearest-even (v_cvt_f16_f32 in the default
// rounding mode); subnormal fp16 results are kept.
__device__ __forceinline__ uint16_t float_to_half_bits(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// fp32 -> fp16 (round to nearest even) of a value that must first exist as
// an fp32 number: the empty asm keeps the compiler from folding the FMA that
// produced x into a mixed-precision FMA with an fp16 result, which would
// round once to fp16 instead of to fp32 and then to fp16 as the format's
// scale is defined (the two differ when the fp32 value lands on an fp16
// rounding boundary).
__device__ __forceinline__ uint16_t fp32_value_to_half_bits(float x) {
  asm volatile("" : "+v"(x));
  return float_to_half_bits(x);
}

// The two divisions of the quantizer, correctly rounded, without the
// general IEEE division sequence.
// s = RN(range / L) for L = 3 or 15: q0 = range * RN(1/L), then one FMA
// residual step (Markstein); equal to the correctly rounded quotient for
// every non-negative finite fp32 range (checked exhaustively on the host by
// the same operation sequence).  L = 1: s = range.
template <int L>
__device__ __forceinline__ float div_by_levels(float range) {
#pragma clang fp contract(off)
  if constexpr (L == 1) {
    return range;
  } else {
    static_assert(L == 3 || L == 15, "levels of 2- or 4-bit codes");
    constexpr float y = L == 3 ? 0.3333333432674408f : 0.06666667014360428f;   // RN(1/L)
    const float q0 = range * y;
    const float r = __builtin_fmaf(-(float)L, q0, range);      // exact residual
    return __builtin_fmaf(r, y, q0);
  }
}

// RN(1/s) for a positive finite fp16 value s (held in fp32): v_rcp_f32
// (within one ulp of 1/s) and one Newton step with FMAs; equal to the
// correctly rounded reciprocal for every such s and every start within two
// ulps of 1/s (checked exhaustively on the host).
__device__ __forceinline__ float recip_of_half_value(float s) {
#pragma clang fp contract(off)
  const float y0 = __builtin_amdgcn_rcpf(s);
  const float e = __builtin_fmaf(-s, y0, 1.0f);
  return __builtin_fmaf(e, y0, y0);
}

// First cache slot of sequence b's new rows: the call's t_offset, or
// offsets[b] for a per-sequence append.
__device__ __forceinline__ int64_t seq_offset(const int32_t *offsets, int64_t t_offset, int64_t b) {
  return offsets != nullptr ? (int64_t)offsets[b] : t_offset;
}

// Cache row of slot `slot` (in [0, T_cap)) of (batch b, KV head h) for a
// write: (b*Hkv + h)*T_cap + slot, or through a block table (slot t of
// sequence b is row t % P of page table[b*max_pages + t / P]; the slot is
// below max_pages * P < 2^31), -1 when the page index is outside the pool.
__device__ __forceinline__ int64_t write_row(const int32_t *table, int64_t max_pages, int64_t n_pages,
                                             int64_t P, int Hkv, int64_t b, int h, int64_t T_cap,
                                             int64_t slot) {
  if (table == nullptr) return (b * Hkv + h) * T_cap + slot;
  const uint32_t sl = (uint32_t)slot, p32 = (uint32_t)P, pi = sl / p32;
  const int64_t page = table[b * max_pages + pi];
  if (page < 0 || page >= n_pages) return -1;
  return (page * Hkv + h) * P + (sl - pi * p32);
}

// Cross-lane moves inside a quad of four lanes (DPP quad_perm).
// kQuadXor1: lane i reads lane i^1; kQuadXor2: lane i reads lane i^2.
constexpr int kQuadXor1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;  // quad_perm [2,3,0,1]

template <int CTRL>
__device__ __forceinline__ float quad_swap(float v) {
  return bits_as_float((uint32_t)__builtin_amdgcn_mov_dpp((int)float_as_bits(v), CTRL, 0xF, 0xF, true));
}

// Butterfly across lanes of a quad: lanes whose bit is 0 get own + partner,
// lanes whose bit is 1 get partner - own.  `neg` is -1.0f on the latter.
template <int CTRL>
__device__ __forceinline__ float quad_butterfly(float own, float neg) {
  float other = quad_swap<CTRL>(own);
  return __builtin_fmaf(own, neg, other);   // exact: own * (+-1) + other, one rounding
}

// Rotate right by N lanes within each row of 16 lanes (DPP row_ror).
template <int N>
__device__ __forceinline__ float row_ror(float v) {
  return bits_as_float((uint32_t)__builtin_amdgcn_mov_dpp((int)float_as_bits(v), 0x120 + N, 0xF, 0xF, false));
}

__device__ __forceinline__ float shfl_xor_f(float v, int mask) {
  return __shfl_xor(v, mask, 64);
}

}  // namespace kvq
