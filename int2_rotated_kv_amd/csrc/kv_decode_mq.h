// Pieces shared by the attention kernels that run on the matrix cores
// (kv_decode_gqa.hip for 2-bit grouped-query attention, kv_decode_gqa_bits.hip
// for other widths, kv_decode_generic.hip for one query head per KV head):
// the operand layouts of the scores and values, row reductions, and the
// conversions of 1- and 4-bit codes to the 2-bit layout.
#pragma once

#include "kv_decode_common.h"

namespace kvq {

typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef float float4v_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef half8_t v8h_t;

constexpr int kMqHeads = 4;          // query heads per wave
constexpr int kMqWaves = 4;          // waves per workgroup
// Score slot k <-> channel of the head: slot 32 kb + 8 u + e holds nibble e
// of unpacked code dword u of group kb (mq_unpack).
__device__ __forceinline__ constexpr int mq_channel(int k) {
  return 32 * (k >> 5) + 16 * ((k >> 4) & 1) + 4 * ((k & 7) >> 1) + 2 * (k & 1) + ((k >> 3) & 1);
}

// One group's 32 codes (two packed dwords) as nibbles 0b00cc: the masked
// copy of a dword keeps channels 4b and 4b+2 of byte b (low and high nibble),
// the shifted copy channels 4b+1 and 4b+3.
__device__ __forceinline__ v8i_t mq_unpack(u32x2_t c) {
  v8i_t b;
  b[0] = (int)(c.x & 0x33333333u);
  b[1] = (int)((c.x >> 2) & 0x33333333u);
  b[2] = (int)(c.y & 0x33333333u);
  b[3] = (int)((c.y >> 2) & 0x33333333u);
  b[4] = 0; b[5] = 0; b[6] = 0; b[7] = 0;
  return b;
}

// The key bytes of one group for one token: 4, 8 or 16 bytes.
template <int KB> struct MbKeyWord;
template <> struct MbKeyWord<1> { typedef uint32_t type; };
template <> struct MbKeyWord<2> { typedef u32x2_t type; };
template <> struct MbKeyWord<4> { typedef u32x4_t type; };

// The fp4 key operand of one group (slot 8 d + j: nibble j of dword d) from
// its packed codes, and the channel each slot holds:
//   - 1 bit: four shifted copies of the group's dword (copy d keeps bits
//     4 j + d in nibble j), so slot 8 d + j holds channel 4 j + d;
//   - 2 bits: mq_unpack (slot order mq_channel);
//   - 4 bits: 2-bit plane p of the nibbles in place (slot = channel); the
//     high plane's product takes the B block scale 2^2.
template <int KB>
__host__ __device__ __forceinline__ constexpr int mq_key_channel(int k) {
  return KB == 4 ? k : KB == 2 ? mq_channel(k) : 32 * (k >> 5) + 4 * (k & 7) + ((k >> 3) & 3);
}
template <int KB>
__device__ __forceinline__ v8i_t mq_key_operand(const typename MbKeyWord<KB>::type &w, int p) {
  v8i_t b;
  if constexpr (KB == 2) {
    b = mq_unpack(w);
  } else {
    if constexpr (KB == 4) {
      b[0] = (int)((w.x >> (2 * p)) & 0x33333333u);
      b[1] = (int)((w.y >> (2 * p)) & 0x33333333u);
      b[2] = (int)((w.z >> (2 * p)) & 0x33333333u);
      b[3] = (int)((w.w >> (2 * p)) & 0x33333333u);
    } else {
      b[0] = (int)(w & 0x11111111u);
      b[1] = (int)((w >> 1) & 0x11111111u);
      b[2] = (int)((w >> 2) & 0x11111111u);
      b[3] = (int)((w >> 3) & 0x11111111u);
    }
    b[4] = 0; b[5] = 0; b[6] = 0; b[7] = 0;
  }
  return b;
}

// Balanced base-32 digit L (0 = most significant) of |q| < 2^19.
__device__ __forceinline__ int mq_digit(int q, int L) {
  int r = q, d = 0;
#pragma unroll
  for (int i = 3; i >= 0; --i) {
    const int di = ((r + 16) & 31) - 16;
    if (i == L) d = di;
    r = (r - di) >> 5;
  }
  return d;
}

// E8M0 block scales of the four digit positions: 2^15, 2^10, 2^5, 1.
__device__ __forceinline__ constexpr int mq_scale(int L) { return 127 + 15 - 5 * L; }

// Sums / maxima over the 16 lanes of a row.
__device__ __forceinline__ float row_sum16(float v) {
  v += row_ror<1>(v);
  v += row_ror<2>(v);
  v += row_ror<4>(v);
  v += row_ror<8>(v);
  return v;
}
__device__ __forceinline__ float row_max16(float v) {
  v = fmaxf(v, row_ror<1>(v));
  v = fmaxf(v, row_ror<2>(v));
  v = fmaxf(v, row_ror<4>(v));
  v = fmaxf(v, row_ror<8>(v));
  return v;
}
__device__ __forceinline__ float lane_read(float v, int l) {
  return bits_as_float((uint32_t)__builtin_amdgcn_readlane((int)float_as_bits(v), l));
}

// Value operand of code byte block BLK: in y (nibble form, positions
// (0, 2) in y02 and (1, 3) in y13), byte BLK is token t0's and byte 2 + BLK
// token t0 + 1's.  Each pair of codes (exact in fp16 after the fp4
// conversion) becomes code * s - nb with (s, nb) the fp16 halves of sv.
template <int BLK>
__device__ __forceinline__ half8_t mq_bvals(uint32_t y02, uint32_t y13, uint32_t sv0, uint32_t sv1) {
  const half2_t c0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(y02, 2.0f, BLK);
  const half2_t c1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(y13, 2.0f, BLK);
  const half2_t c2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(y02, 2.0f, 2 + BLK);
  const half2_t c3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(y13, 2.0f, 2 + BLK);
  const half2_t p0 = __builtin_bit_cast(half2_t, sv0), p1 = __builtin_bit_cast(half2_t, sv1);
  const _Float16 s0 = p0.x, n0 = p0.y, s1 = p1.x, n1 = p1.y;
  const half2_t a = __builtin_elementwise_fma(c0, half2_t{s0, s0}, half2_t{n0, n0});
  const half2_t b = __builtin_elementwise_fma(c1, half2_t{s0, s0}, half2_t{n0, n0});
  const half2_t c = __builtin_elementwise_fma(c2, half2_t{s1, s1}, half2_t{n1, n1});
  const half2_t d = __builtin_elementwise_fma(c3, half2_t{s1, s1}, half2_t{n1, n1});
  return half8_t{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

// The same positions as plain codes (0..3, exact in fp16), for a value step
// whose A operand carries the scale.
template <int BLK>
__device__ __forceinline__ half8_t mq_bcodes(uint32_t y02, uint32_t y13) {
  const half2_t c0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(y02, 2.0f, BLK);
  const half2_t c1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(y13, 2.0f, BLK);
  const half2_t c2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(y02, 2.0f, 2 + BLK);
  const half2_t c3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(y13, 2.0f, 2 + BLK);
  return half8_t{c0.x, c0.y, c1.x, c1.y, c2.x, c2.y, c3.x, c3.y};
}

// Bytes b0, b1 spread to the 2-bit layout: b0 -> bits 0..15, b1 -> bits 16..31.
__device__ __forceinline__ uint32_t mb_spread_pair(uint32_t b0, uint32_t b1) {
  uint32_t x = b0 | (b1 << 16);
  x = (x | (x << 4)) & 0x0F0F0F0Fu;
  x = (x | (x << 2)) & 0x33333333u;
  return (x | (x << 1)) & 0x55555555u;
}
// Plane p of eight 4-bit codes (nibble c = channel c) in the 2-bit layout:
// 16 bits, field c = bits (4c + 2p, 4c + 2p + 1) of w.
__device__ __forceinline__ uint32_t mb_plane16(uint32_t w, int p) {
  uint32_t x = (w >> (2 * p)) & 0x33333333u;
  x = (x | (x >> 2)) & 0x0F0F0F0Fu;
  x = (x | (x >> 4)) & 0x00FF00FFu;
  return (x | (x >> 8)) & 0x0000FFFFu;
}

}  // namespace kvq
