// Write path: rotate -> 2-bit quantize -> pack, one KV-cache row per
// quad of lanes (gfx950, wave64).
//
// The rotation is applied before quantization ("Output-Aware Rotation for
// INT2 KV-Cache Quantization", woor.ai page, "Key Details").  The Hadamard
// case uses the fast Walsh-Hadamard transform (RotateKV, IJCAI 2025
// record, abstract item (i)) computed in registers: lane j of a quad holds
// channels [32j, 32j+32) of one row, so five butterfly stages run inside a
// lane and the two stages across the 32- and 64-channel strides use DPP
// quad permutes.  A quantization group (32 channels) is exactly one lane's
// values, so min/max need no cross-lane traffic, and the lane packs its 32
// codes into 8 bytes.  Consecutive quads handle consecutive tokens of one
// (batch, head), so a wave's code stores cover 512 contiguous bytes.
//
// Every write kernel quantizes with one device function, quantize_group32:
// the exact IEEE fp32 sequence of the format applied to the rotated row the
// kernel computed (the Hadamard output times fp32(1/sqrt(128)), rounded
// once), so codes, scales and zeros are bit-exact given the same rotated
// row.  The conversion to fp32 rides on the first butterfly (v_fma_mix).
#include "kvq_device.h"
#include "kvq_launch.h"

namespace kvq {

// Adding 1.5 * 2^23 to t in [0, 15] rounds t to an integer with round half
// to even and leaves that integer in the low mantissa bits.
constexpr float kRoundMagic = 12582912.0f;          // 0x4B400000
constexpr uint32_t kRoundMagicBits = 0x4B400000u;

// Sum over i < 16 of (kRoundMagicBits << 2i) mod 2^32: what the shift-add
// packing of 16 magic-biased codes adds on top of the codes themselves.
constexpr uint32_t magic_pack_bias() {
  uint32_t s = 0;
  for (int i = 0; i < 16; ++i) s += kRoundMagicBits << (2 * i);
  return s;
}
constexpr uint32_t kPackBias = magic_pack_bias();

// (x << SH) + acc in one instruction (v_lshl_add_u32, SH an inline constant).
template <int SH>
__device__ __forceinline__ uint32_t shl_add(uint32_t x, uint32_t acc) {
  uint32_t r;
  asm("v_lshl_add_u32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "I"(SH), "v"(acc));
  return r;
}

// Pack 16 magic-biased code words: sum_i f(i) << 2i (mod 2^32).
template <typename F, int I = 0>
__device__ __forceinline__ uint32_t pack16(F &&f, uint32_t acc) {
  if constexpr (I == 16) {
    return acc;
  } else {
    return pack16<F, I + 1>(static_cast<F &&>(f), shl_add<2 * I>(f(I), acc));
  }
}

// Group min/max over 32 values.
__device__ __forceinline__ void minmax32(const float (&v)[32], float &mn, float &mx) {
  mn = v[0];
  mx = v[0];
#pragma unroll
  for (int i = 1; i < 32; ++i) {
    mn = fminf(mn, v[i]);
    mx = fmaxf(mx, v[i]);
  }
}

// Quantize one group of 32 values of a row to b-bit codes (L = 2^b - 1
// levels above the zero) with the exact IEEE fp32 sequence of the format:
//   y     = v * c           (SCALED: v is the unnormalized Hadamard output and
//                            c = fp32(1/sqrt(128)); otherwise y = v)
//   s     = fp32(fp32(max y - min y) / L)    correctly rounded (div_by_levels)
//   scale = fp16(s);  zero = fp16(min y + 0) (a zero minimum gives +0)
//   inv   = fp32(1 / scale)                 correctly rounded (recip_of_half_value)
//   code  = clamp(rint_half_even(fp32(fp32(y - zero) * inv)), 0, L)
// and every code 0 when the scale is 0.  min/max of y are taken as c times
// min/max of v: a positive scaling with one rounding is monotonic, so they
// equal the min/max of the rounded y.  Word k of w holds codes
// 32k/b .. 32(k+1)/b - 1, code i of a word at bits b*i.
//
// Two code forms give the same codes.  When every group of the wave has a
// normal fp16 scale and |zero| <= 8 scale, u = fp32(fp32(y - zero) * inv)
// lies in [-0.004, L + 0.012]: the fp16 roundings of the zero and the scale
// move (y - min)/(range/L) in [0, L] by at most 8 2^-11 and L 2^-11.  Then
// v_cvt_pk_u8_f32 (round half to even, saturating below 0) gives
// clamp(rint(u), 0, L) directly and drops it into byte i/P of word i%P.
// Otherwise u is clamped to [0, L] and rounded by adding 1.5 * 2^23 (clamp
// then round equals round then clamp for integer bounds).
// GH > 1: v is the unnormalized transform over the channels of GH heads
// (grouped-head rotation) and c = fp32(1/sqrt(128 GH)).
template <int BITS, bool SCALED, int GH = 1>
__device__ __forceinline__ void quantize_group32(float (&v)[32], uint32_t (&w)[BITS],
                                                 uint16_t &sbits, uint16_t &zbits) {
#pragma clang fp contract(off)
  constexpr int L = (1 << BITS) - 1;
  constexpr int CPW = 32 / BITS;                    // codes per word
  constexpr int P = 8 / BITS;                       // codes per byte
  static_assert(GH == 1 || GH == 2 || GH == 4, "grouped heads");
  // fp32(1/sqrt(128 GH)): 0x3DB504F3, 0x3D800000, 0x3D3504F3
  constexpr float c = GH == 1 ? 0.08838834764831845f : GH == 2 ? 0.0625f : 0.04419417382415922f;
  float mn, mx;
  minmax32(v, mn, mx);
  if constexpr (SCALED) {
    mn = mn * c;
    mx = mx * c;
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = v[i] * c;
  }
  const float range = mx - mn;
  const float s32 = div_by_levels<L>(range);          // RN(range / L)
  sbits = fp32_value_to_half_bits(s32);
  zbits = float_to_half_bits(mn + 0.0f);
  const float sf = half_bits_to_float(sbits);
  const float zf = half_bits_to_float(zbits);
  const bool degenerate = (sf == 0.0f);
  const float inv = recip_of_half_value(degenerate ? 1.0f : sf);   // RN(1 / scale)
  uint32_t r[BITS];
  if (!__builtin_amdgcn_ballot_w64(fabsf(zf) > 8.0f * sf || sf < kMinNormalHalf)) {
#pragma unroll
    for (int k = 0; k < BITS; ++k) {
      uint32_t D[P];
#pragma unroll
      for (int m = 0; m < P; ++m) D[m] = 0u;
#pragma unroll
      for (int i = 0; i < CPW; ++i) {
        const float u = (v[k * CPW + i] - zf) * inv;
        D[i % P] = __builtin_amdgcn_cvt_pk_u8_f32(u, (uint32_t)(i / P), D[i % P]);
      }
      uint32_t word = D[0];
#pragma unroll
      for (int m = 1; m < P; ++m) word |= D[m] << (BITS * m);
      r[k] = word;
    }
  } else {
    uint32_t cb[32];                                  // 0x4B400000 | code
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const float u = (v[i] - zf) * inv;
      const float t = __builtin_amdgcn_fmed3f(u, 0.0f, (float)L);
      cb[i] = float_as_bits(t + kRoundMagic);
    }
    if constexpr (BITS == 2) {
      r[0] = pack16([&](int i) { return cb[i]; }, 0u) - kPackBias;
      r[1] = pack16([&](int i) { return cb[16 + i]; }, 0u) - kPackBias;
    } else {
#pragma unroll
      for (int k = 0; k < BITS; ++k) {
        uint32_t word = 0u;
#pragma unroll
        for (int i = 0; i < CPW; ++i) word |= (cb[k * CPW + i] - kRoundMagicBits) << (BITS * i);
        r[k] = word;
      }
    }
  }
#pragma unroll
  for (int k = 0; k < BITS; ++k) w[k] = degenerate ? 0u : r[k];
}

// lo + hi and lo - hi of the two fp16 halves of a dword, in fp32 with one
// rounding (v_fma_mix_f32 reads fp16 operands directly).
__device__ __forceinline__ float mix_sum(uint32_t w) {
  float r;
  asm("v_fma_mix_f32 %0, %1, 1.0, %1 op_sel:[0,0,1] op_sel_hi:[1,0,1]" : "=v"(r) : "v"(w));
  return r;
}
__device__ __forceinline__ float mix_diff(uint32_t w) {
  float r;
  asm("v_fma_mix_f32 %0, %1, -1.0, %1 op_sel:[1,0,0] op_sel_hi:[1,0,1]" : "=v"(r) : "v"(w));
  return r;
}

// Unnormalized FWHT stages 2..7 of a 128-vector spread over a quad, after
// stage 1 (stride 1) was applied while loading.
__device__ __forceinline__ void fwht128_quad_rest(float (&v)[32], int j) {
#pragma unroll
  for (int hs = 2; hs < 32; hs <<= 1) {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if ((i & hs) == 0) {
        const float a = v[i], b = v[i + hs];
        v[i] = a + b;
        v[i + hs] = a - b;
      }
    }
  }
  const float n1 = (j & 1) ? -1.0f : 1.0f;
  const float n2 = (j & 2) ? -1.0f : 1.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] = quad_butterfly<kQuadXor1>(v[i], n1);
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] = quad_butterfly<kQuadXor2>(v[i], n2);
}

// Load a lane's 32 channels.  ROT: apply FWHT stage 1 on the way in.
template <typename TIn, bool ROT>
__device__ __forceinline__ void load_row32(const TIn *src, float (&v)[32]);

template <>
__device__ __forceinline__ void load_row32<_Float16, true>(const _Float16 *src, float (&v)[32]) {
  const u32x4_t *p = reinterpret_cast<const u32x4_t *>(src);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const u32x4_t u = __builtin_nontemporal_load(p + k);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[8 * k + 2 * e] = mix_sum(w[e]);
      v[8 * k + 2 * e + 1] = mix_diff(w[e]);
    }
  }
}

template <>
__device__ __forceinline__ void load_row32<_Float16, false>(const _Float16 *src, float (&v)[32]) {
  const u32x4_t *p = reinterpret_cast<const u32x4_t *>(src);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const u32x4_t u = __builtin_nontemporal_load(p + k);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[8 * k + 2 * e] = half_bits_to_float((uint16_t)(w[e] & 0xFFFFu));
      v[8 * k + 2 * e + 1] = half_bits_to_float((uint16_t)(w[e] >> 16));
    }
  }
}

template <bool ROT>
__device__ __forceinline__ void load_row32_f32(const float *src, float (&v)[32]) {
  const float4_t *p = reinterpret_cast<const float4_t *>(src);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float4_t u = __builtin_nontemporal_load(p + k);
    if (ROT) {
      v[4 * k] = u.x + u.y;
      v[4 * k + 1] = u.x - u.y;
      v[4 * k + 2] = u.z + u.w;
      v[4 * k + 3] = u.z - u.w;
    } else {
      v[4 * k] = u.x; v[4 * k + 1] = u.y; v[4 * k + 2] = u.z; v[4 * k + 3] = u.w;
    }
  }
}
template <>
__device__ __forceinline__ void load_row32<float, true>(const float *src, float (&v)[32]) {
  load_row32_f32<true>(src, v);
}
template <>
__device__ __forceinline__ void load_row32<float, false>(const float *src, float (&v)[32]) {
  load_row32_f32<false>(src, v);
}

struct RowsKernelArgs {
  QuantSide side[2];
  int64_t stride_b, stride_t, stride_h;
  int64_t T_new, t_offset;
  int Hkv;
  int n_sides;
  const int32_t *perm;   // permuted Hadamard: [Hkv][128] channel order, else unused
  const int32_t *offsets;   // per-sequence first slot (device [B]) or NULL: t_offset
  // paged cache: slot t of sequence b is row t % page_tokens of page
  // block_table[b * max_pages + t / page_tokens]; NULL: row (b*Hkv + h)*T_cap + t
  const int32_t *block_table;
  int64_t max_pages, n_pages, page_tokens;
};

// grid: x = token blocks of 64, y = KV head, z = batch * n_sides + side
template <typename TIn, bool ROT>
__global__ __launch_bounds__(256) void kv_rotate_quant_rows(RowsKernelArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane >> 2;
  const int j = lane & 3;
  const int h = blockIdx.y;
  const int sidx = (int)(blockIdx.z % (unsigned)a.n_sides);
  const int64_t b = blockIdx.z / (unsigned)a.n_sides;
  const QuantSide s = sidx ? a.side[1] : a.side[0];
  const int64_t t = (int64_t)blockIdx.x * 64 + wave * 16 + r;
  const bool valid = t < a.T_new;
  const int64_t tl = valid ? t : 0;
  const TIn *src = reinterpret_cast<const TIn *>(s.x) + b * a.stride_b + tl * a.stride_t +
                   (int64_t)h * a.stride_h + 32 * j;
  float v[32];
  load_row32<TIn, ROT>(src, v);
  uint32_t w2[2];
  uint16_t sb, zb;
  if constexpr (ROT) {
    fwht128_quad_rest(v, j);
    quantize_group32<2, true>(v, w2, sb, zb);
  } else {
    quantize_group32<2, false>(v, w2, sb, zb);
  }
  const uint32_t w0 = w2[0], w1 = w2[1];
  const int64_t slot = seq_offset(a.offsets, a.t_offset, b) + t;
  if (valid && slot >= 0 && slot < s.T_cap) {       // a per-sequence slot outside the cache is skipped
    const int64_t row = write_row(a.block_table, a.max_pages, a.n_pages, a.page_tokens, a.Hkv, b, h, s.T_cap, slot);
    if (row >= 0) {                                  // a page outside the pool is skipped
      *reinterpret_cast<uint2 *>(s.codes + row * kCodeBytes + 8 * j) = make_uint2(w0, w1);
      s.scales[row * kNGroups + j] = sb;
      s.zeros[row * kNGroups + j] = zb;
    }
  }
}

// ---------------------------------------------------------------------------
// fp16 input + Hadamard.  A wave handles 64 consecutive tokens of one
// (batch, head, side).  Rows are first brought into LDS with fully coalesced
// 16-byte loads (16 lanes per 256-byte row); rows are padded by 16 bytes so
// that 16 lanes reading 16 bytes each from 16 different rows hit distinct
// banks.  The transform then takes part of the butterfly onto the matrix
// cores (below), each quantization group is quantized by the lane that
// holds it, and the codes go back through LDS to whole-row stores.
//
// Block order puts the head index fastest, so the waves resident at one
// time read whole token records (all heads of a token are adjacent in the
// input) rather than one head's 256-byte slice of many records.  Code rows
// go back through LDS so that each store instruction writes 1 KiB of
// consecutive cache rows, with non-temporal hints: in a stream that mixes
// reads and writes this measured faster than row-per-lane stores.
// ---------------------------------------------------------------------------
constexpr int kStageRowDwords = 64 + 4;     // 128 fp16 + 16-byte pad

// grid: x = token block * Hkv + KV head, z = batch * n_sides + side;
// block = one wave.  PERM: the rows are reordered to the head's channel
// order pi (x_pi[j] = x[pi[j]], RotateKV's channel reordering ahead of the
// transform) while they are staged: channel c goes to position pinv[c] of
// its LDS row (one 2-byte store each, the row offset in the store's
// immediate), and the rows are read back as in the plain kernel.  Indices
// are taken modulo 128, so any order array stays inside the rows.
// HG = 4: a wave takes 16 consecutive tokens of 4 consecutive heads (64 rows),
// so each staging load reads the 4 heads' rows of one token, 1 KiB of
// contiguous input when heads are adjacent, and each store writes runs of
// 16 rows per head.  HG = 1: 64 consecutive tokens of one head.
// GH > 1 (HG = 4, no reordering): the pre-RoPE grouped-head rotation of
// keys (RotateKV, IJCAI 2025 record, abstract item (ii)): the rows of GH
// consecutive heads of a token are one row of 128 GH channels, head j of
// the group at channels 128 j .. 128 j + 127, rotated by the normalized
// Hadamard matrix of that size.  With the head index as the high bits that
// matrix is H_GH x H_128, so each head's row is transformed as before, then
// butterflies across the GH heads (all four heads of a token sit in one
// lane) complete it, and the normalization is 1/sqrt(128 GH).
template <bool PERM, int BITS, int HG, int GH = 1>
__device__ __forceinline__ void fwht_f16_body(const RowsKernelArgs &a) {
  static_assert(GH == 1 || (HG == 4 && !PERM && (GH == 2 || GH == 4)), "grouped heads need 4 heads per wave");
  constexpr int TPW = 64 / HG;                       // tokens per wave
  __shared__ uint32_t stage[64 * kStageRowDwords];
  const int lane = threadIdx.x;
  const int hgroups = a.Hkv / HG;
  const int h0 = (int)(blockIdx.x % (unsigned)hgroups) * HG;
  const int sidx = (int)(blockIdx.z % (unsigned)a.n_sides);
  const int64_t b = blockIdx.z / (unsigned)a.n_sides;
  const QuantSide s = sidx ? a.side[1] : a.side[0];
  // HG = 4: the 16-token tiles are laid on 16-slot boundaries of the cache
  // (the first tile starts `shift` tokens early, those tokens masked), so
  // each 16-row run of scales or zeros is one whole 128-byte line when T_cap
  // is a multiple of 16; a per-sequence slot gives a per-sequence shift.
  const int64_t slot_base = seq_offset(a.offsets, a.t_offset, b);
  const int64_t shift = HG == 1 ? 0 : ((slot_base % 16) + 16) % 16;
  const int64_t t0 = (int64_t)(blockIdx.x / (unsigned)hgroups) * TPW - shift;
  if (t0 >= a.T_new) return;                         // the extra tile of a shift of 0: no token
  const _Float16 *base = reinterpret_cast<const _Float16 *>(s.x) + b * a.stride_b +
                         (int64_t)h0 * a.stride_h;

  // Coalesced staging: instruction i covers stage rows 4i..4i+3, 16 lanes
  // per row.  Stage row r holds token t0 + r / HG of head h0 + r % HG (HG = 4:
  // instruction i reads token i of the 4 heads; HG = 1: tokens 4i..4i+3).
  const int chunk = lane & 15;
  const int r0 = lane >> 4;
  const int hr = HG == 1 ? 0 : r0;                   // head of this lane's staged rows
  auto tok_of_load = [&](int i) { return HG == 1 ? 4 * i + r0 : i; };
  // PERM: channel c is staged at position pinv[c] of its row (pinv = the
  // inverse of the head's order, built in LDS), so the rows are read back
  // already reordered.  pos[e]: byte offset of channel 8 chunk + e in row r0.
  uint32_t pos[8];
  if constexpr (PERM) {
    __shared__ uint8_t pinv_all[HG][kD];
    for (int g = 0; g < HG; ++g) {
      const int32_t *pi = a.perm + (int64_t)(h0 + g) * kD;
      pinv_all[g][pi[2 * lane] & (kD - 1)] = (uint8_t)(2 * lane);
      pinv_all[g][pi[2 * lane + 1] & (kD - 1)] = (uint8_t)(2 * lane + 1);
    }
    __syncthreads();
    const uint8_t *pinv = pinv_all[hr];
#pragma unroll
    for (int e = 0; e < 8; ++e)
      pos[e] = (uint32_t)(r0 * kStageRowDwords * 4 + 2 * (pinv[8 * chunk + e] & (kD - 1)));
  }
  auto stage_row = [&](int i, const u32x4_t &u) {
    if constexpr (PERM) {
      uint8_t *rb = reinterpret_cast<uint8_t *>(stage) + 4 * i * kStageRowDwords * 4;
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int e = 0; e < 8; ++e)
        *reinterpret_cast<uint16_t *>(rb + pos[e]) = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
    } else {
      *reinterpret_cast<u32x4_t *>(&stage[(4 * i + r0) * kStageRowDwords + 4 * chunk]) = u;
    }
  };
  // all 16 loads of the tile first, then the LDS writes
  u32x4_t ld[16];
  {
    const _Float16 *hb = base + (int64_t)hr * a.stride_h;
    if (t0 >= 0 && t0 + TPW <= a.T_new) {
      const u32x4_t *src = reinterpret_cast<const u32x4_t *>(hb + (t0 + tok_of_load(0)) * a.stride_t) + chunk;
      const int64_t step = (HG == 1 ? 4 : 1) * a.stride_t / 8;   // in 16-byte units
#pragma unroll
      for (int i = 0; i < 16; ++i) ld[i] = __builtin_nontemporal_load(src + i * step);
    } else {                                        // tokens past T_new re-read the first
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int64_t t = t0 + tok_of_load(i);
        const int64_t tl = (t >= 0 && t < a.T_new) ? t : (t0 > 0 ? t0 : 0);   // t0 < T_new here
        ld[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(hb + tl * a.stride_t) + chunk);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) stage_row(i, ld[i]);
  __syncthreads();

  // Transform.  H128 = H16 (channel bits 3..6) x H8 (bits 0..2), and the
  // factors commute.  The H16 part runs on the matrix cores straight from the
  // fp16 rows: for each low index c0 = 0..7, D = H16 * X_c0 with
  // X_c0[k][n] = x[token n][c0 + 8k] (16 tokens per product, fp32
  // accumulation of exact +-x products).  v_mfma_f32_16x16x16_f16 leaves
  // D[4q + r][n] in lane 16q + n, so after the eight products lane (n, q)
  // holds channels c0 + 8(4q + r) of token n: exactly quantization group q.
  // The H8 part (three butterfly stages over c0) then runs in registers, and
  // the group is quantized and stored by the lane that holds it.
  const int n = lane & 15;                 // token within a group of 16
  const int q = lane >> 4;                 // quantization group
  // A operand: H16[m = lane%16][k = 4(lane/16) + i] = (-1)^popcount(m & k)
  half4_t hA;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    hA[i] = (__builtin_popcount((unsigned)(n & (4 * q + i))) & 1) ? (_Float16)-1.0f : (_Float16)1.0f;
  const int64_t slot0 = slot_base + t0;
  const int64_t n_valid = a.T_new - t0;              // >= 1; tokens past it are not ours
  // tokens [lo, hi) of the tile are written: at or after token 0 and slot 0
  const int64_t lo = (slot0 < 0 ? -slot0 : 0) > -t0 ? (slot0 < 0 ? -slot0 : 0) : -t0;
  const int64_t hi = s.T_cap - slot0 < n_valid ? s.T_cap - slot0 : n_valid;
  // Paged cache, HG = 4: the tile's 16 slots start on a 16-slot boundary and
  // pages hold a multiple of 64 tokens, so one page (looked up once, wave-
  // uniform) holds every written row of the tile.
  int64_t tile_page = -1;
  if (HG == 4 && a.block_table != nullptr) {
    const int64_t first = slot0 + lo;                // the tile's first written slot
    if (lo < hi) tile_page = a.block_table[b * a.max_pages + (uint32_t)first / (uint32_t)a.page_tokens];
  }
  // cache row of token tk in [lo, hi) of the tile, head h0 + g; -1 when a
  // paged slot's page index is outside the cache (the row is not written).
  // A paged slot is below max_pages * page_tokens < 2^31.
  auto row_of = [&](int g, int64_t tk) -> int64_t {
    const int64_t slot = slot0 + tk;
    if (a.block_table == nullptr) return (b * a.Hkv + h0 + g) * s.T_cap + slot;
    const uint32_t sl = (uint32_t)slot, P = (uint32_t)a.page_tokens, pi = sl / P;
    const int64_t page = HG == 4 ? tile_page : a.block_table[b * a.max_pages + pi];
    if (page < 0 || page >= a.n_pages) return -1;
    return (page * a.Hkv + h0 + g) * a.page_tokens + (sl - pi * P);
  };

  // lane (n, q): stage row r(g) = 16g + n for HG = 1, 4n + g for HG = 4
  auto srow = [&](int g) { return HG == 1 ? 16 * g + n : 4 * n + g; };
  uint32_t cw[4][BITS], csz[4];                      // codes and scale | zero << 16 of stage row srow(g)
  // the transform of stage row srow(g) into z: channel c0 + 8(4q + r') in z[c0 + 8r']
  auto transform = [&](int g, float (&z)[32]) {
    const int r = srow(g);                           // the lane's stage row
    // channels 8(4q + i) .. 8(4q + i) + 7 of row r, i = 0..3
    u32x4_t u[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      u[i] = *reinterpret_cast<const u32x4_t *>(&stage[r * kStageRowDwords + 4 * (4 * q + i)]);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t w0 = u[0][e], w1 = u[1][e], w2 = u[2][e], w3 = u[3][e];
      // B operands for c0 = 2e (low halves) and 2e + 1 (high halves)
      const uint32_t lo01 = __builtin_amdgcn_perm(w1, w0, 0x05040100u), lo23 = __builtin_amdgcn_perm(w3, w2, 0x05040100u);
      const uint32_t hi01 = __builtin_amdgcn_perm(w1, w0, 0x07060302u), hi23 = __builtin_amdgcn_perm(w3, w2, 0x07060302u);
      const half4_t bl = __builtin_bit_cast(half4_t, u32x2_t{lo01, lo23});
      const half4_t bh = __builtin_bit_cast(half4_t, u32x2_t{hi01, hi23});
      const float4_t dl = __builtin_amdgcn_mfma_f32_16x16x16f16(hA, bl, float4_t{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
      const float4_t dh = __builtin_amdgcn_mfma_f32_16x16x16f16(hA, bh, float4_t{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        z[2 * e + 8 * rr] = dl[rr];
        z[2 * e + 1 + 8 * rr] = dh[rr];
      }
    }
    // H8 over c0 for each r': three butterfly stages in registers
#pragma unroll
    for (int hs = 1; hs < 8; hs <<= 1) {
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        if ((i & hs) == 0) {
          const float x = z[i], y = z[i + hs];
          z[i] = x + y;
          z[i + hs] = x - y;
        }
      }
    }
  };
  if constexpr (GH == 1) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      float z[32];
      transform(g, z);
      uint16_t sb, zb;
      quantize_group32<BITS, true>(z, cw[g], sb, zb);
      csz[g] = (uint32_t)sb | ((uint32_t)zb << 16);
    }
  } else {
    // the four heads of the lane's token, then the butterflies across each
    // group of GH heads (head bits of the grouped transform)
    float z[4][32];
#pragma unroll
    for (int g = 0; g < 4; ++g) transform(g, z[g]);
#pragma unroll
    for (int hs = 1; hs < GH; hs <<= 1) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        if ((g & hs) == 0) {
#pragma unroll
          for (int i = 0; i < 32; ++i) {
            const float x = z[g][i], y = z[g + hs][i];
            z[g][i] = x + y;
            z[g + hs][i] = x - y;
          }
        }
      }
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      uint16_t sb, zb;
      quantize_group32<BITS, true, GH>(z[g], cw[g], sb, zb);
      csz[g] = (uint32_t)sb | ((uint32_t)zb << 16);
    }
  }
  // Back through LDS to one row per lane (codes: the row's 16 b bytes,
  // 16-byte chunk k of row r at entry b r + k; then scale | zero << 16 of
  // each group), so each code store writes 1 KiB of consecutive cache rows
  // and each lane writes its row's scales and zeros as 8 bytes; storing the
  // code pieces and 2-byte scales straight from the transform layout
  // measured slower.
  constexpr int kRowDwords = 4 * BITS;               // code dwords per row
  constexpr int kSzOff = 64 * kRowDwords;            // scale | zero entries
  const int64_t row_bytes = 16 * BITS;
  __syncthreads();                                   // the stage is read
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int r = srow(g);
#pragma unroll
    for (int k = 0; k < BITS; ++k) stage[r * kRowDwords + BITS * q + k] = cw[g][k];
    stage[kSzOff + r * 4 + q] = csz[g];
  }
  __syncthreads();
  {
    // stage row r = token r / HG of head h0 + r % HG (HG = 1: token r)
    const u32x4_t *rows = reinterpret_cast<const u32x4_t *>(stage);
#pragma unroll
    for (int kk = 0; kk < BITS; ++kk) {
      const int c = 64 * kk + lane;                  // 16-byte chunk c % BITS of stage row c / BITS
      const int r = c / BITS, tk = r / HG;
      if (tk >= lo && tk < hi) {
        const int64_t row = row_of(r % HG, tk);
        if (row >= 0)
          __builtin_nontemporal_store(rows[c], reinterpret_cast<u32x4_t *>(s.codes + row * row_bytes) + c % BITS);
      }
    }
    const int tk = lane / HG;
    const int64_t row = (tk >= lo && tk < hi) ? row_of(lane % HG, tk) : -1;
    if (row >= 0) {
      const u32x4_t e = *reinterpret_cast<const u32x4_t *>(&stage[kSzOff + lane * 4]);
      const u32x2_t sv = {__builtin_amdgcn_perm(e.y, e.x, 0x05040100u), __builtin_amdgcn_perm(e.w, e.z, 0x05040100u)};
      const u32x2_t zv = {__builtin_amdgcn_perm(e.y, e.x, 0x07060302u), __builtin_amdgcn_perm(e.w, e.z, 0x07060302u)};
      __builtin_nontemporal_store(sv, reinterpret_cast<u32x2_t *>(s.scales + row * kNGroups));
      __builtin_nontemporal_store(zv, reinterpret_cast<u32x2_t *>(s.zeros + row * kNGroups));
    }
  }
}

template <int HG>
__global__ __launch_bounds__(64) void kv_rotate_quant_fwht_f16(RowsKernelArgs a) {
  fwht_f16_body<false, 2, HG>(a);
}
template <int HG>
__global__ __launch_bounds__(64) void kv_rotate_quant_fwht_perm_f16(RowsKernelArgs a) {
  fwht_f16_body<true, 2, HG>(a);
}
// 1- and 4-bit codes (keys and values may be kept at different widths)
template <int HG>
__global__ __launch_bounds__(64) void kv_rotate_quant_fwht_b1_f16(RowsKernelArgs a) {
  fwht_f16_body<false, 1, HG>(a);
}
template <int HG>
__global__ __launch_bounds__(64) void kv_rotate_quant_fwht_b4_f16(RowsKernelArgs a) {
  fwht_f16_body<false, 4, HG>(a);
}
template <int HG>
__global__ __launch_bounds__(64) void kv_rotate_quant_fwht_perm_b1_f16(RowsKernelArgs a) {
  fwht_f16_body<true, 1, HG>(a);
}
template <int HG>
__global__ __launch_bounds__(64) void kv_rotate_quant_fwht_perm_b4_f16(RowsKernelArgs a) {
  fwht_f16_body<true, 4, HG>(a);
}

// Pre-RoPE keys with the grouped-head rotation over GH heads (2-bit codes).
template <int GH>
__global__ __launch_bounds__(64, 2) void kv_rotate_quant_fwht_grouped_f16(RowsKernelArgs a) {
  fwht_f16_body<false, 2, 4, GH>(a);
}

hipError_t launch_quantize_grouped(const QuantArgs &q, int group_heads, hipStream_t stream) {
  // one side (the keys), fp16 rows, Hkv a multiple of 4 (checked by the caller)
  RowsKernelArgs a;
  a.side[0] = q.side[0];
  a.side[1] = q.side[0];
  a.stride_b = q.stride_b;
  a.stride_t = q.stride_t;
  a.stride_h = q.stride_h;
  a.T_new = q.T_new;
  a.t_offset = q.t_offset;
  a.offsets = q.offsets;
  a.Hkv = (int)q.Hkv;
  a.n_sides = 1;
  a.perm = nullptr;
  a.block_table = nullptr;
  a.max_pages = a.n_pages = a.page_tokens = 0;
  const int64_t tiles = (q.T_new + 15) / 16 + 1;
  const dim3 grid((unsigned)(tiles * (q.Hkv / 4)), 1, (unsigned)q.B), block(64);
  if (group_heads == 2) hipLaunchKernelGGL(kv_rotate_quant_fwht_grouped_f16<2>, grid, block, 0, stream, a);
  else if (group_heads == 4) hipLaunchKernelGGL(kv_rotate_quant_fwht_grouped_f16<4>, grid, block, 0, stream, a);
  else return hipErrorNotSupported;
  return hipGetLastError();
}

// The fp16 Hadamard write kernels: a wave takes 16 tokens of 4 heads when
// the head count allows, else 64 tokens of one head.
template <int HG>
static hipError_t launch_fwht_hg(const RowsKernelArgs &a, int64_t T_new, int64_t Hkv, int64_t zdim,
                                 bool perm, int bits, hipStream_t stream) {
  // HG = 4: one more tile for the shift onto 16-slot boundaries
  const int64_t tiles = HG == 1 ? (T_new + 63) / 64 : (T_new + 15) / 16 + 1;
  const dim3 grid((unsigned)(tiles * (Hkv / HG)), 1, (unsigned)zdim), block(64);
  if (bits == 1) {
    if (perm) hipLaunchKernelGGL(kv_rotate_quant_fwht_perm_b1_f16<HG>, grid, block, 0, stream, a);
    else hipLaunchKernelGGL(kv_rotate_quant_fwht_b1_f16<HG>, grid, block, 0, stream, a);
  } else if (bits == 4) {
    if (perm) hipLaunchKernelGGL(kv_rotate_quant_fwht_perm_b4_f16<HG>, grid, block, 0, stream, a);
    else hipLaunchKernelGGL(kv_rotate_quant_fwht_b4_f16<HG>, grid, block, 0, stream, a);
  } else {
    if (perm) hipLaunchKernelGGL(kv_rotate_quant_fwht_perm_f16<HG>, grid, block, 0, stream, a);
    else hipLaunchKernelGGL(kv_rotate_quant_fwht_f16<HG>, grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

static hipError_t launch_fwht_f16(const RowsKernelArgs &a, int64_t T_new, int64_t Hkv, int64_t zdim,
                                  bool perm, int bits, hipStream_t stream) {
  if (Hkv % 4 == 0) return launch_fwht_hg<4>(a, T_new, Hkv, zdim, perm, bits, stream);
  return launch_fwht_hg<1>(a, T_new, Hkv, zdim, perm, bits, stream);
}

hipError_t launch_quantize_rows(const QuantArgs &q, hipStream_t stream) {
  RowsKernelArgs a;
  a.side[0] = q.side[0];
  a.side[1] = q.n_sides > 1 ? q.side[1] : q.side[0];
  a.stride_b = q.stride_b;
  a.stride_t = q.stride_t;
  a.stride_h = q.stride_h;
  a.T_new = q.T_new;
  a.t_offset = q.t_offset;
  a.offsets = q.offsets;
  a.Hkv = (int)q.Hkv;
  a.n_sides = q.n_sides;
  a.perm = q.perm;
  a.block_table = q.block_table;
  a.max_pages = q.max_pages;
  a.n_pages = q.n_pages;
  a.page_tokens = q.page_tokens;
  const int64_t n_tb = (q.T_new + 63) / 64;
  const int kbits = q.side[0].bits, vbits = q.n_sides > 1 ? q.side[1].bits : kbits;
  if (kbits != 2 || vbits != 2) {
    // 1- and 4-bit codes: fp16 rows with the (reordered) Hadamard rotation;
    // one launch per side when the two widths differ
    if (q.in_f32 || !(q.rot == 1 || q.rot == 3)) return hipErrorNotSupported;   // rejected by the caller
    const bool perm = q.rot == 3;
    for (int sd = 0; sd < q.n_sides; ++sd) {
      if (sd == 1 && kbits == vbits) break;          // both sides in the first launch
      RowsKernelArgs a1 = a;
      int n_sides = q.n_sides;
      if (kbits != vbits) {
        a1.side[0] = q.side[sd];
        a1.side[1] = q.side[sd];
        a1.n_sides = 1;
        n_sides = 1;
      }
      const int bits = q.side[sd].bits;
      const hipError_t e = launch_fwht_f16(a1, q.T_new, q.Hkv, q.B * n_sides, perm, bits, stream);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  dim3 grid((unsigned)n_tb, (unsigned)q.Hkv, (unsigned)(q.B * q.n_sides));
  const bool rot = (q.rot == 1);
  if ((rot || q.rot == 3) && !q.in_f32)
    return launch_fwht_f16(a, q.T_new, q.Hkv, q.B * q.n_sides, q.rot == 3, 2, stream);
  if (q.rot == 3) return hipErrorNotSupported;     // fp32 input: the caller has rejected it
  dim3 block(256);
  if (q.in_f32) {
    if (rot) hipLaunchKernelGGL((kv_rotate_quant_rows<float, true>), grid, block, 0, stream, a);
    else     hipLaunchKernelGGL((kv_rotate_quant_rows<float, false>), grid, block, 0, stream, a);
  } else {
    if (rot) hipLaunchKernelGGL((kv_rotate_quant_rows<_Float16, true>), grid, block, 0, stream, a);
    else     hipLaunchKernelGGL((kv_rotate_quant_rows<_Float16, false>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace kvq
