// Declarations shared by the decode kernels of the kvq library.
#pragma once

#include "kvq_device.h"
#include "kvq_launch.h"

namespace kvq {

constexpr float kNegInf = -__builtin_huge_valf();

struct AttnArgs {
  const uint8_t *kcodes; const uint16_t *kscales; const uint16_t *kzeros; int64_t kT_cap;
  const uint8_t *vcodes; const uint16_t *vscales; const uint16_t *vzeros; int64_t vT_cap;
  int64_t t_begin, n_int2;
  int64_t n_splits;
  int64_t total_waves;  // B * Hq * n_splits
  int Hkv, Hq, G;
  const uint32_t *qprep;
  float *partials;
  // In-wave query preparation (one query head per KV head, Hadamard or no
  // rotation): the attention waves transform q themselves and qprep is unused.
  bool fused_prep;
  const void *q; bool q_f32;
  int rot;
  float qscale;
  // Tile grid shift: tiles start `skip` rows before t_begin (0 <= skip < 16).
  int skip;
  // Variable-length batch: sequence b's INT2 range ends at t_ends[b] (device
  // [B]; clamped to [t_begin, t_begin + n_int2]); NULL: every range is n_int2.
  const int32_t *t_ends;
};

// INT2 tokens of sequence b.
__device__ __forceinline__ int64_t seq_int2(const AttnArgs &a, int64_t b) {
  if (a.t_ends == nullptr) return a.n_int2;
  const int64_t e = (int64_t)a.t_ends[b] - a.t_begin;
  return e < 0 ? 0 : (e > a.n_int2 ? a.n_int2 : e);
}

// Reassemble the fp16 subnormal channel factor: code at position x of a
// 16-bit half is read with weight 2^(2x-24) (x <= 4) or 2^(2x-30) (x >= 5).
__device__ __forceinline__ constexpr float chan_unscale(int x) {
  return x <= 4 ? (float)(1u << (24 - 2 * x)) : (float)(1u << (30 - 2 * x));
}

// Lazy rescaling: the running reference m is moved only when a score
// exceeds it by more than kSlack (log2 units), so p = 2^(s - m) stays below
// 2^kSlack and w = p * s_v stays far inside the fp16 range.  The partial
// (m, l, o') is exact for any reference m, so the merge is unchanged.
constexpr float kSlack = 4.0f;

constexpr uint32_t kHalf2Ones = 0x3C003C00u;   // (1.0, 1.0) in fp16

// Sum / max over the two 16-lane rows of each 32-lane half (xor 16) and over
// the two halves (xor 32) with the gfx950 lane-swap instructions.
__device__ __forceinline__ float sum_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(float_as_bits(v), float_as_bits(v), false, false);
  return bits_as_float(r[0]) + bits_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(float_as_bits(v), float_as_bits(v), false, false);
  return bits_as_float(r[0]) + bits_as_float(r[1]);
}
__device__ __forceinline__ float max_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(float_as_bits(v), float_as_bits(v), false, false);
  return fmaxf(bits_as_float(r[0]), bits_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(float_as_bits(v), float_as_bits(v), false, false);
  return fmaxf(bits_as_float(r[0]), bits_as_float(r[1]));
}

__device__ __forceinline__ float lo_half(uint32_t w) { return half_bits_to_float((uint16_t)(w & 0xFFFFu)); }
__device__ __forceinline__ float hi_half(uint32_t w) { return half_bits_to_float((uint16_t)(w >> 16)); }

// A wave's tiles: the head's INT2 tokens are cut into 64-token tiles and
// wave `split` of S takes tiles split, split + S, ...; mine = how many full
// tiles that is.
// The tiles of a head.  The 64-token tile grid starts `skip` rows before
// the INT2 range, chosen on the host so that tile starts sit on 16-row
// boundaries of the cache arrays: then every 512-byte run of a tile's scales
// or zeros is four whole 128-byte lines.  In the shifted row coordinates the
// valid rows are [skip, n_tok).  Tile t is full when none of its rows is
// masked; wave `split` of S owns tiles split, split + S, ...  Its full tiles
// are split + (i0 + i) S for i < mine; the partial tiles (the first one when
// skip > 0, the last one when n_tok is not a multiple of 64) are processed
// with masks by the wave that owns them.
struct HeadTiles {
  int64_t n_tok, n_full_end, i0, mine;
  __device__ __forceinline__ HeadTiles(int64_t n_int2, int skip, int64_t split, int64_t S) {
    n_tok = n_int2 + skip;
    n_full_end = n_tok >> 6;
    i0 = (skip > 0 && split == 0) ? 1 : 0;
    const int64_t t_first = split + i0 * S;
    mine = t_first < n_full_end ? (n_full_end - 1 - t_first) / S + 1 : 0;
  }
  // first row of the wave's i-th full tile (i clamped to the last one)
  __device__ __forceinline__ int64_t full_row(int64_t i, int64_t split, int64_t S) const {
    return 64 * (split + (i0 + (i < mine - 1 ? i : mine - 1)) * S);
  }
  // the partial tiles this wave owns: t0 (first) and t1 (last), or -1
  __device__ __forceinline__ void partial(int skip, int64_t split, int64_t S, int64_t &t0, int64_t &t1) const {
    t0 = (skip > 0 && split == 0) ? 0 : -1;
    t1 = ((n_tok & 63) != 0 && n_full_end % S == split) ? n_full_end : -1;
    if (t1 == t0) t1 = -1;                         // one tile that is both
  }
};

hipError_t launch_attn_gqa(const AttnArgs &a, hipStream_t stream);

}  // namespace kvq
