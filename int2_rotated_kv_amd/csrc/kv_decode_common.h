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
  int64_t n_splits;     // splits per head planned for the longest sequence
  int64_t total_waves;  // grid size in waves
  int64_t B;
  int Hkv, Hq, G;
  const uint32_t *qprep;
  float *partials;
  // In-wave query preparation (one query head per KV head, Hadamard or no
  // rotation): the attention waves transform q themselves and qprep is unused.
  bool fused_prep;
  const void *q; bool q_f32;
  int rot;
  const int32_t *perm;  // reordered Hadamard: [Hkv][128] (read by the b-bit kernel)
  float qscale;
  // Tile grid shift: tiles start `skip` rows before t_begin (0 <= skip < 16).
  int skip;
  // Variable-length batch: sequence b's INT2 range ends at t_ends[b] (device
  // [B]; clamped to [t_begin, t_begin + n_int2]); NULL: every range is n_int2.
  const int32_t *t_ends;
  // Paged cache: token t of sequence b is row t % page_tokens of page
  // block_table[b * max_pages + t / page_tokens] ([n_pages][Hkv][page_tokens]
  // rows per side); NULL: rows (b*Hkv + h)*T_cap + t.
  const int32_t *block_table;
  int64_t max_pages, n_pages, page_tokens;
  // Precomputed key scores (keys cached with the pre-RoPE grouped-head
  // rotation): [B][Hq][score_rows] in log2 units, row r = shifted-grid row r
  // (token t_begin - skip + r); NULL: scores from the key cache.
  const float *scores;
  int64_t score_rows;
};

// The score launch for keys with the pre-RoPE grouped-head rotation
// (kv_decode_prerope.hip).
struct PreropeArgs {
  const uint8_t *kcodes; const uint16_t *kscales; const uint16_t *kzeros; int64_t kT_cap;
  int64_t t_begin, n_int2;   // INT2 tokens [t_begin, t_begin + n_int2), position = cache slot
  int skip;                  // score row of token t: t - t_begin + skip
  int64_t n_rows;            // score rows per (b, query head)
  int64_t B;
  int Hq, Hkv, G, GH;        // GH: heads per rotation group
  const void *q; bool q_f32;
  float qscale;              // softmax_scale * log2(e) / sqrt(128 GH)
  double log2_base;          // log2 of the RoPE base
  uint32_t *rope_table;      // written by the table kernel, read by the score kernel
  float *scores;
  int64_t tiles, tiles_per_wave, chunks;   // steps of 16 tokens; per wave (<= 128); waves per (b, head group)
};
hipError_t launch_prerope_scores(const PreropeArgs &a, hipStream_t stream);

// First K and V cache rows of the tile that starts at row r0 of a head's
// shifted grid (row 0 = token t_begin - skip).  A paged cache's tiles start on
// 64-token boundaries and pages hold a multiple of 64 tokens, so a tile never
// crosses a page; an out-of-range page index reads page 0 (an unspecified
// result, never an access outside the cache).
struct TileRows {
  int64_t k, v;
};
__device__ __forceinline__ TileRows tile_rows(const AttnArgs &a, int64_t b, int hkv, int64_t krow0,
                                              int64_t vrow0, int64_t r0) {
  if (a.block_table == nullptr) return TileRows{krow0 + r0, vrow0 + r0};
  // a sequence holds fewer than 2^31 tokens (max_pages * page_tokens)
  const uint32_t t = (uint32_t)(a.t_begin - a.skip + r0), P = (uint32_t)a.page_tokens;
  const uint32_t pi = t / P;
  int64_t page = a.block_table[b * a.max_pages + pi];
  page = (page >= 0 && page < a.n_pages) ? page : 0;
  const int64_t row = (page * a.Hkv + hkv) * a.page_tokens + (t - pi * P);
  return TileRows{row, row};
}

// INT2 tokens of sequence b.
__device__ __forceinline__ int64_t seq_int2(const AttnArgs &a, int64_t b) {
  if (a.t_ends == nullptr) return a.n_int2;
  const int64_t e = (int64_t)a.t_ends[b] - a.t_begin;
  return e < 0 ? 0 : (e > a.n_int2 ? a.n_int2 : e);
}

// ---------------------------------------------------------------------------
// Splits of a variable-length batch.
//
// With one length for the whole batch every head of every sequence gets S
// waves (splits), planned on the host so that one round of resident waves
// covers the call.  With per-sequence lengths that plan would leave the waves
// of short sequences idle once they finish, so the B*S split rows of a head
// index are instead shared among the sequences by tile count: with w tiles
// per wave, sequence b gets count_b = ceil(tiles_b / w) rows, and w is the
// least value (at least 4 tiles, i.e. 256 tokens, and at most kMaxSplits rows
// per sequence) whose counts fit in B*S rows.  That minimises the longest
// wave.  Sequence b's rows are first_b .. first_b + count_b - 1, first_b the
// sum of the earlier counts.  With every sequence as long as the longest,
// count_b is S or a smaller count whose longest wave is no longer.
//
// Waves of sequence b sit at [first_b U, (first_b + count_b) U) with U the
// waves of one split row (Hkv per-head waves, or Hkv head quads), ordered
// (KV head, split, sub-wave); partial rows of sequence b sit at
// [first_b Hq, (first_b + count_b) Hq), ordered (query head, split).
// Both the attention kernels and the combine derive the same counts from
// t_ends, so nothing passes between them.  The functions below are
// wave-level: every lane of the wave calls them with the same arguments,
// and their results are wave-uniform.
// ---------------------------------------------------------------------------
constexpr int64_t kMaxSplits = 4096;

// Most split rows one head of a variable-length batch can take.
__host__ __device__ __forceinline__ int64_t varlen_lds_splits(int64_t B, int64_t S) {
  return B * S < kMaxSplits ? B * S : kMaxSplits;
}

struct SplitMap {
  const int32_t *t_ends;
  int64_t B, t_begin, n_int2, S;
  int skip;
  uint32_t t_lane;   // B <= 64: tiles of sequence `lane` (0 past B), loaded once
};

__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)(uint64_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ int64_t wave_sum64(int64_t v) {
  for (int k = 1; k < 64; k <<= 1) v += __shfl_xor(v, k, 64);
  return uniform64(v);
}

// Sum / max of a 32-bit value over the wave with DPP and the lane-swap
// instructions (no LDS round trips); the result is wave-uniform.
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_mov_dpp((int)v, kQuadXor1, 0xF, 0xF, true);
  v += (uint32_t)__builtin_amdgcn_mov_dpp((int)v, kQuadXor2, 0xF, 0xF, true);
  v += (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x124, 0xF, 0xF, false);   // row_ror 4
  v += (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, false);   // row_ror 8
  const auto r16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = r16[0] + r16[1];
  const auto r32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return __builtin_amdgcn_readfirstlane(r32[0] + r32[1]);
}
__device__ __forceinline__ uint32_t umax32(uint32_t a, uint32_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = umax32(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, kQuadXor1, 0xF, 0xF, true));
  v = umax32(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, kQuadXor2, 0xF, 0xF, true));
  v = umax32(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x124, 0xF, 0xF, false));
  v = umax32(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, false));
  const auto r16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = umax32(r16[0], r16[1]);
  const auto r32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return __builtin_amdgcn_readfirstlane(umax32(r32[0], r32[1]));
}

// tiles of sequence b (its INT2 tokens in the shifted 64-row grid); below
// 2^26 since t_ends are int32
__device__ __forceinline__ uint32_t sm_tiles(const SplitMap &m, int64_t b) {
  const int64_t e = (int64_t)m.t_ends[b] - m.t_begin;
  const int64_t n = e < 0 ? 0 : (e > m.n_int2 ? m.n_int2 : e);
  return n > 0 ? (uint32_t)((n + m.skip + 63) >> 6) : 0u;
}

__device__ __forceinline__ SplitMap make_split_map(const int32_t *t_ends, int64_t B, int64_t t_begin,
                                                   int64_t n_int2, int64_t S, int skip) {
  SplitMap m{t_ends, B, t_begin, n_int2, S, skip, 0u};
  const int lane = threadIdx.x & 63;
  if (B <= 64 && lane < B) m.t_lane = sm_tiles(m, lane);
  return m;
}

__device__ __forceinline__ int64_t ceil_div(int64_t x, int64_t w) { return (x + w - 1) / w; }
// ceil(tiles / tiles-per-wave), both below 2^26
__device__ __forceinline__ uint32_t tiles_div(uint32_t t, uint32_t w) { return (t + w - 1u) / w; }

// split rows the batch takes at w tiles per wave
__device__ __forceinline__ int64_t sm_rows(const SplitMap &m, uint32_t w) {
  if (m.B <= 64) return wave_sum_u32(tiles_div(m.t_lane, w));   // <= 64 * 2^24
  int64_t r = 0;
  for (int64_t b = threadIdx.x & 63; b < m.B; b += 64) r += tiles_div(sm_tiles(m, b), w);
  return wave_sum64(r);
}

// Tiles per wave; 0 when the batch has no INT2 token.
__device__ __forceinline__ int64_t sm_wave_tiles(const SplitMap &m) {
  int64_t tot, tmax, nb;
  if (m.B <= 64) {
    tot = wave_sum_u32(m.t_lane);                 // <= 64 * 2^26
    tmax = wave_max_u32(m.t_lane);
    nb = wave_sum_u32(m.t_lane > 0u ? 1u : 0u);
  } else {
    int64_t t0 = 0, n0 = 0;
    uint32_t x0 = 0;
    for (int64_t b = threadIdx.x & 63; b < m.B; b += 64) {
      const uint32_t t = sm_tiles(m, b);
      t0 += t;
      x0 = umax32(x0, t);
      n0 += t > 0u;
    }
    tot = wave_sum64(t0);
    tmax = wave_max_u32(x0);
    nb = wave_sum64(n0);
  }
  if (tmax == 0) return 0;
  const int64_t rows = m.B * m.S;
  // rows(w) >= tot / w, and rows(w) <= tot / w + nb: the least feasible w
  // lies in [lo, hi], and rows(hi) <= B*S
  int64_t lo = ceil_div(tot, rows);
  const int64_t lo_cap = ceil_div(tmax, kMaxSplits);
  lo = lo > 4 ? lo : 4;
  lo = lo > lo_cap ? lo : lo_cap;
  int64_t hi = rows > nb ? ceil_div(tot, rows - nb) : tmax;
  hi = hi > lo ? hi : lo;
  while (lo < hi) {
    const int64_t mid = (lo + hi) >> 1;
    if (sm_rows(m, (uint32_t)mid) <= rows) hi = mid;
    else lo = mid + 1;
  }
  return lo;
}

// Sequence b's first split row and split count, w tiles per wave.
__device__ __forceinline__ void sm_of_seq(const SplitMap &m, int64_t w, int64_t b, int64_t &first,
                                          int64_t &count) {
  if (m.B <= 64) {
    const uint32_t c = tiles_div(m.t_lane, (uint32_t)w);
    uint32_t f = 0;
    for (int i = 0; i < (int)b; ++i) f += __builtin_amdgcn_readlane(c, i);
    first = f;
    count = __builtin_amdgcn_readlane(c, (int)b);
    return;
  }
  int64_t f = 0;
  for (int64_t i = threadIdx.x & 63; i < b; i += 64) f += tiles_div(sm_tiles(m, i), (uint32_t)w);
  first = wave_sum64(f);
  count = __builtin_amdgcn_readfirstlane(tiles_div(sm_tiles(m, b), (uint32_t)w));
}

// The sequence that owns split row r, with its first row and count; false
// when r lies past the last row.
__device__ __forceinline__ bool sm_find_row(const SplitMap &m, int64_t w, int64_t r, int64_t &b,
                                            int64_t &first, int64_t &count) {
  if (m.B <= 64) {
    // one sequence per lane: walk the counts in the scalar unit
    const uint32_t c = tiles_div(m.t_lane, (uint32_t)w);
    int64_t f = 0;
    for (int i = 0; i < (int)m.B; ++i) {
      const int64_t ci = __builtin_amdgcn_readlane(c, i);
      if (r < f + ci) {
        b = i;
        first = f;
        count = ci;
        return true;
      }
      f += ci;
    }
    return false;
  }
  const int lane = threadIdx.x & 63;
  int64_t carry = 0;
  for (int64_t base = 0; base < m.B; base += 64) {
    const int64_t bb = base + lane;
    const int64_t c = bb < m.B ? tiles_div(sm_tiles(m, bb), (uint32_t)w) : 0;
    int64_t incl = c;                           // inclusive prefix over the chunk
    for (int k = 1; k < 64; k <<= 1) {
      const int64_t y = __shfl_up(incl, (unsigned)k, 64);
      if (lane >= k) incl += y;
    }
    incl += carry;
    // the prefix is non-decreasing, so the sequences ending at or before row
    // r are the first k lanes, and lane k (if any) holds row r
    const int k = __popcll(__ballot(bb < m.B && incl <= r));
    if (k < 64 && base + k < m.B) {
      b = base + k;
      count = uniform64(__shfl(c, k, 64));
      first = uniform64(__shfl(incl, k, 64)) - count;
      return true;
    }
    carry = uniform64(__shfl(incl, 63, 64));
  }
  return false;
}

// A wave's place in the grid: sequence, KV head, split, sub-wave (query head
// of a group, or head quad; `per` of them per split), and its sequence's
// split count and first split row.  False for a wave with nothing to do.
struct WavePlace {
  int64_t b, split, S, first;
  int hkv, sub;
};

__device__ __forceinline__ bool wave_place(const AttnArgs &a, int64_t gw, int per, WavePlace &w) {
  if (gw >= a.total_waves) return false;
  if (a.t_ends == nullptr) {
    w.sub = (int)(gw % per);
    const int64_t gs = gw / per;
    w.split = gs % a.n_splits;
    const int64_t bh = gs / a.n_splits;
    w.hkv = (int)(bh % a.Hkv);
    w.b = bh / a.Hkv;
    w.S = a.n_splits;
    w.first = w.b * a.n_splits;
    return true;
  }
  const SplitMap m = make_split_map(a.t_ends, a.B, a.t_begin, a.n_int2, a.n_splits, a.skip);
  const int64_t wt = sm_wave_tiles(m);
  if (wt == 0) return false;
  const int64_t U = (int64_t)a.Hkv * per;
  if (!sm_find_row(m, wt, gw / U, w.b, w.first, w.S)) return false;
  const int64_t local = gw - w.first * U;
  const int64_t per_head = w.S * per;
  w.hkv = (int)(local / per_head);
  const int64_t rem = local - (int64_t)w.hkv * per_head;
  w.split = rem / per;
  w.sub = (int)(rem - w.split * per);
  return true;
}

// Partial row of query head hq for a wave at place w.
__device__ __forceinline__ int64_t partial_row(const AttnArgs &a, const WavePlace &w, int hq) {
  return w.first * a.Hq + (int64_t)hq * w.S + w.split;
}

// Issue priority tied to a wave's progress through its full tiles: 3 in the
// first quarter, 2, 1, then 0 in the last quarter (grouped-query kernels).
// Two attention waves that share a SIMD have the same work, but at equal
// priority the older one wins issue arbitration and finishes well ahead of
// the younger one, which then runs the last part alone.  With the priority
// falling as a wave advances, the wave that is behind is favoured and the
// two finish closer together.  `done` is wave-uniform.
struct ProgressPrio {
  int64_t q1, q2, q3;
  int level;
  __device__ __forceinline__ explicit ProgressPrio(int64_t total)
      : q1(total / 4), q2(total / 2), q3(total - total / 4), level(3) {
    __builtin_amdgcn_s_setprio(3);
  }
  __device__ __forceinline__ void update(int64_t done) {
    const int want = 3 - (done >= q1) - (done >= q2) - (done >= q3);
    if (want == level) return;
    level = want;
    switch (want) {
      case 2: __builtin_amdgcn_s_setprio(2); break;
      case 1: __builtin_amdgcn_s_setprio(1); break;
      case 0: __builtin_amdgcn_s_setprio(0); break;
      default: __builtin_amdgcn_s_setprio(3); break;
    }
  }
};

// Reassemble the fp16 subnormal channel factor: code at position x of a
// 16-bit half is read with weight 2^(2x-24) (x <= 4) or 2^(2x-30) (x >= 5).
__device__ __forceinline__ constexpr float chan_unscale(int x) {
  return x <= 4 ? (float)(1u << (24 - 2 * x)) : (float)(1u << (30 - 2 * x));
}

// Lazy rescaling: the running reference m is moved only when a score
// exceeds it by more than kSlack (log2 units), so p = 2^(s - m) stays below
// 2^kSlack.  The partial (m, l, o') is exact for any reference m, so the
// merge is unchanged.
constexpr float kSlack = 4.0f;

// Value pre-scale of the one-head decode kernels, whose fp16 weights are
// w = fp16(p s 2^kx) with one power of two 2^kx per wave.  kx = 25 - E for
// the largest biased fp16 exponent field E (at least 1) among the value
// scales the wave has met, so s 2^kx < 2^11 and, with p < 2^kSlack,
// w < 2^15 stays inside the fp16 range for every finite scale; the largest
// scales give w >= p 2^10, so the weights stay normal fp16 numbers (2^-11
// relative rounding) even for scales that are fp16 subnormals.  kx only
// goes down; the accumulators that carry the factor are multiplied by
// 2^(new - old) when it does, an exact power of two.
struct ValuePrescale {
  int kx;          // -6 .. 24, wave-uniform
  uint32_t lim;    // scale magnitude bits from which kx must go down: (26 - kx) << 10
  float f, inv;    // 2^kx, 2^-kx
};
__device__ __forceinline__ ValuePrescale prescale_init() {
  return ValuePrescale{24, 2u << 10, 16777216.0f, 1.0f / 16777216.0f};
}
// Largest magnitude bits of four fp16 value scales (two per dword); the
// bits of a magnitude order like its value.
__device__ __forceinline__ uint32_t max_half_bits(uint32_t s0, uint32_t s1) {
  s0 &= 0x7FFF7FFFu;
  s1 &= 0x7FFF7FFFu;
  return umax32(umax32(s0 & 0xFFFFu, s0 >> 16), umax32(s1 & 0xFFFFu, s1 >> 16));
}
// Lowers kx to fit the wave's largest scale (mbits from max_half_bits);
// returns 2^(new - old) for the accumulators.  Call wave-uniformly.
__device__ __forceinline__ float prescale_lower(ValuePrescale &ps, uint32_t mbits) {
  const int E = (int)(wave_max_u32(mbits) >> 10);     // 31 only for inf / nan scales
  const int kx = 25 - (E > 1 ? E : 1);
  const float f = __builtin_amdgcn_ldexpf(1.0f, kx - ps.kx);
  ps.kx = kx;
  ps.lim = (uint32_t)(26 - kx) << 10;
  ps.f = __builtin_amdgcn_ldexpf(1.0f, kx);
  ps.inv = __builtin_amdgcn_ldexpf(1.0f, -kx);
  return f;
}

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

// First rows of a wave's full tiles in a paged cache, fetched 64 tiles at a
// time: lane j holds the row of full tile 64 blk + j (low and high dwords),
// so a tile's row is two lane reads instead of a table load and a division
// in front of the tile's loads.  row(i) takes wave-uniform i, clamped to the
// wave's last full tile as HeadTiles::full_row does.
struct PagedTileRows {
  int64_t blk = -1;
  uint32_t lo = 0, hi = 0;
  __device__ __forceinline__ int64_t row(const AttnArgs &a, int64_t b, int hkv, const HeadTiles &ht,
                                         int64_t split, int64_t S, int64_t i) {
    const int64_t ic = i < ht.mine - 1 ? i : ht.mine - 1;
    if ((ic >> 6) != blk) {                          // wave-uniform
      blk = ic >> 6;
      const int64_t j = (blk << 6) + (threadIdx.x & 63);
      const int64_t r = j < ht.mine ? tile_rows(a, b, hkv, 0, 0, ht.full_row(j, split, S)).k : 0;
      lo = (uint32_t)r;
      hi = (uint32_t)((uint64_t)r >> 32);
    }
    const int l = (int)(ic & 63);
    const uint32_t rl = (uint32_t)__builtin_amdgcn_readlane((int)lo, l);
    const uint32_t rh = (uint32_t)__builtin_amdgcn_readlane((int)hi, l);
    return (int64_t)(((uint64_t)rh << 32) | rl);
  }
};

hipError_t launch_attn_gqa(const AttnArgs &a, hipStream_t stream);
hipError_t launch_attn_generic(const AttnArgs &a, int kbits, int vbits, hipStream_t stream);
hipError_t launch_attn_gqa_bits(const AttnArgs &a, int kbits, int vbits, hipStream_t stream);

}  // namespace kvq
