// Read path for grouped-query attention (G >= 2 query heads per KV head):
// decode attention over the packed INT2 cache with the scores on the gfx950
// matrix cores ("Output-Aware Rotation for INT2 KV-Cache Quantization",
// woor.ai page, "What You Need to Know": scaled dot-product attention over
// the quantized cache; the rotation handling is the same as for G = 1).
//
// One wave owns up to four query heads of one KV head and every S-th
// 64-token tile of it, so each loaded K/V byte serves all of them.
//
// Scores.  With the per-head fixed-point query qi (|qi| < 2^18, written by
// the query preparation) in balanced base-32 digits d_L in [-16, 15]
// (qi = sum_L d_L 32^(3-L)), the per-group dot products of four heads and
// sixteen tokens are four v_mfma_scale_f32_16x16x128_f8f6f4 (one per digit
// position L):
//   A (fp8 e4m3, 16 x 128): row (head g, group j), column = channel slot;
//                           holds d_L of that channel when it lies in group j,
//                           else 0; block scale 2^(5(3-L));
//   B (fp4 e2m1, 128 x 16): a 2-bit code zero-extended to a nibble is the
//                           e2m1 value code/2, so the packed codes become the
//                           operand with two masks and a shift.
// Every product and partial sum is a multiple of 1/2 below 2^25, so D =
// (1/2) sum_{c in j} qi_c code_c up to the last bit of fp32.  D lands as
// lane (head g = lane/16, token lane%16) holding the four groups.
//
// Softmax runs per head on a 16-lane row (lazy reference as for G = 1).  The
// value weights w = fp16(p * scale_v) go through LDS to a second lane layout
// (token pair x 16 channels) where the V codes are accumulated for the four
// heads with v_dot2 on fp16-subnormal code encodings, as for G = 1.
#include "kv_decode_common.h"

namespace kvq {

typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef float float4v_t __attribute__((ext_vector_type(4)));

constexpr int kMqHeads = 4;          // query heads per wave
constexpr int kMqWaves = 4;          // waves per workgroup
constexpr int kMqLdsDwords = 64 * 8 + 4 * 8 * 4 * 4;   // token scales + value weights

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

// Loads of one 64-token tile.  K side: lane (token slot lane%16, group
// lane/16); tokens 16k + lane%16 for block k.  Token scales: lane = token.
// V side: lane (pair slot tp = lane/8, code dword lane%8); tokens 16k + tp
// and 16k + tp + 8.
struct MqTile {
  u32x2_t kc[4];
  u32x2_t ks, kz, vs, vz;
  uint32_t va[4], vb[4];
};

struct MqState {
  float m, l, zacc[4], wsum[4];     // K side: the lane's head
  float acc[kMqHeads][16];          // V side: four heads x the lane's 16 channels
};

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
__device__ __forceinline__ uint32_t row_ror8_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x120 + 8, 0xF, 0xF, false);
}
__device__ __forceinline__ float lane_read(float v, int l) {
  return bits_as_float((uint32_t)__builtin_amdgcn_readlane((int)float_as_bits(v), l));
}

// grid: ceil(total_waves / 4) workgroups of 4 waves; wave index
// gw = ((b*Hkv + hkv)*S + split)*quads + quad.
__global__ __launch_bounds__(64 * kMqWaves) void kv_int2_decode_attn_gqa(AttnArgs a) {
  __shared__ uint32_t lds_all[kMqWaves][kMqLdsDwords];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t gw = (int64_t)blockIdx.x * kMqWaves + wave;
  if (gw >= a.total_waves) return;                  // whole wave leaves; no barrier follows
  uint32_t *tsz = lds_all[wave];                    // [64 tokens][8 dwords]: ks kz vs vz
  uint32_t *wl = lds_all[wave] + 64 * 8;            // [group][pair slot][block][head] half2
  const int quads = (a.G + kMqHeads - 1) / kMqHeads;
  const int quad = (int)(gw % quads);
  const int64_t gs = gw / quads;
  const int64_t split = gs % a.n_splits;
  const int64_t bh = gs / a.n_splits;
  const int hkv = (int)(bh % a.Hkv);
  const int64_t b = bh / a.Hkv;
  const int64_t S = a.n_splits;

  // ---- query: K-side data of head g = lane/16, A operands of row lane%16
  const int gk = lane >> 4;
  const bool head_ok = kMqHeads * quad + gk < a.G;
  float isum[4], qstep = 0.0f;
  {
    const int hq = hkv * a.G + kMqHeads * quad + gk;
    const uint32_t *p = a.qprep + (b * a.Hq + (head_ok ? hq : 0)) * kQprepDwordsPerHead;
#pragma unroll
    for (int j = 0; j < 4; ++j) isum[j] = head_ok ? bits_as_float(p[32 * j + 26]) : 0.0f;
    qstep = head_ok ? bits_as_float(p[25]) : 0.0f;
  }
  v8i_t A[4];
  {
    const int mrow = lane & 15, ga = mrow >> 2, ja = mrow & 3, kba = lane >> 4;
    const bool ok = kMqHeads * quad + ga < a.G;
    const int hq = hkv * a.G + kMqHeads * quad + ga;
    const int32_t *qi = reinterpret_cast<const int32_t *>(a.qprep) +
                        (b * a.Hq + (ok ? hq : 0)) * kQprepDwordsPerHead + kQprepFixedOffset;
    // bytes 0..15 are slots 16 kba + i (group kba/2), bytes 16..31 slots
    // 64 + 16 kba + i (group 2 + kba/2); only the half in group ja is nonzero
    const bool lo_on = ok && (kba >> 1) == ja;
    const bool hi_on = ok && 2 + (kba >> 1) == ja;
    const int kbase = hi_on ? 64 + 16 * kba : 16 * kba;
    int q16[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) q16[i] = (lo_on || hi_on) ? qi[mq_channel(kbase + i)] : 0;
#pragma unroll
    for (int L = 0; L < 4; ++L) {
      int dw[4];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        int v = __builtin_amdgcn_cvt_pk_fp8_f32((float)mq_digit(q16[4 * w], L),
                                                (float)mq_digit(q16[4 * w + 1], L), 0, false);
        v = __builtin_amdgcn_cvt_pk_fp8_f32((float)mq_digit(q16[4 * w + 2], L),
                                            (float)mq_digit(q16[4 * w + 3], L), v, true);
        dw[w] = v;
      }
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        A[L][w] = lo_on ? dw[w] : 0;
        A[L][4 + w] = hi_on ? dw[w] : 0;
      }
    }
  }

  MqState st;
  st.m = kNegInf; st.l = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j) { st.zacc[j] = 0.0f; st.wsum[j] = 0.0f; }
#pragma unroll
  for (int g = 0; g < kMqHeads; ++g)
#pragma unroll
    for (int i = 0; i < 16; ++i) st.acc[g][i] = 0.0f;

  const int64_t krow0 = bh * a.kT_cap + a.t_begin;
  const int64_t vrow0 = bh * a.vT_cap + a.t_begin;
  const uint8_t *kc = a.kcodes + krow0 * kCodeBytes;
  const uint8_t *vc = a.vcodes + vrow0 * kCodeBytes;
  const uint16_t *ks = a.kscales + krow0 * kNGroups, *kz = a.kzeros + krow0 * kNGroups;
  const uint16_t *vs = a.vscales + vrow0 * kNGroups, *vz = a.vzeros + vrow0 * kNGroups;
  const int tk = lane & 15, kgrp = lane >> 4;      // K side
  const int tp = lane >> 3, c4 = lane & 7;          // V side

  // Full tile at row r0 (relative to the head's INT2 start): wave-uniform
  // tile bases plus 32-bit lane offsets.
  const uint32_t o_kc = (uint32_t)(tk * kCodeBytes + 8 * kgrp);
  const uint32_t o_sz = (uint32_t)(lane * kNGroups);
  const uint32_t o_va = (uint32_t)(tp * kCodeBytes + 4 * c4);
  auto load_full = [&](int64_t r0) {
    MqTile t;
    const uint8_t *kct = kc + r0 * kCodeBytes, *vct = vc + r0 * kCodeBytes;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      t.kc[k] = *reinterpret_cast<const u32x2_t *>(kct + o_kc + 16 * k * kCodeBytes);
    t.ks = *reinterpret_cast<const u32x2_t *>(ks + r0 * kNGroups + o_sz);
    t.kz = *reinterpret_cast<const u32x2_t *>(kz + r0 * kNGroups + o_sz);
    t.vs = *reinterpret_cast<const u32x2_t *>(vs + r0 * kNGroups + o_sz);
    t.vz = *reinterpret_cast<const u32x2_t *>(vz + r0 * kNGroups + o_sz);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      t.va[k] = *reinterpret_cast<const uint32_t *>(vct + o_va + 16 * k * kCodeBytes);
      t.vb[k] = *reinterpret_cast<const uint32_t *>(vct + o_va + (16 * k + 8) * kCodeBytes);
    }
    return t;
  };
  // Any tile: rows clamped to rmax (the partial last tile).
  auto load_tile = [&](int64_t r0, int64_t rmax) {
    MqTile t;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      int64_t r = r0 + 16 * k + tk;
      r = r < rmax ? r : rmax;
      t.kc[k] = *reinterpret_cast<const u32x2_t *>(kc + r * kCodeBytes + 8 * kgrp);
    }
    {
      int64_t r = r0 + lane;
      r = r < rmax ? r : rmax;
      t.ks = *reinterpret_cast<const u32x2_t *>(ks + r * kNGroups);
      t.kz = *reinterpret_cast<const u32x2_t *>(kz + r * kNGroups);
      t.vs = *reinterpret_cast<const u32x2_t *>(vs + r * kNGroups);
      t.vz = *reinterpret_cast<const u32x2_t *>(vz + r * kNGroups);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      int64_t ra = r0 + 16 * k + tp, rb = ra + 8;
      ra = ra < rmax ? ra : rmax;
      rb = rb < rmax ? rb : rmax;
      t.va[k] = *reinterpret_cast<const uint32_t *>(vc + ra * kCodeBytes + 4 * c4);
      t.vb[k] = *reinterpret_cast<const uint32_t *>(vc + rb * kCodeBytes + 4 * c4);
    }
    return t;
  };

  // One tile with nvalid (<= 64) valid tokens.
  auto process = [&](const MqTile &t, int nvalid) {
    reinterpret_cast<u32x4_t *>(tsz)[2 * lane] = u32x4_t{t.ks.x, t.ks.y, t.kz.x, t.kz.y};
    reinterpret_cast<u32x4_t *>(tsz)[2 * lane + 1] = u32x4_t{t.vs.x, t.vs.y, t.vz.x, t.vz.y};
    asm volatile("" ::: "memory");     // LDS of one wave is ordered; keep the program order
    // scores of the four 16-token blocks (lane: head gk, token 16k + tk)
    float raw[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int tt = 16 * k + tk;
      const v8i_t Bop = mq_unpack(t.kc[k]);
      float4v_t d = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int L = 0; L < 4; ++L)
        d = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[L], Bop, d, 0, 4, 0, mq_scale(L), 0, 127);
      const u32x4_t kq = reinterpret_cast<const u32x4_t *>(tsz)[2 * tt];
      // vector elements go through scalars: a bit_cast of an element
      // expression reads element 0 with this compiler
      const uint32_t kq0 = kq.x, kq1 = kq.y, kq2 = kq.z, kq3 = kq.w;
      const half2_t ks01 = __builtin_bit_cast(half2_t, kq0), ks23 = __builtin_bit_cast(half2_t, kq1);
      const half2_t kz01 = __builtin_bit_cast(half2_t, kq2), kz23 = __builtin_bit_cast(half2_t, kq3);
      // d[j] = (1/2) sum_{c in j} qi_c code_c
      float sd = d[0] * (float)ks01.x;
      sd = __builtin_fmaf(d[1], (float)ks01.y, sd);
      sd = __builtin_fmaf(d[2], (float)ks23.x, sd);
      sd = __builtin_fmaf(d[3], (float)ks23.y, sd);
      float sz = (float)kz01.x * isum[0];
      sz = __builtin_fmaf((float)kz01.y, isum[1], sz);
      sz = __builtin_fmaf((float)kz23.x, isum[2], sz);
      sz = __builtin_fmaf((float)kz23.y, isum[3], sz);
      raw[k] = __builtin_fmaf(2.0f, sd, sz);           // score in query steps
    }
    // one reference check for the whole tile, before any weight is formed
    float x[4];
    float xmax = kNegInf;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[k] = (16 * k + tk < nvalid) ? __builtin_fmaf(qstep, raw[k], -st.m) : kNegInf;
      xmax = fmaxf(xmax, x[k]);
    }
    if (__builtin_amdgcn_ballot_w64(xmax > kSlack)) {              // wave-uniform
      float y[4];
      float ymax = kNegInf;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        y[k] = (16 * k + tk < nvalid) ? qstep * raw[k] : kNegInf;
        ymax = fmaxf(ymax, y[k]);
      }
      const float mnew = fmaxf(st.m, row_max16(ymax));
      const float alpha = __builtin_amdgcn_exp2f(st.m - mnew);
      st.l *= alpha;
#pragma unroll
      for (int j = 0; j < 4; ++j) { st.zacc[j] *= alpha; st.wsum[j] *= alpha; }
#pragma unroll
      for (int g = 0; g < kMqHeads; ++g) {
        const float ag = lane_read(alpha, 16 * g);
#pragma unroll
        for (int i = 0; i < 16; ++i) st.acc[g][i] *= ag;
      }
      st.m = mnew;
#pragma unroll
      for (int k = 0; k < 4; ++k) x[k] = y[k] - mnew;
    }
    // weights of the value side: w = fp16(p * scale_v) per group
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int tt = 16 * k + tk;
      const float p = __builtin_amdgcn_exp2f(x[k]);          // 0 for masked tokens
      st.l += p;
      const u32x4_t vq = reinterpret_cast<const u32x4_t *>(tsz)[2 * tt + 1];
      const uint32_t vq0 = vq.x, vq1 = vq.y, vq2 = vq.z, vq3 = vq.w;
      const half2_t vs01 = __builtin_bit_cast(half2_t, vq0), vs23 = __builtin_bit_cast(half2_t, vq1);
      const half2_t vz01 = __builtin_bit_cast(half2_t, vq2), vz23 = __builtin_bit_cast(half2_t, vq3);
      const float svj[4] = {(float)vs01.x, (float)vs01.y, (float)vs23.x, (float)vs23.y};
      const float zvj[4] = {(float)vz01.x, (float)vz01.y, (float)vz23.x, (float)vz23.y};
      _Float16 wh[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        wh[j] = (_Float16)(p * svj[j]);
        st.zacc[j] = __builtin_fmaf(p, __builtin_fmaf(1.5f, svj[j], zvj[j]), st.zacc[j]);
        st.wsum[j] += (float)wh[j];
      }
      // token tt + 8's weights from lane tk + 8 of the row; lanes tk < 8
      // store the pairs (token 16k + tk, token 16k + tk + 8) per group
      const uint32_t w01 = __builtin_bit_cast(uint32_t, half2_t{wh[0], wh[1]});
      const uint32_t w23 = __builtin_bit_cast(uint32_t, half2_t{wh[2], wh[3]});
      const uint32_t o01 = row_ror8_u(w01), o23 = row_ror8_u(w23);
      if (tk < 8) {
        const uint32_t pr[4] = {__builtin_amdgcn_perm(o01, w01, 0x05040100u),   // (w0 mine, w0 partner)
                                __builtin_amdgcn_perm(o01, w01, 0x07060302u),
                                __builtin_amdgcn_perm(o23, w23, 0x05040100u),
                                __builtin_amdgcn_perm(o23, w23, 0x07060302u)};
#pragma unroll
        for (int j = 0; j < 4; ++j) wl[((j * 8 + tk) * 4 + k) * 4 + kgrp] = pr[j];
      }
    }
    asm volatile("" ::: "memory");
    // V side: pairs (16k + tp, 16k + tp + 8) x channels 16 c4 .. 16 c4 + 15
    const int jv = c4 >> 1;
    u32x4_t wq[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) wq[k] = reinterpret_cast<const u32x4_t *>(wl)[(jv * 8 + tp) * 4 + k];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t X = __builtin_amdgcn_perm(t.vb[k], t.va[k], 0x05040100u);
      const uint32_t Y = __builtin_amdgcn_perm(t.vb[k], t.va[k], 0x07060302u);
      const uint32_t X6 = X >> 6, Y6 = Y >> 6;
      const uint32_t wk[4] = {wq[k].x, wq[k].y, wq[k].z, wq[k].w};
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        const uint32_t px = x <= 4 ? (X & (0x00030003u << (2 * x))) : (X6 & (0x00030003u << (2 * x - 6)));
        const uint32_t py = x <= 4 ? (Y & (0x00030003u << (2 * x))) : (Y6 & (0x00030003u << (2 * x - 6)));
        const half2_t hx = __builtin_bit_cast(half2_t, px);
        const half2_t hy = __builtin_bit_cast(half2_t, py);
#pragma unroll
        for (int g = 0; g < kMqHeads; ++g) {
          const half2_t wg = __builtin_bit_cast(half2_t, wk[g]);
          st.acc[g][x] = __builtin_amdgcn_fdot2(hx, wg, st.acc[g][x], false);
          st.acc[g][8 + x] = __builtin_amdgcn_fdot2(hy, wg, st.acc[g][8 + x], false);
        }
      }
    }
    asm volatile("" ::: "memory");
  };

  // this wave's full tiles, loads one tile ahead
  const int64_t mine = tiles_of_split(a.n_int2, split, S);
  if (mine > 0) {
    auto row_of = [&](int64_t i) { return 64 * (split + (i < mine - 1 ? i : mine - 1) * S); };
    MqTile t0 = load_full(row_of(0)), t1;
    int64_t i = 0;
    for (; i + 2 <= mine; i += 2) {
      t1 = load_full(row_of(i + 1));
      process(t0, 64);
      t0 = load_full(row_of(i + 2));
      process(t1, 64);
    }
    if (i < mine) process(t0, 64);
  }
  const int64_t n_full = a.n_int2 >> 6;
  const int rem = (int)(a.n_int2 & 63);
  if (rem != 0 && n_full % S == split) {
    const MqTile t = load_tile(64 * n_full, a.n_int2 - 1);
    process(t, rem);
  }

  // ---- reduce and write the partials of the wave's heads
  st.l = row_sum16(st.l);
  float corr[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) corr[j] = row_sum16(__builtin_fmaf(-1.5f, st.wsum[j], st.zacc[j]));
#pragma unroll
  for (int g = 0; g < kMqHeads; ++g)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float v = st.acc[g][i];
      v += row_ror<8>(v);                  // pair slots tp and tp ^ 1 (lanes l, l + 8)
      st.acc[g][i] = sum_xor32(sum_xor16(v));
    }
  const int jv = c4 >> 1;
#pragma unroll
  for (int g = 0; g < kMqHeads; ++g) {
    if (kMqHeads * quad + g >= a.G) break;          // wave-uniform
    const int hq = hkv * a.G + kMqHeads * quad + g;
    float *dst = a.partials + ((b * a.Hq + hq) * S + split) * kPartialStride;
    const float c0 = lane_read(corr[0], 16 * g), c1 = lane_read(corr[1], 16 * g);
    const float c2 = lane_read(corr[2], 16 * g), c3 = lane_read(corr[3], 16 * g);
    const float cj = jv == 0 ? c0 : jv == 1 ? c1 : jv == 2 ? c2 : c3;
    if (tp == 0) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        dst[16 * c4 + i] = __builtin_fmaf(st.acc[g][i], chan_unscale(i & 7), cj);
    }
    const float mg = lane_read(st.m, 16 * g), lg = lane_read(st.l, 16 * g);
    if (lane == 0) {
      dst[128] = mg;
      dst[129] = lg;
    }
  }
}

hipError_t launch_attn_gqa(const AttnArgs &a, hipStream_t stream) {
  hipLaunchKernelGGL(kv_int2_decode_attn_gqa, dim3((unsigned)((a.total_waves + kMqWaves - 1) / kMqWaves)),
                     dim3(64 * kMqWaves), 0, stream, a);
  return hipGetLastError();
}

}  // namespace kvq
