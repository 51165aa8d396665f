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
// With codes <= 3 the result is a multiple of 1/2 below 2^22.6 and the
// partial sums after the leading digits are multiples of larger powers of
// two in the same range, so D = (1/2) sum_{c in j} qi_c code_c exactly.  D lands as
// lane (head g = lane/16, token lane%16) holding the four groups.
//
// Softmax runs per head on a 16-lane row (lazy reference as for G = 1).  The
// weights are rounded once to fp16, p~ = fp16(p), and used everywhere: in
// the normalizer l = sum p~, the zero-point term and the value product, so
// the partial is an exact softmax-weighted sum with weights p~.
//
// Values, also on the matrix cores (v_mfma_f32_16x16x32_f16), per 8 tokens
// and 16 code bytes:
//   A (16 x 32): row (head h, position e of a channel in its byte), column
//                (token t, position e'): p~[h][t] when e' = e, else 0;
//   B (32 x 16): column = code byte; (t, e') holds code * s - fp16(1.5 s)
//                of channel 4 byte + e' (one fp4 -> fp16 conversion and one
//                packed fp16 FMA per two values).
// The accumulator row (h, e), column byte b, is channel 4b + e of head h;
// with the two byte blocks (2n, 2n+1) a lane ends up owning channels
// 8n .. 8n+7 of its head, summed over every token of the split.  The
// zero-point term sum p~ (z + fp16(1.5 s)) is accumulated per group in the
// softmax layout.
#include "kv_decode_mq.h"

namespace kvq {

// LDS per wave, in dwords: per-token records, the tile's value codes and the
// fp16 weights of the four heads.
constexpr int kMqRecDwords = 12;     // ks, kz (4) | (s_j, -fp16(1.5 s_j)) (4) | z_j + fp16(1.5 s_j) fp32 (4)
constexpr int kMqRecOff = 0;
constexpr int kMqCodeOff = kMqRecOff + 64 * kMqRecDwords;          // 64 tokens x 32 bytes
constexpr int kMqPwOff = kMqCodeOff + 64 * kCodeBytes / 4;          // [head][64 tokens] fp16
constexpr int kMqLdsDwords = kMqPwOff + kMqHeads * 64 / 2;

// Loads of one 64-token tile.  K side: lane (token slot lane%16, group
// lane/16); tokens 16k + lane%16 for block k.  Token scales and zeros: lane =
// token.  Value codes: the tile's 2 KB as two 1 KB halves, 16 bytes per lane,
// staged to LDS in token-major order.
struct MqTile {
  u32x2_t kc[4];
  u32x2_t ks, kz, vs, vz;
  u32x4_t vc[2];
};

struct MqState {
  float m, l, zacc[4];     // softmax layout: the lane's head (lane / 16)
  float4v_t o[2];          // value layout: rows (head lane/16, e = 0..3), byte 2 (lane%16) + blk
};

// grid: ceil(total_waves / 4) workgroups of 4 waves; wave index
// gw = ((b*Hkv + hkv)*S + split)*quads + quad for one length, the
// variable-length map of wave_place otherwise.
__global__ __launch_bounds__(64 * kMqWaves) void kv_int2_decode_attn_gqa(AttnArgs a) {
  __shared__ uint32_t lds_all[kMqWaves][kMqLdsDwords];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t gw = (int64_t)blockIdx.x * kMqWaves + wave;
  const int quads = (a.G + kMqHeads - 1) / kMqHeads;
  WavePlace wp;
  if (!wave_place(a, gw, quads, wp)) return;        // whole wave leaves; no barrier follows
  uint32_t *rec = lds_all[wave] + kMqRecOff;        // [64 tokens][kMqRecDwords]
  uint8_t *vcl = reinterpret_cast<uint8_t *>(lds_all[wave] + kMqCodeOff);   // [64 tokens][32 bytes]
  _Float16 *pw = reinterpret_cast<_Float16 *>(lds_all[wave] + kMqPwOff);     // [head][64 tokens]
  const int quad = wp.sub;
  const int64_t split = wp.split;
  const int hkv = wp.hkv;
  const int64_t b = wp.b;
  const int64_t bh = b * a.Hkv + hkv;
  const int64_t S = wp.S;

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

  // ---- value side: lane (byte pair n = lane%16, token pair kb = lane/16) of
  // B; lane (head ha = (lane%16)/4, position e = lane%4, kb) of A.  The A
  // dword d holds token kb*2 + d/2, positions (d%2, d%2 + 2); v_perm
  // selectors pick p~ of that token into the half of position e, or zero.
  const int vn = lane & 15, vkb = lane >> 4;
  const int ha = vn >> 2, ve = vn & 3;
  uint32_t selA[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t src = (d >> 1) ? 0x0706u : 0x0504u;       // p~ of token 2 kb + d/2 in P
    const bool on = (d & 1) == (ve & 1);
    selA[d] = !on ? 0x0C0C0C0Cu : (ve >> 1) ? ((src << 16) | 0x0C0Cu) : (0x0C0C0000u | src);
  }

  MqState st;
  st.m = kNegInf; st.l = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j) st.zacc[j] = 0.0f;
  st.o[0] = float4v_t{0.0f, 0.0f, 0.0f, 0.0f};
  st.o[1] = float4v_t{0.0f, 0.0f, 0.0f, 0.0f};

  const int64_t krow0 = bh * a.kT_cap + a.t_begin - a.skip;   // row 0 of the shifted grid
  const int64_t vrow0 = bh * a.vT_cap + a.t_begin - a.skip;
  const int tk = lane & 15, kgrp = lane >> 4;      // K side

  // Full tile at row r0 (relative to the head's INT2 start): wave-uniform
  // tile bases plus 32-bit lane offsets.
  const uint32_t o_kc = (uint32_t)(tk * kCodeBytes + 8 * kgrp);
  const uint32_t o_sz = (uint32_t)(lane * kNGroups);
  const uint32_t o_vc = (uint32_t)(16 * lane);
  auto load_full = [&](const TileRows &tr) {
    MqTile t;
    const uint8_t *kct = a.kcodes + tr.k * kCodeBytes, *vct = a.vcodes + tr.v * kCodeBytes;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      t.kc[k] = *reinterpret_cast<const u32x2_t *>(kct + o_kc + 16 * k * kCodeBytes);
    t.ks = *reinterpret_cast<const u32x2_t *>(a.kscales + tr.k * kNGroups + o_sz);
    t.kz = *reinterpret_cast<const u32x2_t *>(a.kzeros + tr.k * kNGroups + o_sz);
    t.vs = *reinterpret_cast<const u32x2_t *>(a.vscales + tr.v * kNGroups + o_sz);
    t.vz = *reinterpret_cast<const u32x2_t *>(a.vzeros + tr.v * kNGroups + o_sz);
    t.vc[0] = *reinterpret_cast<const u32x4_t *>(vct + o_vc);
    t.vc[1] = *reinterpret_cast<const u32x4_t *>(vct + 1024 + o_vc);
    return t;
  };
  // Any tile: rows clamped into [rmin, rmax] (a partial tile), then taken
  // relative to the tile's first cache row.
  auto load_tile = [&](int64_t r0, int64_t rmin, int64_t rmax) {
    const TileRows tr = tile_rows(a, b, hkv, krow0, vrow0, r0);
    const uint8_t *kc = a.kcodes + (tr.k - r0) * kCodeBytes, *vc = a.vcodes + (tr.v - r0) * kCodeBytes;
    const uint16_t *ks = a.kscales + (tr.k - r0) * kNGroups, *kz = a.kzeros + (tr.k - r0) * kNGroups;
    const uint16_t *vs = a.vscales + (tr.v - r0) * kNGroups, *vz = a.vzeros + (tr.v - r0) * kNGroups;
    auto clampr = [&](int64_t r) { return r < rmax ? (r > rmin ? r : rmin) : rmax; };
    MqTile t;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int64_t r = clampr(r0 + 16 * k + tk);
      t.kc[k] = *reinterpret_cast<const u32x2_t *>(kc + r * kCodeBytes + 8 * kgrp);
    }
    {
      const int64_t r = clampr(r0 + lane);
      t.ks = *reinterpret_cast<const u32x2_t *>(ks + r * kNGroups);
      t.kz = *reinterpret_cast<const u32x2_t *>(kz + r * kNGroups);
      t.vs = *reinterpret_cast<const u32x2_t *>(vs + r * kNGroups);
      t.vz = *reinterpret_cast<const u32x2_t *>(vz + r * kNGroups);
    }
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int64_t r = clampr(r0 + 32 * hh + (lane >> 1));
      t.vc[hh] = *reinterpret_cast<const u32x4_t *>(vc + r * kCodeBytes + 16 * (lane & 1));
    }
    return t;
  };

  // One tile whose tokens [lo, hi) are valid.  big: the wave has met a value
  // scale of 2^15 or more (fp16 bits 0x7800 and up; adding 0x0800 sets bit
  // 15 of such a half, with no carry for finite halves), for which
  // fp16(1.5 s) and the B entries could overflow; from then on the B entries
  // are built from s/2 and each weight in the A operand is doubled
  // (2 p~ (code s/2 - fp16(0.75 s)) = p~ (code s - 2 fp16(0.75 s)), exact
  // power-of-two scalings), with the zero-point term z + 2 fp16(0.75 s) to
  // match.  Either form may follow the other in one accumulator: each
  // token's product is the same.  The mode enters as wave-uniform factors
  // (1 or 2, 1 or 1/2), not as a second copy of the tile code, so that one
  // tile's value products and the next tile's score products fall in one
  // basic block and can interleave.
  bool big = false;
  auto process = [&](const MqTile &t, int lo, int hi) {
    if (!big && __builtin_amdgcn_ballot_w64(
                    (((t.vs.x + 0x08000800u) | (t.vs.y + 0x08000800u)) & 0x80008000u) != 0u))
      big = true;
    const float kB = big ? 2.0f : 1.0f;
    const _Float16 hb = big ? (_Float16)0.5f : (_Float16)1.0f, wb = big ? (_Float16)2.0f : (_Float16)1.0f;
    {
      // per-token record (lane = token) and the value codes
      uint32_t *rl = rec + lane * kMqRecDwords;
      uint32_t vs0 = t.vs.x, vs1 = t.vs.y;
      const uint32_t vz0 = t.vz.x, vz1 = t.vz.y;
      half2_t s01 = __builtin_bit_cast(half2_t, vs0), s23 = __builtin_bit_cast(half2_t, vs1);
      s01 = s01 * half2_t{hb, hb};
      s23 = s23 * half2_t{hb, hb};
      vs0 = __builtin_bit_cast(uint32_t, s01);
      vs1 = __builtin_bit_cast(uint32_t, s23);
      const half2_t z01 = __builtin_bit_cast(half2_t, vz0), z23 = __builtin_bit_cast(half2_t, vz1);
      const half2_t n01 = s01 * half2_t{(_Float16)-1.5f, (_Float16)-1.5f};   // -fp16(1.5 s)
      const half2_t n23 = s23 * half2_t{(_Float16)-1.5f, (_Float16)-1.5f};
      const uint32_t un01 = __builtin_bit_cast(uint32_t, n01), un23 = __builtin_bit_cast(uint32_t, n23);
      reinterpret_cast<u32x4_t *>(rl)[0] = u32x4_t{t.ks.x, t.ks.y, t.kz.x, t.kz.y};
      reinterpret_cast<u32x4_t *>(rl)[1] =
          u32x4_t{__builtin_amdgcn_perm(un01, vs0, 0x05040100u), __builtin_amdgcn_perm(un01, vs0, 0x07060302u),
                  __builtin_amdgcn_perm(un23, vs1, 0x05040100u), __builtin_amdgcn_perm(un23, vs1, 0x07060302u)};
      reinterpret_cast<float4v_t *>(rl)[2] =
          float4v_t{__builtin_fmaf(-kB, (float)n01.x, (float)z01.x), __builtin_fmaf(-kB, (float)n01.y, (float)z01.y),
                    __builtin_fmaf(-kB, (float)n23.x, (float)z23.x), __builtin_fmaf(-kB, (float)n23.y, (float)z23.y)};
      reinterpret_cast<u32x4_t *>(vcl)[lane] = t.vc[0];
      reinterpret_cast<u32x4_t *>(vcl)[64 + lane] = t.vc[1];
    }
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
      const u32x4_t kq = reinterpret_cast<const u32x4_t *>(rec + tt * kMqRecDwords)[0];
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
      x[k] = (16 * k + tk >= lo && 16 * k + tk < hi) ? __builtin_fmaf(qstep, raw[k], -st.m) : kNegInf;
      xmax = fmaxf(xmax, x[k]);
    }
    if (__builtin_amdgcn_ballot_w64(xmax > kSlack)) {              // wave-uniform
      float y[4];
      float ymax = kNegInf;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        y[k] = (16 * k + tk >= lo && 16 * k + tk < hi) ? qstep * raw[k] : kNegInf;
        ymax = fmaxf(ymax, y[k]);
      }
      const float mnew = fmaxf(st.m, row_max16(ymax));
      const float alpha = __builtin_amdgcn_exp2f(st.m - mnew);   // the row's head = the lane's value rows
      st.l *= alpha;
#pragma unroll
      for (int j = 0; j < 4; ++j) st.zacc[j] *= alpha;
      st.o[0] *= alpha;
      st.o[1] *= alpha;
      st.m = mnew;
#pragma unroll
      for (int k = 0; k < 4; ++k) x[k] = y[k] - mnew;
    }
    // weights p~ = fp16(p), the normalizer and the zero-point term
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int tt = 16 * k + tk;
      const _Float16 ph = (_Float16)__builtin_amdgcn_exp2f(x[k]);   // 0 for masked tokens
      const float pf = (float)ph;
      st.l += pf;
      const float4v_t zb = reinterpret_cast<const float4v_t *>(rec + tt * kMqRecDwords)[2];
      st.zacc[0] = __builtin_fmaf(pf, zb[0], st.zacc[0]);
      st.zacc[1] = __builtin_fmaf(pf, zb[1], st.zacc[1]);
      st.zacc[2] = __builtin_fmaf(pf, zb[2], st.zacc[2]);
      st.zacc[3] = __builtin_fmaf(pf, zb[3], st.zacc[3]);
      pw[gk * 64 + tt] = ph * wb;
    }
    asm volatile("" ::: "memory");
    // values: 8 blocks of 8 tokens; lane's tokens t0 = 8 tb + 2 kb and t0 + 1
    const int jv = vn >> 2;                        // group of bytes 2 vn, 2 vn + 1
#pragma unroll
    for (int tb = 0; tb < 8; ++tb) {
      const int t0 = 8 * tb + 2 * vkb;
      const uint32_t y = (uint32_t)*reinterpret_cast<const uint16_t *>(vcl + t0 * kCodeBytes + 2 * vn) |
                         ((uint32_t)*reinterpret_cast<const uint16_t *>(vcl + (t0 + 1) * kCodeBytes + 2 * vn) << 16);
      const uint32_t sv0 = rec[t0 * kMqRecDwords + 4 + jv];
      const uint32_t sv1 = rec[(t0 + 1) * kMqRecDwords + 4 + jv];
      const uint32_t P = *reinterpret_cast<const uint32_t *>(pw + ha * 64 + t0);
      v8h_t Aop;
      {
        const uint32_t a0 = __builtin_amdgcn_perm(P, P, selA[0]), a1 = __builtin_amdgcn_perm(P, P, selA[1]);
        const uint32_t a2 = __builtin_amdgcn_perm(P, P, selA[2]), a3 = __builtin_amdgcn_perm(P, P, selA[3]);
        const half2_t h0 = __builtin_bit_cast(half2_t, a0), h1 = __builtin_bit_cast(half2_t, a1);
        const half2_t h2 = __builtin_bit_cast(half2_t, a2), h3 = __builtin_bit_cast(half2_t, a3);
        Aop = half8_t{h0.x, h0.y, h1.x, h1.y, h2.x, h2.y, h3.x, h3.y};
      }
      // nibble bytes: positions (0, 2) and (1, 3) of every code byte
      const uint32_t y02 = y & 0x33333333u, y13 = (y >> 2) & 0x33333333u;
      st.o[0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Aop, mq_bvals<0>(y02, y13, sv0, sv1), st.o[0], 0, 0, 0);
      st.o[1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Aop, mq_bvals<1>(y02, y13, sv0, sv1), st.o[1], 0, 0, 0);
    }
    asm volatile("" ::: "memory");
  };

  auto run = process;


  // this wave's full tiles, loads one tile ahead
  const HeadTiles ht(seq_int2(a, b), a.skip, split, S);
  const int64_t mine = ht.mine;
  if (mine > 0) {
    PagedTileRows pages;
    auto row_of = [&](int64_t i) {
      if (a.block_table == nullptr) {
        const int64_t r = ht.full_row(i, split, S);
        return TileRows{krow0 + r, vrow0 + r};
      }
      const int64_t r = pages.row(a, b, hkv, ht, split, S, i);
      return TileRows{r, r};
    };
    MqTile t0 = load_full(row_of(0)), t1;
    ProgressPrio prio(mine);
    int64_t i = 0;
    for (; i + 2 <= mine; i += 2) {
      prio.update(i);
      t1 = load_full(row_of(i + 1));
      run(t0, 0, 64);
      t0 = load_full(row_of(i + 2));
      run(t1, 0, 64);
    }
    if (i < mine) run(t0, 0, 64);
  }
  {
    // partial tiles: masked rows are loaded from the nearest valid row
    int64_t p[2];
    ht.partial(a.skip, split, S, p[0], p[1]);
    for (int e = 0; e < 2; ++e) {
      if (p[e] < 0) continue;
      const int64_t base = 64 * p[e];
      const int lo = a.skip > base ? (int)(a.skip - base) : 0;
      const int hi = ht.n_tok - base < 64 ? (int)(ht.n_tok - base) : 64;
      const MqTile t = load_tile(base, base + lo, base + hi - 1);
      run(t, lo, hi);
    }
  }

  // ---- write the partials of the wave's heads.  Softmax rows: head = lane/16;
  // value lanes: head lane/16, channels 8 (lane%16) .. + 7 (group (lane%16)/4).
  st.l = row_sum16(st.l);
  float corr[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) corr[j] = row_sum16(st.zacc[j]);
  const int g = lane >> 4;
  if (kMqHeads * quad + g < a.G) {
    const int hq = hkv * a.G + kMqHeads * quad + g;
    float *dst = a.partials + partial_row(a, wp, hq) * kPartialStride;
    const int jo = vn >> 2;
    const float cj = jo == 0 ? corr[0] : jo == 1 ? corr[1] : jo == 2 ? corr[2] : corr[3];
    const float4v_t c4v = {cj, cj, cj, cj};
    reinterpret_cast<float4v_t *>(dst + 8 * vn)[0] = st.o[0] + c4v;
    reinterpret_cast<float4v_t *>(dst + 8 * vn)[1] = st.o[1] + c4v;
    if (vn == 0) {
      dst[128] = st.m;
      dst[129] = st.l;
    }
  }
}

hipError_t launch_attn_gqa(const AttnArgs &a, hipStream_t stream) {
  hipLaunchKernelGGL(kv_int2_decode_attn_gqa, dim3((unsigned)((a.total_waves + kMqWaves - 1) / kMqWaves)),
                     dim3(64 * kMqWaves), 0, stream, a);
  return hipGetLastError();
}

}  // namespace kvq
