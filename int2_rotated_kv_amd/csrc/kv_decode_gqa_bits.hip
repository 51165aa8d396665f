// Grouped-query attention (G >= 2 query heads per KV head) over caches of
// other code widths: keys at KB bits and values at VB bits, each 1, 2 or 4,
// not both 2 (the library's b-bit form of the INT2 codec, OptR page,
// future-work paragraph on mixed-bit schemes; the attention is the scaled
// dot product of the page's "What You Need to Know").
//
// The same matrix-core scheme as the 2-bit kernel (kv_decode_gqa.hip): one
// wave owns up to four query heads of one KV head and every S-th 64-token
// tile, so each loaded K/V byte serves all of them.  Every width goes
// through 2-bit operands:
//
// Keys.  The scores are sums of qi_c * code_c per group on
//   v_mfma_scale_f32_16x16x128_f8f6f4 (fp8 digits of the fixed-point query
//   times fp4 nibbles 0b00cc = code/2).
//   - 2 bits: the packed codes as in the 2-bit kernel (slot order mq_channel).
//   - 1 bit: four shifted copies of the group's dword, each masked to the
//     low bit of its nibbles (mq_key_operand).
//   - 4 bits: code = lo + 4 hi with 2-bit planes; a nibble's plane p is
//     (w >> 2p) & 0x33333333 in place, so slot 8u + e of a group is channel
//     8u + e (the query digits are laid out in that order), and the high
//     plane's product carries the B block scale 2^2, so both planes
//     accumulate into one result.
// Values.  On v_mfma_f32_16x16x32_f16 with the 2-bit kernel's operands
//   (A: the fp16 weights p~ per (head, position in a byte); B: code * s -
//   fp16(1.5 s) per code byte column).
//   - 1 bit: the lane's code byte of each token is spread to the two 2-bit
//     bytes first.
//   - 4 bits: two 2-bit planes compacted from the nibbles, the high plane
//     with weights 4 p~ (exact); the zero-point term is then
//     z + 5 fp16(1.5 s).
#include "kv_decode_mq.h"

namespace kvq {

// Per-token record: ks, kz (4) | (s_j, -fp16(1.5 s_j)) (4) | zero-point term fp32 (4)
constexpr int kMbRecDwords = 12;

template <int VB>
struct MbLds {
  static constexpr int kRowBytes = 16 * VB;                        // a value row
  static constexpr int kRecOff = 0;
  static constexpr int kCodeOff = kRecOff + 64 * kMbRecDwords;     // 64 tokens x kRowBytes
  static constexpr int kPwOff = kCodeOff + 64 * kRowBytes / 4;     // [head][64 tokens] fp16
  static constexpr int kDwords = kPwOff + kMqHeads * 64 / 2;
};

template <int KB, int VB>
struct MbTile {
  typename MbKeyWord<KB>::type kc[4];
  u32x2_t ks, kz, vs, vz;
  u32x4_t vc[VB];
};

struct MbState {
  float m, l, zacc[4];
  float4v_t o[2];
};

// grid: ceil(total_waves / 4) workgroups of 4 waves; the wave map of the
// 2-bit grouped-query kernel.
template <int KB, int VB>
__global__ __launch_bounds__(64 * kMqWaves, 2) void kv_quant_decode_attn_gqa(AttnArgs a) {
  typedef MbLds<VB> L;
  constexpr int kKRow = 16 * KB;                   // key row bytes
  constexpr int kPV = VB == 4 ? 2 : 1;             // value planes
  __shared__ uint32_t lds_all[kMqWaves][L::kDwords];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t gw = (int64_t)blockIdx.x * kMqWaves + wave;
  const int quads = (a.G + kMqHeads - 1) / kMqHeads;
  WavePlace wp;
  if (!wave_place(a, gw, quads, wp)) return;        // whole wave leaves; no barrier follows
  uint32_t *rec = lds_all[wave] + L::kRecOff;       // [64 tokens][kMbRecDwords]
  uint8_t *vcl = reinterpret_cast<uint8_t *>(lds_all[wave] + L::kCodeOff);   // [64 tokens][row]
  _Float16 *pw = reinterpret_cast<_Float16 *>(lds_all[wave] + L::kPwOff);     // [head][64 tokens]
  const int quad = wp.sub;
  const int64_t split = wp.split;
  const int hkv = wp.hkv;
  const int64_t b = wp.b;
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
    for (int i = 0; i < 16; ++i) q16[i] = (lo_on || hi_on) ? qi[mq_key_channel<KB>(kbase + i)] : 0;
#pragma unroll
    for (int Ld = 0; Ld < 4; ++Ld) {
      int dw[4];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        int v = __builtin_amdgcn_cvt_pk_fp8_f32((float)mq_digit(q16[4 * w], Ld),
                                                (float)mq_digit(q16[4 * w + 1], Ld), 0, false);
        v = __builtin_amdgcn_cvt_pk_fp8_f32((float)mq_digit(q16[4 * w + 2], Ld),
                                            (float)mq_digit(q16[4 * w + 3], Ld), v, true);
        dw[w] = v;
      }
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        A[Ld][w] = lo_on ? dw[w] : 0;
        A[Ld][4 + w] = hi_on ? dw[w] : 0;
      }
    }
  }

  // ---- value side (as the 2-bit kernel): lane (byte pair n = lane%16,
  // token pair kb = lane/16) of B; lane (head ha, position e, kb) of A
  const int vn = lane & 15, vkb = lane >> 4;
  const int ha = vn >> 2, ve = vn & 3;
  uint32_t selA[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t src = (d >> 1) ? 0x0706u : 0x0504u;
    const bool on = (d & 1) == (ve & 1);
    selA[d] = !on ? 0x0C0C0C0Cu : (ve >> 1) ? ((src << 16) | 0x0C0Cu) : (0x0C0C0000u | src);
  }

  MbState st;
  st.m = kNegInf; st.l = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j) st.zacc[j] = 0.0f;
  st.o[0] = float4v_t{0.0f, 0.0f, 0.0f, 0.0f};
  st.o[1] = float4v_t{0.0f, 0.0f, 0.0f, 0.0f};

  const int64_t bh = b * a.Hkv + hkv;
  const int64_t krow0 = bh * a.kT_cap + a.t_begin - a.skip;
  const int64_t vrow0 = bh * a.vT_cap + a.t_begin - a.skip;
  const int tk = lane & 15, kgrp = lane >> 4;      // K side: token slot, group

  typedef typename MbKeyWord<KB>::type KWord;
  auto load_full = [&](const TileRows &tr) {
    MbTile<KB, VB> t;
    const uint8_t *kct = a.kcodes + tr.k * kKRow, *vct = a.vcodes + tr.v * L::kRowBytes;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      t.kc[k] = *reinterpret_cast<const KWord *>(kct + (16 * k + tk) * kKRow + (kKRow / 4) * kgrp);
    t.ks = *reinterpret_cast<const u32x2_t *>(a.kscales + (tr.k + lane) * kNGroups);
    t.kz = *reinterpret_cast<const u32x2_t *>(a.kzeros + (tr.k + lane) * kNGroups);
    t.vs = *reinterpret_cast<const u32x2_t *>(a.vscales + (tr.v + lane) * kNGroups);
    t.vz = *reinterpret_cast<const u32x2_t *>(a.vzeros + (tr.v + lane) * kNGroups);
#pragma unroll
    for (int hh = 0; hh < VB; ++hh) t.vc[hh] = *reinterpret_cast<const u32x4_t *>(vct + 1024 * hh + 16 * lane);
    return t;
  };
  // Any tile: rows clamped into [rmin, rmax] (a partial tile)
  auto load_tile = [&](int64_t r0, int64_t rmin, int64_t rmax) {
    const TileRows tr = tile_rows(a, b, hkv, krow0, vrow0, r0);
    const uint8_t *kc = a.kcodes + (tr.k - r0) * kKRow, *vc = a.vcodes + (tr.v - r0) * L::kRowBytes;
    const uint16_t *ks = a.kscales + (tr.k - r0) * kNGroups, *kz = a.kzeros + (tr.k - r0) * kNGroups;
    const uint16_t *vs = a.vscales + (tr.v - r0) * kNGroups, *vz = a.vzeros + (tr.v - r0) * kNGroups;
    auto clampr = [&](int64_t r) { return r < rmax ? (r > rmin ? r : rmin) : rmax; };
    MbTile<KB, VB> t;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int64_t r = clampr(r0 + 16 * k + tk);
      t.kc[k] = *reinterpret_cast<const KWord *>(kc + r * kKRow + (kKRow / 4) * kgrp);
    }
    {
      const int64_t r = clampr(r0 + lane);
      t.ks = *reinterpret_cast<const u32x2_t *>(ks + r * kNGroups);
      t.kz = *reinterpret_cast<const u32x2_t *>(kz + r * kNGroups);
      t.vs = *reinterpret_cast<const u32x2_t *>(vs + r * kNGroups);
      t.vz = *reinterpret_cast<const u32x2_t *>(vz + r * kNGroups);
    }
    // 16-byte piece hh of the tile's value rows: token (64/VB) hh + lane/VB,
    // bytes 16 (lane % VB) .. of its row
#pragma unroll
    for (int hh = 0; hh < VB; ++hh) {
      const int64_t r = clampr(r0 + (64 / VB) * hh + lane / VB);
      t.vc[hh] = *reinterpret_cast<const u32x4_t *>(vc + r * L::kRowBytes + 16 * (lane % VB));
    }
    return t;
  };

  // One tile whose tokens [lo, hi) are valid; big as in the 2-bit kernel
  // (value scales of 2^15 or more: entries from s/2, weights doubled; the
  // mode enters as wave-uniform factors).
  bool big = false;
  auto process = [&](const MbTile<KB, VB> &t, int lo, int hi) {
    if (!big && __builtin_amdgcn_ballot_w64(
                    (((t.vs.x + 0x08000800u) | (t.vs.y + 0x08000800u)) & 0x80008000u) != 0u))
      big = true;
    const float kB = big ? 2.0f : 1.0f;
    const _Float16 hb = big ? (_Float16)0.5f : (_Float16)1.0f, wb = big ? (_Float16)2.0f : (_Float16)1.0f;
    constexpr float kZ = VB == 4 ? 5.0f : 1.0f;    // planes: 1.5 s (1 + 4)
    {
      uint32_t *rl = rec + lane * kMbRecDwords;
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
          float4v_t{__builtin_fmaf(-kB * kZ, (float)n01.x, (float)z01.x),
                    __builtin_fmaf(-kB * kZ, (float)n01.y, (float)z01.y),
                    __builtin_fmaf(-kB * kZ, (float)n23.x, (float)z23.x),
                    __builtin_fmaf(-kB * kZ, (float)n23.y, (float)z23.y)};
#pragma unroll
      for (int hh = 0; hh < VB; ++hh) reinterpret_cast<u32x4_t *>(vcl)[64 * hh + lane] = t.vc[hh];
    }
    asm volatile("" ::: "memory");     // LDS of one wave is ordered; keep the program order
    // scores of the four 16-token blocks (lane: head gk, token 16k + tk)
    float raw[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int tt = 16 * k + tk;
      float4v_t d = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int p = 0; p < (KB == 4 ? 2 : 1); ++p) {   // 4 bits: code = lo + 4 hi
        const v8i_t Bop = mq_key_operand<KB>(t.kc[k], p);
#pragma unroll
        for (int Ld = 0; Ld < 4; ++Ld)
          d = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[Ld], Bop, d, 0, 4, 0, mq_scale(Ld), 0, 127 + 2 * p);
      }
      const u32x4_t kq = reinterpret_cast<const u32x4_t *>(rec + tt * kMbRecDwords)[0];
      const uint32_t kq0 = kq.x, kq1 = kq.y, kq2 = kq.z, kq3 = kq.w;
      const half2_t ks01 = __builtin_bit_cast(half2_t, kq0), ks23 = __builtin_bit_cast(half2_t, kq1);
      const half2_t kz01 = __builtin_bit_cast(half2_t, kq2), kz23 = __builtin_bit_cast(half2_t, kq3);
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
      const float alpha = __builtin_amdgcn_exp2f(st.m - mnew);
      st.l *= alpha;
#pragma unroll
      for (int j = 0; j < 4; ++j) st.zacc[j] *= alpha;
      st.o[0] *= alpha;
      st.o[1] *= alpha;
      st.m = mnew;
#pragma unroll
      for (int k = 0; k < 4; ++k) x[k] = y[k] - mnew;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int tt = 16 * k + tk;
      const _Float16 ph = (_Float16)__builtin_amdgcn_exp2f(x[k]);   // 0 for masked tokens
      const float pf = (float)ph;
      st.l += pf;
      const float4v_t zb = reinterpret_cast<const float4v_t *>(rec + tt * kMbRecDwords)[2];
      st.zacc[0] = __builtin_fmaf(pf, zb[0], st.zacc[0]);
      st.zacc[1] = __builtin_fmaf(pf, zb[1], st.zacc[1]);
      st.zacc[2] = __builtin_fmaf(pf, zb[2], st.zacc[2]);
      st.zacc[3] = __builtin_fmaf(pf, zb[3], st.zacc[3]);
      pw[gk * 64 + tt] = ph * wb;
    }
    asm volatile("" ::: "memory");
    // values: 8 blocks of 8 tokens; lane's tokens t0 = 8 tb + 2 kb and t0 + 1,
    // channels 8 vn .. 8 vn + 7 in the 2-bit layout (two bytes per token)
    const int jv = vn >> 2;
#pragma unroll
    for (int tb = 0; tb < 8; ++tb) {
      const int t0 = 8 * tb + 2 * vkb;
      uint32_t y[kPV];
      if constexpr (VB == 2) {
        y[0] = (uint32_t)*reinterpret_cast<const uint16_t *>(vcl + t0 * L::kRowBytes + 2 * vn) |
               ((uint32_t)*reinterpret_cast<const uint16_t *>(vcl + (t0 + 1) * L::kRowBytes + 2 * vn) << 16);
      } else if constexpr (VB == 1) {
        y[0] = mb_spread_pair(vcl[t0 * L::kRowBytes + vn], vcl[(t0 + 1) * L::kRowBytes + vn]);
      } else {
        const uint32_t w0 = *reinterpret_cast<const uint32_t *>(vcl + t0 * L::kRowBytes + 4 * vn);
        const uint32_t w1 = *reinterpret_cast<const uint32_t *>(vcl + (t0 + 1) * L::kRowBytes + 4 * vn);
#pragma unroll
        for (int p = 0; p < kPV; ++p) y[p] = mb_plane16(w0, p) | (mb_plane16(w1, p) << 16);
      }
      const uint32_t sv0 = rec[t0 * kMbRecDwords + 4 + jv];
      const uint32_t sv1 = rec[(t0 + 1) * kMbRecDwords + 4 + jv];
      const uint32_t P = *reinterpret_cast<const uint32_t *>(pw + ha * 64 + t0);
#pragma unroll
      for (int p = 0; p < kPV; ++p) {
        // the high plane's weights are 4 p~ (exact)
        const uint32_t Pp = p == 0 ? P
                                   : __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, P) *
                                                                      half2_t{(_Float16)4.0f, (_Float16)4.0f});
        v8h_t Aop;
        {
          const uint32_t a0 = __builtin_amdgcn_perm(Pp, Pp, selA[0]), a1 = __builtin_amdgcn_perm(Pp, Pp, selA[1]);
          const uint32_t a2 = __builtin_amdgcn_perm(Pp, Pp, selA[2]), a3 = __builtin_amdgcn_perm(Pp, Pp, selA[3]);
          const half2_t h0 = __builtin_bit_cast(half2_t, a0), h1 = __builtin_bit_cast(half2_t, a1);
          const half2_t h2 = __builtin_bit_cast(half2_t, a2), h3 = __builtin_bit_cast(half2_t, a3);
          Aop = half8_t{h0.x, h0.y, h1.x, h1.y, h2.x, h2.y, h3.x, h3.y};
        }
        const uint32_t y02 = y[p] & 0x33333333u, y13 = (y[p] >> 2) & 0x33333333u;
        st.o[0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Aop, mq_bvals<0>(y02, y13, sv0, sv1), st.o[0], 0, 0, 0);
        st.o[1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Aop, mq_bvals<1>(y02, y13, sv0, sv1), st.o[1], 0, 0, 0);
      }
    }
    asm volatile("" ::: "memory");
  };

  auto run = process;

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
    MbTile<KB, VB> t0 = load_full(row_of(0)), t1;
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
    int64_t p[2];
    ht.partial(a.skip, split, S, p[0], p[1]);
    for (int e = 0; e < 2; ++e) {
      if (p[e] < 0) continue;
      const int64_t base = 64 * p[e];
      const int lo = a.skip > base ? (int)(a.skip - base) : 0;
      const int hi = ht.n_tok - base < 64 ? (int)(ht.n_tok - base) : 64;
      const MbTile<KB, VB> t = load_tile(base, base + lo, base + hi - 1);
      run(t, lo, hi);
    }
  }

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

hipError_t launch_attn_gqa_bits(const AttnArgs &a, int kbits, int vbits, hipStream_t stream) {
  const dim3 grid((unsigned)((a.total_waves + kMqWaves - 1) / kMqWaves)), block(64 * kMqWaves);
#define KVQ_GQA_BITS_CASE(KB, VB)                                                      \
  if (kbits == KB && vbits == VB) {                                                    \
    hipLaunchKernelGGL((kv_quant_decode_attn_gqa<KB, VB>), grid, block, 0, stream, a); \
    return hipGetLastError();                                                          \
  }
  KVQ_GQA_BITS_CASE(1, 1) KVQ_GQA_BITS_CASE(1, 2) KVQ_GQA_BITS_CASE(1, 4)
  KVQ_GQA_BITS_CASE(2, 1) KVQ_GQA_BITS_CASE(2, 4)
  KVQ_GQA_BITS_CASE(4, 1) KVQ_GQA_BITS_CASE(4, 2) KVQ_GQA_BITS_CASE(4, 4)
#undef KVQ_GQA_BITS_CASE
  return hipErrorNotSupported;
}

}  // namespace kvq
