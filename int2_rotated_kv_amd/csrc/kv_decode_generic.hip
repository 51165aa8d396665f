// Decode attention over caches of other code widths: keys at KB bits and
// values at VB bits, each 1, 2 or 4 (the pair 2/2 has its own kernels).
//
// Mixed-bit KV caches are named as a direction on the OptR page (future-work
// paragraph); the codec is the library's b-bit generalization of the INT2
// format: L = 2^b - 1 levels above an fp16 zero in groups of 32 channels,
// 8/b codes per byte.  The attention is the same as for the INT2 cache
// (scaled dot product over dequantized rows in the rotated basis, the
// query rotated by R and the output un-rotated by R^T in the combine).
//
// One wave per (batch, query head, split).  The wave rotates and scales its
// query itself (none, Hadamard or reordered Hadamard; a dense R comes from
// the query preparation launch as a fixed point), as a 19-bit fixed point.
// Every 64-token tile gives one token to each lane for the softmax, and the
// wave shares a running maximum.
//   - Key scores run on the matrix cores: the fixed point's four balanced
//     base-32 digits as one fp8 operand (a digit per row block, its weight
//     in the E8M0 A scale) against the codes as fp4, then a sum across the
//     row blocks that leaves each lane its own token's group sums.
//   - Values: at 1- and 2-bit values on the matrix cores (VM), in the
//     operand layout of the grouped-query kernels' value step, with the
//     A rows given to the four value groups instead of four heads: row
//     (group g, position e) carries w = fp16(p s_g) of each token, B the
//     plain codes, so the scale costs nothing per code; at 4-bit values the
//     lane adds its token's weighted codes into 128 fp32 accumulators of its
//     own, summed at the end by a reduce-scatter over the 64 lanes.
// The wave writes the same partial (o', m, l) as the INT2 kernels, so the
// combine and un-rotation are shared.
#include "kv_decode_mq.h"

namespace kvq {

constexpr int kGenWaves = 4;

// Sum / max over the 64 lanes; every lane gets the result.
__device__ __forceinline__ float gen_wave_sum(float v) {
  v += quad_swap<kQuadXor1>(v);
  v += quad_swap<kQuadXor2>(v);
  v += row_ror<4>(v);
  v += row_ror<8>(v);
  return sum_xor32(sum_xor16(v));
}
__device__ __forceinline__ float gen_wave_max(float v) {
  v = fmaxf(v, quad_swap<kQuadXor1>(v));
  v = fmaxf(v, quad_swap<kQuadXor2>(v));
  v = fmaxf(v, row_ror<4>(v));
  v = fmaxf(v, row_ror<8>(v));
  return max_xor32(max_xor16(v));
}

// Code order of a b-bit row: dword j holds channels (32/b) j .. (32/b)(j+1) - 1,
// channel (32/b) j + P k + m (P = 8/b codes per byte) in byte k, field m.
// Reading the dword field by field, k fastest, gives index
// (32/b) j + 4 m + k; the channel of index i:
template <int BITS>
__host__ __device__ __forceinline__ constexpr int chan_of(int i) {
  constexpr int CPW = 32 / BITS, P = 8 / BITS;
  return CPW * (i / CPW) + P * (i % 4) + (i % CPW) / 4;
}

// One token's row of one side: 16*BITS code bytes, then the four fp16
// scales and zeros.
template <int BITS>
struct GenRow {
  u32x4_t w[BITS];
  u32x2_t s, z;
};

template <int BITS>
__device__ __forceinline__ GenRow<BITS> gen_load(const uint8_t *codes, const uint16_t *scales,
                                                 const uint16_t *zeros, int64_t row) {
  GenRow<BITS> r;
  const u32x4_t *cp = reinterpret_cast<const u32x4_t *>(codes + row * (16 * BITS));
#pragma unroll
  for (int k = 0; k < BITS; ++k) r.w[k] = cp[k];
  r.s = *reinterpret_cast<const u32x2_t *>(scales + row * kNGroups);
  r.z = *reinterpret_cast<const u32x2_t *>(zeros + row * kNGroups);
  return r;
}

// Code of index i (code order) of a row held as BITS x 4 dwords.
template <int BITS>
__device__ __forceinline__ float gen_code(const GenRow<BITS> &r, int i) {
  constexpr int CPW = 32 / BITS;
  constexpr uint32_t M = (1u << BITS) - 1u;
  const int j = i / CPW, m = (i % CPW) / 4, k = i % 4;
  const uint32_t w = r.w[j >> 2][j & 3];
  return (float)((w >> (8 * k + BITS * m)) & M);
}

__device__ __forceinline__ float gen_half(const u32x2_t &v, int g) {
  const uint32_t w = g < 2 ? v.x : v.y;
  return half_bits_to_float((uint16_t)((g & 1) ? (w >> 16) : (w & 0xFFFFu)));
}

// Matrix-core key scores: the 4 x 16 tokens of a tile as four B blocks of
// v_mfma_scale_f32_16x16x128_f8f6f4, lane (token 16 k + lane % 16, group
// lane / 16) of block k, the codes as fp4 (mq_key_operand, slot order
// mq_key_channel).

// x_k (k = 0..3) hold, in lane (row block j, n), the part of row j of
// block k.  Returns in lane (r, n) the sum over j of block r's rows: row
// blocks 2,3 of x0 / x1 trade places with rows 0,1 of x2 / x3 and the
// halves add (rows j and j + 2 meet), then the odd rows of the first sum
// trade with the even rows of the second and add (rows j and j + 1 meet).
__device__ __forceinline__ float ms_digit_sum(float x0, float x1, float x2, float x3) {
  const auto a = __builtin_amdgcn_permlane32_swap(float_as_bits(x0), float_as_bits(x2), false, false);
  const float u02 = bits_as_float(a[0]) + bits_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(float_as_bits(x1), float_as_bits(x3), false, false);
  const float u13 = bits_as_float(b[0]) + bits_as_float(b[1]);
  const auto c = __builtin_amdgcn_permlane16_swap(float_as_bits(u02), float_as_bits(u13), false, false);
  return bits_as_float(c[0]) + bits_as_float(c[1]);
}

// A tile's keys for the matrix-core scores: the code words of block k and
// the scale / zero of the lane's own token.
template <int KB>
struct MsKeys {
  typename MbKeyWord<KB>::type kc[4];
  u32x2_t s, z;
};

// Rows r0 + t of a tile; tokens outside [lo, hi) read row r0 + lo.
template <int KB>
__device__ __forceinline__ MsKeys<KB> ms_load(const AttnArgs &a, int64_t r0, int lo, int hi) {
  constexpr int kRow = 16 * KB;
  typedef typename MbKeyWord<KB>::type KWord;
  const int lane = threadIdx.x & 63, tk = lane & 15, kg = lane >> 4;
  MsKeys<KB> r;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int t = 16 * k + tk;
    const int64_t row = r0 + (t >= lo && t < hi ? t : lo);
    r.kc[k] = *reinterpret_cast<const KWord *>(a.kcodes + row * kRow + (kRow / 4) * kg);
  }
  const int64_t row = r0 + (lane >= lo && lane < hi ? lane : lo);
  r.s = *reinterpret_cast<const u32x2_t *>(a.kscales + row * kNGroups);
  r.z = *reinterpret_cast<const u32x2_t *>(a.kzeros + row * kNGroups);
  return r;
}

// Waves per SIMD the register budget is held to: three with the matrix-core
// value step (132-156 registers without spills; the tighter allocation
// measured 1-4% faster even at two resident waves), one with the fp32 value
// step.
template <int KB, int VB, bool VM>
constexpr int gen_min_waves() { return VM ? 3 : 1; }

// grid: ceil(total_waves / 4) blocks of 4 waves; wave index as in
// wave_place with one wave per query head (`per` = G).
template <int KB, int VB, bool VM>
__global__ __launch_bounds__(64 * kGenWaves, (gen_min_waves<KB, VB, VM>())) void kv_quant_decode_attn(AttnArgs a) {
  // the query as a 19-bit fixed point, and its group sums
  __shared__ int32_t qi_all[kGenWaves][kD];
  __shared__ float qsum_all[kGenWaves][4];
  // value step on the matrix cores: the tile's value rows and the fp16
  // weights w = fp16(p s_g), [group][token]
  constexpr int kVRow = 16 * VB;
  __shared__ __attribute__((aligned(16))) uint8_t vcl_all[VM ? kGenWaves : 1][VM ? 64 * kVRow : 16];
  __shared__ __attribute__((aligned(16))) _Float16 pw_all[VM ? kGenWaves : 1][VM ? 4 * 64 : 8];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t gw = (int64_t)blockIdx.x * kGenWaves + wave;
  WavePlace wp;
  if (!wave_place(a, gw, a.G, wp)) return;          // whole wave leaves; no barrier follows
  const int64_t b = wp.b, split = wp.split, S = wp.S;
  const int hkv = wp.hkv;
  const int hq = hkv * a.G + wp.sub;
  const int64_t bh = b * a.Hkv + hkv;
  float qstep;                                        // weight of one qi unit

  // ---- query: q' = qscale * q R, lane l holding channels 2l and 2l + 1
  {
    int q0i, q1i;
    if (a.rot == 2) {
      // dense R: the query preparation launch has written the fixed point
      // (same exponent rule as below) and its step
      const int32_t *qp = reinterpret_cast<const int32_t *>(a.qprep) + (b * a.Hq + hq) * kQprepDwordsPerHead;
      q0i = qp[kQprepFixedOffset + 2 * lane];
      q1i = qp[kQprepFixedOffset + 2 * lane + 1];
      qstep = bits_as_float((uint32_t)qp[25]);
    } else {
    const int64_t qoff = (b * a.Hq + hq) * kD;
    int c0 = 2 * lane, c1 = 2 * lane + 1;
    if (a.rot == 3) {                                // (q_pi)_j = q[pi(j)]
      c0 = a.perm[(int64_t)hkv * kD + c0] & (kD - 1);
      c1 = a.perm[(int64_t)hkv * kD + c1] & (kD - 1);
    }
    float x0, x1;
    if (a.q_f32) {
      x0 = reinterpret_cast<const float *>(a.q)[qoff + c0];
      x1 = reinterpret_cast<const float *>(a.q)[qoff + c1];
    } else {
      x0 = (float)reinterpret_cast<const _Float16 *>(a.q)[qoff + c0];
      x1 = (float)reinterpret_cast<const _Float16 *>(a.q)[qoff + c1];
    }
    float scale = a.qscale;
    if (a.rot == 1 || a.rot == 3) {
      // unnormalized Walsh-Hadamard transform: stride 1 inside the lane,
      // strides 2 .. 64 across lanes (lane distance 1 .. 32)
      const float s0 = x0 + x1, d0 = x0 - x1;
      x0 = s0;
      x1 = d0;
#pragma unroll
      for (int m = 1; m < 64; m <<= 1) {
        const float p0 = __shfl_xor(x0, m, 64), p1 = __shfl_xor(x1, m, 64);
        const bool upper = (lane & m) != 0;
        x0 = upper ? p0 - x0 : x0 + p0;
        x1 = upper ? p1 - x1 : x1 + p1;
      }
      scale *= 0.08838834764831845f;                 // 1/sqrt(128)
    }
    x0 *= scale;
    x1 *= scale;
    // qi = rint(q' 2^E) with |qi| < 2^18 for the head's largest |q'|; the
    // group sums of qi c are integers, exact in fp32 below 2^24 and rounded
    // once above (relative 2^-24), so the fixed-point rounding (below 2^-18
    // of the largest |q'|) is the scores' main approximation
    const float amax = gen_wave_max(fmaxf(fabsf(x0), fabsf(x1)));
    // amax = m 2^e with m in [0.5, 1): E = 18 - e puts amax 2^E in [2^17, 2^18)
    const int E = amax > 0.0f ? 18 - __builtin_amdgcn_frexp_expf(amax) : 0;
    qstep = __builtin_amdgcn_ldexpf(1.0f, -E);
    q0i = (int)__builtin_rintf(__builtin_amdgcn_ldexpf(x0, E));
    q1i = (int)__builtin_rintf(__builtin_amdgcn_ldexpf(x1, E));
    }
    float gs = (float)q0i + (float)q1i;               // group g = lane / 16, exact
    qi_all[wave][2 * lane] = q0i;
    qi_all[wave][2 * lane + 1] = q1i;
    gs += quad_swap<kQuadXor1>(gs);
    gs += quad_swap<kQuadXor2>(gs);
    gs += row_ror<4>(gs);
    gs += row_ror<8>(gs);
    if ((lane & 15) == 0) qsum_all[wave][lane >> 4] = gs;
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // this wave's LDS writes are done
  float qsum[4];                                      // sum of qi over each group
#pragma unroll
  for (int g = 0; g < 4; ++g) qsum[g] = qsum_all[wave][g];
  // Key scores: one fp8 operand for the four digits of the fixed point.  A row
  // (block jr, group ja) holds digit L(jr) of group ja's channels (zero in
  // the other groups' slots), and the lane's E8M0 A scale is that digit's
  // weight 2^(5 (3 - L)).  Rows 0 and 2 carry digits 0 and 1, rows 1 and 3
  // digits 2 and 3, so that the first pairwise sums across the row blocks
  // (below) add digits of neighbouring weight and stay exact.
  v8i_t Aq;
  int sa;
  {
    const int32_t *qi = qi_all[wave];
    const int ja = lane & 3, jr = (lane & 15) >> 2, kba = lane >> 4;
    const int Ld = (jr >> 1) | ((jr & 1) << 1);
    sa = mq_scale(Ld);
    // bytes 0..15: slots 16 kba + i (group kba / 2); bytes 16..31: slots
    // 64 + 16 kba + i (group 2 + kba / 2); only the half in group ja is nonzero
    const bool lo_on = (kba >> 1) == ja, hi_on = 2 + (kba >> 1) == ja;
    const int kbase = hi_on ? 64 + 16 * kba : 16 * kba;
    int dw[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      int d4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) d4[e] = (lo_on || hi_on) ? mq_digit(qi[mq_key_channel<KB>(kbase + 4 * w + e)], Ld) : 0;
      int v = __builtin_amdgcn_cvt_pk_fp8_f32((float)d4[0], (float)d4[1], 0, false);
      dw[w] = __builtin_amdgcn_cvt_pk_fp8_f32((float)d4[2], (float)d4[3], v, true);
    }
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      Aq[w] = lo_on ? dw[w] : 0;
      Aq[4 + w] = hi_on ? dw[w] : 0;
    }
  }

  float acc[VM ? 1 : kD];                             // value accumulators, value-code order
#pragma unroll
  for (int i = 0; i < (VM ? 1 : kD); ++i) acc[i] = 0.0f;
  // matrix-core value step: lane (byte pair vn, token pair vkb) of B; lane
  // (group ga = vn / 4, position e = vn % 4, vkb) of A.  The A dword d holds
  // token 2 vkb + d / 2 at positions (d % 2, d % 2 + 2); v_perm selectors
  // pick that token's weight into the half of position e, or zero.
  float4v_t o[2] = {float4v_t{0.0f, 0.0f, 0.0f, 0.0f}, float4v_t{0.0f, 0.0f, 0.0f, 0.0f}};
  const int vn = lane & 15, vkb = lane >> 4, ga = vn >> 2;
  uint32_t selA[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const int ve = vn & 3;
    const uint32_t src = (d >> 1) ? 0x0706u : 0x0504u;
    const bool on = (d & 1) == (ve & 1);
    selA[d] = !on ? 0x0C0C0C0Cu : (ve >> 1) ? ((src << 16) | 0x0C0Cu) : (0x0C0C0000u | src);
  }
  float zacc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  float l = 0.0f, m_run = kNegInf;

  const int64_t krow0 = bh * a.kT_cap + a.t_begin - a.skip;   // row 0 of the shifted grid
  const int64_t vrow0 = bh * a.vT_cap + a.t_begin - a.skip;

  // matrix-core value step: the weights carry the wave's value pre-scale
  // 2^kx (normal fp16 numbers below 2^15 for every finite scale), and so
  // does o; the fp32 step needs none
  ValuePrescale ps = prescale_init();
  auto token = [&](const auto &kr, const GenRow<VB> &vr, bool valid) {
    float s = 0.0f;
    {
      // block k (tokens 16 k .. 16 k + 15): lane (row block jr, token n) gets
      // digit L(jr)'s part of (1/2) sum qi c for each group of token 16 k + n
      float4v_t d[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        d[k] = float4v_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int p = 0; p < (KB == 4 ? 2 : 1); ++p)   // 4 bits: code = lo + 4 hi
          d[k] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(Aq, mq_key_operand<KB>(kr.kc[k], p), d[k], 0, 4, 0,
                                                                  sa, 0, 127 + 2 * p);
      }
      // sum over the digit rows with the blocks spread over the row blocks:
      // lane (r, n) ends with the group sums of token 16 r + n, its own
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float dot = 2.0f * ms_digit_sum(d[0][g], d[1][g], d[2][g], d[3][g]);   // sum qi c
        s = __builtin_fmaf(gen_half(kr.s, g), dot, __builtin_fmaf(gen_half(kr.z, g), qsum[g], s));
      }
    }
    s *= qstep;
    s = valid ? s : kNegInf;
    const float mt = gen_wave_max(s);
    if (mt > m_run + kSlack) {                         // wave-uniform
      const float f = __builtin_amdgcn_exp2f(m_run - mt);
#pragma unroll
      for (int i = 0; i < (VM ? 1 : kD); ++i) acc[i] *= f;
      o[0] *= f;
      o[1] *= f;
#pragma unroll
      for (int g = 0; g < 4; ++g) zacc[g] *= f;
      l *= f;
      m_run = mt;
    }
    const float p = valid ? __builtin_amdgcn_exp2f(s - m_run) : 0.0f;
    if constexpr (!VM) {
      l += p;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float pv = p * gen_half(vr.s, g);
        zacc[g] = __builtin_fmaf(p, gen_half(vr.z, g), zacc[g]);
#pragma unroll
        for (int i = 0; i < 32; ++i)
          acc[32 * g + i] = __builtin_fmaf(pv, gen_code<VB>(vr, 32 * g + i), acc[32 * g + i]);
      }
    } else {
      // Weights w_g = fp16(p~ s_g 2^kx) with p~ = fp16(p), B entries the
      // plain codes over the 2-bit layout (1-bit codes spread to 2-bit
      // fields).  Centered on c = (2^VB - 1) / 2:
      // o' = 2^-kx (sum w code - c sum w) + sum p~ (z + c s), so the rounding
      // of w multiplies code - c; the last two terms are accumulated per
      // token lane, without the pre-scale.
      static_assert(VB == 1 || VB == 2, "matrix-core value step: 1- and 2-bit values");
      constexpr float kC = 0.5f * (float)((1 << VB) - 1);
      uint8_t *vcl = vcl_all[wave];
      _Float16 *pw = pw_all[wave];
      const _Float16 ph = (_Float16)p;
      const float pf = (float)ph;
      l += pf;
      // vector elements are copied out before the bit casts: hipcc lowers a
      // bit cast of an element such as vr.s.y as a read of the vector's first
      // element
      const uint32_t vs0 = vr.s.x, vs1 = vr.s.y, vz0 = vr.z.x, vz1 = vr.z.y;
      {
        // a value scale beyond the wave's pre-scale: lower it (wave-uniform, rare)
        const uint32_t mb = max_half_bits(vs0, vs1);
        if (__builtin_amdgcn_ballot_w64(mb >= ps.lim)) {
          const float f = prescale_lower(ps, mb);
          o[0] *= f;
          o[1] *= f;
        }
      }
      const half2_t s01 = __builtin_bit_cast(half2_t, vs0), s23 = __builtin_bit_cast(half2_t, vs1);
      const half2_t z01 = __builtin_bit_cast(half2_t, vz0), z23 = __builtin_bit_cast(half2_t, vz1);
      const float sg[4] = {(float)s01.x, (float)s01.y, (float)s23.x, (float)s23.y};
      const float zg[4] = {(float)z01.x, (float)z01.y, (float)z23.x, (float)z23.y};
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const _Float16 w = (_Float16)(pf * (sg[g] * ps.f));
        zacc[g] = __builtin_fmaf(pf, __builtin_fmaf(kC, sg[g], zg[g]), __builtin_fmaf(-kC * ps.inv, (float)w, zacc[g]));
        pw[64 * g + lane] = w;
      }
#pragma unroll
      for (int k = 0; k < VB; ++k) reinterpret_cast<u32x4_t *>(vcl + lane * kVRow)[k] = vr.w[k];
      asm volatile("" ::: "memory");                   // LDS of one wave is ordered; keep the program order
#pragma unroll
      for (int tb = 0; tb < 8; ++tb) {
        const int t0 = 8 * tb + 2 * vkb;
        // byte pair vn of tokens t0 and t0 + 1 in the 2-bit layout
        const uint32_t y =
            VB == 2 ? ((uint32_t)*reinterpret_cast<const uint16_t *>(vcl + t0 * kVRow + 2 * vn) |
                       ((uint32_t)*reinterpret_cast<const uint16_t *>(vcl + (t0 + 1) * kVRow + 2 * vn) << 16))
                    : mb_spread_pair(vcl[t0 * kVRow + vn], vcl[(t0 + 1) * kVRow + vn]);
        const uint32_t P = *reinterpret_cast<const uint32_t *>(pw + 64 * ga + t0);
        v8h_t Aop;
        {
          const uint32_t a0 = __builtin_amdgcn_perm(P, P, selA[0]), a1 = __builtin_amdgcn_perm(P, P, selA[1]);
          const uint32_t a2 = __builtin_amdgcn_perm(P, P, selA[2]), a3 = __builtin_amdgcn_perm(P, P, selA[3]);
          const half2_t h0 = __builtin_bit_cast(half2_t, a0), h1 = __builtin_bit_cast(half2_t, a1);
          const half2_t h2 = __builtin_bit_cast(half2_t, a2), h3 = __builtin_bit_cast(half2_t, a3);
          Aop = half8_t{h0.x, h0.y, h1.x, h1.y, h2.x, h2.y, h3.x, h3.y};
        }
        const uint32_t y02 = y & 0x33333333u, y13 = (y >> 2) & 0x33333333u;
        o[0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Aop, mq_bcodes<0>(y02, y13), o[0], 0, 0, 0);
        o[1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Aop, mq_bcodes<1>(y02, y13), o[1], 0, 0, 0);
      }
      asm volatile("" ::: "memory");                   // the next tile's writes come after these reads
    }
  };
  auto run = token;


  const HeadTiles ht(seq_int2(a, b), a.skip, split, S);
  if (ht.mine > 0) {
    // a tile's rows follow its first row (one page holds the whole tile)
    PagedTileRows pages;
    auto full_rows = [&](int64_t i) {
      if (a.block_table == nullptr) {
        const int64_t r = ht.full_row(i, split, S);
        return TileRows{krow0 + r, vrow0 + r};
      }
      const int64_t r = pages.row(a, b, hkv, ht, split, S, i);
      return TileRows{r, r};
    };
    auto lk = [&](const TileRows &t) {
      return ms_load<KB>(a, t.k, 0, 64);
    };
    auto lv = [&](const TileRows &t) { return gen_load<VB>(a.vcodes, a.vscales, a.vzeros, t.v + lane); };
    if constexpr (KB != 4 && VB != 4) {
      // narrow rows leave registers for a three-deep pipeline: while tile i
      // is computed the loads of tiles i + 1 and i + 2 are in flight (2-5%
      // faster than one tile ahead); prefetches past the wave's last tile
      // re-read it
      TileRows t = full_rows(0);
      auto k0 = lk(t);
      auto v0 = lv(t);
      t = full_rows(1);
      auto k1 = lk(t);
      auto v1 = lv(t);
      decltype(k0) k2;
      decltype(v0) v2;
      int64_t i = 0;
      for (; i + 3 <= ht.mine; i += 3) {
        t = full_rows(i + 2);
        k2 = lk(t);
        v2 = lv(t);
        run(k0, v0, true);
        t = full_rows(i + 3);
        k0 = lk(t);
        v0 = lv(t);
        run(k1, v1, true);
        t = full_rows(i + 4);
        k1 = lk(t);
        v1 = lv(t);
        run(k2, v2, true);
      }
      if (i < ht.mine) run(k0, v0, true);
      if (i + 1 < ht.mine) run(k1, v1, true);
    } else {
      const TileRows t0 = full_rows(0);
      auto kr = lk(t0);
      GenRow<VB> vr = lv(t0);
      for (int64_t i = 0; i < ht.mine; ++i) {
        // the next tile's rows are loaded while this one is computed (the
        // last prefetch re-reads the wave's last tile)
        const TileRows tn = full_rows(i + 1);
        const auto kn = lk(tn);
        const GenRow<VB> vn = lv(tn);
        run(kr, vr, true);
        kr = kn;
        vr = vn;
      }
    }
  }
  {
    // partial tiles: masked rows are loaded from the tile's first valid row
    int64_t p[2];
    ht.partial(a.skip, split, S, p[0], p[1]);
    for (int e = 0; e < 2; ++e) {
      if (p[e] < 0) continue;
      const int64_t base = 64 * p[e];
      const int64_t lo = a.skip > base ? a.skip - base : 0;
      const int64_t hi = ht.n_tok - base < 64 ? ht.n_tok - base : 64;
      const bool valid = lane >= lo && lane < hi;
      const int64_t r = valid ? lane : lo;
      const TileRows tr = tile_rows(a, b, hkv, krow0, vrow0, base);
      const GenRow<VB> vr = gen_load<VB>(a.vcodes, a.vscales, a.vzeros, tr.v + r);
      run(ms_load<KB>(a, tr.k, (int)lo, (int)hi), vr, valid);
    }
  }

  // ---- reduce over the 64 token lanes and write the partial
  l = gen_wave_sum(l);
#pragma unroll
  for (int g = 0; g < 4; ++g) zacc[g] = gen_wave_sum(zacc[g]);
  float *dst = a.partials + partial_row(a, wp, hq) * kPartialStride;
  if constexpr (VM) {
    // lane 16 g + vn holds the rows of group g for byte columns 2 vn and
    // 2 vn + 1, channels 8 vn .. 8 vn + 7, which lie in group vn / 4: the
    // lanes with g = vn / 4 hold the result
    if ((lane >> 4) == ga) {
      const float zl = ga == 0 ? zacc[0] : ga == 1 ? zacc[1] : ga == 2 ? zacc[2] : zacc[3];
      const float4v_t z4 = {zl, zl, zl, zl};
      const float4v_t u4 = {ps.inv, ps.inv, ps.inv, ps.inv};
      reinterpret_cast<float4v_t *>(dst + 8 * vn)[0] = o[0] * u4 + z4;
      reinterpret_cast<float4v_t *>(dst + 8 * vn)[1] = o[1] * u4 + z4;
    }
    if (lane == 0) {
      dst[128] = m_run;
      dst[129] = l;
    }
    return;
  }
  // reduce-scatter: at the step with lane mask M a lane keeps the half of
  // its values whose index bit matches its lane bit and adds the partner's
  // copy of that half; after six steps lane l holds indices 2l and 2l + 1
#pragma unroll
  for (int step = 0; step < 6; ++step) {
    const int M = 32 >> step;                          // lane mask
    const int half = 64 >> step;                       // values kept after this step
    const bool upper = (lane & M) != 0;
#pragma unroll
    for (int i = 0; i < half; ++i) {
      const float keep = upper ? acc[half + i] : acc[i];
      const float send = upper ? acc[i] : acc[half + i];
      acc[i] = keep + __shfl_xor(send, M, 64);
    }
  }
  const float zl = (lane >> 4) == 0 ? zacc[0] : (lane >> 4) == 1 ? zacc[1] : (lane >> 4) == 2 ? zacc[2] : zacc[3];
  // the value at index 2l + e (value-code order) belongs to channel chan_of(2l + e)
  dst[chan_of<VB>(2 * lane)] = acc[0] + zl;
  dst[chan_of<VB>(2 * lane + 1)] = acc[1] + zl;
  if (lane == 0) {
    dst[128] = m_run;
    dst[129] = l;
  }
}

// The matrix-core value step at 1- and 2-bit values; 4-bit values keep the
// fp32 step.
template <int VB>
constexpr bool gen_value_mfma() { return VB != 4; }
hipError_t launch_attn_generic(const AttnArgs &a, int kbits, int vbits, hipStream_t stream) {
  const dim3 grid((unsigned)((a.total_waves + kGenWaves - 1) / kGenWaves)), block(64 * kGenWaves);
#define KVQ_GEN_CASE(KB, VB)                                                                  \
  if (kbits == KB && vbits == VB) {                                                           \
    constexpr bool kVm = gen_value_mfma<VB>();                                                \
    hipLaunchKernelGGL((kv_quant_decode_attn<KB, VB, kVm>), grid, block, 0, stream, a);       \
    return hipGetLastError();                                                                 \
  }
  // 2-bit keys and values take the INT2 kernels
  KVQ_GEN_CASE(1, 1) KVQ_GEN_CASE(1, 2) KVQ_GEN_CASE(1, 4)
  KVQ_GEN_CASE(2, 1) KVQ_GEN_CASE(2, 4)
  KVQ_GEN_CASE(4, 1) KVQ_GEN_CASE(4, 2) KVQ_GEN_CASE(4, 4)
#undef KVQ_GEN_CASE
  return hipErrorNotSupported;
}

}  // namespace kvq
