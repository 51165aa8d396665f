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
// the query preparation launch as a fixed point) and keeps it in LDS as
// a 19-bit fixed point in five 4-bit limbs, laid out in the nibble order of
// the key codes.  Every 64-token tile gives one token to each lane: the lane
// scores its token with v_dot8_i32_i4 on the key codes, the wave shares a
// running maximum, and the lane adds its token's weighted value codes into
// 128 accumulators of its own.  At the end the 64 lanes' accumulators are
// summed by a reduce-scatter that leaves two channels in each lane, and the
// wave writes the same partial (o', m, l) as the INT2 kernels, so the
// combine and un-rotation are shared.
#include "kv_decode_common.h"

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

// Key codes as signed nibbles for v_dot8_i32_i4.  Limb dword u (0..15) of a
// b-bit row is code dword j = u / (4/b), shifted right by b (u mod 4/b) and
// masked to b bits per nibble: nibble h then holds the code of channel
// (32/b) j + (4/b) h + (u mod 4/b).  4-bit codes are flipped in their top bit,
// so that the signed nibble reads c - 8.
template <int BITS>
__host__ __device__ __forceinline__ constexpr int nib_pos(int c) {   // 8 u + h of channel c
  constexpr int CPW = 32 / BITS, SUB = 4 / BITS;
  return 8 * ((c / CPW) * SUB + (c % CPW) % SUB) + (c % CPW) / SUB;
}
template <int BITS>
__device__ __forceinline__ uint32_t key_nibbles(const GenRow<BITS> &r, int u) {
  constexpr int SUB = 4 / BITS;
  const int j = u / SUB;
  const uint32_t w = r.w[j >> 2][j & 3];
  if constexpr (BITS == 4) return w ^ 0x88888888u;
  else if constexpr (BITS == 2) return (w >> (2 * (u % SUB))) & 0x33333333u;
  else return (w >> (u % SUB)) & 0x11111111u;
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

// grid: ceil(total_waves / 4) blocks of 4 waves; wave index as in
// wave_place with one wave per query head (`per` = G).
template <int KB, int VB>
__global__ __launch_bounds__(64 * kGenWaves) void kv_quant_decode_attn(AttnArgs a) {
  // the query as a 19-bit fixed point in five signed 4-bit limbs: limb L,
  // nibble 8u + h at the position of the key nibble it multiplies (nib_pos);
  // nibbles staged one per byte first, then packed; group sums of qi last
  __shared__ __attribute__((aligned(16))) uint32_t ql_all[kGenWaves][5][16];
  __shared__ uint8_t qn_all[kGenWaves][5][kD];
  __shared__ float qsum_all[kGenWaves][4];
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
    // scores are then exact integer dot products of qi with the codes, and
    // the fixed-point rounding (below 2^-18 of the largest |q'|) is their
    // only approximation
    const float amax = gen_wave_max(fmaxf(fabsf(x0), fabsf(x1)));
    // amax = m 2^e with m in [0.5, 1): E = 18 - e puts amax 2^E in [2^17, 2^18)
    const int E = amax > 0.0f ? 18 - __builtin_amdgcn_frexp_expf(amax) : 0;
    qstep = __builtin_amdgcn_ldexpf(1.0f, -E);
    q0i = (int)__builtin_rintf(__builtin_amdgcn_ldexpf(x0, E));
    q1i = (int)__builtin_rintf(__builtin_amdgcn_ldexpf(x1, E));
    }
    float gs = (float)q0i + (float)q1i;               // group g = lane / 16, exact
    uint8_t(*qn)[kD] = qn_all[wave];
#pragma unroll
    for (int L = 0; L < 5; ++L) {                     // balanced base-16 digits
      const int d0 = ((q0i + 8) & 15) - 8, d1 = ((q1i + 8) & 15) - 8;
      q0i = (q0i - d0) >> 4;
      q1i = (q1i - d1) >> 4;
      qn[L][nib_pos<KB>(2 * lane)] = (uint8_t)(d0 & 15);
      qn[L][nib_pos<KB>(2 * lane + 1)] = (uint8_t)(d1 & 15);
    }
    gs += quad_swap<kQuadXor1>(gs);
    gs += quad_swap<kQuadXor2>(gs);
    gs += row_ror<4>(gs);
    gs += row_ror<8>(gs);
    if ((lane & 15) == 0) qsum_all[wave][lane >> 4] = gs;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // this wave's LDS writes are done
    uint8_t *lb = reinterpret_cast<uint8_t *>(ql_all[wave]);
#pragma unroll
    for (int L = 0; L < 5; ++L) lb[64 * L + lane] = (uint8_t)(qn[L][2 * lane] | (qn[L][2 * lane + 1] << 4));
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  float qsum[4];                                      // sum of qi over each group
#pragma unroll
  for (int g = 0; g < 4; ++g) qsum[g] = qsum_all[wave][g];

  float acc[kD];                                      // value accumulators, value-code order
#pragma unroll
  for (int i = 0; i < kD; ++i) acc[i] = 0.0f;
  float zacc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  float l = 0.0f, m_run = kNegInf;

  const int64_t krow0 = bh * a.kT_cap + a.t_begin - a.skip;   // row 0 of the shifted grid
  const int64_t vrow0 = bh * a.vT_cap + a.t_begin - a.skip;

  auto token = [&](const GenRow<KB> &kr, const GenRow<VB> &vr, bool valid) {
    // The query limbs are re-read from LDS for every token: a query held
    // in registers leaves one wave per SIMD (measured 12-19% slower).
    asm volatile("" ::: "memory");
    // per group: sum qi c from v_dot8_i32_i4, one accumulator per limb
    // (4-bit codes read as c - 8, so + 8 sum qi restores sum qi c)
    float s = 0.0f;
    const uint32_t *ql = &ql_all[wave][0][0];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      int acc5[5] = {0, 0, 0, 0, 0};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int kn = (int)key_nibbles<KB>(kr, 4 * g + e);
#pragma unroll
        for (int L = 0; L < 5; ++L) acc5[L] = __builtin_amdgcn_sdot8((int)ql[16 * L + 4 * g + e], kn, acc5[L], false);
      }
      const int v = acc5[0] + (acc5[1] << 4) + (acc5[2] << 8) + (acc5[3] << 12) + (acc5[4] << 16);
      const float dot = KB == 4 ? (float)v + 8.0f * qsum[g] : (float)v;   // exact in fp32 (< 2^24)
      s = __builtin_fmaf(gen_half(kr.s, g), dot, __builtin_fmaf(gen_half(kr.z, g), qsum[g], s));
    }
    s *= qstep;
    s = valid ? s : kNegInf;
    const float mt = gen_wave_max(s);
    if (mt > m_run + kSlack) {                         // wave-uniform
      const float f = __builtin_amdgcn_exp2f(m_run - mt);
#pragma unroll
      for (int i = 0; i < kD; ++i) acc[i] *= f;
#pragma unroll
      for (int g = 0; g < 4; ++g) zacc[g] *= f;
      l *= f;
      m_run = mt;
    }
    const float p = valid ? __builtin_amdgcn_exp2f(s - m_run) : 0.0f;
    l += p;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float pv = p * gen_half(vr.s, g);
      zacc[g] = __builtin_fmaf(p, gen_half(vr.z, g), zacc[g]);
#pragma unroll
      for (int i = 0; i < 32; ++i) acc[32 * g + i] = __builtin_fmaf(pv, gen_code<VB>(vr, 32 * g + i), acc[32 * g + i]);
    }
  };

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
    const TileRows t0 = full_rows(0);
    GenRow<KB> kr = gen_load<KB>(a.kcodes, a.kscales, a.kzeros, t0.k + lane);
    GenRow<VB> vr = gen_load<VB>(a.vcodes, a.vscales, a.vzeros, t0.v + lane);
    for (int64_t i = 0; i < ht.mine; ++i) {
      // the next tile's rows are loaded while this one is computed (the
      // last prefetch re-reads the wave's last tile)
      const TileRows tn = full_rows(i + 1);
      const GenRow<KB> kn = gen_load<KB>(a.kcodes, a.kscales, a.kzeros, tn.k + lane);
      const GenRow<VB> vn = gen_load<VB>(a.vcodes, a.vscales, a.vzeros, tn.v + lane);
      token(kr, vr, true);
      kr = kn;
      vr = vn;
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
      token(gen_load<KB>(a.kcodes, a.kscales, a.kzeros, tr.k + r),
            gen_load<VB>(a.vcodes, a.vscales, a.vzeros, tr.v + r), valid);
    }
  }

  // ---- reduce over the 64 token lanes and write the partial
  l = gen_wave_sum(l);
#pragma unroll
  for (int g = 0; g < 4; ++g) zacc[g] = gen_wave_sum(zacc[g]);
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
  float *dst = a.partials + partial_row(a, wp, hq) * kPartialStride;
  const float zl = (lane >> 4) == 0 ? zacc[0] : (lane >> 4) == 1 ? zacc[1] : (lane >> 4) == 2 ? zacc[2] : zacc[3];
  // the value at index 2l + e (value-code order) belongs to channel chan_of(2l + e)
  dst[chan_of<VB>(2 * lane)] = acc[0] + zl;
  dst[chan_of<VB>(2 * lane + 1)] = acc[1] + zl;
  if (lane == 0) {
    dst[128] = m_run;
    dst[129] = l;
  }
}

hipError_t launch_attn_generic(const AttnArgs &a, int kbits, int vbits, hipStream_t stream) {
  const dim3 grid((unsigned)((a.total_waves + kGenWaves - 1) / kGenWaves)), block(64 * kGenWaves);
#define KVQ_GEN_CASE(KB, VB)                                                       \
  if (kbits == KB && vbits == VB) {                                                \
    hipLaunchKernelGGL((kv_quant_decode_attn<KB, VB>), grid, block, 0, stream, a); \
    return hipGetLastError();                                                      \
  }
  KVQ_GEN_CASE(1, 1) KVQ_GEN_CASE(1, 2) KVQ_GEN_CASE(1, 4)
  KVQ_GEN_CASE(2, 1) KVQ_GEN_CASE(2, 2) KVQ_GEN_CASE(2, 4)
  KVQ_GEN_CASE(4, 1) KVQ_GEN_CASE(4, 2) KVQ_GEN_CASE(4, 4)
#undef KVQ_GEN_CASE
  return hipErrorNotSupported;
}

}  // namespace kvq
