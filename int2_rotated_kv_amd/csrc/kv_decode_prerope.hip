// Scores for keys cached with the pre-RoPE grouped-head rotation (RotateKV,
// IJCAI 2025 record, abstract item (ii): keys are rotated before the rotary
// position embedding, across a group of heads).
//
// The cache holds, for each token, the Hadamard rotation over the channels
// of GH consecutive KV heads of the keys before RoPE, quantized like any
// other row.  RoPE turns channel pairs (i, i + 64) by angles that depend on
// the token's position, so it does not commute with the rotation: the key
// of every token has to be brought back to the original basis and embedded
// at its own position before the dot product with the (position-embedded)
// query.  This kernel does that for every INT2 token and writes the scores,
// in log2 units, to the workspace; the split-K attention then reads them in
// place of its own key scores (its values and merge are unchanged).
//
// Un-rotation.  With the head index as the high bits, the rotation over GH
// heads is H_GH x H_4 x H_32 (Sylvester), with the 32-channel quantization
// group as the H_4 index.  Per head and per group G, D_G = H_32 C_G (C_G the
// group's 2-bit codes of 16 tokens) runs on the matrix cores:
// v_mfma_scale_f32_16x16x128_f8f6f4 with fp4 operands, A = +-1 rows of H_32
// in the K slots of group G (zero elsewhere), B = the codes as nibbles (the
// e2m1 value code/2).  Every product and sum is exact.  The scales enter
// after the product, v_G = 2 s_G D_G, with the zero-point term 32 z_G on
// output channel 0 of the group (the only nonzero column sum of H_32); then
// butterflies over the groups (H_4) and over the GH heads (H_GH) finish the
// transform in fp32.  The normalization 1/sqrt(128 GH) is folded into the
// query.
//
// Lane layout: lane (n = lane % 16, kq = lane / 16) loads the codes of group
// kq of token n (8 bytes) as its part of the B operand, and receives output
// channels c' = 16 mb + 4 kq + e (mb = 0, 1; e = 0..3) of every group for
// token n.  RoPE pairs channel i with i + 64, i.e. group G with G + 2 at the
// same c', so both halves of every pair sit in one lane.
//
// RoPE angles.  Pair i turns by t * base^(-2i/128) at position t (the
// token's cache slot).  Each lane holds the 16 frequencies of its pairs in
// revolutions per position as 64-bit fixed point (computed once in fp64),
// takes the fractional revolutions of t * f exactly from the low 64 bits of
// the product, and evaluates v_sin_f32 / v_cos_f32 (which take revolutions).
#include "kv_decode_common.h"

namespace kvq {

typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef float float4v_t __attribute__((ext_vector_type(4)));

constexpr int kPrWaves = 4;                // waves per workgroup

// Channel (within a 32-channel group) of K slot 8u + e of a lane's group:
// the masked code dword (w & 0x33333333) holds channels 4b and 4b + 2 of byte
// b in nibbles 2b and 2b + 1, the shifted one ((w >> 2) & 0x33333333) channels
// 4b + 1 and 4b + 3; dwords u = 0, 1 come from the group's first code dword,
// u = 2, 3 from its second (channels 16 ..).
__device__ __forceinline__ constexpr int pr_chan(int u, int e) {
  return 16 * (u >> 1) + 4 * (e >> 1) + 2 * (e & 1) + (u & 1);
}

constexpr uint32_t kFp4PlusOne = 0x2u;     // e2m1 +1.0
constexpr uint32_t kFp4MinusOne = 0xAu;    // e2m1 -1.0

// Fractional revolutions of t * f for f in 64-bit fixed point (fhi, flo)
// revolutions per position: the top 32 bits of the low 64 bits of the
// product, as a signed fraction in [-1/2, 1/2).
__device__ __forceinline__ double frac_revolutions(uint32_t t, uint32_t fhi, uint32_t flo) {
  const uint32_t top = __umulhi(t, flo) + t * fhi;
  return (double)(int32_t)top * 2.3283064365386963e-10;   // 2^-32
}

// sin and cos of 2 pi rev for rev in [-1/2, 1/2], in fp64: quadrant k =
// round(4 rev), remainder r = 2 pi (rev - k / 4) in [-pi/4, pi/4], Taylor
// series of sin r and cos r to degree 19 and 18 (truncation below 1e-19),
// then the quarter turns.  No large-argument reduction is needed here.
// 1/i! for i <= 22 (each rounded once from the exact factorial, which is
// exact in fp64 up to 22!)
struct InvFactorials {
  double v[23];
  constexpr InvFactorials() : v() {
    double f = 1.0;
    for (int i = 0; i < 23; ++i) {
      if (i > 0) f *= i;
      v[i] = 1.0 / f;
    }
  }
};
__device__ constexpr InvFactorials kInvFact{};
__device__ __forceinline__ void sincos_turns(double rev, double *sn, double *cs) {
  const double k = rint(4.0 * rev);
  const double r = (rev - 0.25 * k) * 6.283185307179586;
  const double r2 = r * r;
  double ps = kInvFact.v[19], pc = kInvFact.v[18];
#pragma unroll
  for (int i = 17; i >= 3; i -= 2) ps = fma(ps, -r2, kInvFact.v[i]);
#pragma unroll
  for (int i = 16; i >= 2; i -= 2) pc = fma(pc, -r2, kInvFact.v[i]);
  const double sr = r * fma(ps, -r2, 1.0), cr = fma(pc, -r2, 1.0);
  const int q = (int)k & 3;
  *sn = q == 0 ? sr : q == 1 ? cr : q == 2 ? -sr : -cr;
  *cs = q == 0 ? cr : q == 1 ? -sr : q == 2 ? -cr : sr;
}

// 2^x in fp64 for x <= 0 of moderate size: 2^floor(x) exactly (ldexp) times
// e^(r ln 2), r = x - floor(x) in [0, 1), by its Taylor series to degree 22
// (truncation below 1e-24).  Written out so that the table kernel needs no
// library call (and no call stack).
__device__ __forceinline__ double exp2_f64(double x) {
  const double k = floor(x);
  const double u = (x - k) * 0.6931471805599453;                    // ln 2
  double p = kInvFact.v[22];
#pragma unroll
  for (int i = 21; i >= 0; --i) p = fma(p, u, kInvFact.v[i]);
  return ldexp(p, (int)k);
}

// The RoPE table: thread i (< 64) writes pair i's frequency base^(-i/64)
// / (2 pi) revolutions per position as 64-bit fixed point (computed in fp64)
// and the cosine and sine of 16 positions' angle.
__global__ __launch_bounds__(64) void kv_rope_table(double log2_base, uint32_t *tab) {
  const int i = threadIdx.x;
  const double f = exp2_f64(-(double)i / 64.0 * log2_base) * 0.15915494309189535;   // / (2 pi)
  const double hi = floor(f * 4294967296.0);
  const uint32_t fhi = (uint32_t)hi, flo = (uint32_t)((f * 4294967296.0 - hi) * 4294967296.0);
  double sv, cv;
  sincos_turns(frac_revolutions(16u, fhi, flo), &sv, &cv);
  tab[4 * i] = fhi;
  tab[4 * i + 1] = flo;
  tab[4 * i + 2] = float_as_bits((float)cv);
  tab[4 * i + 3] = float_as_bits((float)sv);
}

// cos and sin, in fp32, of the angle t * f for f in 64-bit fixed point
// revolutions: the fraction's top 32 bits are split exactly (integers) into a
// quarter turn k and a remainder of at most 1/8 turn, whose angle r (|r| <=
// pi/4) goes through Taylor series to degree 11 and 10 (truncation below
// 2e-10), then the quarter turns.
__device__ __forceinline__ void cossin_at(uint32_t t, uint32_t fhi, uint32_t flo, float *cs, float *sn) {
  const uint32_t top = __umulhi(t, flo) + t * fhi;
  const uint32_t k = (top + 0x20000000u) >> 30;
  const int32_t rem = (int32_t)(top - (k << 30));
  const float r = (float)rem * 1.4629180792671596e-09f;             // 2 pi / 2^32
  const float r2 = r * r;
  float ps = -1.0f / 39916800.0f, pc = -1.0f / 3628800.0f;           // -1/11!, -1/10!
  ps = __builtin_fmaf(ps, r2, 1.0f / 362880.0f);
  ps = __builtin_fmaf(ps, r2, -1.0f / 5040.0f);
  ps = __builtin_fmaf(ps, r2, 1.0f / 120.0f);
  ps = __builtin_fmaf(ps, r2, -1.0f / 6.0f);
  const float sr = __builtin_fmaf(r * r2, ps, r);
  pc = __builtin_fmaf(pc, r2, 1.0f / 40320.0f);
  pc = __builtin_fmaf(pc, r2, -1.0f / 720.0f);
  pc = __builtin_fmaf(pc, r2, 1.0f / 24.0f);
  pc = __builtin_fmaf(pc, r2, -0.5f);
  const float cr = __builtin_fmaf(r2, pc, 1.0f);
  const uint32_t q = k & 3u;
  *sn = q == 0 ? sr : q == 1 ? cr : q == 2 ? -sr : -cr;
  *cs = q == 0 ? cr : q == 1 ? -sr : q == 2 ? -cr : sr;
}

// LDS per wave: the group's queries [GH G][128], then the per-step turn
// (cos, sin of 16 positions' angle) of the 16 pairs of each lane row kq.
template <int GH, int G>
__host__ __device__ constexpr int pr_lds_floats() {
  return GH * G * kD + 4 * 16 * 2;
}

// GH heads per rotation group, G query heads per KV head.  The two blocks of
// output channels (mb = 0, 1) are processed one after the other, so that
// only half of the group's un-rotated channels are live at a time; the
// partial dot products of each (head, query head) carry over.
template <int GH, int G>
__global__ __launch_bounds__(64 * kPrWaves, 2) void kv_prerope_scores(PreropeArgs a) {
  extern __shared__ float pr_lds[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t gw = (int64_t)blockIdx.x * kPrWaves + wave;
  const int ngroups = a.Hkv / GH;
  if (gw >= a.B * ngroups * a.chunks) return;      // whole wave; no barrier follows
  const int64_t chunk = gw % a.chunks;
  const int64_t bg = gw / a.chunks;
  const int grp = (int)(bg % ngroups);
  const int64_t b = bg / ngroups;
  const int h0 = grp * GH;                          // first KV head of the group
  constexpr int NQ = GH * G;                        // query heads h0 G .. (h0 + GH) G - 1
  float *qs = pr_lds + (int64_t)wave * pr_lds_floats<GH, G>();
  float *wt = qs + NQ * kD;
  const int n = lane & 15, kq = lane >> 4;

  // the group's queries, times softmax_scale * log2(e) / sqrt(128 GH)
  for (int i = lane; i < NQ * kD; i += 64) {
    const int64_t off = (b * a.Hq + (int64_t)h0 * G) * kD + i;
    const float v = a.q_f32 ? reinterpret_cast<const float *>(a.q)[off]
                            : (float)reinterpret_cast<const _Float16 *>(a.q)[off];
    qs[i] = v * a.qscale;
  }

  // A operands, one per (block mb, group Gi): H_32 rows 16 mb + n over the K
  // slots of group Gi (lanes kq = Gi), zero in the other groups' slots, fp4
  uint32_t Am[2][4][4];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      uint32_t w = 0u;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const bool neg = (__builtin_popcount((unsigned)((16 * mb + n) & pr_chan(u, e))) & 1) != 0;
        w |= (neg ? kFp4MinusOne : kFp4PlusOne) << (4 * e);
      }
#pragma unroll
      for (int Gi = 0; Gi < 4; ++Gi) Am[mb][Gi][u] = kq == Gi ? w : 0u;
    }
  }

  const int64_t step_first = chunk * a.tiles_per_wave;
  int64_t step_last = step_first + a.tiles_per_wave;
  step_last = step_last < a.tiles ? step_last : a.tiles;
  const int64_t t_end = a.t_begin + a.n_int2;
  const int64_t t_first = a.t_begin + 16 * step_first + n;   // the lane's token at the first step

  // RoPE of the lane's pairs x = 8 Go + 4 mb + e (Go = 0, 1): channels i and
  // i + 64 with i = 32 Go + 16 mb + 4 kq + e, kept as (C, S) = (cos - sin,
  // cos + sin) of the current angle and turned by 16 positions per step
  // (the turns go to LDS, one row kq at a time).  Angles exact in the
  // position (64-bit fixed-point revolutions).
  float Cp[16], Sp[16];
#pragma unroll
  for (int x = 0; x < 16; ++x) {
    const int i = 32 * (x >> 3) + 16 * ((x >> 2) & 1) + 4 * kq + (x & 3);
    const u32x4_t e = *reinterpret_cast<const u32x4_t *>(a.rope_table + 4 * i);
    float cv, sv;
    cossin_at((uint32_t)t_first, e[0], e[1], &cv, &sv);
    Cp[x] = cv - sv;
    Sp[x] = cv + sv;
    if (n == 0) {                                   // one lane per row kq writes the row's turns
      wt[(kq * 16 + x) * 2] = bits_as_float(e[2]);
      wt[(kq * 16 + x) * 2 + 1] = bits_as_float(e[3]);
    }
  }
  asm volatile("" ::: "memory");                    // LDS of one wave is ordered; keep the program order
  const float z_mul = kq == 0 ? 32.0f : 0.0f;       // 32 z on output channel c' = 0 (lanes kq = 0)

  // the group's key rows of token t (clamped to the range): codes of group
  // kq, the four scales and zeros; loaded one step ahead
  auto load_rows = [&](int64_t t, u32x2_t *cw, u32x2_t *sw, u32x2_t *zw) {
    const int64_t tr = t < t_end ? t : t_end - 1;   // rows past the range re-read the last
#pragma unroll
    for (int j = 0; j < GH; ++j) {
      const int64_t row = (b * a.Hkv + h0 + j) * a.kT_cap + tr;
      cw[j] = *reinterpret_cast<const u32x2_t *>(a.kcodes + row * kCodeBytes + 8 * kq);
      sw[j] = *reinterpret_cast<const u32x2_t *>(a.kscales + row * kNGroups);
      zw[j] = *reinterpret_cast<const u32x2_t *>(a.kzeros + row * kNGroups);
    }
  };
  u32x2_t ncw[GH], nsw[GH], nzw[GH];
  if (step_first < step_last) load_rows(t_first, ncw, nsw, nzw);

  for (int64_t step = step_first; step < step_last; ++step) {
    const int64_t t = t_first + 16 * (step - step_first);
    const bool valid = t < t_end;
    // the queries and turns are read from LDS at every step: the barrier
    // keeps those reads in the loop instead of holding them all in registers
    asm volatile("" ::: "memory");
    uint32_t bw[GH][4];
    u32x2_t sw[GH], zw[GH];
#pragma unroll
    for (int j = 0; j < GH; ++j) {
      const u32x2_t cw = ncw[j];
      sw[j] = nsw[j];
      zw[j] = nzw[j];
      bw[j][0] = cw.x & 0x33333333u;
      bw[j][1] = (cw.x >> 2) & 0x33333333u;
      bw[j][2] = cw.y & 0x33333333u;
      bw[j][3] = (cw.y >> 2) & 0x33333333u;
    }
    if (step + 1 < step_last) load_rows(t + 16, ncw, nsw, nzw);
    float part[GH][G];
#pragma unroll
    for (int j = 0; j < GH; ++j)
#pragma unroll
      for (int g = 0; g < G; ++g) part[j][g] = 0.0f;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      // u[j][G1][Go0][e]: scales applied, butterfly over bit 0 of the group
      // index done, at output channel c' = 16 mb + 4 kq + e
      float u[GH][2][2][4];
#pragma unroll
      for (int j = 0; j < GH; ++j) {
        v8i_t Bv;
#pragma unroll
        for (int w = 0; w < 4; ++w) Bv[w] = (int)bw[j][w];
        Bv[4] = 0; Bv[5] = 0; Bv[6] = 0; Bv[7] = 0;
        float4v_t D[4];
#pragma unroll
        for (int Gi = 0; Gi < 4; ++Gi) {
          v8i_t A;
#pragma unroll
          for (int w = 0; w < 4; ++w) A[w] = (int)Am[mb][Gi][w];
          A[4] = 0; A[5] = 0; A[6] = 0; A[7] = 0;
          // A scaled by 2: D = sum over group Gi of H_32[c'][.] codes, exactly
          D[Gi] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, Bv, float4v_t{0.0f, 0.0f, 0.0f, 0.0f},
                                                                  4, 4, 0, 128, 0, 127);
        }
        const float sc[4] = {lo_half(sw[j].x), hi_half(sw[j].x), lo_half(sw[j].y), hi_half(sw[j].y)};
#pragma unroll
        for (int G1 = 0; G1 < 2; ++G1) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (mb == 0 && e == 0) {
              const float z0 = z_mul * (G1 == 0 ? lo_half(zw[j].x) : lo_half(zw[j].y));
              const float z1 = z_mul * (G1 == 0 ? hi_half(zw[j].x) : hi_half(zw[j].y));
              const float v0 = __builtin_fmaf(sc[2 * G1], D[2 * G1][0], z0);
              const float v1 = __builtin_fmaf(sc[2 * G1 + 1], D[2 * G1 + 1][0], z1);
              u[j][G1][0][0] = v0 + v1;
              u[j][G1][1][0] = v0 - v1;
            } else {
              const float v0 = sc[2 * G1] * D[2 * G1][e];
              u[j][G1][0][e] = __builtin_fmaf(sc[2 * G1 + 1], D[2 * G1 + 1][e], v0);
              u[j][G1][1][e] = __builtin_fmaf(-sc[2 * G1 + 1], D[2 * G1 + 1][e], v0);
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);          // one head's products at a time
      }
      // butterflies over the group's heads
#pragma unroll
      for (int hs = 1; hs < GH; hs <<= 1) {
#pragma unroll
        for (int j = 0; j < GH; ++j) {
          if ((j & hs) == 0) {
#pragma unroll
            for (int G1 = 0; G1 < 2; ++G1)
#pragma unroll
              for (int Go0 = 0; Go0 < 2; ++Go0)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  const float x0 = u[j][G1][Go0][e], x1 = u[j + hs][G1][Go0][e];
                  u[j][G1][Go0][e] = x0 + x1;
                  u[j + hs][G1][Go0][e] = x0 - x1;
                }
          }
        }
      }
      // butterfly over bit 1 of the group index fused with RoPE: with
      // a = u[.][0], b = u[.][1], channel i holds a + b and channel i + 64
      // holds a - b, so the embedded pair is (a C + b S, a S - b C); then the
      // dot products with the head's queries
#pragma unroll
      for (int Go0 = 0; Go0 < 2; ++Go0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int x = 8 * Go0 + 4 * mb + e;
          const float Ck = Cp[x], Sk = Sp[x];
#pragma unroll
          for (int j = 0; j < GH; ++j) {
            asm volatile("" ::: "memory");            // the queries are read where they are used
            const float av = u[j][0][Go0][e], bv = u[j][1][Go0][e];
            const float lo = __builtin_fmaf(bv, Sk, av * Ck);
            const float hi = __builtin_fmaf(-bv, Ck, av * Sk);
#pragma unroll
            for (int g = 0; g < G; ++g) {
              const float *qh = qs + (j * G + g) * kD + 32 * Go0 + 16 * mb + 4 * kq + e;
              part[j][g] = __builtin_fmaf(qh[64], hi, __builtin_fmaf(qh[0], lo, part[j][g]));
            }
          }
        }
      }
    }
    // sums over the four lanes of token n, stored from one branch (a branch
    // per store would keep every sum live across all of them)
    float tot[GH][G];
#pragma unroll
    for (int j = 0; j < GH; ++j)
#pragma unroll
      for (int g = 0; g < G; ++g) tot[j][g] = sum_xor32(sum_xor16(part[j][g]));
    if (kq == 0 && valid) {
      float *dst = a.scores + (b * a.Hq + (int64_t)h0 * G) * a.n_rows + (t - a.t_begin) + a.skip;
#pragma unroll
      for (int j = 0; j < GH; ++j)
#pragma unroll
        for (int g = 0; g < G; ++g) dst[(j * G + g) * a.n_rows] = tot[j][g];
    }
    // next step: turn every pair by 16 positions (turns read here, not held
    // across the step)
    asm volatile("" ::: "memory");
#pragma unroll
    for (int x = 0; x < 16; ++x) {
      const float wc = wt[(kq * 16 + x) * 2], ws = wt[(kq * 16 + x) * 2 + 1];
      const float c = Cp[x], s = Sp[x];
      Cp[x] = __builtin_fmaf(-s, ws, c * wc);
      Sp[x] = __builtin_fmaf(c, ws, s * wc);
    }
  }
}

template <int GH>
static hipError_t launch_prerope_g(const PreropeArgs &a, dim3 grid, dim3 block, size_t lds, hipStream_t stream) {
  switch (a.G) {
    case 1: hipLaunchKernelGGL((kv_prerope_scores<GH, 1>), grid, block, lds, stream, a); break;
    case 2: hipLaunchKernelGGL((kv_prerope_scores<GH, 2>), grid, block, lds, stream, a); break;
    case 4: hipLaunchKernelGGL((kv_prerope_scores<GH, 4>), grid, block, lds, stream, a); break;
    case 8: hipLaunchKernelGGL((kv_prerope_scores<GH, 8>), grid, block, lds, stream, a); break;
    default: return hipErrorNotSupported;
  }
  return hipGetLastError();
}

hipError_t launch_prerope_scores(const PreropeArgs &a, hipStream_t stream) {
  hipLaunchKernelGGL(kv_rope_table, dim3(1), dim3(64), 0, stream, a.log2_base, a.rope_table);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t waves = a.B * (a.Hkv / a.GH) * a.chunks;
  const dim3 grid((unsigned)((waves + kPrWaves - 1) / kPrWaves)), block(64 * kPrWaves);
  const size_t lds = (size_t)kPrWaves * (a.GH * a.G * kD + 4 * 16 * 2) * sizeof(float);
  switch (a.GH) {
    case 1: return launch_prerope_g<1>(a, grid, block, lds, stream);
    case 2: return launch_prerope_g<2>(a, grid, block, lds, stream);
    case 4: return launch_prerope_g<4>(a, grid, block, lds, stream);
    default: return hipErrorNotSupported;
  }
}

}  // namespace kvq
