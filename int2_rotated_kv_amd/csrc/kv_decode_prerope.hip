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
constexpr int kPrTileTokens = 16;

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

template <int GH>
__global__ __launch_bounds__(64 * kPrWaves) void kv_prerope_scores(PreropeArgs a) {
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
  const int nq = GH * a.G;                          // query heads h0 G .. (h0 + GH) G - 1
  float *qs = pr_lds + (int64_t)wave * nq * kD;

  // the group's queries, times softmax_scale * log2(e) / sqrt(128 GH)
  for (int i = lane; i < nq * kD; i += 64) {
    const int64_t off = (b * a.Hq + (int64_t)h0 * a.G) * kD + i;
    const float v = a.q_f32 ? reinterpret_cast<const float *>(a.q)[off]
                            : (float)reinterpret_cast<const _Float16 *>(a.q)[off];
    qs[i] = v * a.qscale;
  }
  asm volatile("" ::: "memory");                    // LDS of one wave is ordered; keep the program order

  const int n = lane & 15, kq = lane >> 4;
  // A operands: H_32 rows 16 mb + n over the lane's K slots (group kq), fp4
  uint32_t hA[2][4];
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
      hA[mb][u] = w;
    }
  }
  // RoPE frequencies of the lane's pairs, revolutions per position in 64-bit
  // fixed point: pair index k = 8 gp + 4 mb + e is channel i = 32 gp + 16 mb + 4 kq + e
  uint32_t flo[16], fhi[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int i = 32 * (k >> 3) + 16 * ((k >> 2) & 1) + 4 * kq + (k & 3);
    const double f = exp2(-(double)i / 64.0 * a.log2_base) * 0.15915494309189535;   // / (2 pi)
    const double hi = floor(f * 4294967296.0);
    fhi[k] = (uint32_t)hi;
    flo[k] = (uint32_t)((f * 4294967296.0 - hi) * 4294967296.0);
  }

  const int64_t t_first = chunk * a.tiles_per_wave;
  int64_t t_last = t_first + a.tiles_per_wave;
  t_last = t_last < a.tiles ? t_last : a.tiles;
  const int64_t t_end = a.t_begin + a.n_int2;
  for (int64_t ti = t_first; ti < t_last; ++ti) {
    const int64_t t = a.t_begin + kPrTileTokens * ti + n;        // the lane's token (cache slot)
    const bool valid = t < t_end;
    const int64_t tr = valid ? t : t_end - 1;                   // rows past the range re-read the last
    // cos / sin of the lane's 16 pairs at position tr
    float cs[16], sn[16];
    {
      const uint32_t tp = (uint32_t)tr;
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        // top 32 bits of the low 64 bits of tp * F: the fractional revolutions
        const uint32_t top = __umulhi(tp, flo[k]) + tp * fhi[k];
        const float rev = (float)(int32_t)top * 2.3283064365386963e-10f;   // 2^-32, in [-0.5, 0.5)
        cs[k] = __builtin_amdgcn_cosf(rev);
        sn[k] = __builtin_amdgcn_sinf(rev);
      }
    }
    // un-rotated (unnormalized) keys of the group's heads at the lane's
    // channels: u[j][8 G + 4 mb + e] is channel 32 G + 16 mb + 4 kq + e
    float uk[GH][32];
#pragma unroll
    for (int j = 0; j < GH; ++j) {
      const int64_t row = (b * a.Hkv + h0 + j) * a.kT_cap + tr;
      const u32x2_t cw = *reinterpret_cast<const u32x2_t *>(a.kcodes + row * kCodeBytes + 8 * kq);
      const u32x2_t sw = *reinterpret_cast<const u32x2_t *>(a.kscales + row * kNGroups);
      const u32x2_t zw = *reinterpret_cast<const u32x2_t *>(a.kzeros + row * kNGroups);
      v8i_t Bop;
      Bop[0] = (int)(cw.x & 0x33333333u);
      Bop[1] = (int)((cw.x >> 2) & 0x33333333u);
      Bop[2] = (int)(cw.y & 0x33333333u);
      Bop[3] = (int)((cw.y >> 2) & 0x33333333u);
      Bop[4] = 0; Bop[5] = 0; Bop[6] = 0; Bop[7] = 0;
      float4v_t D[4][2];
#pragma unroll
      for (int G = 0; G < 4; ++G) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          v8i_t A;
#pragma unroll
          for (int u = 0; u < 4; ++u) A[u] = kq == G ? (int)hA[mb][u] : 0;
          A[4] = 0; A[5] = 0; A[6] = 0; A[7] = 0;
          D[G][mb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, Bop, float4v_t{0.0f, 0.0f, 0.0f, 0.0f},
                                                                     4, 4, 0, 127, 0, 127);
        }
      }
      // D[G][mb][e] = (1/2) sum_{j' in group G} H_32[c'][j'] code_j' for c' = 16 mb + 4 kq + e
      const float s2[4] = {2.0f * lo_half(sw.x), 2.0f * hi_half(sw.x), 2.0f * lo_half(sw.y), 2.0f * hi_half(sw.y)};
      const bool c0 = kq == 0;                      // e = 0, mb = 0 is output channel c' = 0
      const float z32[4] = {c0 ? 32.0f * lo_half(zw.x) : 0.0f, c0 ? 32.0f * hi_half(zw.x) : 0.0f,
                            c0 ? 32.0f * lo_half(zw.y) : 0.0f, c0 ? 32.0f * hi_half(zw.y) : 0.0f};
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float v[4];
#pragma unroll
          for (int G = 0; G < 4; ++G)
            v[G] = (mb == 0 && e == 0) ? __builtin_fmaf(s2[G], D[G][mb][e], z32[G]) : s2[G] * D[G][mb][e];
          // H_4 over the groups
          const float a0 = v[0] + v[1], a1 = v[0] - v[1], a2 = v[2] + v[3], a3 = v[2] - v[3];
          uk[j][0 + 4 * mb + e] = a0 + a2;
          uk[j][8 + 4 * mb + e] = a1 + a3;
          uk[j][16 + 4 * mb + e] = a0 - a2;
          uk[j][24 + 4 * mb + e] = a1 - a3;
        }
      }
    }
    // H_GH over the heads of the group
#pragma unroll
    for (int hs = 1; hs < GH; hs <<= 1) {
#pragma unroll
      for (int j = 0; j < GH; ++j) {
        if ((j & hs) == 0) {
#pragma unroll
          for (int i = 0; i < 32; ++i) {
            const float x = uk[j][i], y = uk[j + hs][i];
            uk[j][i] = x + y;
            uk[j + hs][i] = x - y;
          }
        }
      }
    }
    // RoPE at position tr, then the dot products with the head's queries
#pragma unroll
    for (int j = 0; j < GH; ++j) {
      float kr[32];
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int gp = k >> 3, idx = k & 7;         // channel 32 gp + c' and its partner + 64
        const float x0 = uk[j][8 * gp + idx], x1 = uk[j][8 * (gp + 2) + idx];
        kr[8 * gp + idx] = __builtin_fmaf(-x1, sn[k], x0 * cs[k]);
        kr[8 * (gp + 2) + idx] = __builtin_fmaf(x0, sn[k], x1 * cs[k]);
      }
      for (int g = 0; g < a.G; ++g) {
        const float *qh = qs + (int64_t)(j * a.G + g) * kD + 4 * kq;
        float acc = 0.0f;
#pragma unroll
        for (int G = 0; G < 4; ++G) {
#pragma unroll
          for (int mb = 0; mb < 2; ++mb) {
            const float4v_t qv = *reinterpret_cast<const float4v_t *>(qh + 32 * G + 16 * mb);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc = __builtin_fmaf(qv[e], kr[8 * G + 4 * mb + e], acc);
          }
        }
        acc = sum_xor32(sum_xor16(acc));              // the four lanes of token n
        if (kq == 0 && valid) {
          const int hq = (h0 + j) * a.G + g;
          a.scores[(b * a.Hq + hq) * a.n_rows + (t - a.t_begin) + a.skip] = acc;
        }
      }
    }
  }
}

hipError_t launch_prerope_scores(const PreropeArgs &a, hipStream_t stream) {
  const int64_t waves = a.B * (a.Hkv / a.GH) * a.chunks;
  const dim3 grid((unsigned)((waves + kPrWaves - 1) / kPrWaves)), block(64 * kPrWaves);
  const size_t lds = (size_t)kPrWaves * a.GH * a.G * kD * sizeof(float);
  switch (a.GH) {
    case 1: hipLaunchKernelGGL(kv_prerope_scores<1>, grid, block, lds, stream, a); break;
    case 2: hipLaunchKernelGGL(kv_prerope_scores<2>, grid, block, lds, stream, a); break;
    case 4: hipLaunchKernelGGL(kv_prerope_scores<4>, grid, block, lds, stream, a); break;
    default: return hipErrorNotSupported;
  }
  return hipGetLastError();
}

}  // namespace kvq
