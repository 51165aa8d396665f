// Write path with a dense per-head rotation (OptR style: one learned
// orthogonal matrix per head, "Output-Aware Rotation for INT2 KV-Cache
// Quantization", woor.ai page, "Key Details"): y = x R_h, then the same
// 2-bit group quantizer as the Hadamard path.
//
// The 128x128 contraction over many tokens runs on MFMA.  Computing
// y^T = R^T x^T with v_mfma_f32_32x32x8f16 puts one token per lane column
// and 32 output channels (exactly one quantization group) per 32x32 tile:
// lane (j, half) holds 16 of the group's channels for token j and the
// other 16 sit in lane j + 32, so group min/max need one cross-half
// exchange.  R is fp32; it is split into fp16 hi + lo parts (R = hi + lo to
// about 2^-22 relative) and both are applied with fp32 accumulation, while
// the fp16 inputs are exact in the MFMA.  The split fragments are staged
// once per workgroup into LDS in A-operand order (one 8-byte LDS read per
// lane per MFMA).
#include "kvq_device.h"
#include "kvq_launch.h"

namespace kvq {

typedef _Float16 half4v_t __attribute__((ext_vector_type(4)));

constexpr int kDenseWaves = 4;
constexpr int kDenseTilesPerWave = 4;                        // 32 tokens each
constexpr int kDenseTokensPerBlock = kDenseWaves * kDenseTilesPerWave * 32;

// K-slot (k-step s of 8 slots, lane half h, element v) <-> input channel:
// lane half h covers input channels [64h, 64h + 64), k-step s channels
// 64h + 4s .. 64h + 4s + 3.  Any bijection works as long as the A and B
// operands use the same one; this one lets a lane load its 64 input
// channels as 128 contiguous bytes.
__device__ __forceinline__ int dense_in_channel(int s, int h, int v) { return 64 * h + 4 * s + v; }

struct DenseKernelArgs {
  QuantSide side[2];
  int64_t stride_b, stride_t, stride_h;
  int64_t T_new, t_offset;
  int Hkv;
  int n_sides;
  const float *R;     // [Hkv][128][128], y = x R
};

// Quantize the 16 values this lane holds of one group; the partner lane
// (lane ^ 32) holds the other 16.  Returns this lane's 4 code bytes (group
// bytes 2q + half, q = 0..3) and the group's scale / zero bits.
__device__ __forceinline__ uint32_t dense_group_codes(const float (&y)[16], uint16_t &sbits,
                                                      uint16_t &zbits) {
#pragma clang fp contract(off)
  float mn = y[0], mx = y[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) {
    mn = fminf(mn, y[r]);
    mx = fmaxf(mx, y[r]);
  }
  mn = fminf(mn, __shfl_xor(mn, 32, 64));
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
  const float range = mx - mn;
  const float s32 = range / 3.0f;
  sbits = float_to_half_bits(s32);
  zbits = float_to_half_bits(mn + 0.0f);
  const float sf = half_bits_to_float(sbits);
  const float zf = half_bits_to_float(zbits);
  const bool degenerate = (sf == 0.0f);
  const float inv = 1.0f / (degenerate ? 1.0f : sf);
  uint32_t out = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t byte = 0;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float u = (y[4 * q + v] - zf) * inv;
      const float t = __builtin_amdgcn_fmed3f(u, 0.0f, 3.0f);
      const uint32_t code = float_as_bits(t + 12582912.0f) & 3u;   // round half to even
      byte |= code << (2 * v);
    }
    out |= byte << (8 * q);
  }
  return degenerate ? 0u : out;
}

// grid: x = blocks of kDenseTokensPerBlock tokens, y = KV head,
// z = batch * n_sides + side.  256 threads.
__global__ __launch_bounds__(256) void kv_rotate_quant_dense(DenseKernelArgs a) {
  // A fragments: [group g][k-step s][hi/lo] x 64 lanes x 4 halves
  __shared__ uint2 frag[4 * 16 * 2 * 64];   // 64 KB
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = blockIdx.y;
  const int sidx = (int)(blockIdx.z % (unsigned)a.n_sides);
  const int64_t b = blockIdx.z / (unsigned)a.n_sides;
  const QuantSide s = sidx ? a.side[1] : a.side[0];

  // stage R_h^T as fp16 hi / lo A fragments
  {
    const float *R = a.R + (int64_t)h * kD * kD;
    _Float16 *fh = reinterpret_cast<_Float16 *>(frag);
    for (int idx = tid; idx < kD * kD; idx += 256) {
      const int k = idx >> 7, c = idx & 127;                 // R[k][c]: input k, output c
      const float r = R[idx];
      const _Float16 hi = (_Float16)r;
      const _Float16 lo = (_Float16)(r - (float)hi);
      const int g = c >> 5, i = c & 31;
      const int hh = k >> 6, st = (k >> 2) & 15, v = k & 3;   // inverse of dense_in_channel
      const int ln = i + 32 * hh;
      const int f0 = ((g * 16 + st) * 2 + 0) * 64 + ln;
      const int f1 = ((g * 16 + st) * 2 + 1) * 64 + ln;
      fh[f0 * 4 + v] = hi;
      fh[f1 * 4 + v] = lo;
    }
  }
  __syncthreads();

  const int j = lane & 31;           // token column
  const int half = lane >> 5;
  const _Float16 *xbase = reinterpret_cast<const _Float16 *>(s.x) + b * a.stride_b +
                          (int64_t)h * a.stride_h + 64 * half;
  for (int tile = 0; tile < kDenseTilesPerWave; ++tile) {
    const int64_t t0 = (int64_t)blockIdx.x * kDenseTokensPerBlock + (wave * kDenseTilesPerWave + tile) * 32;
    if (t0 >= a.T_new) break;                                // wave-uniform
    const int64_t t = t0 + j;
    const bool valid = t < a.T_new;
    const int64_t tl = valid ? t : t0;
    // B operand: this lane's 64 input channels of token t (128 bytes)
    const u32x4_t *src = reinterpret_cast<const u32x4_t *>(xbase + tl * a.stride_t);
    uint32_t xw[32];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const u32x4_t u = __builtin_nontemporal_load(src + k);
      xw[4 * k] = u.x; xw[4 * k + 1] = u.y; xw[4 * k + 2] = u.z; xw[4 * k + 3] = u.w;
    }
    float16_t acc[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      acc[g] = float16_t{};
#pragma unroll
      for (int st = 0; st < 16; ++st) {
        const half4v_t bx = __builtin_bit_cast(half4v_t, make_uint2(xw[2 * st], xw[2 * st + 1]));
        const half4v_t ahi = __builtin_bit_cast(half4v_t, frag[((g * 16 + st) * 2 + 0) * 64 + lane]);
        const half4v_t alo = __builtin_bit_cast(half4v_t, frag[((g * 16 + st) * 2 + 1) * 64 + lane]);
        acc[g] = __builtin_amdgcn_mfma_f32_32x32x8f16(ahi, bx, acc[g], 0, 0, 0);
        acc[g] = __builtin_amdgcn_mfma_f32_32x32x8f16(alo, bx, acc[g], 0, 0, 0);
      }
    }
    // epilogue: acc[g][r] = y[t][32g + 8(r/4) + 4*half + r%4]
    const int64_t row = (b * a.Hkv + h) * s.T_cap + a.t_offset + t;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      float y[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) y[r] = acc[g][r];
      uint16_t sb, zb;
      const uint32_t mine = dense_group_codes(y, sb, zb);
      const uint32_t other = (uint32_t)__shfl_xor((int)mine, 32, 64);
      // group bytes 0..7: even bytes from half 0, odd bytes from half 1
      const uint32_t e = half ? other : mine, o = half ? mine : other;
      const uint32_t w0 = __builtin_amdgcn_perm(o, e, 0x05010400u);   // e0 o0 e1 o1
      const uint32_t w1 = __builtin_amdgcn_perm(o, e, 0x07030602u);   // e2 o2 e3 o3
      if (valid && half == (g & 1)) {
        *reinterpret_cast<uint2 *>(s.codes + row * kCodeBytes + 8 * g) = make_uint2(w0, w1);
        s.scales[row * kNGroups + g] = sb;
        s.zeros[row * kNGroups + g] = zb;
      }
    }
  }
}

hipError_t launch_quantize_dense(const QuantArgs &q, hipStream_t stream) {
  DenseKernelArgs a;
  a.side[0] = q.side[0];
  a.side[1] = q.n_sides > 1 ? q.side[1] : q.side[0];
  a.stride_b = q.stride_b;
  a.stride_t = q.stride_t;
  a.stride_h = q.stride_h;
  a.T_new = q.T_new;
  a.t_offset = q.t_offset;
  a.Hkv = (int)q.Hkv;
  a.n_sides = q.n_sides;
  a.R = q.R;
  dim3 grid((unsigned)((q.T_new + kDenseTokensPerBlock - 1) / kDenseTokensPerBlock),
            (unsigned)q.Hkv, (unsigned)(q.B * q.n_sides));
  hipLaunchKernelGGL(kv_rotate_quant_dense, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace kvq
