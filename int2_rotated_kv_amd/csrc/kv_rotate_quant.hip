// Write path: rotate -> 2-bit quantize -> pack, one KV-cache row per
// quad of lanes (gfx950, wave64).
//
// The rotation is applied before quantization ("Output-Aware Rotation for
// INT2 KV-Cache Quantization", woor.ai page, "Key Details").  The Hadamard
// case uses the fast Walsh-Hadamard transform (RotateKV, IJCAI 2025
// record, abstract item (i)) computed in registers: lane j of a quad holds
// channels [32j, 32j+32) of one row, so five butterfly stages run inside a
// lane and the two stages across the 32- and 64-channel strides use DPP
// quad permutes.  A quantization group (32 channels) is exactly one lane's
// values, so min/max need no cross-lane traffic, and the lane packs its 32
// codes into 8 bytes.  Consecutive quads handle consecutive tokens of one
// (batch, head), so a wave's code stores cover 512 contiguous bytes.
#include "kvq_device.h"
#include "kvq_launch.h"

namespace kvq {

// The quantizer as a fixed sequence of IEEE fp32 operations (no fused
// multiply-add): s = fp32(fp32(max - min) / 3); scale = fp16(s);
// zero = fp16(min + 0) (a zero minimum is +0 whatever the signs of the
// group's zeros); code = clamp(rint((y - zero) * fp32(1/scale)), 0, 3).
__device__ __forceinline__ void quantize_group32(const float (&v)[32], uint32_t &w0,
                                                 uint32_t &w1, uint16_t &sbits,
                                                 uint16_t &zbits) {
#pragma clang fp contract(off)
  float mn = v[0], mx = v[0];
#pragma unroll
  for (int i = 1; i < 32; ++i) {
    mn = fminf(mn, v[i]);
    mx = fmaxf(mx, v[i]);
  }
  const float range = mx - mn;
  const float s32 = range / 3.0f;            // correctly rounded fp32 division
  sbits = float_to_half_bits(s32);
  zbits = float_to_half_bits(mn + 0.0f);   // -0 + 0 = +0 in round-to-nearest
  const float sf = half_bits_to_float(sbits);
  const float zf = half_bits_to_float(zbits);
  const bool degenerate = (sf == 0.0f);
  const float inv = 1.0f / (degenerate ? 1.0f : sf);
  uint32_t a = 0, b = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const float u = (v[i] - zf) * inv;
    float r = __builtin_rintf(u);           // round half to even
    r = fminf(fmaxf(r, 0.0f), 3.0f);
    const uint32_t c = (uint32_t)r;
    if (i < 16) a |= c << (2 * i);
    else        b |= c << (2 * (i - 16));
  }
  w0 = degenerate ? 0u : a;
  w1 = degenerate ? 0u : b;
}

template <typename TIn>
__device__ __forceinline__ void load_row32(const TIn *src, float (&v)[32]);

template <>
__device__ __forceinline__ void load_row32<_Float16>(const _Float16 *src, float (&v)[32]) {
  const u32x4_t *p = reinterpret_cast<const u32x4_t *>(src);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const u32x4_t u = __builtin_nontemporal_load(p + k);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[8 * k + 2 * e] = half_bits_to_float((uint16_t)(w[e] & 0xFFFFu));
      v[8 * k + 2 * e + 1] = half_bits_to_float((uint16_t)(w[e] >> 16));
    }
  }
}

template <>
__device__ __forceinline__ void load_row32<float>(const float *src, float (&v)[32]) {
  const float4_t *p = reinterpret_cast<const float4_t *>(src);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float4_t u = __builtin_nontemporal_load(p + k);
    v[4 * k] = u.x; v[4 * k + 1] = u.y; v[4 * k + 2] = u.z; v[4 * k + 3] = u.w;
  }
}

// Normalized FWHT of a 128-vector spread over a quad (32 values per lane).
__device__ __forceinline__ void fwht128_quad(float (&v)[32], int j) {
#pragma unroll
  for (int hs = 1; hs < 32; hs <<= 1) {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if ((i & hs) == 0) {
        const float a = v[i], b = v[i + hs];
        v[i] = a + b;
        v[i + hs] = a - b;
      }
    }
  }
  const float n1 = (j & 1) ? -1.0f : 1.0f;
  const float n2 = (j & 2) ? -1.0f : 1.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] = quad_butterfly<kQuadXor1>(v[i], n1);
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] = quad_butterfly<kQuadXor2>(v[i], n2);
  const float norm = 0.08838834764831845f;  // fp32(1/sqrt(128))
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] *= norm;
}

struct RowsKernelArgs {
  QuantSide side[2];
  int64_t stride_b, stride_t, stride_h;
  int64_t T_new, t_offset;
  int Hkv;
  int n_sides;
};

// grid: x = token blocks of 64, y = KV head, z = batch * n_sides + side
template <typename TIn, bool ROT>
__global__ __launch_bounds__(256) void kv_rotate_quant_rows(RowsKernelArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane >> 2;
  const int j = lane & 3;
  const int h = blockIdx.y;
  const int sidx = (int)(blockIdx.z % (unsigned)a.n_sides);
  const int64_t b = blockIdx.z / (unsigned)a.n_sides;
  const QuantSide s = sidx ? a.side[1] : a.side[0];
  const int64_t t = (int64_t)blockIdx.x * 64 + wave * 16 + r;
  const bool valid = t < a.T_new;
  const int64_t tl = valid ? t : 0;
  const TIn *src = reinterpret_cast<const TIn *>(s.x) + b * a.stride_b + tl * a.stride_t +
                   (int64_t)h * a.stride_h + 32 * j;
  float v[32];
  load_row32<TIn>(src, v);
  if (ROT) fwht128_quad(v, j);
  uint32_t w0, w1;
  uint16_t sb, zb;
  quantize_group32(v, w0, w1, sb, zb);
  if (valid) {
    const int64_t row = (b * a.Hkv + h) * s.T_cap + a.t_offset + t;
    *reinterpret_cast<uint2 *>(s.codes + row * kCodeBytes + 8 * j) = make_uint2(w0, w1);
    s.scales[row * kNGroups + j] = sb;
    s.zeros[row * kNGroups + j] = zb;
  }
}

hipError_t launch_quantize_rows(const QuantArgs &q, hipStream_t stream) {
  RowsKernelArgs a;
  a.side[0] = q.side[0];
  a.side[1] = q.n_sides > 1 ? q.side[1] : q.side[0];
  a.stride_b = q.stride_b;
  a.stride_t = q.stride_t;
  a.stride_h = q.stride_h;
  a.T_new = q.T_new;
  a.t_offset = q.t_offset;
  a.Hkv = (int)q.Hkv;
  a.n_sides = q.n_sides;
  dim3 grid((unsigned)((q.T_new + 63) / 64), (unsigned)q.Hkv, (unsigned)(q.B * q.n_sides));
  dim3 block(256);
  const bool rot = (q.rot == 1);
  if (q.in_f32) {
    if (rot) hipLaunchKernelGGL((kv_rotate_quant_rows<float, true>), grid, block, 0, stream, a);
    else     hipLaunchKernelGGL((kv_rotate_quant_rows<float, false>), grid, block, 0, stream, a);
  } else {
    if (rot) hipLaunchKernelGGL((kv_rotate_quant_rows<_Float16, true>), grid, block, 0, stream, a);
    else     hipLaunchKernelGGL((kv_rotate_quant_rows<_Float16, false>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace kvq
