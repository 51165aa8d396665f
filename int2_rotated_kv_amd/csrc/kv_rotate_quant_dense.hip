// Write path with a dense per-head rotation (OptR style: one learned
// orthogonal matrix per head, "Output-Aware Rotation for INT2 KV-Cache
// Quantization", woor.ai page, "Key Details"): y = x R_h, then the same
// 2-bit group quantizer as the Hadamard path.
//
// The 128x128 contraction over many tokens runs on the matrix cores.
// Computing y^T = R^T x^T with v_mfma_f32_32x32x16_f16 puts one token per
// lane column and 32 output channels (exactly one quantization group) per
// 32x32 tile: lane (j, half) holds 16 of the group's channels for token j and
// the other 16 sit in lane j + 32, so group min/max need one cross-half
// exchange.  R is fp32; it is split into fp16 hi + lo parts (R = hi + lo to
// about 2^-22 relative) and both are applied with fp32 accumulation, while
// the fp16 inputs and the fp16 x fp16 products are exact.
//
// A workgroup owns one (batch, KV head) and a range of 32-token tiles of
// both sides.  It converts R_h into A-operand fragments in LDS once (64 KiB)
// and then streams its tiles; each wave loads the next tile's inputs while
// the current tile's 64 MFMAs and its quantization run.
#include "kvq_device.h"
#include "kvq_launch.h"

namespace kvq {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));

constexpr int kDenseWaves = 4;
constexpr int64_t kDenseTargetBlocks = 512;   // 256 CUs x 2 workgroups (64 KiB LDS each)
constexpr int64_t kDenseMinItemsPerBlock = 16;

// K-slot (k-step s of 8, lane half h, element i) <-> input channel: lane
// half h supplies input channels [64h, 64h + 64), k-step s the channels
// 64h + 8s .. 64h + 8s + 7.  Any bijection works as long as the A and B
// operands agree; this one lets a lane load its 64 input channels as 128
// contiguous bytes.
__device__ __forceinline__ constexpr int dense_in_channel(int s, int h, int i) { return 64 * h + 8 * s + i; }

// LDS slot of the A operand (group g, k-step s, hi/lo part, lane): 16 bytes.
__device__ __forceinline__ constexpr int dense_frag(int g, int s, int part, int lane) {
  return ((g * 8 + s) * 2 + part) * 64 + lane;
}

struct DenseKernelArgs {
  QuantSide side[2];
  int64_t stride_b, stride_t, stride_h;
  int64_t T_new, t_offset;
  int Hkv;
  int n_sides;
  int64_t n_items;          // n_sides * 32-token tiles; item i = (side i % n_sides, tile i / n_sides)
  int64_t items_per_block;
  const float *R;           // [Hkv][128][128], y = x R
};

// (x << SH) + acc in one instruction (v_lshl_add_u32, SH an inline constant).
template <int SH>
__device__ __forceinline__ uint32_t dshl_add(uint32_t x, uint32_t acc) {
  uint32_t r;
  asm("v_lshl_add_u32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "I"(SH), "v"(acc));
  return r;
}

// Pack 16 magic-biased code words: word q*4 + e goes to bits 8q + 2e.
template <typename F, int I = 0>
__device__ __forceinline__ uint32_t dense_pack16(F &&f, uint32_t acc) {
  if constexpr (I == 16) {
    return acc;
  } else {
    return dense_pack16<F, I + 1>(static_cast<F &&>(f), dshl_add<8 * (I / 4) + 2 * (I % 4)>(f(I), acc));
  }
}

constexpr float kDenseRoundMagic = 12582912.0f;                  // 1.5 * 2^23
constexpr uint32_t kDensePackBias = 0x4B400000u * 0x55555555u;   // sum of the biases, mod 2^32

// Both halves' values of a lane pair: r[0] = the lower half's, r[1] = the upper half's.
__device__ __forceinline__ float pair_min(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(float_as_bits(v), float_as_bits(v), false, false);
  return __builtin_fminf(bits_as_float(r[0]), bits_as_float(r[1]));
}
__device__ __forceinline__ float pair_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(float_as_bits(v), float_as_bits(v), false, false);
  return __builtin_fmaxf(bits_as_float(r[0]), bits_as_float(r[1]));
}

// Quantize the 16 values this lane holds of one group; the partner lane
// (lane ^ 32) holds the other 16.  y[r] is channel 8(r/4) + 4*half + r%4 of
// the group, so y[4q .. 4q+3] are the four codes of group byte 2q + half.
// Returns the group's 8 code bytes (w0: bytes 0..3, w1: bytes 4..7) and its
// scale / zero bits, identical in both lanes of the pair.
__device__ __forceinline__ void dense_group_codes(const float16_t &y, uint32_t &w0, uint32_t &w1,
                                                  uint16_t &sbits, uint16_t &zbits) {
#pragma clang fp contract(off)
  float mn = y[0], mx = y[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) {
    mn = __builtin_fminf(mn, y[r]);
    mx = __builtin_fmaxf(mx, y[r]);
  }
  mn = pair_min(mn);
  mx = pair_max(mx);
  const float s32 = (mx - mn) / 3.0f;                         // correctly rounded
  sbits = float_to_half_bits(s32);
  zbits = float_to_half_bits(mn + 0.0f);
  const float sf = half_bits_to_float(sbits);
  const float zf = half_bits_to_float(zbits);
  // scale 0: every code is 0 (inv = 1 and the clamp to [0, 0] give that)
  const float inv = 1.0f / (sf == 0.0f ? 1.0f : sf);
  const float top = 3.0f * sf;
  // code = rint((y - zero) / scale) clamped to [0, 3]: clamp the difference to
  // [0, 3 scale], then one fma with the magic constant rounds to an integer
  auto code = [&](int r) {
    const float d = __builtin_amdgcn_fmed3f(y[r] - zf, 0.0f, top);
    return float_as_bits(__builtin_fmaf(d, inv, kDenseRoundMagic));
  };
  const uint32_t mine = dense_pack16(code, 0u) - kDensePackBias;   // byte q = group byte 2q + half
  const auto ex = __builtin_amdgcn_permlane32_swap(mine, mine, false, false);
  const uint32_t e = ex[0], o = ex[1];          // bytes of the lower / upper half
  w0 = __builtin_amdgcn_perm(o, e, 0x05010400u);   // e0 o0 e1 o1
  w1 = __builtin_amdgcn_perm(o, e, 0x07030602u);   // e2 o2 e3 o3
}

// grid: x = chunk of items, y = KV head, z = batch; 256 threads, two
// workgroups per CU (LDS), so at most 256 registers per lane.
__global__ __launch_bounds__(256, 2) void kv_rotate_quant_dense(DenseKernelArgs a) {
  __shared__ half8_t frag[4 * 8 * 2 * 64];      // 64 KiB of A fragments
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = blockIdx.y;
  const int64_t b = blockIdx.z;

  // Stage R_h^T as fp16 hi / lo A fragments: slot (g, s, lane = (m, kh))
  // holds R[dense_in_channel(s, kh, i)][32g + m] for i = 0..7.
  {
    const float *R = a.R + (int64_t)h * kD * kD;
    for (int f = tid; f < 4 * 8 * 64; f += 256) {
      const int ln = f & 63, s = (f >> 6) & 7, g = f >> 9;
      const int m = ln & 31, kh = ln >> 5;
      half8_t hi, lo;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float r = R[dense_in_channel(s, kh, i) * kD + 32 * g + m];
        hi[i] = (_Float16)r;
        lo[i] = (_Float16)(r - (float)hi[i]);
      }
      frag[dense_frag(g, s, 0, ln)] = hi;
      frag[dense_frag(g, s, 1, ln)] = lo;
    }
  }
  __syncthreads();

  const int j = lane & 31;            // token column of the tile
  const int half = lane >> 5;
  const int64_t i0 = (int64_t)blockIdx.x * a.items_per_block;
  const int64_t i1 = (i0 + a.items_per_block < a.n_items) ? i0 + a.items_per_block : a.n_items;

  // this lane's 64 input channels of its token in the tile of item `it`
  const int side_shift = a.n_sides - 1;                   // n_sides is 1 or 2
  auto load_item = [&](int64_t it, uint32_t (&xw)[32]) {
    const int sidx = (int)(it & side_shift);
    const int64_t t0 = (it >> side_shift) * 32;
    const QuantSide s = sidx ? a.side[1] : a.side[0];       // by value: scalar selects
    const int64_t t = (t0 + j < a.T_new) ? t0 + j : a.T_new - 1;
    const u32x4_t *src = reinterpret_cast<const u32x4_t *>(
        reinterpret_cast<const _Float16 *>(s.x) + b * a.stride_b + t * a.stride_t +
        (int64_t)h * a.stride_h + 64 * half);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const u32x4_t u = __builtin_nontemporal_load(src + k);
      xw[4 * k] = u.x; xw[4 * k + 1] = u.y; xw[4 * k + 2] = u.z; xw[4 * k + 3] = u.w;
    }
  };

  // rotate-quantize-store one tile from the lane's inputs xw
  auto tile = [&](int64_t it, const uint32_t (&xw)[32]) {
    // four independent accumulators (one per group) keep the matrix pipe
    // busy; acc[g][r] = y[token j][32g + 8(r/4) + 4*half + r%4].  The eight
    // A fragments of k-step s+1 are read from LDS while the eight MFMAs of
    // step s run (scheduling barriers pin that order).
    float16_t acc[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) acc[g] = float16_t{};
    half8_t fr[2][8];
    auto read_frags = [&](int s, half8_t (&f)[8]) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f[2 * g] = frag[dense_frag(g, s, 0, lane)];
        f[2 * g + 1] = frag[dense_frag(g, s, 1, lane)];
      }
    };
    read_frags(0, fr[0]);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      if (s + 1 < 8) read_frags(s + 1, fr[(s + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
      const half8_t bx = __builtin_bit_cast(
          half8_t, u32x4_t{xw[4 * s], xw[4 * s + 1], xw[4 * s + 2], xw[4 * s + 3]});
#pragma unroll
      for (int g = 0; g < 4; ++g)
        acc[g] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fr[s & 1][2 * g], bx, acc[g], 0, 0, 0);
#pragma unroll
      for (int g = 0; g < 4; ++g)
        acc[g] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fr[s & 1][2 * g + 1], bx, acc[g], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    uint32_t w0[4], w1[4];
    uint16_t sb[4], zb[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) dense_group_codes(acc[g], w0[g], w1[g], sb[g], zb[g]);
    const int sidx = (int)(it & side_shift);
    const int64_t t = (it >> side_shift) * 32 + j;
    const QuantSide s = sidx ? a.side[1] : a.side[0];
    if (t < a.T_new) {
      const int64_t row = (b * a.Hkv + h) * s.T_cap + a.t_offset + t;
      // lane half h stores code bytes [16h, 16h + 16) of the row (groups 2h,
      // 2h+1): one instruction covers 32 consecutive rows; half 0 stores the
      // four scales, half 1 the four zeros
      const u32x4_t cw = half ? u32x4_t{w0[2], w1[2], w0[3], w1[3]} : u32x4_t{w0[0], w1[0], w0[1], w1[1]};
      __builtin_nontemporal_store(cw, reinterpret_cast<u32x4_t *>(s.codes + row * kCodeBytes) + half);
      const uint16_t *v4 = half ? zb : sb;
      const u32x2_t sv = {(uint32_t)v4[0] | ((uint32_t)v4[1] << 16), (uint32_t)v4[2] | ((uint32_t)v4[3] << 16)};
      uint16_t *dst = half ? s.zeros : s.scales;
      __builtin_nontemporal_store(sv, reinterpret_cast<u32x2_t *>(dst + row * kNGroups));
    }
  };

  // The wave's items are it0, it0 + 4, it0 + 8, ... < i1.  The next tile's
  // inputs are loaded while the current one computes (two register buffers
  // used in turn); a prefetch past the block's items re-reads its last item
  // (unused), which keeps every path's load count the same.
  constexpr int64_t W = kDenseWaves;
  int64_t it = i0 + wave;
  if (it >= i1) return;               // wave-uniform; no barrier follows
  auto clampi = [&](int64_t i) { return i < i1 ? i : i1 - 1; };
  uint32_t xa[32], xb[32];
  load_item(it, xa);
  for (;;) {
    load_item(clampi(it + W), xb);
    __builtin_amdgcn_sched_barrier(0);    // keep the prefetch ahead of the tile's work
    tile(it, xa);
    it += W;
    if (it >= i1) break;
    load_item(clampi(it + W), xa);
    __builtin_amdgcn_sched_barrier(0);
    tile(it, xb);
    it += W;
    if (it >= i1) break;
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
  a.n_items = (int64_t)q.n_sides * ((q.T_new + 31) / 32);
  // about two resident workgroups per CU in total, each with >= 4 tiles per wave
  const int64_t heads = q.B * q.Hkv;
  int64_t chunks = (kDenseTargetBlocks + heads - 1) / heads;
  const int64_t by_items = (a.n_items + kDenseMinItemsPerBlock - 1) / kDenseMinItemsPerBlock;
  if (chunks > by_items) chunks = by_items;
  if (chunks < 1) chunks = 1;
  a.items_per_block = (a.n_items + chunks - 1) / chunks;
  chunks = (a.n_items + a.items_per_block - 1) / a.items_per_block;
  dim3 grid((unsigned)chunks, (unsigned)q.Hkv, (unsigned)q.B);
  hipLaunchKernelGGL(kv_rotate_quant_dense, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace kvq
