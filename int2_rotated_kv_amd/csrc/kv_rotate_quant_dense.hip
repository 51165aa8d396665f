// Write path with a dense per-head rotation (OptR style: one learned
// orthogonal matrix per head, "Output-Aware Rotation for INT2 KV-Cache
// Quantization", woor.ai page, "Key Details"): y = x R_h, then the same
// group quantizer as the Hadamard path, at 2 bits per code or at the
// library's other widths (1 and 4 bits).
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
// both sides.  Wave w computes quantization group w, so its 16 A fragments
// (R_h columns 32w .. 32w+31, hi and lo) stay in registers for the whole
// kernel.  The workgroup stages the inputs of four tiles at a time in LDS
// with fully coalesced loads (16 lanes per 256-byte row), XOR-swizzled so
// that the B-operand reads (one token per lane) hit distinct banks; the next
// four tiles are loaded while the current ones compute.  Output rows are
// assembled in LDS and written with whole-line stores one iteration later
// (per-wave 4-byte pieces left partial lines in the cache and cost extra
// HBM traffic).
#include "kvq_device.h"
#include "kvq_launch.h"

namespace kvq {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));

constexpr int kDenseTiles = 4;                 // 32-token tiles per iteration
constexpr int kDenseSlots = kDenseTiles * 32 * 16;        // 16-byte input chunks per iteration
constexpr int kDenseLoadsPerThread = kDenseSlots / 256;
// output staging per iteration: codes [tile][32 rows][16 b B], then scales
// and zeros [tile][32 rows][8 B] each
constexpr int dense_out_codes(int bits) { return kDenseTiles * 32 * 16 * bits; }
constexpr int dense_out_bytes(int bits) { return dense_out_codes(bits) + 2 * kDenseTiles * 32 * 8; }
constexpr int64_t kDenseTargetBlocks = 512;   // 256 CUs x 2 workgroups
constexpr int64_t kDenseMinItemsPerBlock = 16;

// K-slot (k-step s of 8, lane half h, element i) <-> input channel: lane
// half h supplies input channels [64h, 64h + 64), k-step s the channels
// 64h + 8s .. 64h + 8s + 7.  Any bijection works as long as the A and B
// operands agree; this one lets a lane load its 64 input channels as 128
// contiguous bytes.
__device__ __forceinline__ constexpr int dense_in_channel(int s, int h, int i) { return 64 * h + 8 * s + i; }

// LDS slot (16-byte units) of position p of row r of tile u; the slot holds
// input chunk p ^ (r & 15) of that row (bytes 16c .. 16c+15 for chunk c).
__device__ __forceinline__ constexpr int dense_slot(int u, int r, int p) { return (u * 32 + r) * 16 + p; }

struct DenseKernelArgs {
  QuantSide side[2];
  int64_t stride_b, stride_t, stride_h;
  int64_t T_new, t_offset;
  int Hkv;
  int n_sides;
  int64_t n_items;          // n_sides * 32-token tiles; item i = (side i % n_sides, tile i / n_sides)
  int64_t items_per_block;
  const float *R;           // [Hkv][128][128], y = x R
  const int32_t *offsets;   // per-sequence first slot (device [B]) or NULL: t_offset
  // paged cache: block_table[b * max_pages + t / page_tokens]; NULL: contiguous
  const int32_t *block_table;
  int64_t max_pages, n_pages, page_tokens;
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
// the group.  Returns the group's 4 BITS code bytes in w (dword k = bytes
// 4k .. 4k+3) and its scale / zero bits, identical in both lanes of the pair.
// At 2 bits y[4q .. 4q+3] are the four codes of group byte 2q + half.
//
// The codes follow the exact IEEE fp32 sequence of the format on the
// rotated row y (the matrix cores' fp32 result): s = fp32(fp32(max - min)/L)
// and inv = fp32(1/scale) as correctly rounded divisions, scale = fp16(s),
// zero = fp16(min + 0), code = clamp(rint_half_even(fp32(fp32(y - zero) *
// inv)), 0, L), all codes 0 for a zero scale.  While every group of the
// wave has a normal fp16 scale and |zero| <= 8 scale the argument lies in
// [-0.004, L + 0.012] (the fp16 roundings of the zero and the scale move
// (y - min)/(range/L) by at most 8 2^-11 and L 2^-11), so v_cvt_pk_u8_f32
// (round half to even, saturating below 0) gives the clamped code
// directly; otherwise the argument is clamped to [0, L] and rounded by
// adding 1.5 * 2^23.
template <int BITS>
__device__ __forceinline__ void dense_group_codes(const float16_t &y, uint32_t (&w)[BITS],
                                                  uint16_t &sbits, uint16_t &zbits) {
#pragma clang fp contract(off)
  constexpr int L = (1 << BITS) - 1;
  float mn = y[0], mx = y[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) {
    mn = __builtin_fminf(mn, y[r]);
    mx = __builtin_fmaxf(mx, y[r]);
  }
  mn = pair_min(mn);
  mx = pair_max(mx);
  const float range = mx - mn;
  const float s32 = div_by_levels<L>(range);          // RN(range / L)
  sbits = fp32_value_to_half_bits(s32);
  zbits = float_to_half_bits(mn + 0.0f);
  const float sf = half_bits_to_float(sbits);
  const float zf = half_bits_to_float(zbits);
  const bool degenerate = (sf == 0.0f);
  const float inv = recip_of_half_value(degenerate ? 1.0f : sf);   // RN(1 / scale)
  const bool fast = !__builtin_amdgcn_ballot_w64(fabsf(zf) > 8.0f * sf || sf < kMinNormalHalf);
  // code r of the lane, in byte r/4 of word r%4 (fast) or as 0x4B400000 | code
  uint32_t D[4] = {0u, 0u, 0u, 0u};
  uint32_t cb[16];
  if (fast) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float u = (y[r] - zf) * inv;
      D[r & 3] = __builtin_amdgcn_cvt_pk_u8_f32(u, (uint32_t)(r >> 2), D[r & 3]);
    }
  } else {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float u = (y[r] - zf) * inv;
      const float t = __builtin_amdgcn_fmed3f(u, 0.0f, (float)L);
      cb[r] = float_as_bits(t + kDenseRoundMagic);
    }
  }
  if constexpr (BITS != 2) {
    // D[e] byte q = code of the lane's channel 8q + 4 half + e
    if (!fast) {
#pragma unroll
      for (int r = 0; r < 16; ++r) D[r & 3] |= (cb[r] - 0x4B400000u) << (8 * (r >> 2));
    }
    if constexpr (BITS == 1) {
      // channel 8q + 4 half + e is bit 4 half + e of group byte q
      const uint32_t mine = D[0] | (D[1] << 1) | (D[2] << 2) | (D[3] << 3);
      const auto ex = __builtin_amdgcn_permlane32_swap(mine, mine, false, false);
      w[0] = degenerate ? 0u : (ex[0] | (ex[1] << 4));
    } else {
      // channel 8q + 4 half + e is nibble e % 2 of group byte 4q + 2 half + e / 2
      const uint32_t a = D[0] | (D[1] << 4), c = D[2] | (D[3] << 4);
      const auto ea = __builtin_amdgcn_permlane32_swap(a, a, false, false);
      const auto ec = __builtin_amdgcn_permlane32_swap(c, c, false, false);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        // bytes 4q .. 4q+3: lower half's (a, c) byte q, then the upper half's
        const uint32_t lo = __builtin_amdgcn_perm(ec[0], ea[0], (uint32_t)(q | (q + 4) << 8) | 0x0C0C0000u);
        const uint32_t hi = __builtin_amdgcn_perm(ec[1], ea[1], 0x0C0Cu | (uint32_t)(q << 16 | (q + 4) << 24));
        w[q] = degenerate ? 0u : (lo | hi);
      }
    }
    return;
  }
  uint32_t mine;
  if (fast) {
    mine = D[0] | (D[1] << 2) | (D[2] << 4) | (D[3] << 6);
  } else {
    mine = dense_pack16([&](int r) { return cb[r]; }, 0u) - kDensePackBias;   // byte q = group byte 2q + half
  }
  mine = degenerate ? 0u : mine;
  const auto ex = __builtin_amdgcn_permlane32_swap(mine, mine, false, false);
  const uint32_t e = ex[0], o = ex[1];          // bytes of the lower / upper half
  w[0] = __builtin_amdgcn_perm(o, e, 0x05010400u);   // e0 o0 e1 o1
  w[BITS - 1] = __builtin_amdgcn_perm(o, e, 0x07030602u);   // e2 o2 e3 o3
}

// grid: x = chunk of items, y = KV head, z = batch; 256 threads = four
// waves, one per quantization group.
// At 4 bits two output buffers (2 x 10 KiB) would leave room for only one
// workgroup per CU, so one buffer is used: an iteration's rows leave before
// the next iteration's are staged, one barrier apart.
template <int BITS>
__global__ __launch_bounds__(256, 2) void kv_rotate_quant_dense(DenseKernelArgs a) {
  constexpr int kOutCodes = dense_out_codes(BITS);
  constexpr int kRowBytes = 16 * BITS;
  constexpr int kOutBufs = BITS == 4 ? 1 : 2;
  __shared__ u32x4_t xs[2][kDenseSlots];      // 2 x 32 KiB of staged inputs
  __shared__ __attribute__((aligned(16))) uint8_t out[kOutBufs][dense_out_bytes(BITS)];   // (4 + 2 b) KiB each
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int g = __builtin_amdgcn_readfirstlane(tid >> 6);   // this wave's group
  const int h = blockIdx.y;
  const int64_t b = blockIdx.z;
  const int j = lane & 31;            // token column of a tile
  const int half = lane >> 5;

  // A fragments of group g: rf[s][part] of lane (m = j, kh = half) holds
  // R[dense_in_channel(s, half, i)][32g + j], i = 0..7, as fp16 hi / lo.
  half8_t rf[8][2];
  {
    const float *R = a.R + (int64_t)h * kD * kD + 32 * g + j;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float r = R[dense_in_channel(s, half, i) * kD];
        rf[s][0][i] = (_Float16)r;
        rf[s][1][i] = (_Float16)(r - (float)rf[s][0][i]);
      }
    }
  }

  const int64_t i0 = (int64_t)blockIdx.x * a.items_per_block;
  const int64_t i1 = (i0 + a.items_per_block < a.n_items) ? i0 + a.items_per_block : a.n_items;
  const int64_t n_iter = (i1 - i0 + kDenseTiles - 1) / kDenseTiles;
  const int side_shift = a.n_sides - 1;                   // n_sides is 1 or 2

  // Loads of iteration k: thread tid fetches slots q = c*256 + tid.  Items
  // past the block's range re-read its last item (results unused).
  auto load_iter = [&](int64_t k, u32x4_t (&P)[kDenseLoadsPerThread]) {
#pragma unroll
    for (int c = 0; c < kDenseLoadsPerThread; ++c) {
      const int q = c * 256 + tid;
      const int u = q >> 9, r = (q >> 4) & 31, p = q & 15;
      int64_t it = i0 + k * kDenseTiles + u;
      it = it < i1 ? it : i1 - 1;
      const QuantSide sd = (it & side_shift) ? a.side[1] : a.side[0];
      const int64_t t0 = (it >> side_shift) * 32;
      const int64_t t = (t0 + r < a.T_new) ? t0 + r : a.T_new - 1;
      const u32x4_t *src = reinterpret_cast<const u32x4_t *>(
          reinterpret_cast<const _Float16 *>(sd.x) + b * a.stride_b + t * a.stride_t +
          (int64_t)h * a.stride_h) + (p ^ (r & 15));
      P[c] = __builtin_nontemporal_load(src);
    }
  };
  auto stage = [&](int buf, const u32x4_t (&P)[kDenseLoadsPerThread]) {
#pragma unroll
    for (int c = 0; c < kDenseLoadsPerThread; ++c) xs[buf][c * 256 + tid] = P[c];
  };

  // Output rows of iteration k (from LDS buffer ob) go to the cache: 16-byte
  // code chunk c (piece c % BITS of row (c / BITS) % 32 of tile c / (32 BITS))
  // from thread c % 256, and 8 bytes of scales (tid < 128) or zeros.
  auto store_out = [&](int64_t k, const uint8_t *ob) {
#pragma unroll
    for (int c = tid; c < kOutCodes / 16; c += 256) {
      const int u = c / (32 * BITS), r = (c % (32 * BITS)) / BITS, piece = c % BITS;
      const int64_t it = i0 + k * kDenseTiles + u;
      const QuantSide sd = (it & side_shift) ? a.side[1] : a.side[0];
      const int64_t t = (it >> side_shift) * 32 + r;
      const int64_t slot = seq_offset(a.offsets, a.t_offset, b) + t;
      if (it < i1 && t < a.T_new && slot >= 0 && slot < sd.T_cap) {   // per-sequence slot inside the cache
        const int64_t row = write_row(a.block_table, a.max_pages, a.n_pages, a.page_tokens, a.Hkv, b, h,
                                      sd.T_cap, slot);
        if (row >= 0)                                // a page outside the pool is skipped
          __builtin_nontemporal_store(*reinterpret_cast<const u32x4_t *>(ob + 16 * c),
                                      reinterpret_cast<u32x4_t *>(sd.codes + row * kRowBytes) + piece);
      }
    }
    {
      const int zs = tid >> 7, u = (tid >> 5) & 3, r = tid & 31;
      const int64_t it = i0 + k * kDenseTiles + u;
      const QuantSide sd = (it & side_shift) ? a.side[1] : a.side[0];
      const int64_t t = (it >> side_shift) * 32 + r;
      const int64_t slot = seq_offset(a.offsets, a.t_offset, b) + t;
      const int64_t row = (it < i1 && t < a.T_new && slot >= 0 && slot < sd.T_cap)   // per-sequence slot inside the cache
                              ? write_row(a.block_table, a.max_pages, a.n_pages, a.page_tokens, a.Hkv, b, h,
                                          sd.T_cap, slot)
                              : -1;
      if (row >= 0) {
        uint16_t *dst = zs ? sd.zeros : sd.scales;
        __builtin_nontemporal_store(
            *reinterpret_cast<const u32x2_t *>(ob + kOutCodes + zs * kDenseTiles * 256 + (u * 32 + r) * 8),
            reinterpret_cast<u32x2_t *>(dst + row * kNGroups));
      }
    }
  };

  // MFMAs and quantization of the iteration's tiles for group g into the
  // output staging buffer ob; stage_next runs after that, then store_prev.
  auto compute = [&](int buf, uint8_t *ob, auto &&stage_next, auto &&store_prev) {
    float16_t acc[kDenseTiles];
#pragma unroll
    for (int u = 0; u < kDenseTiles; ++u) acc[u] = float16_t{};
    half8_t bx[2][kDenseTiles];
    auto read_b = [&](int s, half8_t (&dst)[kDenseTiles]) {
      const int pos = (8 * half + s) ^ (j & 15);
#pragma unroll
      for (int u = 0; u < kDenseTiles; ++u) dst[u] = __builtin_bit_cast(half8_t, xs[buf][dense_slot(u, j, pos)]);
    };
    read_b(0, bx[0]);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      if (s + 1 < 8) read_b(s + 1, bx[(s + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < kDenseTiles; ++u)
        acc[u] = __builtin_amdgcn_mfma_f32_32x32x16_f16(rf[s][0], bx[s & 1][u], acc[u], 0, 0, 0);
#pragma unroll
      for (int u = 0; u < kDenseTiles; ++u)
        acc[u] = __builtin_amdgcn_mfma_f32_32x32x16_f16(rf[s][1], bx[s & 1][u], acc[u], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    // acc[u][r] = y[token j of tile u][32g + 8(r/4) + 4*half + r%4]; half 0
    // puts group bytes 0..3 and the scale in the row, half 1 bytes 4..7 and
    // the zero
#pragma unroll
    for (int u = 0; u < kDenseTiles; ++u) {
      uint32_t w[BITS];
      uint16_t sb, zb;
      dense_group_codes<BITS>(acc[u], w, sb, zb);
      // group g's 4 BITS code bytes: each half of the lane pair writes half
      // of them (at 1 bit, the lower half writes the one dword)
      uint8_t *gc = ob + (u * 32 + j) * kRowBytes + 4 * BITS * g;
      if constexpr (BITS == 4) {
        *reinterpret_cast<u32x2_t *>(gc + 8 * half) = half ? u32x2_t{w[2], w[3]} : u32x2_t{w[0], w[1]};
      } else if constexpr (BITS == 2) {
        *reinterpret_cast<uint32_t *>(gc + 4 * half) = half ? w[1] : w[0];
      } else {
        if (half == 0) *reinterpret_cast<uint32_t *>(gc) = w[0];
      }
      *reinterpret_cast<uint16_t *>(ob + kOutCodes + half * kDenseTiles * 256 + (u * 32 + j) * 8 + 2 * g) =
          half ? zb : sb;
    }
    // Loads are waited for before the stores are issued: those waits also
    // cover every earlier memory operation, stores included.
    stage_next();
    store_prev();
  };

  u32x4_t P[kDenseLoadsPerThread];
  load_iter(0, P);
  stage(0, P);
  __syncthreads();
  for (int64_t k = 0; k < n_iter; ++k) {              // block-uniform trip count
    const bool more = k + 1 < n_iter;
    if (more) load_iter(k + 1, P);
    if constexpr (kOutBufs == 1) {
      // the previous iteration's rows leave before this one's are staged
      if (k > 0) {
        store_out(k - 1, out[0]);
        __syncthreads();
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // buffers last read before the previous barrier: input (k+1)&1, output k&1
    compute((int)(k & 1), out[k & (kOutBufs - 1)],
            [&] { if (more) stage((int)((k + 1) & 1), P); },
            [&] { if (kOutBufs == 2 && k > 0) store_out(k - 1, out[(k - 1) & (kOutBufs - 1)]); });
    __syncthreads();
  }
  store_out(n_iter - 1, out[(n_iter - 1) & (kOutBufs - 1)]);   // published by the last barrier
}

// Both sides at one code width.
static hipError_t launch_quantize_dense_one(const QuantArgs &q, hipStream_t stream) {
  DenseKernelArgs a;
  a.side[0] = q.side[0];
  a.side[1] = q.n_sides > 1 ? q.side[1] : q.side[0];
  a.stride_b = q.stride_b;
  a.stride_t = q.stride_t;
  a.stride_h = q.stride_h;
  a.T_new = q.T_new;
  a.t_offset = q.t_offset;
  a.offsets = q.offsets;
  a.block_table = q.block_table;
  a.max_pages = q.max_pages;
  a.n_pages = q.n_pages;
  a.page_tokens = q.page_tokens;
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
  switch (a.side[0].bits) {
    case 1: hipLaunchKernelGGL(kv_rotate_quant_dense<1>, grid, dim3(256), 0, stream, a); break;
    case 4: hipLaunchKernelGGL(kv_rotate_quant_dense<4>, grid, dim3(256), 0, stream, a); break;
    default: hipLaunchKernelGGL(kv_rotate_quant_dense<2>, grid, dim3(256), 0, stream, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_quantize_dense(const QuantArgs &q, hipStream_t stream) {
  // sides of different code widths: one launch each
  if (q.n_sides == 2 && q.side[0].bits != q.side[1].bits) {
    for (int sd = 0; sd < 2; ++sd) {
      QuantArgs q1 = q;
      q1.side[0] = q.side[sd];
      q1.n_sides = 1;
      const hipError_t e = launch_quantize_dense_one(q1, stream);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  return launch_quantize_dense_one(q, stream);
}

}  // namespace kvq
