// Read path: decode attention over the packed INT2 cache (gfx950, wave64).
//
// out = softmax(scale * (q R) . k_hat) v_hat R^T, jointly normalized with
// optional fp16 sink / residual tokens kept in the original basis.  The
// readout is scaled dot-product attention and the rotation is removed
// after the attention computation ("Output-Aware Rotation for INT2
// KV-Cache Quantization", woor.ai page, "What You Need to Know" and "Key
// Details"); sinks stay unquantized (RotateKV abstract, item (iii)).
//
// Three launches on the caller's stream:
//   1. kv_prep_query     per (b, query head): q' = q R (FWHT or dense), scaled
//                        by softmax_scale*log2(e), turned into a per-group
//                        19-bit fixed-point vector split into five signed
//                        4-bit limbs.
//   2. kv_int2_decode_attn  one wave per (b, kv head, token split): flash-
//                        decoding over its tokens with an online softmax; every
//                        loaded K/V row serves all G query heads of the group.
//   3. kv_combine_unrotate  per (b, query head): log-sum-exp merge of the wave
//                        partials staged through LDS, un-rotation by R^T
//                        (linear, so applied once after the merge), fp16
//                        tokens, normalization, store.
//
// Scores never dequantize a key: with per-group scale s and zero z,
//   q'.k_hat = sum_j s_j * (sum_{c in j} q'_c code_c) + z_j * (sum_{c in j} q'_c),
// and the inner sum is an exact int32 dot product (v_dot8 on 4-bit code
// nibbles and 4-bit query limbs).  Values: with w_t = fp16(p_t s_{t,j}),
//   o'_c = sum_t w_t code_{t,c} - 1.5 sum_t w_t + sum_t p_t (z_{t,j} + 1.5 s_{t,j});
// the first term runs as v_dot2 over token pairs with codes placed in fp16
// subnormal encodings (code * 2^(e-24)), accumulated in fp32.  Centering the
// codes on 1.5 makes the fp16 rounding of w multiply code - 1.5 in
// [-1.5, 1.5], so it does not get amplified by the cancellation between the
// code and zero-point terms.
#include "kvq_device.h"
#include "kvq_launch.h"

namespace kvq {

constexpr float kNegInf = -__builtin_huge_valf();

// ---------------------------------------------------------------------------
// 128-point normalized FWHT / dense rotation across a 128-thread block (LDS)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float block_fwht128(float x, float *buf) {
  const int c = threadIdx.x;
  buf[c] = x;
  __syncthreads();
#pragma unroll
  for (int h = 1; h < 128; h <<= 1) {
    if (c < 64) {
      const int i = (c / h) * (2 * h) + (c % h);
      const float a = buf[i], b = buf[i + h];
      buf[i] = a + b;
      buf[i + h] = a - b;
    }
    __syncthreads();
  }
  const float y = buf[c] * 0.08838834764831845f;
  __syncthreads();
  return y;
}

// y_c = sum_k x_k M[k][c]  (transpose=false)  or  sum_k x_k M[c][k] (true)
__device__ __forceinline__ float block_matvec128(float x, const float *__restrict__ M,
                                                 bool transpose, float *buf) {
  const int c = threadIdx.x;
  buf[c] = x;
  __syncthreads();
  float acc = 0.0f;
  if (!transpose) {
#pragma unroll 8
    for (int k = 0; k < 128; ++k) acc = __builtin_fmaf(buf[k], M[k * 128 + c], acc);
  } else {
#pragma unroll 8
    for (int k = 0; k < 128; ++k) acc = __builtin_fmaf(buf[k], M[c * 128 + k], acc);
  }
  __syncthreads();
  return acc;
}

// ---------------------------------------------------------------------------
// 1. query preparation
// ---------------------------------------------------------------------------
struct PrepArgs {
  const void *q;
  bool q_f32;
  int Hq, Hkv;
  int rot;
  const float *R;
  float qscale;
  uint8_t *qprep;    // [B][Hq][128 dwords]
};


// grid: B*Hq blocks of 128 threads; thread c owns channel c.
__global__ __launch_bounds__(128) void kv_prep_query(PrepArgs a) {
  __shared__ float buf[128];
  const int c = threadIdx.x;
  const int64_t bh = blockIdx.x;            // b*Hq + hq
  const int hq = (int)(bh % a.Hq);
  const int hkv = hq / (a.Hq / a.Hkv);
  float x = a.q_f32 ? reinterpret_cast<const float *>(a.q)[bh * kD + c]
                    : (float)reinterpret_cast<const _Float16 *>(a.q)[bh * kD + c];
  if (a.rot == 1) x = block_fwht128(x, buf);
  else if (a.rot == 2) x = block_matvec128(x, a.R + (int64_t)hkv * kD * kD, false, buf);
  x *= a.qscale;

  // per-group (32 lanes) maximum magnitude -> exponent of the fixed point
  float amax = fabsf(x);
#pragma unroll
  for (int m = 1; m < 32; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 32));
  int e = 0;
  (void)frexpf(amax, &e);                    // amax < 2^e
  const bool zero_group = !(amax > 0.0f);
  const int E = 18 - e;                      // |x| * 2^E < 2^18
  const int qi = zero_group ? 0 : (int)__builtin_rintf(ldexpf(x, E));
  const float step = zero_group ? 0.0f : ldexpf(1.0f, -E);
  int isum = qi;
#pragma unroll
  for (int m = 1; m < 32; m <<= 1) isum += __shfl_xor(isum, m, 32);

  // balanced base-16 digits in [-8, 7]: qi = sum_L d_L * 16^(4-L), L = 0 most
  // significant.  |qi| <= 2^18 fits five digits.
  int dig[5];
  int r = qi;
#pragma unroll
  for (int L = 4; L >= 0; --L) {
    const int dl = ((r + 8) & 15) - 8;
    dig[L] = dl;
    r = (r - dl) >> 4;
  }

  // Codes arrive as nibbles: of a code dword w (channels 16w..16w+15 of the
  // group), the masked copy (w & 0x33333333) holds channel 16w + 2k in nibble
  // k and ((w >> 2) & 0x33333333) holds channel 16w + 2k + 1.  Limb dword
  // (L, w, parity) packs the matching digits of the query the same way.
  const int j = c >> 5, cg = c & 31;
  const int w = cg >> 4, par = cg & 1, k = (cg & 15) >> 1;
  uint32_t *base = reinterpret_cast<uint32_t *>(a.qprep) + bh * kQprepDwordsPerHead + j * 32;
  // assemble limb dwords with a 16-lane OR-reduction of shifted digits
#pragma unroll
  for (int L = 0; L < 5; ++L) {
    uint32_t part = ((uint32_t)dig[L] & 15u) << (4 * k);
    // lanes of one dword: same (w, par), k = 0..7 -> lane offsets 2k within cg
    part |= __shfl_xor(part, 2, 32);
    part |= __shfl_xor(part, 4, 32);
    part |= __shfl_xor(part, 8, 32);
    if (k == 0) base[L * 4 + w * 2 + par] = part;
  }
  if (cg == 0) {
    float *fb = reinterpret_cast<float *>(base);
    fb[24] = (float)isum * step;             // sum of the group's fixed-point q
    fb[25] = step;
  }
}

// ---------------------------------------------------------------------------
// 2. split-K attention over INT2 tokens
// ---------------------------------------------------------------------------
struct AttnArgs {
  const uint8_t *kcodes; const uint16_t *kscales; const uint16_t *kzeros; int64_t kT_cap;
  const uint8_t *vcodes; const uint16_t *vscales; const uint16_t *vzeros; int64_t vT_cap;
  int64_t t_begin, n_int2;
  int64_t n_splits, tps;
  int64_t total_waves;
  int Hkv, Hq, G, g0;   // heads [g0, g0 + GC) of each group
  const uint32_t *qprep;
  float *partials;
};

// Reassemble the fp16 subnormal channel factor: code at position x of a
// 16-bit half is read with weight 2^(2x-24) (x <= 4) or 2^(2x-30) (x >= 5).
__device__ __forceinline__ constexpr float chan_unscale(int x) {
  return x <= 4 ? (float)(1u << (24 - 2 * x)) : (float)(1u << (30 - 2 * x));
}

// Lane layout of the attention kernel: lane l handles token slot ts = l/2 of
// a 64-token tile (tokens ts and 32 + ts) on channel half h = l%2, i.e. the
// two groups 2h and 2h+1 (64 channels).  Codes arrive as one 16-byte load
// per token and lane (1 KB per wave instruction); scales and zeros as one
// 4-byte load (both groups) per token and lane.
struct TileRegs {
  u32x4_t kA, kB, vA, vB;          // codes of tokens A (= ts) and B (= 32 + ts)
  uint32_t ksA, kzA, ksB, kzB;     // two fp16 scales / zeros each
  uint32_t vsA, vzA, vsB, vzB;
};

template <int GC>
struct AttnState {
  float m[GC], l[GC], zacc[GC][2], wsum[GC][2], acc[GC][64];
};

constexpr uint32_t kHalf2Ones = 0x3C003C00u;   // (1.0, 1.0) in fp16

// Per-lane query data for the lane's two channel groups of GC heads.
template <int GC>
struct QueryLimbs {
  uint32_t limb[GC][2][20];   // [head][group in half][L*4 + w*2 + parity]
  float qsum[GC][2], qstep[GC][2];
};

__device__ __forceinline__ float lo_half(uint32_t w) { return half_bits_to_float((uint16_t)(w & 0xFFFFu)); }
__device__ __forceinline__ float hi_half(uint32_t w) { return half_bits_to_float((uint16_t)(w >> 16)); }

// exact int32 dot product of one group's 32 codes (two code dwords) with the
// five 4-bit limbs of the fixed-point query
__device__ __forceinline__ int group_dot(const uint32_t (&limb)[20], uint32_t c0, uint32_t c1) {
  const uint32_t n[4] = {c0 & 0x33333333u, (c0 >> 2) & 0x33333333u,
                         c1 & 0x33333333u, (c1 >> 2) & 0x33333333u};
  int acc = 0;
#pragma unroll
  for (int L = 0; L < 5; ++L) {
    if (L) acc <<= 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_sdot8((int)limb[4 * L + i], (int)n[i], acc, false);
  }
  return acc;
}

template <int GC>
__device__ __forceinline__ void attn_tile(AttnState<GC> &st, const QueryLimbs<GC> &q,
                                          const TileRegs &r, bool va, bool vb) {
  const uint32_t kAw[4] = {r.kA.x, r.kA.y, r.kA.z, r.kA.w};
  const uint32_t kBw[4] = {r.kB.x, r.kB.y, r.kB.z, r.kB.w};
  half2_t wp[GC][2];
#pragma unroll
  for (int g = 0; g < GC; ++g) {
    float sa = 0.0f, sb = 0.0f;
#pragma unroll
    for (int gi = 0; gi < 2; ++gi) {
      const int ia = group_dot(q.limb[g][gi], kAw[2 * gi], kAw[2 * gi + 1]);
      const int ib = group_dot(q.limb[g][gi], kBw[2 * gi], kBw[2 * gi + 1]);
      const float skA = gi ? hi_half(r.ksA) : lo_half(r.ksA);
      const float zkA = gi ? hi_half(r.kzA) : lo_half(r.kzA);
      const float skB = gi ? hi_half(r.ksB) : lo_half(r.ksB);
      const float zkB = gi ? hi_half(r.kzB) : lo_half(r.kzB);
      sa += __builtin_fmaf((float)ia, skA * q.qstep[g][gi], zkA * q.qsum[g][gi]);
      sb += __builtin_fmaf((float)ib, skB * q.qstep[g][gi], zkB * q.qsum[g][gi]);
    }
    sa += quad_swap<kQuadXor1>(sa);          // the other half of the row
    sb += quad_swap<kQuadXor1>(sb);
    sa = va ? sa : kNegInf;
    sb = vb ? sb : kNegInf;

    // online softmax (log2 domain); the tile max is wave-uniform
    float mx = fmaxf(sa, sb);
    mx = fmaxf(mx, row_ror<2>(mx));
    mx = fmaxf(mx, row_ror<4>(mx));
    mx = fmaxf(mx, row_ror<8>(mx));
    mx = fmaxf(mx, shfl_xor_f(mx, 16));
    mx = fmaxf(mx, shfl_xor_f(mx, 32));
    if (mx > st.m[g]) {
      const float alpha = __builtin_amdgcn_exp2f(st.m[g] - mx);
      st.l[g] *= alpha;
      st.zacc[g][0] *= alpha;
      st.zacc[g][1] *= alpha;
      st.wsum[g][0] *= alpha;
      st.wsum[g][1] *= alpha;
#pragma unroll
      for (int i = 0; i < 64; ++i) st.acc[g][i] *= alpha;
      st.m[g] = mx;
    }
    const float pA = __builtin_amdgcn_exp2f(sa - st.m[g]);   // 0 for masked tokens
    const float pB = __builtin_amdgcn_exp2f(sb - st.m[g]);
    st.l[g] += pA + pB;
#pragma unroll
    for (int gi = 0; gi < 2; ++gi) {
      const float svA = gi ? hi_half(r.vsA) : lo_half(r.vsA);
      const float zvA = gi ? hi_half(r.vzA) : lo_half(r.vzA);
      const float svB = gi ? hi_half(r.vsB) : lo_half(r.vsB);
      const float zvB = gi ? hi_half(r.vzB) : lo_half(r.vzB);
      st.zacc[g][gi] = __builtin_fmaf(pA, __builtin_fmaf(1.5f, svA, zvA),
                                      __builtin_fmaf(pB, __builtin_fmaf(1.5f, svB, zvB), st.zacc[g][gi]));
      wp[g][gi].x = (_Float16)(pA * svA);
      wp[g][gi].y = (_Float16)(pB * svB);
      st.wsum[g][gi] = __builtin_amdgcn_fdot2(wp[g][gi], __builtin_bit_cast(half2_t, kHalf2Ones),
                                              st.wsum[g][gi], false);
    }
  }

  // V: token pair (A in the low half, B in the high half) per channel
  const uint32_t vAw[4] = {r.vA.x, r.vA.y, r.vA.z, r.vA.w};
  const uint32_t vBw[4] = {r.vB.x, r.vB.y, r.vB.z, r.vB.w};
#pragma unroll
  for (int d = 0; d < 4; ++d) {               // code dword d: group d/2, dword w = d%2
    const int gi = d >> 1, w = d & 1;
    const uint32_t X = __builtin_amdgcn_perm(vBw[d], vAw[d], 0x05040100u);   // lo16(A) | lo16(B) << 16
    const uint32_t Y = __builtin_amdgcn_perm(vBw[d], vAw[d], 0x07060302u);   // hi16(A) | hi16(B) << 16
    const uint32_t X6 = X >> 6, Y6 = Y >> 6;
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      const uint32_t px = x <= 4 ? (X & (0x00030003u << (2 * x))) : (X6 & (0x00030003u << (2 * x - 6)));
      const uint32_t py = x <= 4 ? (Y & (0x00030003u << (2 * x))) : (Y6 & (0x00030003u << (2 * x - 6)));
      const half2_t hx = __builtin_bit_cast(half2_t, px);
      const half2_t hy = __builtin_bit_cast(half2_t, py);
#pragma unroll
      for (int g = 0; g < GC; ++g) {
        float &ax = st.acc[g][32 * gi + 16 * w + x];
        float &ay = st.acc[g][32 * gi + 16 * w + 8 + x];
        ax = __builtin_amdgcn_fdot2(hx, wp[g][gi], ax, false);
        ay = __builtin_amdgcn_fdot2(hy, wp[g][gi], ay, false);
      }
    }
  }
}

template <int GC>
__global__ __launch_bounds__(256) void kv_int2_decode_attn(AttnArgs a) {
  const int lane = threadIdx.x & 63;
  // wave index made explicitly uniform so every per-wave quantity is scalar
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t gw = (int64_t)blockIdx.x * 4 + wave;
  if (gw >= a.total_waves) return;           // whole wave leaves together
  const int64_t split = gw % a.n_splits;
  const int64_t bh = gw / a.n_splits;        // b*Hkv + hkv
  const int hkv = (int)(bh % a.Hkv);
  const int64_t b = bh / a.Hkv;
  const int ts = lane >> 1;                  // token slot 0..31
  const int h = lane & 1;                    // channel half: groups 2h, 2h+1
  const int64_t s0 = split * a.tps;
  const int64_t s1 = (s0 + a.tps < a.n_int2) ? s0 + a.tps : a.n_int2;

  QueryLimbs<GC> q;
#pragma unroll
  for (int g = 0; g < GC; ++g) {
    const int hq = hkv * a.G + a.g0 + g;
#pragma unroll
    for (int gi = 0; gi < 2; ++gi) {
      const uint32_t *p = a.qprep + (b * a.Hq + hq) * kQprepDwordsPerHead + (2 * h + gi) * 32;
#pragma unroll
      for (int i = 0; i < 20; ++i) q.limb[g][gi][i] = p[i];
      q.qsum[g][gi] = bits_as_float(p[24]);
      q.qstep[g][gi] = bits_as_float(p[25]);
    }
  }

  AttnState<GC> st;
#pragma unroll
  for (int g = 0; g < GC; ++g) {
    st.m[g] = kNegInf; st.l[g] = 0.0f; st.zacc[g][0] = 0.0f; st.zacc[g][1] = 0.0f;
    st.wsum[g][0] = 0.0f; st.wsum[g][1] = 0.0f;
#pragma unroll
    for (int i = 0; i < 64; ++i) st.acc[g][i] = 0.0f;
  }

  // Row r of the split: codes at *c + r*32 bytes, scales/zeros at *s + r*4
  // halves.  Lane offsets are 32-bit; tile bases are wave-uniform.
  const int64_t krow0 = bh * a.kT_cap + a.t_begin + s0;
  const int64_t vrow0 = bh * a.vT_cap + a.t_begin + s0;
  const uint8_t *kc = a.kcodes + krow0 * kCodeBytes;
  const uint8_t *vc = a.vcodes + vrow0 * kCodeBytes;
  const uint16_t *ks = a.kscales + krow0 * kNGroups, *kz = a.kzeros + krow0 * kNGroups;
  const uint16_t *vs = a.vscales + vrow0 * kNGroups, *vz = a.vzeros + vrow0 * kNGroups;
  const int64_t n = s1 - s0;
  const int64_t nfull = n & ~(int64_t)63;

  // Loads of one lane: codes at tile base + oc (+1 KB for token B), scales
  // and zeros at tile base + os halves (+64 halves for token B).  Tile bases
  // are wave-uniform, lane offsets 32-bit.
  const uint32_t oc = (uint32_t)(ts * kCodeBytes + 16 * h);
  const uint32_t os = (uint32_t)(ts * kNGroups + 2 * h);
  auto load_tile = [&](int64_t first_row) {
    TileRegs r;
    const uint8_t *kct = kc + first_row * kCodeBytes, *vct = vc + first_row * kCodeBytes;
    const uint16_t *kst = ks + first_row * kNGroups, *kzt = kz + first_row * kNGroups;
    const uint16_t *vst = vs + first_row * kNGroups, *vzt = vz + first_row * kNGroups;
    r.kA = *reinterpret_cast<const u32x4_t *>(kct + oc);
    r.kB = *reinterpret_cast<const u32x4_t *>(kct + oc + 32 * kCodeBytes);
    r.vA = *reinterpret_cast<const u32x4_t *>(vct + oc);
    r.vB = *reinterpret_cast<const u32x4_t *>(vct + oc + 32 * kCodeBytes);
    r.ksA = *reinterpret_cast<const uint32_t *>(kst + os);
    r.kzA = *reinterpret_cast<const uint32_t *>(kzt + os);
    r.ksB = *reinterpret_cast<const uint32_t *>(kst + os + 32 * kNGroups);
    r.kzB = *reinterpret_cast<const uint32_t *>(kzt + os + 32 * kNGroups);
    r.vsA = *reinterpret_cast<const uint32_t *>(vst + os);
    r.vzA = *reinterpret_cast<const uint32_t *>(vzt + os);
    r.vsB = *reinterpret_cast<const uint32_t *>(vst + os + 32 * kNGroups);
    r.vzB = *reinterpret_cast<const uint32_t *>(vzt + os + 32 * kNGroups);
    return r;
  };

  // Full tiles, software-pipelined two deep: while tile i is computed the
  // loads of tile i+1 are in flight.  A prefetch past the last full tile is
  // clamped to it (a re-read of valid rows, result unused).
  const int64_t ntiles = nfull >> 6;
  if (ntiles > 0) {
    const int64_t last = ntiles - 1;
    TileRegs r0 = load_tile(0), r1;
    int64_t i = 0;
    for (; i + 2 <= ntiles; i += 2) {
      r1 = load_tile(64 * (i + 1));
      attn_tile<GC>(st, q, r0, true, true);
      r0 = load_tile(64 * (i + 2 < last ? i + 2 : last));
      attn_tile<GC>(st, q, r1, true, true);
    }
    if (i < ntiles) attn_tile<GC>(st, q, r0, true, true);
  }
  if (nfull < n) {                          // tail tile: clamp rows into the split
    const int64_t ta = nfull + ts, tb = nfull + 32 + ts;
    const bool va = ta < n, vb = tb < n;
    const int64_t ra = va ? ta : 0, rb = vb ? tb : 0;
    TileRegs r;
    r.kA = *reinterpret_cast<const u32x4_t *>(kc + ra * kCodeBytes + 16 * h);
    r.kB = *reinterpret_cast<const u32x4_t *>(kc + rb * kCodeBytes + 16 * h);
    r.vA = *reinterpret_cast<const u32x4_t *>(vc + ra * kCodeBytes + 16 * h);
    r.vB = *reinterpret_cast<const u32x4_t *>(vc + rb * kCodeBytes + 16 * h);
    r.ksA = *reinterpret_cast<const uint32_t *>(ks + ra * kNGroups + 2 * h);
    r.kzA = *reinterpret_cast<const uint32_t *>(kz + ra * kNGroups + 2 * h);
    r.ksB = *reinterpret_cast<const uint32_t *>(ks + rb * kNGroups + 2 * h);
    r.kzB = *reinterpret_cast<const uint32_t *>(kz + rb * kNGroups + 2 * h);
    r.vsA = *reinterpret_cast<const uint32_t *>(vs + ra * kNGroups + 2 * h);
    r.vzA = *reinterpret_cast<const uint32_t *>(vz + ra * kNGroups + 2 * h);
    r.vsB = *reinterpret_cast<const uint32_t *>(vs + rb * kNGroups + 2 * h);
    r.vzB = *reinterpret_cast<const uint32_t *>(vz + rb * kNGroups + 2 * h);
    attn_tile<GC>(st, q, r, va, vb);
  }

  // reduce over the 32 token slots (lanes sharing h), then write the partial
#pragma unroll
  for (int g = 0; g < GC; ++g) {
    float l = st.l[g];
    float z0 = __builtin_fmaf(-1.5f, st.wsum[g][0], st.zacc[g][0]);
    float z1 = __builtin_fmaf(-1.5f, st.wsum[g][1], st.zacc[g][1]);
#pragma unroll
    for (int msk = 2; msk < 64; msk <<= 1) {
      l += shfl_xor_f(l, msk);
      z0 += shfl_xor_f(z0, msk);
      z1 += shfl_xor_f(z1, msk);
#pragma unroll
      for (int i = 0; i < 64; ++i) st.acc[g][i] += shfl_xor_f(st.acc[g][i], msk);
    }
    if (ts == 0) {
      const int hq = hkv * a.G + a.g0 + g;
      float *dst = a.partials + ((b * a.Hq + hq) * a.n_splits + split) * kPartialStride;
#pragma unroll
      for (int i = 0; i < 64; ++i) {
        const int x = i & 7;
        dst[64 * h + i] = __builtin_fmaf(st.acc[g][i], chan_unscale(x), i < 32 ? z0 : z1);
      }
      if (h == 0) {
        dst[128] = st.m[g];
        dst[129] = l;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// GQA variant: lane (ts, j) = (l/4, l%4) handles tokens ts and 16 + ts of a
// 32-token tile on channel group j for GC query heads at once, so each
// loaded K/V code serves GC heads.  Registers allow GC = 2 with a three-deep
// load pipeline.
// ---------------------------------------------------------------------------
struct QuadTileRegs {
  uint2 kA, kB, vA, vB;
  uint16_t h[8];   // kscale A, kzero A, kscale B, kzero B, vscale A, vzero A, vscale B, vzero B
};

template <int GC>
struct QuadState {
  float m[GC], l[GC], zacc[GC], wsum[GC], acc[GC][32];
};

template <int GC>
struct QuadQuery {
  uint32_t limb[GC][20];
  float qsum[GC], qstep[GC];
};

template <int GC>
__device__ __forceinline__ void quad_tile(QuadState<GC> &st, const QuadQuery<GC> &q,
                                          const QuadTileRegs &r, bool va, bool vb) {
  const float skA = half_bits_to_float(r.h[0]), zkA = half_bits_to_float(r.h[1]);
  const float skB = half_bits_to_float(r.h[2]), zkB = half_bits_to_float(r.h[3]);
  const float svA = half_bits_to_float(r.h[4]), zvA = half_bits_to_float(r.h[5]);
  const float svB = half_bits_to_float(r.h[6]), zvB = half_bits_to_float(r.h[7]);
  half2_t wp[GC];
#pragma unroll
  for (int g = 0; g < GC; ++g) {
    const int ia = group_dot(q.limb[g], r.kA.x, r.kA.y);
    const int ib = group_dot(q.limb[g], r.kB.x, r.kB.y);
    float sa = __builtin_fmaf((float)ia, skA * q.qstep[g], zkA * q.qsum[g]);
    float sb = __builtin_fmaf((float)ib, skB * q.qstep[g], zkB * q.qsum[g]);
    sa += quad_swap<kQuadXor1>(sa);
    sb += quad_swap<kQuadXor1>(sb);
    sa += quad_swap<kQuadXor2>(sa);
    sb += quad_swap<kQuadXor2>(sb);
    sa = va ? sa : kNegInf;
    sb = vb ? sb : kNegInf;
    float mx = fmaxf(sa, sb);
    mx = fmaxf(mx, row_ror<4>(mx));
    mx = fmaxf(mx, row_ror<8>(mx));
    mx = fmaxf(mx, shfl_xor_f(mx, 16));
    mx = fmaxf(mx, shfl_xor_f(mx, 32));
    if (mx > st.m[g]) {
      const float alpha = __builtin_amdgcn_exp2f(st.m[g] - mx);
      st.l[g] *= alpha;
      st.zacc[g] *= alpha;
      st.wsum[g] *= alpha;
#pragma unroll
      for (int i = 0; i < 32; ++i) st.acc[g][i] *= alpha;
      st.m[g] = mx;
    }
    const float pA = __builtin_amdgcn_exp2f(sa - st.m[g]);
    const float pB = __builtin_amdgcn_exp2f(sb - st.m[g]);
    st.l[g] += pA + pB;
    st.zacc[g] = __builtin_fmaf(pA, __builtin_fmaf(1.5f, svA, zvA),
                                __builtin_fmaf(pB, __builtin_fmaf(1.5f, svB, zvB), st.zacc[g]));
    wp[g].x = (_Float16)(pA * svA);
    wp[g].y = (_Float16)(pB * svB);
    st.wsum[g] = __builtin_amdgcn_fdot2(wp[g], __builtin_bit_cast(half2_t, kHalf2Ones), st.wsum[g], false);
  }
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    const uint32_t a32 = w ? r.vA.y : r.vA.x;
    const uint32_t b32 = w ? r.vB.y : r.vB.x;
    const uint32_t X = __builtin_amdgcn_perm(b32, a32, 0x05040100u);
    const uint32_t Y = __builtin_amdgcn_perm(b32, a32, 0x07060302u);
    const uint32_t X6 = X >> 6, Y6 = Y >> 6;
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      const uint32_t px = x <= 4 ? (X & (0x00030003u << (2 * x))) : (X6 & (0x00030003u << (2 * x - 6)));
      const uint32_t py = x <= 4 ? (Y & (0x00030003u << (2 * x))) : (Y6 & (0x00030003u << (2 * x - 6)));
      const half2_t hx = __builtin_bit_cast(half2_t, px);
      const half2_t hy = __builtin_bit_cast(half2_t, py);
#pragma unroll
      for (int g = 0; g < GC; ++g) {
        st.acc[g][16 * w + x] = __builtin_amdgcn_fdot2(hx, wp[g], st.acc[g][16 * w + x], false);
        st.acc[g][16 * w + 8 + x] = __builtin_amdgcn_fdot2(hy, wp[g], st.acc[g][16 * w + 8 + x], false);
      }
    }
  }
}

template <int GC>
__global__ __launch_bounds__(256) void kv_int2_decode_attn_gqa(AttnArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t gw = (int64_t)blockIdx.x * 4 + wave;
  if (gw >= a.total_waves) return;
  const int64_t split = gw % a.n_splits;
  const int64_t bh = gw / a.n_splits;
  const int hkv = (int)(bh % a.Hkv);
  const int64_t b = bh / a.Hkv;
  const int ts = lane >> 2;
  const int j = lane & 3;
  const int64_t s0 = split * a.tps;
  const int64_t s1 = (s0 + a.tps < a.n_int2) ? s0 + a.tps : a.n_int2;

  QuadQuery<GC> q;
#pragma unroll
  for (int g = 0; g < GC; ++g) {
    const int hq = hkv * a.G + a.g0 + g;
    const uint32_t *p = a.qprep + (b * a.Hq + hq) * kQprepDwordsPerHead + j * 32;
#pragma unroll
    for (int i = 0; i < 20; ++i) q.limb[g][i] = p[i];
    q.qsum[g] = bits_as_float(p[24]);
    q.qstep[g] = bits_as_float(p[25]);
  }
  QuadState<GC> st;
#pragma unroll
  for (int g = 0; g < GC; ++g) {
    st.m[g] = kNegInf; st.l[g] = 0.0f; st.zacc[g] = 0.0f; st.wsum[g] = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) st.acc[g][i] = 0.0f;
  }
  const int64_t krow0 = bh * a.kT_cap + a.t_begin + s0;
  const int64_t vrow0 = bh * a.vT_cap + a.t_begin + s0;
  const uint8_t *kc = a.kcodes + krow0 * kCodeBytes, *vc = a.vcodes + vrow0 * kCodeBytes;
  const uint16_t *ks = a.kscales + krow0 * kNGroups, *kz = a.kzeros + krow0 * kNGroups;
  const uint16_t *vs = a.vscales + vrow0 * kNGroups, *vz = a.vzeros + vrow0 * kNGroups;
  const uint32_t oc = (uint32_t)(ts * kCodeBytes + 8 * j);
  const uint32_t os = (uint32_t)(ts * kNGroups + j);
  const int64_t n = s1 - s0;
  const int64_t nfull = n & ~(int64_t)31;
  auto load_tile = [&](int64_t first_row) {
    QuadTileRegs r;
    const uint8_t *kct = kc + first_row * kCodeBytes, *vct = vc + first_row * kCodeBytes;
    const uint16_t *kst = ks + first_row * kNGroups, *kzt = kz + first_row * kNGroups;
    const uint16_t *vst = vs + first_row * kNGroups, *vzt = vz + first_row * kNGroups;
    r.kA = *reinterpret_cast<const uint2 *>(kct + oc);
    r.kB = *reinterpret_cast<const uint2 *>(kct + oc + 16 * kCodeBytes);
    r.vA = *reinterpret_cast<const uint2 *>(vct + oc);
    r.vB = *reinterpret_cast<const uint2 *>(vct + oc + 16 * kCodeBytes);
    r.h[0] = kst[os]; r.h[1] = kzt[os];
    r.h[2] = kst[os + 16 * kNGroups]; r.h[3] = kzt[os + 16 * kNGroups];
    r.h[4] = vst[os]; r.h[5] = vzt[os];
    r.h[6] = vst[os + 16 * kNGroups]; r.h[7] = vzt[os + 16 * kNGroups];
    return r;
  };
  const int64_t ntiles = nfull >> 5;
  if (ntiles > 0) {
    const int64_t last = ntiles - 1;
    QuadTileRegs r0 = load_tile(0), r1 = load_tile(32 * (last < 1 ? last : 1)), r2;
    int64_t i = 0;
    for (; i + 3 <= ntiles; i += 3) {
      r2 = load_tile(32 * (i + 2 < last ? i + 2 : last));
      quad_tile<GC>(st, q, r0, true, true);
      r0 = load_tile(32 * (i + 3 < last ? i + 3 : last));
      quad_tile<GC>(st, q, r1, true, true);
      r1 = load_tile(32 * (i + 4 < last ? i + 4 : last));
      quad_tile<GC>(st, q, r2, true, true);
    }
    if (i < ntiles) quad_tile<GC>(st, q, r0, true, true);
    if (i + 1 < ntiles) quad_tile<GC>(st, q, r1, true, true);
  }
  if (nfull < n) {
    const int64_t ta = nfull + ts, tb = nfull + 16 + ts;
    const bool va = ta < n, vb = tb < n;
    const int64_t ra = va ? ta : 0, rb = vb ? tb : 0;
    QuadTileRegs r;
    r.kA = *reinterpret_cast<const uint2 *>(kc + ra * kCodeBytes + 8 * j);
    r.kB = *reinterpret_cast<const uint2 *>(kc + rb * kCodeBytes + 8 * j);
    r.vA = *reinterpret_cast<const uint2 *>(vc + ra * kCodeBytes + 8 * j);
    r.vB = *reinterpret_cast<const uint2 *>(vc + rb * kCodeBytes + 8 * j);
    r.h[0] = ks[ra * kNGroups + j]; r.h[1] = kz[ra * kNGroups + j];
    r.h[2] = ks[rb * kNGroups + j]; r.h[3] = kz[rb * kNGroups + j];
    r.h[4] = vs[ra * kNGroups + j]; r.h[5] = vz[ra * kNGroups + j];
    r.h[6] = vs[rb * kNGroups + j]; r.h[7] = vz[rb * kNGroups + j];
    quad_tile<GC>(st, q, r, va, vb);
  }
#pragma unroll
  for (int g = 0; g < GC; ++g) {
    st.zacc[g] = __builtin_fmaf(-1.5f, st.wsum[g], st.zacc[g]);
#pragma unroll
    for (int msk = 4; msk < 64; msk <<= 1) {
      st.l[g] += shfl_xor_f(st.l[g], msk);
      st.zacc[g] += shfl_xor_f(st.zacc[g], msk);
#pragma unroll
      for (int i = 0; i < 32; ++i) st.acc[g][i] += shfl_xor_f(st.acc[g][i], msk);
    }
    if (ts == 0) {
      const int hq = hkv * a.G + a.g0 + g;
      float *dst = a.partials + ((b * a.Hq + hq) * a.n_splits + split) * kPartialStride;
#pragma unroll
      for (int i = 0; i < 32; ++i) dst[32 * j + i] = __builtin_fmaf(st.acc[g][i], chan_unscale(i & 7), st.zacc[g]);
      if (j == 0) {
        dst[128] = st.m[g];
        dst[129] = st.l[g];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// 3. combine splits, un-rotate, fp16 tokens, normalize
// ---------------------------------------------------------------------------
struct CombineArgs {
  const void *q;
  bool q_f32, out_f32;
  int Hq, Hkv;
  int rot;
  const float *R;
  float qscale;
  const float *partials;
  int64_t n_splits;
  const uint16_t *sink_k, *sink_v; int64_t n_sink;
  const uint16_t *res_k, *res_v; int64_t n_res;
  void *out;
};

__device__ __forceinline__ float block_max128(float v, float *red) {
  for (int m = 1; m < 64; m <<= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  const float r = fmaxf(red[0], red[1]);
  __syncthreads();
  return r;
}

__device__ __forceinline__ float block_sum128(float v, float *red) {
  for (int m = 1; m < 64; m <<= 1) v += __shfl_xor(v, m, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  const float r = red[0] + red[1];
  __syncthreads();
  return r;
}

// grid: B*Hq blocks of 128 threads.  Dynamic LDS: n_splits + n_sink + n_res floats.
__global__ __launch_bounds__(128) void kv_combine_unrotate(CombineArgs a) {
  extern __shared__ float lds[];
  __shared__ float buf[128];
  __shared__ float red[2];
  const int c = threadIdx.x;
  const int64_t bh = blockIdx.x;             // b*Hq + hq
  const int hq = (int)(bh % a.Hq);
  const int64_t b = bh / a.Hq;
  const int hkv = hq / (a.Hq / a.Hkv);
  float *wsplit = lds;
  float *pf = lds + a.n_splits;

  // INT2 partials: M = max m_i, weights 2^(m_i - M)
  const float *part = a.partials + bh * a.n_splits * kPartialStride;
  float mloc = kNegInf;
  for (int64_t i = c; i < a.n_splits; i += 128) mloc = fmaxf(mloc, part[i * kPartialStride + 128]);
  const float M2 = block_max128(mloc, red);
  float lloc = 0.0f;
  for (int64_t i = c; i < a.n_splits; i += 128) {
    const float mi = part[i * kPartialStride + 128];
    const float wi = (mi == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f(mi - M2);
    wsplit[i] = wi;
    lloc += wi * part[i * kPartialStride + 129];
  }
  __syncthreads();
  const float L2 = block_sum128(lloc, red);
  float o = 0.0f;
  for (int64_t i = 0; i < a.n_splits; ++i) o = __builtin_fmaf(wsplit[i], part[i * kPartialStride + c], o);

  // un-rotate the INT2 part (linear, so once after the merge)
  if (a.rot == 1) o = block_fwht128(o, buf);
  else if (a.rot == 2) o = block_matvec128(o, a.R + (int64_t)hkv * kD * kD, true, buf);

  // fp16 tokens in the original basis
  const int64_t nf = a.n_sink + a.n_res;
  float Mf = kNegInf, Lf = 0.0f, of = 0.0f;
  if (nf > 0) {
    float qv = a.q_f32 ? reinterpret_cast<const float *>(a.q)[bh * kD + c]
                       : (float)reinterpret_cast<const _Float16 *>(a.q)[bh * kD + c];
    buf[c] = qv * a.qscale;
    __syncthreads();
    const int64_t bkv = b * a.Hkv + hkv;
    float sl = kNegInf;
    for (int64_t t = c; t < nf; t += 128) {
      const uint16_t *row = t < a.n_sink ? a.sink_k + (bkv * a.n_sink + t) * kD
                                         : a.res_k + (bkv * a.n_res + (t - a.n_sink)) * kD;
      float s = 0.0f;
      for (int k = 0; k < kD; ++k) s = __builtin_fmaf(buf[k], half_bits_to_float(row[k]), s);
      pf[t] = s;
      sl = fmaxf(sl, s);
    }
    Mf = block_max128(sl, red);
  }
  const float M = fmaxf(M2, Mf);
  if (nf > 0) {
    float ll = 0.0f;
    for (int64_t t = c; t < nf; t += 128) {
      const float p = __builtin_amdgcn_exp2f(pf[t] - M);
      pf[t] = p;
      ll += p;
    }
    __syncthreads();
    Lf = block_sum128(ll, red);
    const int64_t bkv = b * a.Hkv + hkv;
    for (int64_t t = 0; t < nf; ++t) {
      const uint16_t *row = t < a.n_sink ? a.sink_v + (bkv * a.n_sink + t) * kD
                                         : a.res_v + (bkv * a.n_res + (t - a.n_sink)) * kD;
      of = __builtin_fmaf(pf[t], half_bits_to_float(row[c]), of);
    }
  }
  const float wint = (M2 == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f(M2 - M);
  const float res = (o * wint + of) / (L2 * wint + Lf);
  if (a.out_f32) reinterpret_cast<float *>(a.out)[bh * kD + c] = res;
  else reinterpret_cast<_Float16 *>(a.out)[bh * kD + c] = (_Float16)res;
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
SplitPlan plan_splits(int64_t B, int64_t Hkv, int64_t n_int2) {
  SplitPlan p{0, 0};
  if (n_int2 <= 0 || B <= 0 || Hkv <= 0) return p;
  const int64_t pairs = B * Hkv;
  const int64_t target_waves = 8192;
  int64_t s = (target_waves + pairs - 1) / pairs;
  const int64_t by_len = (n_int2 + 255) / 256;   // at least ~256 tokens per wave
  if (s > by_len) s = by_len;
  if (s > 4096) s = 4096;
  if (s < 1) s = 1;
  int64_t tps = (n_int2 + s - 1) / s;
  tps = (tps + 31) / 32 * 32;
  p.tokens_per_split = tps;
  p.n_splits = (n_int2 + tps - 1) / tps;
  return p;
}

hipError_t launch_decode(const DecodeArgs &d, hipStream_t stream) {
  const int G = (int)(d.Hq / d.Hkv);
  {
    PrepArgs p;
    p.q = d.q; p.q_f32 = d.q_f32; p.Hq = (int)d.Hq; p.Hkv = (int)d.Hkv;
    p.rot = d.rot; p.R = d.R; p.qscale = d.qscale;
    p.qprep = reinterpret_cast<uint8_t *>(d.qprep);
    hipLaunchKernelGGL(kv_prep_query, dim3((unsigned)(d.B * d.Hq)), dim3(128), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (d.n_splits > 0) {
    AttnArgs a;
    a.kcodes = d.kcodes; a.kscales = d.kscales; a.kzeros = d.kzeros; a.kT_cap = d.kT_cap;
    a.vcodes = d.vcodes; a.vscales = d.vscales; a.vzeros = d.vzeros; a.vT_cap = d.vT_cap;
    a.t_begin = d.t_begin; a.n_int2 = d.n_int2;
    a.n_splits = d.n_splits; a.tps = d.tokens_per_split;
    a.total_waves = d.B * d.Hkv * d.n_splits;
    a.Hkv = (int)d.Hkv; a.Hq = (int)d.Hq; a.G = G;
    a.qprep = reinterpret_cast<const uint32_t *>(d.qprep);
    a.partials = d.partials;
    const dim3 grid((unsigned)((a.total_waves + 3) / 4));
    if (G == 1) {
      a.g0 = 0;
      hipLaunchKernelGGL(kv_int2_decode_attn<1>, grid, dim3(256), 0, stream, a);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    } else {
      const int GC = (G % 2 == 0) ? 2 : 1;
      for (int g0 = 0; g0 < G; g0 += GC) {
        a.g0 = g0;
        if (GC == 2) hipLaunchKernelGGL(kv_int2_decode_attn_gqa<2>, grid, dim3(256), 0, stream, a);
        else hipLaunchKernelGGL(kv_int2_decode_attn_gqa<1>, grid, dim3(256), 0, stream, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
      }
    }
  }
  {
    CombineArgs c;
    c.q = d.q; c.q_f32 = d.q_f32; c.out_f32 = d.out_f32;
    c.Hq = (int)d.Hq; c.Hkv = (int)d.Hkv; c.rot = d.rot; c.R = d.R; c.qscale = d.qscale;
    c.partials = d.partials; c.n_splits = d.n_splits;
    c.sink_k = d.sink_k; c.sink_v = d.sink_v; c.n_sink = d.n_sink;
    c.res_k = d.res_k; c.res_v = d.res_v; c.n_res = d.n_res;
    c.out = d.out;
    const size_t lds = (size_t)(d.n_splits + d.n_sink + d.n_res) * sizeof(float);
    hipLaunchKernelGGL(kv_combine_unrotate, dim3((unsigned)(d.B * d.Hq)), dim3(128), lds, stream, c);
    return hipGetLastError();
  }
}

}  // namespace kvq
