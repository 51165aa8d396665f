// Read path: decode attention over the packed INT2 cache (gfx950, wave64).
//
// out = softmax(scale * (q R) . k_hat) v_hat R^T, jointly normalized with
// optional fp16 sink / residual tokens kept in the original basis.  The
// readout is scaled dot-product attention and the rotation is removed
// after the attention computation ("Output-Aware Rotation for INT2
// KV-Cache Quantization", woor.ai page, "What You Need to Know" and "Key
// Details"); sinks stay unquantized (RotateKV abstract, item (iii)).
//
// Launches on the caller's stream:
//   1. kv_prep_query     per (b, query head): q' = q R (FWHT or dense), scaled
//                        by softmax_scale*log2(e), turned into a per-group
//                        19-bit fixed-point vector split into five signed
//                        4-bit limbs.  Only for a dense rotation or grouped-
//                        query attention: otherwise every attention wave
//                        does the same steps for its head (wave_prep_query).
//   2. kv_int2_decode_attn  (one query head per KV head) one wave per
//                        (b, head, split): flash-decoding over every S-th
//                        64-token tile of the head with an online softmax.
//                        Grouped-query attention (several query heads per KV
//                        head) takes the matrix-core kernel of
//                        kv_decode_gqa.hip instead, which writes the same
//                        partials.
//   3. kv_combine_unrotate  per (b, query head): log-sum-exp merge of the wave
//                        partials staged through LDS, un-rotation by R^T
//                        (linear, so applied once after the merge), fp16
//                        tokens, normalization, store.
//
// Scores never dequantize a key: with per-group scale s and zero z,
//   q'.k_hat = sum_j s_j * (sum_{c in j} q'_c code_c) + z_j * (sum_{c in j} q'_c),
// and the inner sum is an exact int32 dot product (v_dot8 on 4-bit code
// nibbles and 4-bit query limbs).  Values: with w_t = fp16(p_t s_{t,j} 2^kx)
// (2^kx the wave's value pre-scale, which keeps every w a normal fp16
// number below 2^15),
//   o'_c = 2^-kx (sum_t w_t code_{t,c} - 1.5 sum_t w_t) + sum_t p_t (z_{t,j} + 1.5 s_{t,j});
// the first term runs as v_dot2 over token pairs with codes placed in fp16
// subnormal encodings (code * 2^(e-24)), accumulated in fp32.  Centering the
// codes on 1.5 makes the fp16 rounding of w multiply code - 1.5 in
// [-1.5, 1.5], so it does not get amplified by the cancellation between the
// code and zero-point terms.
#include <math.h>

#include "kv_decode_common.h"

namespace kvq {


// ---------------------------------------------------------------------------
// 128-point normalized FWHT / dense rotation across a block of >= 128 threads (LDS)
// ---------------------------------------------------------------------------
// Threads 0..127 own channel c; wider blocks pass through the barriers.
__device__ __forceinline__ float block_fwht128(float x, float *buf) {
  const int c = threadIdx.x;
  if (c < 128) buf[c] = x;
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
  const float y = c < 128 ? buf[c] * 0.08838834764831845f : 0.0f;
  __syncthreads();
  return y;
}

// y_c = sum_k x_k M[k][c]  (transpose=false)  or  sum_k x_k M[c][k] (true),
// spread over a block of kMatThreads threads so that every thread has 16
// independent 16-byte loads in flight:
//   M[k][c]: thread t owns columns 4 (t%32) .. +3 over rows 16 (t/32) .. +15;
//   M[c][k]: thread t owns row c = t%128 over columns 64 (t/128) .. +63.
// The thread's part of M is loaded first (mat_load128, which the callers
// issue before the loads that x depends on), then block_matvec128 takes it.
// Partial sums meet in `red` (8 x 128 floats).
constexpr int kMatThreads = 256;
struct MatRegs {
  float4_t m[16];
};
__device__ __forceinline__ MatRegs mat_load128(const float *__restrict__ M, bool transpose) {
  const int t = threadIdx.x;
  MatRegs r;
  if (!transpose) {
    const float4_t *col = reinterpret_cast<const float4_t *>(M + 16 * (t >> 5) * 128) + (t & 31);
#pragma unroll
    for (int i = 0; i < 16; ++i) r.m[i] = col[32 * i];
  } else {
    const float4_t *row = reinterpret_cast<const float4_t *>(M + (t & 127) * 128 + 64 * (t >> 7));
#pragma unroll
    for (int i = 0; i < 16; ++i) r.m[i] = row[i];
  }
  return r;
}
__device__ __forceinline__ float block_matvec128(float x, const MatRegs &mr, bool transpose, float *buf,
                                                 float *red) {
  const int t = threadIdx.x;
  if (t < 128) buf[t] = x;
  __syncthreads();
  if (!transpose) {
    const int cg = t & 31, sl = t >> 5;
    float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float xk = buf[16 * sl + i];
      acc.x = __builtin_fmaf(xk, mr.m[i].x, acc.x);
      acc.y = __builtin_fmaf(xk, mr.m[i].y, acc.y);
      acc.z = __builtin_fmaf(xk, mr.m[i].z, acc.z);
      acc.w = __builtin_fmaf(xk, mr.m[i].w, acc.w);
    }
    reinterpret_cast<float4_t *>(red + 128 * sl)[cg] = acc;
  } else {
    const int c = t & 127, hh = t >> 7;
    float acc0 = 0.0f, acc1 = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float *xb = buf + 64 * hh + 4 * i;
      acc0 = __builtin_fmaf(xb[0], mr.m[i].x, acc0);
      acc1 = __builtin_fmaf(xb[1], mr.m[i].y, acc1);
      acc0 = __builtin_fmaf(xb[2], mr.m[i].z, acc0);
      acc1 = __builtin_fmaf(xb[3], mr.m[i].w, acc1);
    }
    red[128 * hh + c] = acc0 + acc1;
  }
  __syncthreads();
  float y = 0.0f;
  if (t < 128) {
    if (!transpose) {
#pragma unroll
      for (int sl = 0; sl < kMatThreads / 32; ++sl) y += red[128 * sl + t];
    } else {
      y = red[t] + red[128 + t];
    }
  }
  __syncthreads();
  return y;
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
  const int32_t *perm;   // permuted Hadamard: [Hkv][128]
  float qscale;
  uint8_t *qprep;    // [B][Hq][128 dwords]
};


// grid: B*Hq blocks of kMatThreads threads; thread c < 128 owns channel c,
// the others only help with a dense rotation.
__global__ __launch_bounds__(kMatThreads) void kv_prep_query(PrepArgs a) {
  __shared__ float buf[128];
  __shared__ float red[8 * 128];
  const int c = threadIdx.x;
  const bool own = c < kD;
  const int64_t bh = blockIdx.x;            // b*Hq + hq
  const int hq = (int)(bh % a.Hq);
  const int hkv = hq / (a.Hq / a.Hkv);
  float x = 0.0f;
  // dense R: the thread's part of R is requested together with q
  MatRegs Rm;
  if (a.rot == 2) Rm = mat_load128(a.R + (int64_t)hkv * kD * kD, false);
  // permuted Hadamard: thread c takes channel pi[c] of q (q_pi), then the transform
  const int cin = a.rot == 3 ? (a.perm[(int64_t)hkv * kD + (c & (kD - 1))] & (kD - 1)) : c;
  if (own) x = a.q_f32 ? reinterpret_cast<const float *>(a.q)[bh * kD + cin]
                       : (float)reinterpret_cast<const _Float16 *>(a.q)[bh * kD + cin];
  if (a.rot == 1 || a.rot == 3) x = block_fwht128(x, buf);
  else if (a.rot == 2) x = block_matvec128(x, Rm, false, buf, red);
  x *= a.qscale;

  // maximum magnitude over the head -> exponent of the fixed point (one step
  // for all four groups, so the step can be applied once per token score)
  __shared__ float wmax[kMatThreads / 64];
  float amax = fabsf(x);
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
  if ((c & 63) == 0) wmax[c >> 6] = amax;
  __syncthreads();
  amax = fmaxf(wmax[0], wmax[1]);
  int e = 0;
  (void)frexpf(amax, &e);                    // amax < 2^e
  const bool zero_head = !(amax > 0.0f);
  const int E = 18 - e;                      // |x| * 2^E < 2^18
  const int qi = zero_head ? 0 : (int)__builtin_rintf(ldexpf(x, E));
  const float step = zero_head ? 0.0f : ldexpf(1.0f, -E);
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
    if (own && k == 0) base[L * 4 + w * 2 + par] = part;
  }
  // the fixed-point query itself, for the matrix-core GQA kernel
  if (own) reinterpret_cast<int32_t *>(a.qprep)[bh * kQprepDwordsPerHead + kQprepFixedOffset + c] = qi;
  if (own && cg == 0) {
    float *fb = reinterpret_cast<float *>(base);
    fb[24] = (float)isum * step;             // sum of the group's fixed-point q
    fb[25] = step;
    fb[26] = (float)isum;                    // the same sum in steps (exact: |isum| < 2^23)
  }
}

// ---------------------------------------------------------------------------
// 2. split-K attention over INT2 tokens
// ---------------------------------------------------------------------------
// Lane layout of the attention kernel: lane l handles token slot ts = l/2 of
// a 64-token tile (tokens ts and 32 + ts) on channel half h = l%2, i.e. the
// two groups 2h and 2h+1 (64 channels).  Codes arrive as one 16-byte load
// per token and lane (1 KB per wave instruction); scales and zeros as one
// 4-byte load (both groups) per token and lane.
struct TileRegs {
  u32x4_t kA, kB, vA, vB;          // codes of tokens A (= ts) and B (= 32 + ts)
  uint32_t ksA, kzA, ksB, kzB;     // two fp16 scales / zeros each
  uint32_t vsA, vzA, vsB, vzB;
  float sA, sB;                    // precomputed scores (log2 units), PRE only
};

template <int GC>
struct AttnState {
  float m[GC], l[GC], zacc[GC][2], wsum[GC][2], acc[GC][64];
  ValuePrescale ps;           // acc and wsum carry the factor 2^kx
};


// Per-lane query data for the lane's two channel groups of GC heads.
template <int GC>
struct QueryLimbs {
  uint32_t limb[GC][2][20];   // [head][group in half][L*4 + w*2 + parity]
  float isum[GC][2];          // group sums of the fixed-point query, in steps
  float qstep[GC];            // fixed-point step of the head (log2 units)
};

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

// PRE: the key scores come precomputed in r.sA / r.sB (log2 units) and the
// key fields of r are unused.
template <int GC, bool PRE = false>
__device__ __forceinline__ void attn_tile(AttnState<GC> &st, const QueryLimbs<GC> &q,
                                          const TileRegs &r, bool va, bool vb) {
  const uint32_t kAw[4] = {r.kA.x, r.kA.y, r.kA.z, r.kA.w};
  const uint32_t kBw[4] = {r.kB.x, r.kB.y, r.kB.z, r.kB.w};
  const half2_t ksA = __builtin_bit_cast(half2_t, r.ksA), kzA = __builtin_bit_cast(half2_t, r.kzA);
  const half2_t ksB = __builtin_bit_cast(half2_t, r.ksB), kzB = __builtin_bit_cast(half2_t, r.kzB);
  const half2_t vsA = __builtin_bit_cast(half2_t, r.vsA), vzA = __builtin_bit_cast(half2_t, r.vzA);
  const half2_t vsB = __builtin_bit_cast(half2_t, r.vsB), vzB = __builtin_bit_cast(half2_t, r.vzB);
  half2_t wp[GC][2];
  {
    // a value scale beyond the wave's pre-scale: lower it (wave-uniform, rare)
    const uint32_t mb = max_half_bits(r.vsA, r.vsB);
    if (__builtin_amdgcn_ballot_w64(mb >= st.ps.lim)) {
      const float f = prescale_lower(st.ps, mb);
#pragma unroll
      for (int g = 0; g < GC; ++g) {
        st.wsum[g][0] *= f;
        st.wsum[g][1] *= f;
#pragma unroll
        for (int i = 0; i < 64; ++i) st.acc[g][i] *= f;
      }
    }
  }
#pragma unroll
  for (int g = 0; g < GC; ++g) {
    float xa, xb;
    float ra = 0.0f, rb = 0.0f;
    if constexpr (PRE) {
      xa = va ? r.sA - st.m[g] : kNegInf;
      xb = vb ? r.sB - st.m[g] : kNegInf;
    } else {
      // score in units of the query step: sum_j s_j * dot_j + z_j * isum_j
#pragma unroll
      for (int gi = 0; gi < 2; ++gi) {
        const int ia = group_dot(q.limb[g][gi], kAw[2 * gi], kAw[2 * gi + 1]);
        const int ib = group_dot(q.limb[g][gi], kBw[2 * gi], kBw[2 * gi + 1]);
        ra = __builtin_fmaf((float)ia, (float)ksA[gi], __builtin_fmaf((float)kzA[gi], q.isum[g][gi], ra));
        rb = __builtin_fmaf((float)ib, (float)ksB[gi], __builtin_fmaf((float)kzB[gi], q.isum[g][gi], rb));
      }
      ra += quad_swap<kQuadXor1>(ra);        // the other half of the row
      rb += quad_swap<kQuadXor1>(rb);
      // log2-domain score minus the running reference
      xa = va ? __builtin_fmaf(q.qstep[g], ra, -st.m[g]) : kNegInf;
      xb = vb ? __builtin_fmaf(q.qstep[g], rb, -st.m[g]) : kNegInf;
    }
    if (__builtin_amdgcn_ballot_w64(fmaxf(xa, xb) > kSlack)) {     // wave-uniform
      const float ya = va ? (PRE ? r.sA : q.qstep[g] * ra) : kNegInf;
      const float yb = vb ? (PRE ? r.sB : q.qstep[g] * rb) : kNegInf;
      float mx = fmaxf(ya, yb);
      mx = fmaxf(mx, row_ror<2>(mx));
      mx = fmaxf(mx, row_ror<4>(mx));
      mx = fmaxf(mx, row_ror<8>(mx));
      mx = max_xor16(mx);
      mx = max_xor32(mx);
      mx = fmaxf(mx, st.m[g]);               // the reference never moves down
      if (mx != kNegInf) {                   // wave-uniform; else no token so far
        const float alpha = __builtin_amdgcn_exp2f(st.m[g] - mx);
        st.l[g] *= alpha;
        st.zacc[g][0] *= alpha;
        st.zacc[g][1] *= alpha;
        st.wsum[g][0] *= alpha;
        st.wsum[g][1] *= alpha;
#pragma unroll
        for (int i = 0; i < 64; ++i) st.acc[g][i] *= alpha;
        st.m[g] = mx;
        xa = ya - mx;
        xb = yb - mx;
      }
    }
    const float pA = __builtin_amdgcn_exp2f(xa);   // 0 for masked tokens
    const float pB = __builtin_amdgcn_exp2f(xb);
    st.l[g] += pA + pB;
#pragma unroll
    for (int gi = 0; gi < 2; ++gi) {
      const float svA = (float)vsA[gi], svB = (float)vsB[gi];
      st.zacc[g][gi] = __builtin_fmaf(pA, __builtin_fmaf(1.5f, svA, (float)vzA[gi]),
                                      __builtin_fmaf(pB, __builtin_fmaf(1.5f, svB, (float)vzB[gi]),
                                                     st.zacc[g][gi]));
      wp[g][gi].x = (_Float16)(pA * (svA * st.ps.f));
      wp[g][gi].y = (_Float16)(pB * (svB * st.ps.f));
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

// The query preparation of kv_prep_query done by one wave for its own head
// (no rotation or the Hadamard rotation): lane l holds channels 2l, 2l+1.
// The butterfly stages, the fixed-point exponent and the digits are the same
// operations in the same order as in kv_prep_query, so the results are
// bitwise identical.  The limb dwords of the four groups (20 each) and the
// group sums go to `lds` (84 dwords); returns the fixed-point step.
__device__ __forceinline__ float wave_prep_query(const void *q, bool q_f32, int64_t qoff, int rot,
                                                 float qscale, uint32_t *lds) {
  const int lane = threadIdx.x & 63;
  float x0, x1;
  if (q_f32) {
    const float *qp = reinterpret_cast<const float *>(q) + qoff + 2 * lane;
    x0 = qp[0]; x1 = qp[1];
  } else {
    const uint32_t u = *reinterpret_cast<const uint32_t *>(reinterpret_cast<const _Float16 *>(q) + qoff + 2 * lane);
    const half2_t hq = __builtin_bit_cast(half2_t, u);
    x0 = (float)hq.x; x1 = (float)hq.y;
  }
  if (rot == 1) {
    float y0 = x0 + x1, y1 = x0 - x1;                      // distance 1: inside the lane
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {                    // distance 2m: lane partner l ^ m
      const float p0 = __shfl_xor(y0, m, 64), p1 = __shfl_xor(y1, m, 64);
      const bool hi = (lane & m) != 0;
      y0 = hi ? p0 - y0 : y0 + p0;
      y1 = hi ? p1 - y1 : y1 + p1;
    }
    x0 = y0 * 0.08838834764831845f;
    x1 = y1 * 0.08838834764831845f;
  }
  x0 *= qscale;
  x1 *= qscale;
  float amax = fmaxf(fabsf(x0), fabsf(x1));
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
  int e = 0;
  (void)frexpf(amax, &e);
  const bool zero_head = !(amax > 0.0f);
  const int E = 18 - e;
  const int qi0 = zero_head ? 0 : (int)__builtin_rintf(ldexpf(x0, E));
  const int qi1 = zero_head ? 0 : (int)__builtin_rintf(ldexpf(x1, E));
  const float step = zero_head ? 0.0f : ldexpf(1.0f, -E);
  int isum = qi0 + qi1;                                   // group j = lane / 16
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) isum += __shfl_xor(isum, m, 64);
  // limb dword (L, w, parity) of group j: nibble k holds digit L of channel
  // 32 j + 16 w + 2 k + parity, i.e. lane 16 j + 8 w + k, element `parity`
  const int j = lane >> 4, w = (lane >> 3) & 1, k = lane & 7;
  int r0 = qi0, r1 = qi1;
#pragma unroll
  for (int L = 4; L >= 0; --L) {
    const int d0 = ((r0 + 8) & 15) - 8, d1 = ((r1 + 8) & 15) - 8;
    r0 = (r0 - d0) >> 4;
    r1 = (r1 - d1) >> 4;
    uint32_t p0 = ((uint32_t)d0 & 15u) << (4 * k), p1 = ((uint32_t)d1 & 15u) << (4 * k);
    p0 |= __shfl_xor(p0, 1, 64); p1 |= __shfl_xor(p1, 1, 64);
    p0 |= __shfl_xor(p0, 2, 64); p1 |= __shfl_xor(p1, 2, 64);
    p0 |= __shfl_xor(p0, 4, 64); p1 |= __shfl_xor(p1, 4, 64);
    if (k == 0) {
      lds[20 * j + 4 * L + 2 * w] = p0;
      lds[20 * j + 4 * L + 2 * w + 1] = p1;
    }
  }
  if ((lane & 15) == 0) lds[80 + j] = float_as_bits((float)isum);
  return step;
}

// WPB waves per workgroup; wave index gw = ((b*Hkv + hkv)*S + split)*G + g
// for one length (the variable-length map of wave_place otherwise), so the
// G heads of a group (same tiles) are neighbours in one workgroup.
// PRE: the key scores are read from a.scores (keys cached with the pre-RoPE
// grouped-head rotation, scored by kv_prerope_scores); the key cache and the
// query are not read.
template <int WPB, bool PRE = false>
__global__ __launch_bounds__(64 * WPB) void kv_int2_decode_attn(AttnArgs a) {
  constexpr int GC = 1;
  const int lane = threadIdx.x & 63;
  // wave index made explicitly uniform so every per-wave quantity is scalar
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t gw = (int64_t)blockIdx.x * WPB + wave;
  WavePlace wp;
  if (!wave_place(a, gw, a.G, wp)) return;   // whole wave leaves together
  const int gq = wp.sub;
  const int64_t split = wp.split;
  const int hkv = wp.hkv;
  const int64_t b = wp.b;
  const int64_t bh = b * a.Hkv + hkv;
  const int ts = lane >> 1;                  // token slot 0..31
  const int h = lane & 1;                    // channel half: groups 2h, 2h+1
  // The head's INT2 tokens are cut into 64-token tiles; wave `split` takes
  // tiles split, split + S, split + 2S, ... (S waves per head: the call's
  // split count, or the sequence's own in a variable-length batch), so the waves
  // of a head stream through adjacent tiles together rather than each
  // through a region of its own.
  const int64_t S = wp.S;
  const HeadTiles ht(seq_int2(a, b), a.skip, split, S);
  const int64_t mine = ht.mine;

  QueryLimbs<GC> q;
  __shared__ uint32_t qlds[WPB][84];
  if constexpr (PRE) {
    // scores come precomputed
  } else if (a.fused_prep) {                 // one head per KV head: hq = b*Hq + hkv
    q.qstep[0] = wave_prep_query(a.q, a.q_f32, (b * a.Hq + hkv) * kD, a.rot, a.qscale, qlds[wave]);
    asm volatile("" ::: "memory");           // LDS of one wave is ordered; keep the program order
#pragma unroll
    for (int gi = 0; gi < 2; ++gi) {
      const uint32_t *p = qlds[wave] + 20 * (2 * h + gi);
#pragma unroll
      for (int i = 0; i < 20; ++i) q.limb[0][gi][i] = p[i];
      q.isum[0][gi] = bits_as_float(qlds[wave][80 + 2 * h + gi]);
    }
  } else {
#pragma unroll
  for (int g = 0; g < GC; ++g) {
    const int hq = hkv * a.G + gq + g;
#pragma unroll
    for (int gi = 0; gi < 2; ++gi) {
      const uint32_t *p = a.qprep + (b * a.Hq + hq) * kQprepDwordsPerHead + (2 * h + gi) * 32;
#pragma unroll
      for (int i = 0; i < 20; ++i) q.limb[g][gi][i] = p[i];
      q.isum[g][gi] = bits_as_float(p[26]);
      if (gi == 0) q.qstep[g] = bits_as_float(p[25]);   // the same for every group
    }
  }
  }

  AttnState<GC> st;
  st.ps = prescale_init();
#pragma unroll
  for (int g = 0; g < GC; ++g) {
    st.m[g] = kNegInf; st.l[g] = 0.0f; st.zacc[g][0] = 0.0f; st.zacc[g][1] = 0.0f;
    st.wsum[g][0] = 0.0f; st.wsum[g][1] = 0.0f;
#pragma unroll
    for (int i = 0; i < 64; ++i) st.acc[g][i] = 0.0f;
  }

  // Row r of the head's INT2 range: codes at *c + r*32 bytes, scales/zeros
  // at *s + r*4 halves.  Lane offsets are 32-bit; tile bases are wave-uniform.
  const int64_t krow0 = bh * a.kT_cap + a.t_begin - a.skip;   // row 0 of the shifted grid
  const int64_t vrow0 = bh * a.vT_cap + a.t_begin - a.skip;

  // Loads of one lane: codes at tile base + oc (+1 KB for token B), scales
  // and zeros at tile base + os halves (+64 halves for token B).  Tile bases
  // are wave-uniform, lane offsets 32-bit.
  const uint32_t oc = (uint32_t)(ts * kCodeBytes + 16 * h);
  const uint32_t os = (uint32_t)(ts * kNGroups + 2 * h);
  // PRE: the wave's query head's precomputed scores, by shifted-grid row
  const float *srow = PRE ? a.scores + (b * a.Hq + hkv * a.G + gq) * a.score_rows : nullptr;
  auto load_tile = [&](const TileRows &tr) {
    TileRegs r;
    const uint8_t *kct = a.kcodes + tr.k * kCodeBytes, *vct = a.vcodes + tr.v * kCodeBytes;
    const uint16_t *kst = a.kscales + tr.k * kNGroups, *kzt = a.kzeros + tr.k * kNGroups;
    const uint16_t *vst = a.vscales + tr.v * kNGroups, *vzt = a.vzeros + tr.v * kNGroups;
    if constexpr (PRE) {
      const int64_t g0 = tr.k - krow0;               // the tile's first shifted-grid row
      r.sA = srow[g0 + ts];
      r.sB = srow[g0 + 32 + ts];
    } else {
      r.kA = *reinterpret_cast<const u32x4_t *>(kct + oc);
      r.kB = *reinterpret_cast<const u32x4_t *>(kct + oc + 32 * kCodeBytes);
      r.ksA = *reinterpret_cast<const uint32_t *>(kst + os);
      r.kzA = *reinterpret_cast<const uint32_t *>(kzt + os);
      r.ksB = *reinterpret_cast<const uint32_t *>(kst + os + 32 * kNGroups);
      r.kzB = *reinterpret_cast<const uint32_t *>(kzt + os + 32 * kNGroups);
    }
    r.vA = *reinterpret_cast<const u32x4_t *>(vct + oc);
    r.vB = *reinterpret_cast<const u32x4_t *>(vct + oc + 32 * kCodeBytes);
    r.vsA = *reinterpret_cast<const uint32_t *>(vst + os);
    r.vzA = *reinterpret_cast<const uint32_t *>(vzt + os);
    r.vsB = *reinterpret_cast<const uint32_t *>(vst + os + 32 * kNGroups);
    r.vzB = *reinterpret_cast<const uint32_t *>(vzt + os + 32 * kNGroups);
    return r;
  };

  // This wave's full tiles, software-pipelined three deep: while tile i is
  // computed the loads of tiles i+1 and i+2 are in flight.  A prefetch past
  // the wave's last tile is clamped to it (a re-read of valid rows, unused).
  if (mine > 0) {
    PagedTileRows pages;
    auto at = [&](int64_t i) {
      if (a.block_table == nullptr) {
        const int64_t r = ht.full_row(i, split, S);
        return TileRows{krow0 + r, vrow0 + r};
      }
      const int64_t r = pages.row(a, b, hkv, ht, split, S, i);
      return TileRows{r, r};
    };
    TileRegs r0 = load_tile(at(0)), r1 = load_tile(at(1)), r2;
    int64_t i = 0;
    for (; i + 3 <= mine; i += 3) {
      r2 = load_tile(at(i + 2));
      attn_tile<GC, PRE>(st, q, r0, true, true);
      r0 = load_tile(at(i + 3));
      attn_tile<GC, PRE>(st, q, r1, true, true);
      r1 = load_tile(at(i + 4));
      attn_tile<GC, PRE>(st, q, r2, true, true);
    }
    if (i < mine) attn_tile<GC, PRE>(st, q, r0, true, true);
    if (i + 1 < mine) attn_tile<GC, PRE>(st, q, r1, true, true);
  }
  // partial tiles: masked rows are loaded from the tile's first valid row
  auto masked_tile = [&](int64_t t) {
    const int64_t base = 64 * t;
    const int64_t lo = a.skip > base ? a.skip - base : 0;
    const int64_t hi = ht.n_tok - base < 64 ? ht.n_tok - base : 64;
    const bool va = ts >= lo && ts < hi, vb = 32 + ts >= lo && 32 + ts < hi;
    const TileRows tr = tile_rows(a, b, hkv, krow0, vrow0, base);
    const uint8_t *kc = a.kcodes + tr.k * kCodeBytes, *vc = a.vcodes + tr.v * kCodeBytes;
    const uint16_t *ks = a.kscales + tr.k * kNGroups, *kz = a.kzeros + tr.k * kNGroups;
    const uint16_t *vs = a.vscales + tr.v * kNGroups, *vz = a.vzeros + tr.v * kNGroups;
    const int64_t ra = va ? ts : lo, rb = vb ? 32 + ts : lo;   // rows inside the tile
    TileRegs r;
    if constexpr (PRE) {
      r.sA = srow[base + ra];
      r.sB = srow[base + rb];
    } else {
      r.kA = *reinterpret_cast<const u32x4_t *>(kc + ra * kCodeBytes + 16 * h);
      r.kB = *reinterpret_cast<const u32x4_t *>(kc + rb * kCodeBytes + 16 * h);
      r.ksA = *reinterpret_cast<const uint32_t *>(ks + ra * kNGroups + 2 * h);
      r.kzA = *reinterpret_cast<const uint32_t *>(kz + ra * kNGroups + 2 * h);
      r.ksB = *reinterpret_cast<const uint32_t *>(ks + rb * kNGroups + 2 * h);
      r.kzB = *reinterpret_cast<const uint32_t *>(kz + rb * kNGroups + 2 * h);
    }
    r.vA = *reinterpret_cast<const u32x4_t *>(vc + ra * kCodeBytes + 16 * h);
    r.vB = *reinterpret_cast<const u32x4_t *>(vc + rb * kCodeBytes + 16 * h);
    r.vsA = *reinterpret_cast<const uint32_t *>(vs + ra * kNGroups + 2 * h);
    r.vzA = *reinterpret_cast<const uint32_t *>(vz + ra * kNGroups + 2 * h);
    r.vsB = *reinterpret_cast<const uint32_t *>(vs + rb * kNGroups + 2 * h);
    r.vzB = *reinterpret_cast<const uint32_t *>(vz + rb * kNGroups + 2 * h);
    attn_tile<GC, PRE>(st, q, r, va, vb);
  };
  {
    int64_t p0, p1;
    ht.partial(a.skip, split, S, p0, p1);
    if (p0 >= 0) masked_tile(p0);
    if (p1 >= 0) masked_tile(p1);
  }

  // reduce over the 32 token slots (lanes sharing h), then write the partial
#pragma unroll
  for (int g = 0; g < GC; ++g) {
    float l = st.l[g];
    // acc and wsum carry the pre-scale 2^kx, zacc does not
    float z0 = __builtin_fmaf(-1.5f * st.ps.inv, st.wsum[g][0], st.zacc[g][0]);
    float z1 = __builtin_fmaf(-1.5f * st.ps.inv, st.wsum[g][1], st.zacc[g][1]);
    // sum over the 32 token slots sharing h: lane bits 1..3 inside the row
    // (DPP), then the rows (xor 16, xor 32)
    auto reduce = [](float v) {
      v += quad_swap<kQuadXor2>(v);
      v += row_ror<4>(v);
      v += row_ror<8>(v);
      return sum_xor32(sum_xor16(v));
    };
    l = reduce(l);
    z0 = reduce(z0);
    z1 = reduce(z1);
#pragma unroll
    for (int i = 0; i < 64; ++i) st.acc[g][i] = reduce(st.acc[g][i]);
    if (ts == 0) {
      const int hq = hkv * a.G + gq + g;
      float *dst = a.partials + partial_row(a, wp, hq) * kPartialStride;
#pragma unroll
      for (int i = 0; i < 64; ++i) {
        const int x = i & 7;
        dst[64 * h + i] = __builtin_fmaf(st.acc[g][i], chan_unscale(x) * st.ps.inv, i < 32 ? z0 : z1);
      }
      if (h == 0) {
        dst[128] = st.m[g];
        dst[129] = l;
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
  const int32_t *perm;   // permuted Hadamard: [Hkv][128]
  float qscale;
  const float *partials;
  int64_t n_splits;
  // variable-length batch (t_ends != NULL): the split map of the attention call
  const int32_t *t_ends; int64_t B, t_begin, n_int2; int skip;
  const uint16_t *sink_k, *sink_v; int64_t n_sink;
  const uint16_t *res_k, *res_v; int64_t n_res;
  void *out;
};

constexpr int kCombineThreads = 256;
static_assert(kCombineThreads == kMatThreads, "the combine block runs the block-wide matvec");
constexpr int kCombineWaves = kCombineThreads / 64;
// fp16 tokens: a 16-lane row per token (8 channels per lane, one 16-byte
// load), kFpRows tokens per step across the block, kFpUnroll steps whose loads
// are issued together.
constexpr int kFpRows = kCombineThreads / 16;
constexpr int kFpUnroll = 9;

__device__ __forceinline__ float block_max(float v, float *red) {
  for (int m = 1; m < 64; m <<= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int i = 1; i < kCombineWaves; ++i) r = fmaxf(r, red[i]);
  __syncthreads();
  return r;
}

__device__ __forceinline__ float block_sum(float v, float *red) {
  for (int m = 1; m < 64; m <<= 1) v += __shfl_xor(v, m, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int i = 1; i < kCombineWaves; ++i) r += red[i];
  __syncthreads();
  return r;
}

// Row t of the fp16 segment: sinks first, then residual tokens.
__device__ __forceinline__ const uint16_t *fp16_row(const uint16_t *sink, const uint16_t *res, int64_t bkv,
                                                    int64_t n_sink, int64_t n_res, int64_t t) {
  return t < n_sink ? sink + (bkv * n_sink + t) * kD : res + (bkv * n_res + (t - n_sink)) * kD;
}

// Merge of one (b, query head) by one wave, for the common case: one INT2
// range for the whole batch, no fp16 tokens, and no rotation, the Hadamard
// or the reordered Hadamard.  Lane l owns channels 2l and 2l + 1; the split
// weights 2^(m_i - M) and the sums are wave reductions.  Un-rotation: the
// FWHT over the 128 merged channels is one in-lane butterfly and six lane
// exchanges, then, for the reordered Hadamard, output j goes to channel
// pi(j).  No LDS or barrier.  Same merge as kv_combine_unrotate (summation
// order aside).  (A dense R^T applied by one wave, from the lane's two rows
// of R, measured slower than the block's matvec.)
// grid: ceil(B*Hq / kWaveCombineWaves) workgroups of kWaveCombineWaves waves.
constexpr int kWaveCombineWaves = 4;
__global__ __launch_bounds__(64 * kWaveCombineWaves) void kv_combine_wave(CombineArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t bh = (int64_t)blockIdx.x * kWaveCombineWaves + (threadIdx.x >> 6);   // b*Hq + hq
  if (bh >= a.B * a.Hq) return;                  // whole wave leaves; no barrier follows
  const int64_t ns = a.n_splits;
  const float *part = a.partials + bh * ns * kPartialStride;   // rows (b*Hq + hq)*S + split
  // M = max m_i, L = sum 2^(m_i - M) l_i
  float mloc = kNegInf;
  for (int64_t i = lane; i < ns; i += 64) mloc = fmaxf(mloc, part[i * kPartialStride + 128]);
  for (int k = 1; k < 64; k <<= 1) mloc = fmaxf(mloc, __shfl_xor(mloc, k, 64));
  const float M = mloc;
  float lloc = 0.0f;
  for (int64_t i = lane; i < ns; i += 64) {
    const float mi = part[i * kPartialStride + 128];
    const float wi = (mi == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f(mi - M);
    lloc = __builtin_fmaf(wi, part[i * kPartialStride + 129], lloc);
  }
  for (int k = 1; k < 64; k <<= 1) lloc += __shfl_xor(lloc, k, 64);
  const float L = lloc;
  // weighted sum of the partial outputs, eight splits' loads in flight
  float o0[2] = {0.0f, 0.0f}, o1[2] = {0.0f, 0.0f};
  int64_t i = 0;
  for (; i + 8 <= ns; i += 8) {
    float2_t v[8];
    float m8[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      v[u] = *reinterpret_cast<const float2_t *>(part + (i + u) * kPartialStride + 2 * lane);
      m8[u] = part[(i + u) * kPartialStride + 128];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float w = (m8[u] == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f(m8[u] - M);
      o0[u & 1] = __builtin_fmaf(w, v[u].x, o0[u & 1]);
      o1[u & 1] = __builtin_fmaf(w, v[u].y, o1[u & 1]);
    }
  }
  for (; i < ns; ++i) {
    const float2_t v = *reinterpret_cast<const float2_t *>(part + i * kPartialStride + 2 * lane);
    const float mi = part[i * kPartialStride + 128];
    const float w = (mi == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f(mi - M);
    o0[0] = __builtin_fmaf(w, v.x, o0[0]);
    o1[0] = __builtin_fmaf(w, v.y, o1[0]);
  }
  float x0 = o0[0] + o0[1], x1 = o1[0] + o1[1];
  const int hq = (int)(bh % a.Hq);
  const int hkv = hq / (a.Hq / a.Hkv);
  if (a.rot == 1 || a.rot == 3) {
    // normalized FWHT: channels (2l, 2l+1) in lane, then channel c pairs with
    // c ^ 2k, i.e. lane l with lane l ^ k; the lower channel takes the sum
    {
      const float s = x0 + x1, d = x0 - x1;
      x0 = s;
      x1 = d;
    }
#pragma unroll
    for (int k = 1; k < 64; k <<= 1) {
      const float p0 = __shfl_xor(x0, k, 64), p1 = __shfl_xor(x1, k, 64);
      const bool upper = (lane & k) != 0;
      x0 = upper ? p0 - x0 : x0 + p0;
      x1 = upper ? p1 - x1 : x1 + p1;
    }
    x0 *= 0.08838834764831845f;
    x1 *= 0.08838834764831845f;
  }
  const bool any = M != kNegInf && L > 0.0f;     // no token at all: 0
  const float r0 = any ? x0 / L : 0.0f, r1 = any ? x1 / L : 0.0f;
  if (a.rot == 3) {
    // o' R^T = (o' H / sqrt(d)) P^T: output j goes to channel pi(j)
    const int32_t *pi = a.perm + (int64_t)hkv * kD;
    const int c0 = pi[2 * lane] & (kD - 1), c1 = pi[2 * lane + 1] & (kD - 1);
    if (a.out_f32) {
      reinterpret_cast<float *>(a.out)[bh * kD + c0] = r0;
      reinterpret_cast<float *>(a.out)[bh * kD + c1] = r1;
    } else {
      reinterpret_cast<_Float16 *>(a.out)[bh * kD + c0] = (_Float16)r0;
      reinterpret_cast<_Float16 *>(a.out)[bh * kD + c1] = (_Float16)r1;
    }
    return;
  }
  if (a.out_f32) {
    *reinterpret_cast<float2_t *>(reinterpret_cast<float *>(a.out) + bh * kD + 2 * lane) = float2_t{r0, r1};
  } else {
    const half2_t h2 = {(_Float16)r0, (_Float16)r1};
    *reinterpret_cast<half2_t *>(reinterpret_cast<_Float16 *>(a.out) + bh * kD + 2 * lane) = h2;
  }
}

// grid: B*Hq blocks of kCombineThreads threads; threads c < 128 own channel c
// in the merge and the un-rotation.  Dynamic LDS: (most splits of one head)
// + n_sink + n_res floats.
__global__ __launch_bounds__(kCombineThreads) void kv_combine_unrotate(CombineArgs a) {
  extern __shared__ float lds[];
  __shared__ float buf[kD];
  __shared__ float red[kCombineWaves];
  __shared__ float vred[kFpRows * kD];
  const int c = threadIdx.x;
  const bool own = c < kD;
  const int64_t bh = blockIdx.x;             // b*Hq + hq
  const int hq = (int)(bh % a.Hq);
  const int64_t b = bh / a.Hq;
  const int hkv = hq / (a.Hq / a.Hkv);
  const int64_t bkv = b * a.Hkv + hkv;
  // the head's partial rows: S splits, or its sequence's own count
  int64_t first, ns;
  int64_t lds_splits = a.n_splits;
  if (a.t_ends == nullptr) {
    first = b * a.n_splits;
    ns = a.n_splits;
  } else {
    const SplitMap m = make_split_map(a.t_ends, a.B, a.t_begin, a.n_int2, a.n_splits, a.skip);
    const int64_t wt = sm_wave_tiles(m);
    if (wt > 0) {
      sm_of_seq(m, wt, b, first, ns);
    } else {
      first = 0;
      ns = 0;
    }
    lds_splits = varlen_lds_splits(a.B, a.n_splits);
  }
  float *wsplit = lds;
  float *pf = lds + lds_splits;
  const int64_t nf = a.n_sink + a.n_res;
  const int rs = c >> 4;                     // token row slot of the fp16 phases
  const int cl = c & 15;                     // channels 8cl .. 8cl+7

  // Loads that no reduction waits for go out first, so that their latency
  // overlaps the fp16 phase and the first reductions: the thread's part of a
  // dense R, the (m, l) of split c, and the values of channel c % 128 in the
  // first 2 kPre splits of parity c / 128.
  MatRegs Rm;
  if (a.rot == 2) Rm = mat_load128(a.R + (int64_t)hkv * kD * kD, true);
  const float *part = a.partials + (first * a.Hq + hq * ns) * kPartialStride;
  const int ch = c & 127, par = c >> 7;
  constexpr int kPre = 32;
  float pv[kPre];
#pragma unroll
  for (int u = 0; u < kPre; ++u) {
    const int64_t i = par + 2 * u;
    pv[u] = i < ns ? part[i * kPartialStride + ch] : 0.0f;
  }
  const float m0 = c < ns ? part[c * kPartialStride + 128] : kNegInf;
  const float l0 = c < ns ? part[c * kPartialStride + 129] : 0.0f;

  // fp16 token scores in the original basis (independent of the partials,
  // so they go first): scale * q . k, log2 units
  float Mf = kNegInf;
  if (nf > 0) {
    float q8[8];
    {
      const int64_t qoff = bh * kD + 8 * cl;
      if (a.q_f32) {
        const float4_t *qp = reinterpret_cast<const float4_t *>(reinterpret_cast<const float *>(a.q) + qoff);
        const float4_t x0 = qp[0], x1 = qp[1];
        q8[0] = x0.x; q8[1] = x0.y; q8[2] = x0.z; q8[3] = x0.w;
        q8[4] = x1.x; q8[5] = x1.y; q8[6] = x1.z; q8[7] = x1.w;
      } else {
        const u32x4_t u = *reinterpret_cast<const u32x4_t *>(reinterpret_cast<const _Float16 *>(a.q) + qoff);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const half2_t hq2 = __builtin_bit_cast(half2_t, w[i]);
          q8[2 * i] = (float)hq2.x;
          q8[2 * i + 1] = (float)hq2.y;
        }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) q8[i] *= a.qscale;
    }
    float sl = kNegInf;
    for (int64_t t0 = 0; t0 < nf; t0 += kFpRows * kFpUnroll) {
      u32x4_t u[kFpUnroll];
#pragma unroll
      for (int k = 0; k < kFpUnroll; ++k) {
        const int64_t t = t0 + k * kFpRows + rs;
        const int64_t tt = t < nf ? t : 0;
        u[k] = *reinterpret_cast<const u32x4_t *>(fp16_row(a.sink_k, a.res_k, bkv, a.n_sink, a.n_res, tt) + 8 * cl);
      }
#pragma unroll
      for (int k = 0; k < kFpUnroll; ++k) {
        const uint32_t w[4] = {u[k].x, u[k].y, u[k].z, u[k].w};
        float sacc = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const half2_t k2 = __builtin_bit_cast(half2_t, w[i]);
          sacc = __builtin_fmaf(q8[2 * i], (float)k2.x, sacc);
          sacc = __builtin_fmaf(q8[2 * i + 1], (float)k2.y, sacc);
        }
        sacc += quad_swap<kQuadXor1>(sacc);
        sacc += quad_swap<kQuadXor2>(sacc);
        sacc += row_ror<4>(sacc);
        sacc += row_ror<8>(sacc);
        const int64_t t = t0 + k * kFpRows + rs;
        if (t < nf) {
          if (cl == 0) pf[t] = sacc;
          sl = fmaxf(sl, sacc);
        }
      }
    }
    Mf = block_max(sl, red);                 // its barrier also publishes pf
  }

  // INT2 partials: M2 = max m_i, weights 2^(m_i - M2)
  float mloc = m0;
  for (int64_t i = c + kCombineThreads; i < ns; i += kCombineThreads)
    mloc = fmaxf(mloc, part[i * kPartialStride + 128]);
  const float M2 = block_max(mloc, red);
  float lloc = 0.0f;
  if (c < ns) {
    const float w0 = (m0 == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f(m0 - M2);
    wsplit[c] = w0;
    lloc = w0 * l0;
  }
  for (int64_t i = c + kCombineThreads; i < ns; i += kCombineThreads) {
    const float mi = part[i * kPartialStride + 128];
    const float wi = (mi == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f(mi - M2);
    wsplit[i] = wi;
    lloc += wi * part[i * kPartialStride + 129];
  }
  const float L2 = block_sum(lloc, red);     // its barrier also publishes wsplit
  // weighted sum of the partial outputs: thread t takes channel t%128 of the
  // splits with parity t/128; split par + 2u goes to accumulator u % 8, the
  // first 2 kPre from the early loads, the rest eight loads in flight
  float o = 0.0f;
  {
    float o8[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int u = 0; u < kPre; ++u) {
      const int64_t i = par + 2 * u;
      if (i < ns) o8[u & 7] = __builtin_fmaf(wsplit[i], pv[u], o8[u & 7]);
    }
    int64_t i = par + 2 * kPre;
    for (; i + 14 < ns; i += 16) {
#pragma unroll
      for (int u = 0; u < 8; ++u)
        o8[u] = __builtin_fmaf(wsplit[i + 2 * u], part[(i + 2 * u) * kPartialStride + ch], o8[u]);
    }
    for (; i < ns; i += 2) o8[0] = __builtin_fmaf(wsplit[i], part[i * kPartialStride + ch], o8[0]);
    vred[c] = ((o8[0] + o8[1]) + (o8[2] + o8[3])) + ((o8[4] + o8[5]) + (o8[6] + o8[7]));
    __syncthreads();
    if (own) o = vred[c] + vred[128 + c];
    __syncthreads();
  }

  // un-rotate the INT2 part (linear, so once after the merge)
  if (a.rot == 1) o = block_fwht128(o, buf);
  else if (a.rot == 2) o = block_matvec128(o, Rm, true, buf, vred);
  else if (a.rot == 3) {
    // o' R^T = (o' H / sqrt(d)) P^T: transform, then output j goes to channel pi[j]
    o = block_fwht128(o, buf);
    if (own) buf[a.perm[(int64_t)hkv * kD + c] & (kD - 1)] = o;
    __syncthreads();
    o = own ? buf[c] : 0.0f;
    __syncthreads();
  }

  // fp16 token weights and values, all in the original basis
  const float M = fmaxf(M2, Mf);
  float Lf = 0.0f, of = 0.0f;
  if (nf > 0) {
    float ll = 0.0f;
    for (int64_t t = c; t < nf; t += kCombineThreads) {
      const float p = __builtin_amdgcn_exp2f(pf[t] - M);
      pf[t] = p;
      ll += p;
    }
    Lf = block_sum(ll, red);                 // its barrier also publishes the weights
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    for (int64_t t0 = 0; t0 < nf; t0 += kFpRows * kFpUnroll) {
      u32x4_t u[kFpUnroll];
#pragma unroll
      for (int k = 0; k < kFpUnroll; ++k) {
        const int64_t t = t0 + k * kFpRows + rs;
        const int64_t tt = t < nf ? t : 0;
        u[k] = *reinterpret_cast<const u32x4_t *>(fp16_row(a.sink_v, a.res_v, bkv, a.n_sink, a.n_res, tt) + 8 * cl);
      }
#pragma unroll
      for (int k = 0; k < kFpUnroll; ++k) {
        const int64_t t = t0 + k * kFpRows + rs;
        const float p = t < nf ? pf[t] : 0.0f;
        const uint32_t w[4] = {u[k].x, u[k].y, u[k].z, u[k].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const half2_t v2 = __builtin_bit_cast(half2_t, w[i]);
          acc[2 * i] = __builtin_fmaf(p, (float)v2.x, acc[2 * i]);
          acc[2 * i + 1] = __builtin_fmaf(p, (float)v2.y, acc[2 * i + 1]);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) vred[rs * kD + 8 * cl + i] = acc[i];
    __syncthreads();
    if (own) {
      float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
      for (int r = 0; r < kFpRows; r += 2) {
        s0 += vred[r * kD + c];
        s1 += vred[(r + 1) * kD + c];
      }
      of = s0 + s1;
    }
  }
  if (own) {
    const float wint = (M2 == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f(M2 - M);
    const float den = L2 * wint + Lf;
    const float res = den > 0.0f ? (o * wint + of) / den : 0.0f;   // no token at all: 0
    if (a.out_f32) reinterpret_cast<float *>(a.out)[bh * kD + c] = res;
    else reinterpret_cast<_Float16 *>(a.out)[bh * kD + c] = (_Float16)res;
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
// Tile grid shift: start the grid t_begin mod 16 rows early when both caches
// keep the rows of a head on 16-row boundaries.
// A paged cache starts the grid on a 64-token boundary instead, so that no
// tile crosses a page.
static int grid_skip(const DecodeArgs &d) {
  if (d.block_table != nullptr) return (int)(d.t_begin % 64);
  return (d.kT_cap % 16 == 0 && d.vT_cap % 16 == 0) ? (int)(d.t_begin % 16) : 0;
}

// Keys with the pre-RoPE grouped-head rotation: the score launch, then the
// attention over the values with those scores (one wave per query head and
// split), then the combine with the values' Hadamard un-rotation.
static hipError_t launch_decode_prerope(const DecodeArgs &d, hipStream_t stream) {
  const int G = (int)(d.Hq / d.Hkv);
  const int skip = grid_skip(d);
  if (d.n_splits > 0) {
    PreropeArgs p;
    p.kcodes = d.kcodes; p.kscales = d.kscales; p.kzeros = d.kzeros; p.kT_cap = d.kT_cap;
    p.t_begin = d.t_begin; p.n_int2 = d.n_int2; p.skip = skip; p.n_rows = d.score_rows;
    p.B = d.B; p.Hq = (int)d.Hq; p.Hkv = (int)d.Hkv; p.G = G; p.GH = d.group_heads;
    p.q = d.q; p.q_f32 = d.q_f32;
    p.qscale = (float)((double)d.qscale / sqrt(128.0 * d.group_heads));
    p.log2_base = d.log2_rope_base;
    p.rope_table = d.rope_table;
    p.scores = d.scores;
    // steps of 16 tokens; at most 128 steps per wave (the kernel turns its
    // RoPE angles step by step from an exact start), at least 8, and about
    // two rounds of the chip's resident waves
    p.tiles = (d.n_int2 + 15) / 16;
    const int64_t groups = d.B * (d.Hkv / d.group_heads);
    int64_t chunks = (8192 + groups - 1) / groups;
    const int64_t by_tiles = (p.tiles + 7) / 8;
    chunks = chunks < by_tiles ? chunks : by_tiles;
    const int64_t min_chunks = (p.tiles + 127) / 128;
    chunks = chunks > min_chunks ? chunks : min_chunks;
    chunks = chunks > 0 ? chunks : 1;
    p.tiles_per_wave = (p.tiles + chunks - 1) / chunks;
    p.chunks = (p.tiles + p.tiles_per_wave - 1) / p.tiles_per_wave;
    hipError_t e = p.tiles > 0 ? launch_prerope_scores(p, stream) : hipSuccess;
    if (e != hipSuccess) return e;
    AttnArgs a;
    a.kcodes = d.kcodes; a.kscales = d.kscales; a.kzeros = d.kzeros; a.kT_cap = d.kT_cap;
    a.vcodes = d.vcodes; a.vscales = d.vscales; a.vzeros = d.vzeros; a.vT_cap = d.vT_cap;
    a.t_begin = d.t_begin; a.n_int2 = d.n_int2; a.t_ends = nullptr;
    a.n_splits = d.n_splits;
    a.B = d.B;
    a.total_waves = d.B * d.Hq * d.n_splits;       // one wave per query head and split
    a.Hkv = (int)d.Hkv; a.Hq = (int)d.Hq; a.G = G;
    a.qprep = nullptr;
    a.partials = d.partials;
    a.fused_prep = false;
    a.skip = skip;
    a.block_table = nullptr;
    a.max_pages = a.n_pages = a.page_tokens = 0;
    a.q = d.q; a.q_f32 = d.q_f32; a.rot = 1; a.perm = nullptr; a.qscale = d.qscale;
    a.scores = d.scores; a.score_rows = d.score_rows;
    hipLaunchKernelGGL((kv_int2_decode_attn<4, true>), dim3((unsigned)((a.total_waves + 3) / 4)), dim3(256), 0,
                       stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  CombineArgs c;
  c.q = d.q; c.q_f32 = d.q_f32; c.out_f32 = d.out_f32;
  c.Hq = (int)d.Hq; c.Hkv = (int)d.Hkv; c.rot = 1; c.R = nullptr; c.perm = nullptr; c.qscale = d.qscale;
  c.partials = d.partials; c.n_splits = d.n_splits;
  c.t_ends = nullptr;
  c.B = d.B; c.t_begin = d.t_begin; c.n_int2 = d.n_int2; c.skip = skip;
  c.sink_k = d.sink_k; c.sink_v = d.sink_v; c.n_sink = d.n_sink;
  c.res_k = d.res_k; c.res_v = d.res_v; c.n_res = d.n_res;
  c.out = d.out;
  const size_t lds = (size_t)(d.n_splits + d.n_sink + d.n_res) * sizeof(float);
  if (c.t_ends == nullptr && c.n_sink == 0 && c.n_res == 0 && c.rot != 2)
      hipLaunchKernelGGL(kv_combine_wave, dim3((unsigned)((d.B * d.Hq + kWaveCombineWaves - 1) / kWaveCombineWaves)),
                         dim3(64 * kWaveCombineWaves), 0, stream, c);
    else
      hipLaunchKernelGGL(kv_combine_unrotate, dim3((unsigned)(d.B * d.Hq)), dim3(kCombineThreads), lds, stream, c);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs &d, hipStream_t stream) {
  if (d.group_heads > 0) return launch_decode_prerope(d, stream);
  const int G = (int)(d.Hq / d.Hkv);
  // one query head per KV head without a dense rotation: the attention waves
  // prepare the query themselves
  const bool fused_prep = G == 1 && (d.rot == 0 || d.rot == 1);
  // other code widths: the b-bit kernel for one query head per KV head
  // (which prepares its query itself), the b-bit grouped-query kernel
  // otherwise (which reads the prepared query like the 2-bit one)
  const bool generic = d.kbits != 2 || d.vbits != 2;
  const bool generic_gqa = generic && G >= 2;
  // the b-bit kernel takes a dense R's query from the preparation launch
  if (((!generic && !fused_prep) || (generic && (d.rot == 2 || generic_gqa))) && d.n_splits > 0) {
    PrepArgs p;
    p.q = d.q; p.q_f32 = d.q_f32; p.Hq = (int)d.Hq; p.Hkv = (int)d.Hkv;
    p.rot = d.rot; p.R = d.R; p.perm = d.perm; p.qscale = d.qscale;
    p.qprep = reinterpret_cast<uint8_t *>(d.qprep);
    hipLaunchKernelGGL(kv_prep_query, dim3((unsigned)(d.B * d.Hq)), dim3(kMatThreads), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (d.n_splits > 0) {
    AttnArgs a;
    a.kcodes = d.kcodes; a.kscales = d.kscales; a.kzeros = d.kzeros; a.kT_cap = d.kT_cap;
    a.vcodes = d.vcodes; a.vscales = d.vscales; a.vzeros = d.vzeros; a.vT_cap = d.vT_cap;
    a.t_begin = d.t_begin; a.n_int2 = d.n_int2; a.t_ends = d.t_ends;
    a.n_splits = d.n_splits;
    a.B = d.B;
    // B*S split rows; the b-bit kernel for G = 1 runs one wave per query head
    a.total_waves = (generic && !generic_gqa ? d.B * d.Hq : split_units(d.B, d.Hq, d.Hkv)) * d.n_splits;
    a.Hkv = (int)d.Hkv; a.Hq = (int)d.Hq; a.G = G;
    a.qprep = reinterpret_cast<const uint32_t *>(d.qprep);
    a.partials = d.partials;
    a.fused_prep = fused_prep;
    a.skip = grid_skip(d);
    a.block_table = d.block_table;
    a.max_pages = d.max_pages; a.n_pages = d.n_pages; a.page_tokens = d.page_tokens;
    a.q = d.q; a.q_f32 = d.q_f32; a.rot = d.rot; a.perm = d.perm; a.qscale = d.qscale;
    if (generic_gqa) {
      hipError_t e = launch_attn_gqa_bits(a, d.kbits, d.vbits, stream);
      if (e != hipSuccess) return e;
    } else if (generic) {
      hipError_t e = launch_attn_generic(a, d.kbits, d.vbits, stream);
      if (e != hipSuccess) return e;
    } else if (G == 1) {
      hipLaunchKernelGGL(kv_int2_decode_attn<4>, dim3((unsigned)((a.total_waves + 3) / 4)), dim3(256), 0,
                         stream, a);
    } else {
      hipError_t e = launch_attn_gqa(a, stream);
      if (e != hipSuccess) return e;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    CombineArgs c;
    c.q = d.q; c.q_f32 = d.q_f32; c.out_f32 = d.out_f32;
    c.Hq = (int)d.Hq; c.Hkv = (int)d.Hkv; c.rot = d.rot; c.R = d.R; c.perm = d.perm; c.qscale = d.qscale;
    c.partials = d.partials; c.n_splits = d.n_splits;
    c.t_ends = d.n_splits > 0 ? d.t_ends : nullptr;
    c.B = d.B; c.t_begin = d.t_begin; c.n_int2 = d.n_int2; c.skip = grid_skip(d);
    c.sink_k = d.sink_k; c.sink_v = d.sink_v; c.n_sink = d.n_sink;
    c.res_k = d.res_k; c.res_v = d.res_v; c.n_res = d.n_res;
    c.out = d.out;
    const int64_t lds_splits = c.t_ends != nullptr ? varlen_lds_splits(d.B, d.n_splits) : d.n_splits;
    const size_t lds = (size_t)(lds_splits + d.n_sink + d.n_res) * sizeof(float);
    if (c.t_ends == nullptr && c.n_sink == 0 && c.n_res == 0 && c.rot != 2)
      hipLaunchKernelGGL(kv_combine_wave, dim3((unsigned)((d.B * d.Hq + kWaveCombineWaves - 1) / kWaveCombineWaves)),
                         dim3(64 * kWaveCombineWaves), 0, stream, c);
    else
      hipLaunchKernelGGL(kv_combine_unrotate, dim3((unsigned)(d.B * d.Hq)), dim3(kCombineThreads), lds, stream, c);
    return hipGetLastError();
  }
}

}  // namespace kvq
