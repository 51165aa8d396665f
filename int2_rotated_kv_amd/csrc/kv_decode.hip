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
//                        23-bit fixed-point vector split into three int8 limbs.
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
// and the inner sum is an exact int32 dot product (v_dot4 on int8 code
// bytes and int8 query limbs).  Values: o'_c += sum_t p_t s_{t,j} code_{t,c}
// + sum_t p_t z_{t,j}; the first term runs as v_dot2 over token pairs with
// codes placed in fp16 subnormal encodings (code * 2^(e-24)) and the
// weights p*s in fp16, accumulated in fp32.
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
  const int E = 22 - e;                      // |x| * 2^E < 2^22
  const int qi = zero_group ? 0 : (int)__builtin_rintf(ldexpf(x, E));
  const float step = zero_group ? 0.0f : ldexpf(1.0f, -E);
  int isum = qi;
#pragma unroll
  for (int m = 1; m < 32; m <<= 1) isum += __shfl_xor(isum, m, 32);

  // balanced base-256 digits: qi = hi*65536 + mid*256 + lo, each in int8
  const int lo = (int)(int8_t)(qi & 0xFF);
  const int r1 = (qi - lo) >> 8;
  const int mid = (int)(int8_t)(r1 & 0xFF);
  const int hi = (r1 - mid) >> 8;

  const int j = c >> 5, cg = c & 31;
  const int w = cg >> 4, bsel = (cg >> 2) & 3, k = cg & 3;
  uint8_t *base = a.qprep + bh * (kQprepDwordsPerHead * 4) + j * 128;
  const int off = (w * 4 + k) * 4 + bsel;
  base[0 * 32 + off] = (uint8_t)hi;
  base[1 * 32 + off] = (uint8_t)mid;
  base[2 * 32 + off] = (uint8_t)lo;
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

template <int GC>
__global__ __launch_bounds__(256) void kv_int2_decode_attn(AttnArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t gw = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (gw >= a.total_waves) return;           // whole wave leaves together
  const int64_t split = gw % a.n_splits;
  const int64_t bh = gw / a.n_splits;        // b*Hkv + hkv
  const int hkv = (int)(bh % a.Hkv);
  const int64_t b = bh / a.Hkv;
  const int ts = lane >> 2;                  // token slot 0..15
  const int j = lane & 3;                    // channel group
  const int64_t s0 = split * a.tps;
  const int64_t s1 = (s0 + a.tps < a.n_int2) ? s0 + a.tps : a.n_int2;

  uint32_t qh[GC][8], qm[GC][8], ql[GC][8];
  float qsum[GC], qstep[GC];
#pragma unroll
  for (int g = 0; g < GC; ++g) {
    const int hq = hkv * a.G + a.g0 + g;
    const uint32_t *p = a.qprep + (b * a.Hq + hq) * kQprepDwordsPerHead + j * 32;
#pragma unroll
    for (int i = 0; i < 8; ++i) { qh[g][i] = p[i]; qm[g][i] = p[8 + i]; ql[g][i] = p[16 + i]; }
    qsum[g] = bits_as_float(p[24]);
    qstep[g] = bits_as_float(p[25]);
  }

  float m[GC], l[GC], zacc[GC], acc[GC][32];
#pragma unroll
  for (int g = 0; g < GC; ++g) {
    m[g] = kNegInf; l[g] = 0.0f; zacc[g] = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) acc[g][i] = 0.0f;
  }

  const int64_t krow0 = bh * a.kT_cap + a.t_begin;
  const int64_t vrow0 = bh * a.vT_cap + a.t_begin;
  const uint8_t *kc = a.kcodes + krow0 * kCodeBytes + 8 * j;
  const uint16_t *ks = a.kscales + krow0 * kNGroups + j;
  const uint16_t *kz = a.kzeros + krow0 * kNGroups + j;
  const uint8_t *vc = a.vcodes + vrow0 * kCodeBytes + 8 * j;
  const uint16_t *vs = a.vscales + vrow0 * kNGroups + j;
  const uint16_t *vz = a.vzeros + vrow0 * kNGroups + j;

  for (int64_t t = s0; t < s1; t += 32) {
    const int64_t ta = t + ts, tb = t + 16 + ts;
    const bool va = ta < s1, vb = tb < s1;
    const int64_t la = va ? ta : s0, lb = vb ? tb : s0;
    const uint2 kA = *reinterpret_cast<const uint2 *>(kc + la * kCodeBytes);
    const uint2 kB = *reinterpret_cast<const uint2 *>(kc + lb * kCodeBytes);
    const uint2 vA = *reinterpret_cast<const uint2 *>(vc + la * kCodeBytes);
    const uint2 vB = *reinterpret_cast<const uint2 *>(vc + lb * kCodeBytes);
    const float skA = half_bits_to_float(ks[la * kNGroups]);
    const float zkA = half_bits_to_float(kz[la * kNGroups]);
    const float skB = half_bits_to_float(ks[lb * kNGroups]);
    const float zkB = half_bits_to_float(kz[lb * kNGroups]);
    const float svA = half_bits_to_float(vs[la * kNGroups]);
    const float zvA = half_bits_to_float(vz[la * kNGroups]);
    const float svB = half_bits_to_float(vs[lb * kNGroups]);
    const float zvB = half_bits_to_float(vz[lb * kNGroups]);

    // K codes -> int8 bytes: cX[w*4+k] byte b = code of channel 16w+4b+k
    uint32_t cA[8], cB[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      cA[k] = (kA.x >> (2 * k)) & 0x03030303u;
      cA[4 + k] = (kA.y >> (2 * k)) & 0x03030303u;
      cB[k] = (kB.x >> (2 * k)) & 0x03030303u;
      cB[4 + k] = (kB.y >> (2 * k)) & 0x03030303u;
    }

    half2_t wp[GC];
    float pA[GC], pB[GC];
#pragma unroll
    for (int g = 0; g < GC; ++g) {
      int ia = 0, ib = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        ia = __builtin_amdgcn_sdot4((int)qh[g][i], (int)cA[i], ia, false);
        ib = __builtin_amdgcn_sdot4((int)qh[g][i], (int)cB[i], ib, false);
      }
      ia <<= 8; ib <<= 8;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        ia = __builtin_amdgcn_sdot4((int)qm[g][i], (int)cA[i], ia, false);
        ib = __builtin_amdgcn_sdot4((int)qm[g][i], (int)cB[i], ib, false);
      }
      ia <<= 8; ib <<= 8;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        ia = __builtin_amdgcn_sdot4((int)ql[g][i], (int)cA[i], ia, false);
        ib = __builtin_amdgcn_sdot4((int)ql[g][i], (int)cB[i], ib, false);
      }
      float sa = (float)ia * (skA * qstep[g]) + zkA * qsum[g];
      float sb = (float)ib * (skB * qstep[g]) + zkB * qsum[g];
      sa += quad_swap<kQuadXor1>(sa);
      sb += quad_swap<kQuadXor1>(sb);
      sa += quad_swap<kQuadXor2>(sa);
      sb += quad_swap<kQuadXor2>(sb);
      sa = va ? sa : kNegInf;
      sb = vb ? sb : kNegInf;

      // online softmax (log2 domain); the tile max is wave-uniform
      float mx = fmaxf(sa, sb);
      mx = fmaxf(mx, shfl_xor_f(mx, 4));
      mx = fmaxf(mx, shfl_xor_f(mx, 8));
      mx = fmaxf(mx, shfl_xor_f(mx, 16));
      mx = fmaxf(mx, shfl_xor_f(mx, 32));
      if (mx > m[g]) {
        const float alpha = __builtin_amdgcn_exp2f(m[g] - mx);
        l[g] *= alpha;
        zacc[g] *= alpha;
#pragma unroll
        for (int i = 0; i < 32; ++i) acc[g][i] *= alpha;
        m[g] = mx;
      }
      pA[g] = va ? __builtin_amdgcn_exp2f(sa - m[g]) : 0.0f;
      pB[g] = vb ? __builtin_amdgcn_exp2f(sb - m[g]) : 0.0f;
      l[g] += pA[g] + pB[g];
      zacc[g] = __builtin_fmaf(pA[g], zvA, __builtin_fmaf(pB[g], zvB, zacc[g]));
      wp[g].x = (_Float16)(pA[g] * svA);
      wp[g].y = (_Float16)(pB[g] * svB);
    }

    // V: token pair (A in the low half, B in the high half) per channel
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const uint32_t a32 = w ? vA.y : vA.x;
      const uint32_t b32 = w ? vB.y : vB.x;
      const uint32_t X = (a32 & 0xFFFFu) | (b32 << 16);           // channels 16w+0..7
      const uint32_t Y = (a32 >> 16) | (b32 & 0xFFFF0000u);       // channels 16w+8..15
      const uint32_t X6 = X >> 6, Y6 = Y >> 6;
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        const uint32_t px = x <= 4 ? (X & (0x00030003u << (2 * x))) : (X6 & (0x00030003u << (2 * x - 6)));
        const uint32_t py = x <= 4 ? (Y & (0x00030003u << (2 * x))) : (Y6 & (0x00030003u << (2 * x - 6)));
        const half2_t hx = __builtin_bit_cast(half2_t, px);
        const half2_t hy = __builtin_bit_cast(half2_t, py);
#pragma unroll
        for (int g = 0; g < GC; ++g) {
          acc[g][16 * w + x] = __builtin_amdgcn_fdot2(hx, wp[g], acc[g][16 * w + x], false);
          acc[g][16 * w + 8 + x] = __builtin_amdgcn_fdot2(hy, wp[g], acc[g][16 * w + 8 + x], false);
        }
      }
    }
  }

  // reduce over the 16 token slots (lanes sharing j), then write the partial
#pragma unroll
  for (int g = 0; g < GC; ++g) {
#pragma unroll
    for (int msk = 4; msk < 64; msk <<= 1) {
      l[g] += shfl_xor_f(l[g], msk);
      zacc[g] += shfl_xor_f(zacc[g], msk);
#pragma unroll
      for (int i = 0; i < 32; ++i) acc[g][i] += shfl_xor_f(acc[g][i], msk);
    }
    if (ts == 0) {
      const int hq = hkv * a.G + a.g0 + g;
      float *dst = a.partials + ((b * a.Hq + hq) * a.n_splits + split) * kPartialStride;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const int x = i & 7;
        dst[32 * j + i] = __builtin_fmaf(acc[g][i], chan_unscale(x), zacc[g]);
      }
      if (j == 0) {
        dst[128] = m[g];
        dst[129] = l[g];
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
    const int GC = (G % 4 == 0) ? 4 : (G % 2 == 0) ? 2 : 1;
    const dim3 grid((unsigned)((a.total_waves + 3) / 4));
    for (int g0 = 0; g0 < G; g0 += GC) {
      a.g0 = g0;
      if (GC == 4) hipLaunchKernelGGL(kv_int2_decode_attn<4>, grid, dim3(256), 0, stream, a);
      else if (GC == 2) hipLaunchKernelGGL(kv_int2_decode_attn<2>, grid, dim3(256), 0, stream, a);
      else hipLaunchKernelGGL(kv_int2_decode_attn<1>, grid, dim3(256), 0, stream, a);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
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
