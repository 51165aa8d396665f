// C ABI of the kvq library: argument validation (host only, before any HIP
// call) and dispatch to the gfx950 kernels.  The operations are defined in
// include/kvq.h.
#include "kvq.h"

#include <math.h>

#include "kvq_launch.h"

namespace {

constexpr int64_t kMaxFp16Tokens = 8192;   // sink + residual tokens per call

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

bool valid_dtype(kvq_dtype t) { return t == KVQ_F16 || t == KVQ_F32; }
bool valid_rot(kvq_rot r) {
  return r == KVQ_ROT_NONE || r == KVQ_ROT_HADAMARD || r == KVQ_ROT_DENSE ||
         r == KVQ_ROT_PERM_HADAMARD;
}

kvq_status check_rotation(kvq_rot rot, const void *R) {
  if (!valid_rot(rot)) return KVQ_ERR_INVALID_ARG;
  if (rot == KVQ_ROT_DENSE || rot == KVQ_ROT_PERM_HADAMARD) {
    if (R == nullptr || !aligned16(R)) return KVQ_ERR_INVALID_ARG;
  } else if (R != nullptr) {
    return KVQ_ERR_INVALID_ARG;
  }
  return KVQ_OK;
}

kvq_status check_cache(const kvq_quant_cache *c) {
  if (c == nullptr) return KVQ_ERR_INVALID_ARG;
  if (c->codes == nullptr || c->scales == nullptr || c->zeros == nullptr) return KVQ_ERR_INVALID_ARG;
  if (!aligned16(c->codes) || !aligned16(c->scales) || !aligned16(c->zeros)) return KVQ_ERR_INVALID_ARG;
  if (c->T_cap <= 0) return KVQ_ERR_INVALID_ARG;
  if (c->bits != 1 && c->bits != 2 && c->bits != 4) return KVQ_ERR_INVALID_ARG;
  return KVQ_OK;
}

// Block table of a paged cache (both sides share it).
struct Paging {
  const int32_t *block_table;
  int64_t max_pages, n_pages, page_tokens;
};

// Checks a paged side pair and the table; on success fills the cache views
// (T_cap = the logical capacity max_pages * page_tokens) and pg.  The widths
// are checked with the views.
kvq_status check_paged(const kvq_paged_cache *kc, const kvq_paged_cache *vc, const int32_t *block_table,
                       int64_t B, int64_t max_pages, kvq_quant_cache &kq, kvq_quant_cache &vq, Paging &pg) {
  if (block_table == nullptr || ((uintptr_t)block_table & 3u) != 0) return KVQ_ERR_INVALID_ARG;
  if (max_pages <= 0 || B < 0 || B * max_pages > 0x7FFFFFFF) return KVQ_ERR_INVALID_ARG;
  const kvq_paged_cache *cs[2] = {kc, vc};
  kvq_quant_cache *qs[2] = {&kq, &vq};
  int64_t np = -1, pt = -1;
  for (int i = 0; i < 2; ++i) {
    const kvq_paged_cache *c = cs[i];
    if (c == nullptr) continue;
    if (c->codes == nullptr || c->scales == nullptr || c->zeros == nullptr) return KVQ_ERR_INVALID_ARG;
    if (!aligned16(c->codes) || !aligned16(c->scales) || !aligned16(c->zeros)) return KVQ_ERR_INVALID_ARG;
    if (c->n_pages <= 0 || c->page_tokens < 64 || c->page_tokens % 64 != 0) return KVQ_ERR_INVALID_ARG;
    if (np >= 0 && (c->n_pages != np || c->page_tokens != pt)) return KVQ_ERR_INVALID_ARG;
    np = c->n_pages;
    pt = c->page_tokens;
    if (max_pages > (int64_t)0x7FFFFFFF / pt) return KVQ_ERR_INVALID_ARG;   // < 2^31 tokens per sequence
    qs[i]->codes = c->codes; qs[i]->scales = c->scales; qs[i]->zeros = c->zeros;
    qs[i]->T_cap = max_pages * c->page_tokens;
    qs[i]->bits = c->bits;
  }
  pg.block_table = block_table;
  pg.max_pages = max_pages;
  pg.n_pages = np;
  pg.page_tokens = pt;
  return KVQ_OK;
}

// An INT2 cache side as a 2-bit cache side (NULL stays NULL).
struct AsQuant {
  kvq_quant_cache c;
  const kvq_quant_cache *p;
  explicit AsQuant(const kvq_int2_cache *x) : c{}, p(nullptr) {
    if (x != nullptr) {
      c.codes = x->codes; c.scales = x->scales; c.zeros = x->zeros; c.T_cap = x->T_cap; c.bits = 2;
      p = &c;
    }
  }
};

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

size_t workspace_bytes(int64_t B, int64_t Hq, int64_t n_splits) {
  const size_t qprep = align256((size_t)B * Hq * kvq::kQprepDwordsPerHead * 4);
  const size_t parts = (size_t)B * Hq * n_splits * kvq::kPartialStride * sizeof(float);
  return qprep + parts;
}

// Score rows per (b, query head) of the pre-RoPE decode: the INT2 tokens plus
// the attention grid's shift (below 16), rounded up to 16.
int64_t prerope_score_rows(int64_t n_int2) { return (n_int2 + 16 + 15) / 16 * 16; }

// Pre-RoPE decode workspace: the split partials, fp32 key scores, then the
// RoPE table (frequencies and per-step turns of the 64 channel pairs).
size_t workspace_bytes_prerope(int64_t B, int64_t Hq, int64_t n_splits, int64_t n_int2) {
  const size_t parts = (size_t)B * Hq * n_splits * kvq::kPartialStride * sizeof(float);
  const size_t scores = (size_t)B * Hq * prerope_score_rows(n_int2) * sizeof(float);
  return align256(parts) + align256(scores) + kvq::kRopeTableBytes;
}


// Shared by the common-offset and the per-sequence-offset entry points.
// offsets == NULL: every sequence's rows start at t_offset (checked against
// T_cap here); otherwise at offsets[b] (device), where a row whose slot falls
// outside [0, T_cap) is skipped by the kernels.
kvq_status quantize_impl(const void *K, const void *V, kvq_dtype in_dtype, int64_t B,
                         int64_t T_new, int64_t Hkv, int64_t d, int64_t stride_b,
                         int64_t stride_t, int64_t stride_h, kvq_rot rot, const void *R,
                         int group, int64_t t_offset, const int32_t *offsets,
                         const kvq_quant_cache *kc, const kvq_quant_cache *vc, void *stream,
                         const Paging *pg = nullptr, int key_group_heads = 1) {
  if (!valid_dtype(in_dtype)) return KVQ_ERR_INVALID_ARG;
  if (B < 0 || T_new < 0 || Hkv <= 0 || t_offset < 0) return KVQ_ERR_INVALID_ARG;
  if (stride_b < 0 || stride_t < 0 || stride_h < 0) return KVQ_ERR_INVALID_ARG;
  if (d != 128 || group != 32) return KVQ_ERR_UNSUPPORTED;
  kvq_status st = check_rotation(rot, R);
  if (st != KVQ_OK) return st;
  if ((rot == KVQ_ROT_DENSE || rot == KVQ_ROT_PERM_HADAMARD) && in_dtype != KVQ_F16)
    return KVQ_ERR_UNSUPPORTED;
  if ((K == nullptr) != (kc == nullptr) || (V == nullptr) != (vc == nullptr)) return KVQ_ERR_INVALID_ARG;
  if (K == nullptr && V == nullptr) return KVQ_ERR_INVALID_ARG;
  const int64_t esize = in_dtype == KVQ_F32 ? 4 : 2;
  if ((stride_b * esize) % 16 || (stride_t * esize) % 16 || (stride_h * esize) % 16) return KVQ_ERR_INVALID_ARG;

  kvq::QuantArgs a{};
  a.n_sides = 0;
  const void *xs[2] = {K, V};
  const kvq_quant_cache *cs[2] = {kc, vc};
  for (int s = 0; s < 2; ++s) {
    if (xs[s] == nullptr) continue;
    if (!aligned16(xs[s])) return KVQ_ERR_INVALID_ARG;
    st = check_cache(cs[s]);
    if (st != KVQ_OK) return st;
    if (offsets == nullptr && (t_offset > cs[s]->T_cap || T_new > cs[s]->T_cap - t_offset))
      return KVQ_ERR_INVALID_ARG;
    if (offsets != nullptr && T_new > cs[s]->T_cap) return KVQ_ERR_INVALID_ARG;
    kvq::QuantSide &q = a.side[a.n_sides++];
    q.x = xs[s];
    q.codes = cs[s]->codes;
    q.scales = cs[s]->scales;
    q.zeros = cs[s]->zeros;
    q.T_cap = cs[s]->T_cap;
    q.bits = cs[s]->bits;
    // 1- and 4-bit codes: fp16 rows with a Hadamard (plain or reordered) or dense rotation
    if (q.bits != 2 && (in_dtype != KVQ_F16 || rot == KVQ_ROT_NONE)) return KVQ_ERR_UNSUPPORTED;
  }
  if (B * a.n_sides > 65535 || Hkv > 65535 || (T_new + 63) / 64 * Hkv > 0x7FFFFFFF)
    return KVQ_ERR_UNSUPPORTED;
  if (B == 0 || T_new == 0) return KVQ_OK;

  a.in_f32 = in_dtype == KVQ_F32;
  a.B = B; a.T_new = T_new; a.Hkv = Hkv;
  a.stride_b = stride_b; a.stride_t = stride_t; a.stride_h = stride_h;
  a.t_offset = t_offset;
  a.offsets = offsets;
  a.rot = (int)rot;
  a.R = rot == KVQ_ROT_DENSE ? static_cast<const float *>(R) : nullptr;
  a.perm = rot == KVQ_ROT_PERM_HADAMARD ? static_cast<const int32_t *>(R) : nullptr;
  if (pg != nullptr) {
    a.block_table = pg->block_table;
    a.max_pages = pg->max_pages; a.n_pages = pg->n_pages; a.page_tokens = pg->page_tokens;
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  if (key_group_heads > 1) {
    // keys with the pre-RoPE grouped-head rotation, values with the per-head
    // Hadamard rotation: one launch each
    e = hipSuccess;
    int next = 0;
    if (K != nullptr) {
      kvq::QuantArgs ak = a;
      ak.n_sides = 1;
      e = kvq::launch_quantize_grouped(ak, key_group_heads, s);
      next = 1;
    }
    if (e == hipSuccess && V != nullptr) {
      kvq::QuantArgs av = a;
      av.side[0] = a.side[next];
      av.n_sides = 1;
      e = kvq::launch_quantize_rows(av, s);
    }
  } else {
    e = (rot == KVQ_ROT_DENSE) ? kvq::launch_quantize_dense(a, s) : kvq::launch_quantize_rows(a, s);
  }
  if (e == hipErrorNotSupported) return KVQ_ERR_UNSUPPORTED;
  return e == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

}  // namespace

extern "C" {

kvq_status kvq_quantize(const void *K, const void *V, kvq_dtype in_dtype, int64_t B,
                        int64_t T_new, int64_t Hkv, int64_t d, int64_t stride_b,
                        int64_t stride_t, int64_t stride_h, kvq_rot rot, const void *R,
                        int group, int64_t t_offset, const kvq_int2_cache *kc,
                        const kvq_int2_cache *vc, void *stream) {
  const AsQuant k2(kc), v2(vc);
  return quantize_impl(K, V, in_dtype, B, T_new, Hkv, d, stride_b, stride_t, stride_h, rot, R,
                       group, t_offset, nullptr, k2.p, v2.p, stream);
}

kvq_status kvq_quantize_bits(const void *K, const void *V, kvq_dtype in_dtype, int64_t B,
                             int64_t T_new, int64_t Hkv, int64_t d, int64_t stride_b,
                             int64_t stride_t, int64_t stride_h, kvq_rot rot, const void *R,
                             int group, int64_t t_offset, const kvq_quant_cache *kc,
                             const kvq_quant_cache *vc, void *stream) {
  return quantize_impl(K, V, in_dtype, B, T_new, Hkv, d, stride_b, stride_t, stride_h, rot, R,
                       group, t_offset, nullptr, kc, vc, stream);
}

kvq_status kvq_quantize_at(const void *K, const void *V, kvq_dtype in_dtype, int64_t B,
                           int64_t T_new, int64_t Hkv, int64_t d, int64_t stride_b,
                           int64_t stride_t, int64_t stride_h, kvq_rot rot, const void *R,
                           int group, const int32_t *t_offsets, const kvq_int2_cache *kc,
                           const kvq_int2_cache *vc, void *stream) {
  if (t_offsets == nullptr || ((uintptr_t)t_offsets & 3u) != 0) return KVQ_ERR_INVALID_ARG;
  const AsQuant k2(kc), v2(vc);
  return quantize_impl(K, V, in_dtype, B, T_new, Hkv, d, stride_b, stride_t, stride_h, rot, R,
                       group, 0, t_offsets, k2.p, v2.p, stream);
}

size_t kvq_decode_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t d,
                                  int64_t n_int2_tokens, int64_t n_sink, int64_t n_res) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || d != 128) return 0;
  if (n_int2_tokens < 0 || n_sink < 0 || n_res < 0) return 0;
  const kvq::SplitPlan p = kvq::plan_splits(B, Hq, Hkv, n_int2_tokens, kvq::workspace_target_waves(Hq / Hkv));
  return workspace_bytes(B, Hq, p.n_splits);
}

}  // extern "C"

namespace {

// Shared by the fixed-length and the variable-length entry points: t_end is
// the (upper bound of the) end of every sequence's INT2 range; t_ends, when
// not NULL, holds each sequence's own end (device).
kvq_status decode_impl(const void *q, kvq_dtype q_dtype, int64_t B, int64_t Hq,
                       int64_t Hkv, int64_t d, const kvq_quant_cache *kc,
                       const kvq_quant_cache *vc, int64_t t_begin, int64_t t_end,
                       const int32_t *t_ends, kvq_rot rot, const void *R, int group,
                       const uint16_t *sink_k, const uint16_t *sink_v, int64_t n_sink,
                       const uint16_t *res_k, const uint16_t *res_v, int64_t n_res,
                       float softmax_scale, void *out, kvq_dtype out_dtype,
                       void *workspace, size_t workspace_bytes_given, void *stream,
                       const Paging *pg = nullptr, bool static_scratch = false,
                       int group_heads = 0, double rope_base = 0.0) {
  if (!valid_dtype(q_dtype) || !valid_dtype(out_dtype)) return KVQ_ERR_INVALID_ARG;
  if (q == nullptr || out == nullptr || !aligned16(q) || !aligned16(out)) return KVQ_ERR_INVALID_ARG;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0) return KVQ_ERR_INVALID_ARG;
  if (d != 128 || group != 32) return KVQ_ERR_UNSUPPORTED;
  kvq_status st = check_rotation(rot, R);
  if (st != KVQ_OK) return st;
  if (t_begin < 0 || t_end < t_begin) return KVQ_ERR_INVALID_ARG;
  const int64_t n_int2 = t_end - t_begin;
  if (n_int2 > 0) {
    if ((st = check_cache(kc)) != KVQ_OK) return st;
    if ((st = check_cache(vc)) != KVQ_OK) return st;
    if (t_end > kc->T_cap || t_end > vc->T_cap) return KVQ_ERR_INVALID_ARG;
  }
  if (n_sink < 0 || n_res < 0) return KVQ_ERR_INVALID_ARG;
  if (n_sink > 0 && (sink_k == nullptr || sink_v == nullptr || !aligned16(sink_k) || !aligned16(sink_v)))
    return KVQ_ERR_INVALID_ARG;
  if (n_res > 0 && (res_k == nullptr || res_v == nullptr || !aligned16(res_k) || !aligned16(res_v)))
    return KVQ_ERR_INVALID_ARG;
  if (n_int2 + n_sink + n_res < 1) return KVQ_ERR_INVALID_ARG;
  if (n_sink + n_res > kMaxFp16Tokens) return KVQ_ERR_UNSUPPORTED;
  if (B * Hq > 0x7FFFFFFF) return KVQ_ERR_UNSUPPORTED;
  if (!(softmax_scale == softmax_scale)) return KVQ_ERR_INVALID_ARG;   // NaN
  // keys with the pre-RoPE grouped-head rotation: one attention wave per
  // query head, and the score rows after the partials
  const int kbits = n_int2 > 0 ? kc->bits : 2, vbits = n_int2 > 0 ? vc->bits : 2;
  const kvq::SplitPlan plan =
      group_heads > 0 ? kvq::plan_splits(B, Hq, Hq, n_int2)
                      : kvq::plan_splits(B, Hq, Hkv, n_int2, kvq::decode_target_waves(Hq / Hkv, kbits, vbits));
  const size_t need = group_heads > 0 ? workspace_bytes_prerope(B, Hq, plan.n_splits, n_int2)
                                      : workspace_bytes(B, Hq, plan.n_splits);
  if (static_scratch) {
    // the library's own scratch array of this GPU (every argument is checked
    // by now: this is the call's first HIP call)
    if (need > (size_t)KVQ_NOALLOC_SCRATCH_BYTES) return KVQ_ERR_WORKSPACE_TOO_SMALL;
    if (kvq::noalloc_scratch(&workspace) != hipSuccess) return KVQ_ERR_HIP;
    workspace_bytes_given = KVQ_NOALLOC_SCRATCH_BYTES;
  }
  if (workspace == nullptr || ((uintptr_t)workspace & 255u) != 0) return KVQ_ERR_INVALID_ARG;
  if (workspace_bytes_given < need) return KVQ_ERR_WORKSPACE_TOO_SMALL;

  kvq::DecodeArgs a{};
  a.q = q;
  a.q_f32 = q_dtype == KVQ_F32;
  a.out_f32 = out_dtype == KVQ_F32;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv;
  if (n_int2 > 0) {
    a.kcodes = kc->codes; a.kscales = kc->scales; a.kzeros = kc->zeros; a.kT_cap = kc->T_cap;
    a.vcodes = vc->codes; a.vscales = vc->scales; a.vzeros = vc->zeros; a.vT_cap = vc->T_cap;
  }
  a.kbits = kbits;
  a.vbits = vbits;
  if (pg != nullptr && n_int2 > 0) {
    // paged caches: rows per page instead of per (b, head)
    a.block_table = pg->block_table;
    a.max_pages = pg->max_pages; a.n_pages = pg->n_pages; a.page_tokens = pg->page_tokens;
    a.kT_cap = a.vT_cap = pg->page_tokens;
  }
  a.t_begin = t_begin;
  a.n_int2 = n_int2;
  a.t_ends = n_int2 > 0 ? t_ends : nullptr;
  a.rot = (int)rot;
  a.R = rot == KVQ_ROT_DENSE ? static_cast<const float *>(R) : nullptr;
  a.perm = rot == KVQ_ROT_PERM_HADAMARD ? static_cast<const int32_t *>(R) : nullptr;
  a.sink_k = sink_k; a.sink_v = sink_v; a.n_sink = n_sink;
  a.res_k = res_k; a.res_v = res_v; a.n_res = n_res;
  const double scale = softmax_scale > 0.0f ? (double)softmax_scale : 1.0 / sqrt(128.0);
  a.qscale = (float)(scale * 1.4426950408889634);   // natural -> base-2 exponent
  a.out = out;
  a.qprep = reinterpret_cast<int32_t *>(workspace);
  a.partials = reinterpret_cast<float *>(reinterpret_cast<char *>(workspace) +
                                         align256((size_t)B * Hq * kvq::kQprepDwordsPerHead * 4));
  a.n_splits = plan.n_splits;
  if (group_heads > 0) {
    const size_t parts = (size_t)B * Hq * plan.n_splits * kvq::kPartialStride * sizeof(float);
    a.qprep = nullptr;
    a.partials = reinterpret_cast<float *>(workspace);
    a.scores = reinterpret_cast<float *>(reinterpret_cast<char *>(workspace) + align256(parts));
    a.score_rows = prerope_score_rows(n_int2);
    a.rope_table = reinterpret_cast<uint32_t *>(
        reinterpret_cast<char *>(a.scores) + align256((size_t)B * Hq * a.score_rows * sizeof(float)));
    a.group_heads = group_heads;
    a.log2_rope_base = log2(rope_base);
  }
  hipError_t e = kvq::launch_decode(a, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

}  // namespace

extern "C" {

kvq_status kvq_decode_attention(const void *q, kvq_dtype q_dtype, int64_t B, int64_t Hq,
                                int64_t Hkv, int64_t d, const kvq_int2_cache *kc,
                                const kvq_int2_cache *vc, int64_t t_begin, int64_t t_end,
                                kvq_rot rot, const void *R, int group,
                                const uint16_t *sink_k, const uint16_t *sink_v, int64_t n_sink,
                                const uint16_t *res_k, const uint16_t *res_v, int64_t n_res,
                                float softmax_scale, void *out, kvq_dtype out_dtype,
                                void *workspace, size_t workspace_bytes_given, void *stream) {
  const AsQuant k2(kc), v2(vc);
  return decode_impl(q, q_dtype, B, Hq, Hkv, d, k2.p, v2.p, t_begin, t_end, nullptr, rot, R, group,
                     sink_k, sink_v, n_sink, res_k, res_v, n_res, softmax_scale, out, out_dtype,
                     workspace, workspace_bytes_given, stream);
}

kvq_status kvq_decode_attention_noalloc(const void *q, kvq_dtype q_dtype, int64_t B, int64_t Hq,
                                        int64_t Hkv, int64_t d, const kvq_int2_cache *kc,
                                        const kvq_int2_cache *vc, int64_t t_begin, int64_t t_end,
                                        kvq_rot rot, const void *R, int group,
                                        const uint16_t *sink_k, const uint16_t *sink_v, int64_t n_sink,
                                        const uint16_t *res_k, const uint16_t *res_v, int64_t n_res,
                                        float softmax_scale, void *out, kvq_dtype out_dtype, void *stream) {
  const AsQuant k2(kc), v2(vc);
  return decode_impl(q, q_dtype, B, Hq, Hkv, d, k2.p, v2.p, t_begin, t_end, nullptr, rot, R, group,
                     sink_k, sink_v, n_sink, res_k, res_v, n_res, softmax_scale, out, out_dtype,
                     nullptr, 0, stream, nullptr, true);
}

kvq_status kvq_decode_attention_bits(const void *q, kvq_dtype q_dtype, int64_t B, int64_t Hq,
                                     int64_t Hkv, int64_t d, const kvq_quant_cache *kc,
                                     const kvq_quant_cache *vc, int64_t t_begin, int64_t t_end,
                                     kvq_rot rot, const void *R, int group,
                                     const uint16_t *sink_k, const uint16_t *sink_v, int64_t n_sink,
                                     const uint16_t *res_k, const uint16_t *res_v, int64_t n_res,
                                     float softmax_scale, void *out, kvq_dtype out_dtype,
                                     void *workspace, size_t workspace_bytes_given, void *stream) {
  return decode_impl(q, q_dtype, B, Hq, Hkv, d, kc, vc, t_begin, t_end, nullptr, rot, R, group,
                     sink_k, sink_v, n_sink, res_k, res_v, n_res, softmax_scale, out, out_dtype,
                     workspace, workspace_bytes_given, stream);
}

kvq_status kvq_decode_attention_varlen(const void *q, kvq_dtype q_dtype, int64_t B, int64_t Hq,
                                       int64_t Hkv, int64_t d, const kvq_int2_cache *kc,
                                       const kvq_int2_cache *vc, int64_t t_begin,
                                       const int32_t *t_ends, int64_t t_end_max,
                                       kvq_rot rot, const void *R, int group,
                                       const uint16_t *sink_k, const uint16_t *sink_v, int64_t n_sink,
                                       const uint16_t *res_k, const uint16_t *res_v, int64_t n_res,
                                       float softmax_scale, void *out, kvq_dtype out_dtype,
                                       void *workspace, size_t workspace_bytes_given, void *stream) {
  if (t_ends == nullptr || ((uintptr_t)t_ends & 3u) != 0) return KVQ_ERR_INVALID_ARG;
  const AsQuant k2(kc), v2(vc);
  return decode_impl(q, q_dtype, B, Hq, Hkv, d, k2.p, v2.p, t_begin, t_end_max, t_ends, rot, R, group,
                     sink_k, sink_v, n_sink, res_k, res_v, n_res, softmax_scale, out, out_dtype,
                     workspace, workspace_bytes_given, stream);
}

kvq_status kvq_quantize_at_bits(const void *K, const void *V, kvq_dtype in_dtype, int64_t B,
                                int64_t T_new, int64_t Hkv, int64_t d, int64_t stride_b,
                                int64_t stride_t, int64_t stride_h, kvq_rot rot, const void *R,
                                int group, const int32_t *t_offsets, const kvq_quant_cache *kc,
                                const kvq_quant_cache *vc, void *stream) {
  if (t_offsets == nullptr || ((uintptr_t)t_offsets & 3u) != 0) return KVQ_ERR_INVALID_ARG;
  return quantize_impl(K, V, in_dtype, B, T_new, Hkv, d, stride_b, stride_t, stride_h, rot, R,
                       group, 0, t_offsets, kc, vc, stream);
}

kvq_status kvq_decode_attention_varlen_bits(const void *q, kvq_dtype q_dtype, int64_t B, int64_t Hq,
                                            int64_t Hkv, int64_t d, const kvq_quant_cache *kc,
                                            const kvq_quant_cache *vc, int64_t t_begin,
                                            const int32_t *t_ends, int64_t t_end_max,
                                            kvq_rot rot, const void *R, int group,
                                            const uint16_t *sink_k, const uint16_t *sink_v,
                                            int64_t n_sink,
                                            const uint16_t *res_k, const uint16_t *res_v,
                                            int64_t n_res, float softmax_scale, void *out,
                                            kvq_dtype out_dtype, void *workspace,
                                            size_t workspace_bytes_given, void *stream) {
  if (t_ends == nullptr || ((uintptr_t)t_ends & 3u) != 0) return KVQ_ERR_INVALID_ARG;
  return decode_impl(q, q_dtype, B, Hq, Hkv, d, kc, vc, t_begin, t_end_max, t_ends, rot, R, group,
                     sink_k, sink_v, n_sink, res_k, res_v, n_res, softmax_scale, out, out_dtype,
                     workspace, workspace_bytes_given, stream);
}

kvq_status kvq_quantize_paged(const void *K, const void *V, kvq_dtype in_dtype, int64_t B,
                              int64_t T_new, int64_t Hkv, int64_t d, int64_t stride_b,
                              int64_t stride_t, int64_t stride_h, kvq_rot rot, const void *R,
                              int group, const int32_t *t_offsets, const int32_t *block_table,
                              int64_t max_pages, const kvq_paged_cache *kc,
                              const kvq_paged_cache *vc, void *stream) {
  if (t_offsets == nullptr || ((uintptr_t)t_offsets & 3u) != 0) return KVQ_ERR_INVALID_ARG;
  kvq_quant_cache kq{}, vq{};
  Paging pg{};
  const kvq_status st = check_paged(kc, vc, block_table, B, max_pages, kq, vq, pg);
  if (st != KVQ_OK) return st;
  return quantize_impl(K, V, in_dtype, B, T_new, Hkv, d, stride_b, stride_t, stride_h, rot, R,
                       group, 0, t_offsets, kc ? &kq : nullptr, vc ? &vq : nullptr, stream, &pg);
}

kvq_status kvq_decode_attention_paged(const void *q, kvq_dtype q_dtype, int64_t B, int64_t Hq,
                                      int64_t Hkv, int64_t d, const kvq_paged_cache *kc,
                                      const kvq_paged_cache *vc, int64_t t_begin,
                                      const int32_t *t_ends, int64_t t_end_max,
                                      const int32_t *block_table, int64_t max_pages,
                                      kvq_rot rot, const void *R, int group,
                                      const uint16_t *sink_k, const uint16_t *sink_v, int64_t n_sink,
                                      const uint16_t *res_k, const uint16_t *res_v, int64_t n_res,
                                      float softmax_scale, void *out, kvq_dtype out_dtype,
                                      void *workspace, size_t workspace_bytes_given, void *stream) {
  if (t_ends == nullptr || ((uintptr_t)t_ends & 3u) != 0) return KVQ_ERR_INVALID_ARG;
  if (kc == nullptr || vc == nullptr) return KVQ_ERR_INVALID_ARG;
  kvq_quant_cache kq{}, vq{};
  Paging pg{};
  const kvq_status st = check_paged(kc, vc, block_table, B, max_pages, kq, vq, pg);
  if (st != KVQ_OK) return st;
  return decode_impl(q, q_dtype, B, Hq, Hkv, d, &kq, &vq, t_begin, t_end_max, t_ends, rot, R, group,
                     sink_k, sink_v, n_sink, res_k, res_v, n_res, softmax_scale, out, out_dtype,
                     workspace, workspace_bytes_given, stream, &pg);
}

kvq_status kvq_quantize_prerope(const void *K, const void *V, kvq_dtype in_dtype, int64_t B,
                                int64_t T_new, int64_t Hkv, int64_t d, int64_t stride_b,
                                int64_t stride_t, int64_t stride_h, int group_heads, int group,
                                int64_t t_offset, const kvq_int2_cache *kc,
                                const kvq_int2_cache *vc, void *stream) {
  if (group_heads != 1 && group_heads != 2 && group_heads != 4) return KVQ_ERR_INVALID_ARG;
  if (Hkv <= 0 || Hkv % group_heads != 0) return KVQ_ERR_INVALID_ARG;
  if (group_heads > 1 && Hkv % 4 != 0) return KVQ_ERR_UNSUPPORTED;   // four heads per wave
  if (in_dtype == KVQ_F32) return KVQ_ERR_UNSUPPORTED;
  const AsQuant k2(kc), v2(vc);
  return quantize_impl(K, V, in_dtype, B, T_new, Hkv, d, stride_b, stride_t, stride_h, KVQ_ROT_HADAMARD,
                       nullptr, group, t_offset, nullptr, k2.p, v2.p, stream, nullptr, group_heads);
}

size_t kvq_decode_workspace_bytes_prerope(int64_t B, int64_t Hq, int64_t Hkv, int64_t d,
                                          int64_t n_int2_tokens, int64_t n_sink, int64_t n_res) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || d != 128) return 0;
  if (n_int2_tokens < 0 || n_sink < 0 || n_res < 0) return 0;
  const kvq::SplitPlan p = kvq::plan_splits(B, Hq, Hq, n_int2_tokens);
  return workspace_bytes_prerope(B, Hq, p.n_splits, n_int2_tokens);
}

kvq_status kvq_decode_attention_prerope(const void *q, kvq_dtype q_dtype, int64_t B, int64_t Hq,
                                        int64_t Hkv, int64_t d, const kvq_int2_cache *kc,
                                        const kvq_int2_cache *vc, int64_t t_begin, int64_t t_end,
                                        int group_heads, float rope_base, int group,
                                        const uint16_t *sink_k, const uint16_t *sink_v, int64_t n_sink,
                                        const uint16_t *res_k, const uint16_t *res_v, int64_t n_res,
                                        float softmax_scale, void *out, kvq_dtype out_dtype,
                                        void *workspace, size_t workspace_bytes_given, void *stream) {
  if (group_heads != 1 && group_heads != 2 && group_heads != 4) return KVQ_ERR_INVALID_ARG;
  if (Hkv <= 0 || Hkv % group_heads != 0) return KVQ_ERR_INVALID_ARG;
  if (!(rope_base > 1.0f) || !(rope_base <= 3.0e38f)) return KVQ_ERR_INVALID_ARG;
  if (Hq > 0 && Hq % Hkv == 0 && group_heads * (Hq / Hkv) > 32) return KVQ_ERR_UNSUPPORTED;
  if (t_end > 0x7FFFFFFF) return KVQ_ERR_UNSUPPORTED;            // positions are 32-bit
  const AsQuant k2(kc), v2(vc);
  return decode_impl(q, q_dtype, B, Hq, Hkv, d, k2.p, v2.p, t_begin, t_end, nullptr, KVQ_ROT_HADAMARD,
                     nullptr, group, sink_k, sink_v, n_sink, res_k, res_v, n_res, softmax_scale, out,
                     out_dtype, workspace, workspace_bytes_given, stream, nullptr, false, group_heads,
                     (double)rope_base);
}

const char *kvq_status_str(kvq_status s) {
  switch (s) {
    case KVQ_OK: return "KVQ_OK";
    case KVQ_ERR_INVALID_ARG: return "KVQ_ERR_INVALID_ARG";
    case KVQ_ERR_UNSUPPORTED: return "KVQ_ERR_UNSUPPORTED";
    case KVQ_ERR_WORKSPACE_TOO_SMALL: return "KVQ_ERR_WORKSPACE_TOO_SMALL";
    case KVQ_ERR_HIP: return "KVQ_ERR_HIP";
  }
  return "KVQ_ERR_UNKNOWN";
}

int kvq_abi_version(void) { return KVQ_ABI_VERSION; }

}  // extern "C"
