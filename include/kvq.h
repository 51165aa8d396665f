/*
 * kvq.h -- C ABI of the rotated INT2 KV-cache library (MI355X / gfx950).
 *
 * Two operations make up the hot path:
 *
 *   kvq_quantize          write path: rotate K and V rows by a per-head
 *                         orthogonal R, quantize them to asymmetric 2-bit
 *                         codes in channel groups, pack four codes per byte.
 *   kvq_decode_attention  read path: one decode query per (batch, query
 *                         head) attends over the packed cache (plus optional
 *                         fp16 sink / residual tokens); the query is rotated
 *                         by R, the output un-rotated by R^T.
 *
 * The method: "Output-Aware Rotation for INT2 KV-Cache Quantization"
 * (woor.ai page, section "Key Details": K and V rows of each head are
 * turned by that head's orthogonal matrix before the 2-bit quantizer sees
 * them, and the attention output is turned back afterwards; section "What
 * You Need to Know": the readout is scaled dot-product attention).  The
 * Hadamard form and its fast transform: RotateKV (IJCAI 2025 record,
 * abstract item (i)) and KVLinC (fugumt page, abstract).  Sinks kept at higher precision: RotateKV abstract, item (iii).
 * The pages fix no group size, scale format, rounding rule or bit layout;
 * the format below is this library's.
 *
 * Conventions for every entry point
 *  - Tensor pointers are DEVICE pointers (HIP global memory) owned by the
 *    caller.  The library never allocates, frees or synchronizes on these
 *    calls; work is enqueued on `stream` (a hipStream_t; NULL = the null
 *    stream) and runs asynchronously.
 *  - Arguments are validated on the host before anything is enqueued.  A
 *    failed check returns an error status and enqueues nothing.  A failed
 *    kernel launch returns KVQ_ERR_HIP.  No C++ exception crosses the ABI.
 *  - Device pointers must be 16-byte aligned (checked).
 *  - Preconditions not checked: inputs are finite; on the write path every
 *    rotated group's (max - min) / L and its minimum are within the fp16
 *    range (else the stored scale or zero is infinite); buffers are as large
 *    as the shapes say.  The decode handles every finite fp16 scale and
 *    zero; an output beyond the range of the output dtype rounds to inf.
 *  - There is no mutable global state; calls on different streams may run
 *    concurrently as long as they do not write the same memory.
 *
 * Cache format (one side, K or V), head-major:
 *    codes  uint8  [B][Hkv][T_cap][d/4]   channel 4b+i in bits 2i..2i+1 of
 *                                          byte b
 *    scales fp16   [B][Hkv][T_cap][d/32]   fp32(max-min)/3 rounded to fp16
 *    zeros  fp16   [B][Hkv][T_cap][d/32]   group minimum rounded to fp16
 *  with channel groups of 32 contiguous channels of the rotated row and
 *    code = clamp(rint_half_even((y - zero) * fp32(1/scale)), 0, 3)
 *  (all codes 0 when scale == 0), so that y ~= code * scale + zero.
 *  3 bits per element; 18.75% of an fp16 cache.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVQ_ABI_VERSION 7

typedef enum {
  KVQ_OK = 0,
  KVQ_ERR_INVALID_ARG = 1,        /* NULL/misaligned pointer, bad shape or range */
  KVQ_ERR_UNSUPPORTED = 2,        /* valid but not implemented (d != 128, group != 32, ...) */
  KVQ_ERR_WORKSPACE_TOO_SMALL = 3,
  KVQ_ERR_HIP = 4                 /* a HIP runtime call or kernel launch failed */
} kvq_status;

typedef enum { KVQ_F16 = 0, KVQ_F32 = 1 } kvq_dtype;

typedef enum {
  KVQ_ROT_NONE = 0,      /* identity: rows are quantized as given            */
  KVQ_ROT_HADAMARD = 1,  /* R = H_d / sqrt(d), H[i][j] = (-1)^popcount(i&j)  */
  KVQ_ROT_DENSE = 2,     /* R = caller's fp32 [Hkv][d][d] row-major, y = x R */
  KVQ_ROT_PERM_HADAMARD = 3  /* R = P_h H_d / sqrt(d): channels reordered by a
                              * per-head permutation pi_h, then the Hadamard
                              * transform, y_j = (H x_pi / sqrt(d))_j with
                              * (x_pi)_j = x[pi_h(j)]; the outlier-aware
                              * rotation of RotateKV (IJCAI 2025 record,
                              * abstract item (i): channel reordering ahead of
                              * the fast Walsh-Hadamard transform) */
} kvq_rot;

/* One side (K or V) of an INT2 cache; all three arrays are device memory
 * laid out as described above, sized for T_cap tokens per (b, head). */
typedef struct {
  uint8_t *codes;
  uint16_t *scales;
  uint16_t *zeros;
  int64_t T_cap;
} kvq_int2_cache;

/* One side of a cache whose codes are `bits` wide (1, 2 or 4; 2 is the INT2
 * format above, kvq_int2_cache's).  b-bit codes use L = 2^b - 1 levels
 * above the zero-point and pack 8/b codes per byte:
 *    codes  uint8  [B][Hkv][T_cap][d*b/8]  channel (8/b)j+i in bits
 *                                           b*i .. b*i+b-1 of byte j
 *    scales fp16   [B][Hkv][T_cap][d/32]   fp32(max-min)/L rounded to fp16
 *    zeros  fp16   [B][Hkv][T_cap][d/32]   group minimum rounded to fp16
 *    code = clamp(rint_half_even((y - zero) * fp32(1/scale)), 0, L).
 * Keys and values may be kept at different widths (for example 4-bit keys
 * with 2-bit values).  The pages name mixed-bit schemes and binary codes as
 * directions without fixing them (OptR page, the future-work paragraph and
 * "Why It Matters"); these widths are this library's. */
typedef struct {
  uint8_t *codes;
  uint16_t *scales;
  uint16_t *zeros;
  int64_t T_cap;
  int32_t bits;
} kvq_quant_cache;

/* One side (K or V) of a paged cache: fixed-size pages of page_tokens
 * token rows each, [n_pages][Hkv][page_tokens][...] per array, row formats as
 * above for codes `bits` wide (1, 2 or 4; 2 is the INT2 format).  A block
 * table int32 [B][max_pages] (device) maps sequence b's token t to row
 * t % page_tokens of page table[b][t / page_tokens]; page_tokens must be a
 * multiple of 64, and max_pages * page_tokens below 2^31.  Serving stacks
 * keep caches in such pages (the pages name serving stacks as the setting:
 * OptR page, "Why It Matters"). */
typedef struct {
  uint8_t *codes;
  uint16_t *scales;
  uint16_t *zeros;
  int64_t n_pages;
  int64_t page_tokens;
  int32_t bits;
} kvq_paged_cache;

/*
 * kvq_quantize -- rotate, quantize and pack T_new new tokens of K and V.
 *
 *  K, V       token rows, element type in_dtype; row (b, t, h) starts at
 *             element b*stride_b + t*stride_t + h*stride_h and its d
 *             channels are contiguous (channel stride 1).  For token-major
 *             [B][T_new][Hkv][d]: stride_b = T_new*Hkv*d, stride_t = Hkv*d,
 *             stride_h = d.  Either side may be skipped by passing NULL for
 *             both its input and its cache; not both.
 *  rot, R     KVQ_ROT_NONE / KVQ_ROT_HADAMARD with R == NULL;
 *             KVQ_ROT_DENSE with R = fp32 [Hkv][d][d] (device), y = x R_h;
 *             KVQ_ROT_PERM_HADAMARD with R = int32 [Hkv][d] (device), row h
 *             a permutation pi_h of 0..d-1 (entries are used modulo d; a
 *             row that is not a permutation gives unspecified codes, never
 *             an out-of-bounds access).  The dense and permuted paths need
 *             in_dtype == KVQ_F16.
 *  group      channels per scale/zero group; must be 32.
 *  t_offset   the rows land in cache slots [t_offset, t_offset + T_new) of
 *             every (b, h); must satisfy 0 <= t_offset, t_offset + T_new <=
 *             T_cap of each cache.
 *  d          head dimension; must be 128.
 *  T_new == 0 (or B == 0) is a no-op returning KVQ_OK.
 */
kvq_status kvq_quantize(const void *K, const void *V, kvq_dtype in_dtype,
                        int64_t B, int64_t T_new, int64_t Hkv, int64_t d,
                        int64_t stride_b, int64_t stride_t, int64_t stride_h,
                        kvq_rot rot, const void *R, int group,
                        int64_t t_offset, const kvq_int2_cache *kc,
                        const kvq_int2_cache *vc, void *stream);

/*
 * kvq_quantize_at -- kvq_quantize with a cache slot per sequence: the T_new
 * rows of sequence b land in slots [t_offsets[b], t_offsets[b] + T_new) of
 * every (b, h) (a decode-step append with sequences of different lengths
 * writes T_new = 1 row per sequence at its current length).
 *
 *  t_offsets  int32 [B], device, 4-byte aligned.  Read by the kernels, so
 *             not checked on the host: a row whose slot falls outside
 *             [0, T_cap) is not written.  T_new <= T_cap is checked.
 *  Every other argument as for kvq_quantize.
 * Serving stacks need this alongside variable-length decode (the pages
 * name serving stacks as the setting, OptR page, "Why It Matters").
 */
kvq_status kvq_quantize_at(const void *K, const void *V, kvq_dtype in_dtype,
                           int64_t B, int64_t T_new, int64_t Hkv, int64_t d,
                           int64_t stride_b, int64_t stride_t, int64_t stride_h,
                           kvq_rot rot, const void *R, int group,
                           const int32_t *t_offsets, const kvq_int2_cache *kc,
                           const kvq_int2_cache *vc, void *stream);

/*
 * kvq_decode_workspace_bytes -- bytes of device workspace that
 * kvq_decode_attention and kvq_decode_attention_varlen need for these sizes
 * (0 on invalid sizes; n_int2_tokens = t_end - t_begin, or t_end_max -
 * t_begin for the variable-length call).  Pure host arithmetic; calls
 * nothing in HIP.
 */
size_t kvq_decode_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t d,
                                  int64_t n_int2_tokens, int64_t n_sink,
                                  int64_t n_res);

/*
 * kvq_decode_attention -- out[b][h] = softmax(q' K_hat^T * scale) V_hat R^T
 * over INT2 tokens [t_begin, t_end) of the cache, jointly normalized with
 * the optional fp16 tokens, for every batch b and query head h.
 *
 *  q          [B][Hq][d] contiguous, q_dtype.  Query head h reads KV head
 *             h / (Hq/Hkv); Hq must be a multiple of Hkv.
 *  kc, vc     INT2 caches (rotated basis); t_begin <= t_end <= T_cap.
 *  rot, R     as for kvq_quantize; must match what wrote the cache.
 *  sink_k/v   fp16 [B][Hkv][n_sink][d] tokens kept unquantized in the
 *             ORIGINAL basis (NULL allowed when n_sink == 0).
 *  res_k/v    fp16 [B][Hkv][n_res][d], same (a recent-token window).
 *  softmax_scale  score multiplier; <= 0 selects 1/sqrt(d).
 *  out        [B][Hq][d] contiguous, out_dtype.
 *  workspace  device scratch of at least
 *             kvq_decode_workspace_bytes(B, Hq, Hkv, d, t_end - t_begin,
 *             n_sink, n_res) bytes; contents on entry are ignored.
 *  The total token count (t_end - t_begin + n_sink + n_res) must be >= 1.
 */
kvq_status kvq_decode_attention(const void *q, kvq_dtype q_dtype,
                                int64_t B, int64_t Hq, int64_t Hkv, int64_t d,
                                const kvq_int2_cache *kc,
                                const kvq_int2_cache *vc,
                                int64_t t_begin, int64_t t_end,
                                kvq_rot rot, const void *R, int group,
                                const uint16_t *sink_k, const uint16_t *sink_v,
                                int64_t n_sink,
                                const uint16_t *res_k, const uint16_t *res_v,
                                int64_t n_res, float softmax_scale,
                                void *out, kvq_dtype out_dtype,
                                void *workspace, size_t workspace_bytes,
                                void *stream);

/*
 * kvq_decode_attention_varlen -- kvq_decode_attention over a batch of
 * sequences of different lengths: sequence b attends to INT2 tokens
 * [t_begin, t_ends[b]) (plus the fp16 tokens, common to the batch).  The
 * attention waves are shared among the sequences in proportion to their
 * lengths, so a mixed batch costs about what its tokens cost.
 *
 *  t_ends     int32 [B], device, 4-byte aligned.  Read by the kernels and
 *             clamped to [t_begin, t_end_max].  A sequence left with no
 *             token at all (no INT2 and no fp16 token) gets a zero output.
 *  t_end_max  host upper bound of every t_ends[b]: sizes the split plan
 *             and the workspace (kvq_decode_workspace_bytes with
 *             n_int2_tokens = t_end_max - t_begin); t_end_max <= T_cap.
 *  Every other argument as for kvq_decode_attention.
 */
kvq_status kvq_decode_attention_varlen(const void *q, kvq_dtype q_dtype,
                                       int64_t B, int64_t Hq, int64_t Hkv, int64_t d,
                                       const kvq_int2_cache *kc,
                                       const kvq_int2_cache *vc, int64_t t_begin,
                                       const int32_t *t_ends, int64_t t_end_max,
                                       kvq_rot rot, const void *R, int group,
                                       const uint16_t *sink_k, const uint16_t *sink_v,
                                       int64_t n_sink,
                                       const uint16_t *res_k, const uint16_t *res_v,
                                       int64_t n_res, float softmax_scale,
                                       void *out, kvq_dtype out_dtype,
                                       void *workspace, size_t workspace_bytes,
                                       void *stream);

/*
 * kvq_quantize_bits -- kvq_quantize into caches of any supported code width
 * (kvq_quant_cache; keys and values may differ).  With both sides at 2 bits
 * it is kvq_quantize.  A side at 1 or 4 bits needs in_dtype == KVQ_F16 and
 * a rotation: KVQ_ROT_HADAMARD, KVQ_ROT_PERM_HADAMARD or KVQ_ROT_DENSE
 * (KVQ_ROT_NONE gives KVQ_ERR_UNSUPPORTED); bits outside {1, 2, 4} give
 * KVQ_ERR_INVALID_ARG.  Every other argument as for kvq_quantize.
 * Mixed-bit caches: OptR page, future-work paragraph.
 */
kvq_status kvq_quantize_bits(const void *K, const void *V, kvq_dtype in_dtype,
                             int64_t B, int64_t T_new, int64_t Hkv, int64_t d,
                             int64_t stride_b, int64_t stride_t, int64_t stride_h,
                             kvq_rot rot, const void *R, int group,
                             int64_t t_offset, const kvq_quant_cache *kc,
                             const kvq_quant_cache *vc, void *stream);

/*
 * kvq_decode_attention_bits -- kvq_decode_attention over caches of any
 * supported code width (kvq_quant_cache; keys and values may differ).  With
 * both sides at 2 bits it is kvq_decode_attention; otherwise a kernel for
 * the other widths runs, with every rotation.  Workspace as for
 * kvq_decode_attention (kvq_decode_workspace_bytes); every other argument
 * likewise.
 */
kvq_status kvq_decode_attention_bits(const void *q, kvq_dtype q_dtype,
                                     int64_t B, int64_t Hq, int64_t Hkv, int64_t d,
                                     const kvq_quant_cache *kc,
                                     const kvq_quant_cache *vc,
                                     int64_t t_begin, int64_t t_end,
                                     kvq_rot rot, const void *R, int group,
                                     const uint16_t *sink_k, const uint16_t *sink_v,
                                     int64_t n_sink,
                                     const uint16_t *res_k, const uint16_t *res_v,
                                     int64_t n_res, float softmax_scale,
                                     void *out, kvq_dtype out_dtype,
                                     void *workspace, size_t workspace_bytes,
                                     void *stream);

/*
 * kvq_quantize_at_bits -- kvq_quantize_at into caches of any supported code
 * width: the per-sequence slots of kvq_quantize_at with the caches and
 * width rules of kvq_quantize_bits.  Mixed-bit caches (OptR page, the
 * future-work paragraph) in the serving setting the pages name (OptR page,
 * "Why It Matters").
 */
kvq_status kvq_quantize_at_bits(const void *K, const void *V, kvq_dtype in_dtype,
                                int64_t B, int64_t T_new, int64_t Hkv, int64_t d,
                                int64_t stride_b, int64_t stride_t, int64_t stride_h,
                                kvq_rot rot, const void *R, int group,
                                const int32_t *t_offsets, const kvq_quant_cache *kc,
                                const kvq_quant_cache *vc, void *stream);

/*
 * kvq_decode_attention_varlen_bits -- kvq_decode_attention_varlen over
 * caches of any supported code width: the per-sequence ends of
 * kvq_decode_attention_varlen with the caches and rotation rules of
 * kvq_decode_attention_bits.  Workspace as for kvq_decode_attention_varlen.
 * Same sources as kvq_quantize_at_bits.
 */
kvq_status kvq_decode_attention_varlen_bits(const void *q, kvq_dtype q_dtype,
                                            int64_t B, int64_t Hq, int64_t Hkv, int64_t d,
                                            const kvq_quant_cache *kc,
                                            const kvq_quant_cache *vc, int64_t t_begin,
                                            const int32_t *t_ends, int64_t t_end_max,
                                            kvq_rot rot, const void *R, int group,
                                            const uint16_t *sink_k, const uint16_t *sink_v,
                                            int64_t n_sink,
                                            const uint16_t *res_k, const uint16_t *res_v,
                                            int64_t n_res, float softmax_scale,
                                            void *out, kvq_dtype out_dtype,
                                            void *workspace, size_t workspace_bytes,
                                            void *stream);

/*
 * kvq_quantize_paged -- kvq_quantize_at into a paged cache: sequence b's
 * T_new rows are its tokens t_offsets[b] .. t_offsets[b] + T_new - 1, each
 * written to its page through block_table.  A token outside
 * [0, max_pages * page_tokens), or whose page index is outside [0, n_pages),
 * is not written.  Input rows, rotations and code widths follow the rules
 * of kvq_quantize and kvq_quantize_bits.  kc and vc (either may be NULL with
 * its input) must agree on n_pages and page_tokens; each has its own bits
 * (1, 2 or 4, else KVQ_ERR_INVALID_ARG).
 */
kvq_status kvq_quantize_paged(const void *K, const void *V, kvq_dtype in_dtype,
                              int64_t B, int64_t T_new, int64_t Hkv, int64_t d,
                              int64_t stride_b, int64_t stride_t, int64_t stride_h,
                              kvq_rot rot, const void *R, int group,
                              const int32_t *t_offsets, const int32_t *block_table,
                              int64_t max_pages, const kvq_paged_cache *kc,
                              const kvq_paged_cache *vc, void *stream);

/*
 * kvq_decode_attention_paged -- kvq_decode_attention_varlen over a paged
 * cache: sequence b attends to its tokens [t_begin, t_ends[b]) found through
 * block_table [B][max_pages] (device, 4-byte aligned); t_end_max <=
 * max_pages * page_tokens.  A page index outside [0, n_pages) reads page 0
 * (an unspecified result, never an access outside the cache).  Workspace:
 * kvq_decode_workspace_bytes with n_int2_tokens = t_end_max - t_begin.
 * With either side at 1 or 4 bits the rotation rules of
 * kvq_decode_attention_bits apply.  Every other argument as for
 * kvq_decode_attention_varlen.
 */
kvq_status kvq_decode_attention_paged(const void *q, kvq_dtype q_dtype,
                                      int64_t B, int64_t Hq, int64_t Hkv, int64_t d,
                                      const kvq_paged_cache *kc,
                                      const kvq_paged_cache *vc, int64_t t_begin,
                                      const int32_t *t_ends, int64_t t_end_max,
                                      const int32_t *block_table, int64_t max_pages,
                                      kvq_rot rot, const void *R, int group,
                                      const uint16_t *sink_k, const uint16_t *sink_v,
                                      int64_t n_sink,
                                      const uint16_t *res_k, const uint16_t *res_v,
                                      int64_t n_res, float softmax_scale,
                                      void *out, kvq_dtype out_dtype,
                                      void *workspace, size_t workspace_bytes,
                                      void *stream);

/*
 * Pre-RoPE grouped-head rotation of the keys (RotateKV, IJCAI 2025 record,
 * abstract item (ii): keys are rotated before the rotary position embedding,
 * and across a group of heads, so that RoPE does not disturb the rotation
 * and outliers spread over heads).  The record fixes neither the embedding
 * nor the grouping; this library reads them as follows.
 *  - Keys are given BEFORE RoPE.  The rows of group_heads (g) consecutive KV
 *    heads of a token form one row of 128 g channels (head j of the group at
 *    channels 128 j .. 128 j + 127), rotated by the normalized Sylvester
 *    Hadamard matrix of size 128 g; head j's 128-channel slice is its cache
 *    row, in the INT2 format above.  g = 1 is the per-head Hadamard rotation.
 *  - Values carry no RoPE and keep the per-head Hadamard rotation.
 *  - RoPE is the rotate-half form: channel i pairs with i + 64, and pair i
 *    turns by the angle t * rope_base^(-2i/128) at position t.  An INT2 key's
 *    position is its cache slot t.
 *  - The decode query is given AFTER RoPE (at its own position), as a model
 *    produces it; fp16 sink / residual keys are kept as a plain fp16 cache
 *    keeps them: after RoPE, unrotated.  Their values are unrotated.
 * The decode therefore computes, for INT2 token t of KV head h,
 *    s_t = softmax_scale * q . rope_t(slice_h(k_hat_group,t R_g^T)).
 */

/*
 * kvq_quantize_prerope -- write pre-RoPE keys with the grouped-head rotation
 * and values with the per-head Hadamard rotation into INT2 caches.
 *  group_heads  1, 2 or 4 heads per rotation group; Hkv must be a multiple
 *               of it (KVQ_ERR_INVALID_ARG), and of 4 when group_heads > 1
 *               (KVQ_ERR_UNSUPPORTED).
 *  in_dtype     KVQ_F16 (KVQ_F32 gives KVQ_ERR_UNSUPPORTED).
 *  Every other argument as for kvq_quantize (rot = KVQ_ROT_HADAMARD, R = NULL).
 */
kvq_status kvq_quantize_prerope(const void *K, const void *V, kvq_dtype in_dtype,
                                int64_t B, int64_t T_new, int64_t Hkv, int64_t d,
                                int64_t stride_b, int64_t stride_t, int64_t stride_h,
                                int group_heads, int group, int64_t t_offset,
                                const kvq_int2_cache *kc, const kvq_int2_cache *vc,
                                void *stream);

/*
 * kvq_decode_workspace_bytes_prerope -- workspace bytes of
 * kvq_decode_attention_prerope (0 on invalid sizes): the split partials and
 * one fp32 key score per (b, query head, INT2 token).  Pure host arithmetic.
 */
size_t kvq_decode_workspace_bytes_prerope(int64_t B, int64_t Hq, int64_t Hkv, int64_t d,
                                          int64_t n_int2_tokens, int64_t n_sink,
                                          int64_t n_res);

/*
 * kvq_decode_attention_prerope -- decode attention over caches written by
 * kvq_quantize_prerope: INT2 tokens [t_begin, t_end) (positions t_begin ..
 * t_end - 1, t_end < 2^31) plus the fp16 tokens, as described above.
 *  group_heads  as written (1, 2 or 4; Hkv a multiple of it); group_heads *
 *               (Hq / Hkv) must be at most 32 (KVQ_ERR_UNSUPPORTED).
 *  rope_base    > 1 and finite (10000 for LLaMA-2).
 *  workspace    at least kvq_decode_workspace_bytes_prerope(...) bytes.
 *  Every other argument as for kvq_decode_attention (no rotation argument).
 */
kvq_status kvq_decode_attention_prerope(const void *q, kvq_dtype q_dtype,
                                        int64_t B, int64_t Hq, int64_t Hkv, int64_t d,
                                        const kvq_int2_cache *kc, const kvq_int2_cache *vc,
                                        int64_t t_begin, int64_t t_end,
                                        int group_heads, float rope_base, int group,
                                        const uint16_t *sink_k, const uint16_t *sink_v,
                                        int64_t n_sink,
                                        const uint16_t *res_k, const uint16_t *res_v,
                                        int64_t n_res, float softmax_scale,
                                        void *out, kvq_dtype out_dtype,
                                        void *workspace, size_t workspace_bytes,
                                        void *stream);

/*
 * kvq_decode_attention_noalloc -- kvq_decode_attention without a workspace
 * argument, for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * call allocates nothing (no hipMalloc, no hipFree): its scratch memory (the
 * prepared queries and the split partials) is a static device array of
 * KVQ_NOALLOC_SCRATCH_BYTES bytes per GPU, which each GPU the library runs on
 * holds until the process ends.  Its device address is looked up on the first
 * call on a GPU (that GPU current), so the first call also makes that lookup;
 * `stream` must belong to the current GPU.
 *
 *  - Sizes whose scratch (kvq_decode_workspace_bytes of the same arguments)
 *    exceeds KVQ_NOALLOC_SCRATCH_BYTES return KVQ_ERR_WORKSPACE_TOO_SMALL and
 *    enqueue nothing; use kvq_decode_attention with a workspace there.
 *  - Every call on one GPU shares that GPU's array, which keeps the last
 *    call's contents; nothing in it needs to start at zero (each call writes
 *    every byte it reads).  Calls that overlap on one GPU (different streams,
 *    or host threads racing) race on the array and give unspecified results;
 *    calls in one stream are ordered and safe.
 *  Every other argument, and the result, as for kvq_decode_attention.
 */
#define KVQ_NOALLOC_SCRATCH_BYTES (16u << 20)
kvq_status kvq_decode_attention_noalloc(const void *q, kvq_dtype q_dtype,
                                        int64_t B, int64_t Hq, int64_t Hkv, int64_t d,
                                        const kvq_int2_cache *kc,
                                        const kvq_int2_cache *vc,
                                        int64_t t_begin, int64_t t_end,
                                        kvq_rot rot, const void *R, int group,
                                        const uint16_t *sink_k, const uint16_t *sink_v,
                                        int64_t n_sink,
                                        const uint16_t *res_k, const uint16_t *res_v,
                                        int64_t n_res, float softmax_scale,
                                        void *out, kvq_dtype out_dtype, void *stream);

/* Human-readable name of a status code (static storage). */
const char *kvq_status_str(kvq_status s);

/* KVQ_ABI_VERSION of the built library. */
int kvq_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
