// Internal host-side interface between the C ABI (api.cpp) and the kernel
// translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kvq {

// One side (K or V) of a quantize call.
struct QuantSide {
  const void *x;        // token rows, channel stride 1
  uint8_t *codes;
  uint16_t *scales;
  uint16_t *zeros;
  int64_t T_cap;
  int bits;             // code width: 1, 2 or 4 (codes per row: 16 * bits bytes)
};

struct QuantArgs {
  QuantSide side[2];    // K, V (a side with x == nullptr is skipped)
  int n_sides;
  bool in_f32;
  int64_t B, T_new, Hkv;
  int64_t stride_b, stride_t, stride_h;
  int64_t t_offset;
  const int32_t *offsets;   // per-sequence append: sequence b's rows start at slot offsets[b] (device [B]) or NULL
  int rot;              // 0 none, 1 Hadamard, 2 dense, 3 permuted Hadamard
  const float *R;       // dense: [Hkv][128][128]
  const int32_t *perm;  // permuted Hadamard: [Hkv][128]
  // paged cache (rows kernels for fp16 + Hadamard only): side T_cap is then
  // max_pages * page_tokens, the logical capacity of a sequence
  const int32_t *block_table;
  int64_t max_pages, n_pages, page_tokens;
};

hipError_t launch_quantize_rows(const QuantArgs &a, hipStream_t stream);
hipError_t launch_quantize_dense(const QuantArgs &a, hipStream_t stream);
// Keys with the pre-RoPE grouped-head rotation over group_heads (2 or 4)
// heads: side[0] only, fp16 rows, Hkv a multiple of 4.
hipError_t launch_quantize_grouped(const QuantArgs &a, int group_heads, hipStream_t stream);

// Decode.
struct DecodeArgs {
  const void *q;
  bool q_f32, out_f32;
  int64_t B, Hq, Hkv;
  const uint8_t *kcodes; const uint16_t *kscales; const uint16_t *kzeros; int64_t kT_cap;
  const uint8_t *vcodes; const uint16_t *vscales; const uint16_t *vzeros; int64_t vT_cap;
  int kbits, vbits;        // code widths (2: the INT2 kernels; else the b-bit kernel)
  int64_t t_begin, n_int2;
  const int32_t *t_ends;   // variable-length batch: per-sequence end (device [B]) or NULL
  int rot; const float *R; const int32_t *perm;
  // paged cache: [n_pages][Hkv][page_tokens] rows per side, block_table
  // [B][max_pages] (device); NULL: contiguous [B][Hkv][T_cap]
  const int32_t *block_table;
  int64_t max_pages, n_pages, page_tokens;
  const uint16_t *sink_k, *sink_v; int64_t n_sink;
  const uint16_t *res_k, *res_v; int64_t n_res;
  float qscale;         // softmax_scale * log2(e)
  void *out;
  // workspace carve-up (device pointers)
  int32_t *qprep;       // [B][Hq][kQprepDwordsPerHead] dwords
  float *partials;      // [B][Hq][n_splits][kPartialStride]; variable length: the same
                        // B*Hq*n_splits rows, shared by sequence
  int64_t n_splits;     // waves per (b, query head), each taking every n_splits-th tile
                        // (variable length: planned for the longest sequence)
  // keys with the pre-RoPE grouped-head rotation over group_heads heads
  // (0: not this mode); scores [B][Hq][score_rows] fp32 in the workspace
  int group_heads;
  double log2_rope_base;
  uint32_t *rope_table;      // kRopeTableBytes of the workspace
  float *scores;
  int64_t score_rows;
};

// Split plan shared by the workspace query and the attention call.
struct SplitPlan {
  int64_t n_splits;
};
// target_waves: the attention waves of one resident round (2048 at two
// waves per SIMD); decode_target_waves picks it for a call, and
// workspace_target_waves bounds it for the workspace query, which does not
// see the code widths.
SplitPlan plan_splits(int64_t B, int64_t Hq, int64_t Hkv, int64_t n_int2, int64_t target_waves = 2048);
int64_t decode_target_waves(int64_t G, int kbits, int vbits);
int64_t workspace_target_waves(int64_t G);
// attention waves per split: one per query head for G = 1, one per four
// query heads of a KV head for G >= 2 (the matrix-core GQA kernel)
int64_t split_units(int64_t B, int64_t Hq, int64_t Hkv);

// Per query head: 128 dwords of nibble limbs and group sums, then the 128
// fixed-point query values (int32).
constexpr int kQprepDwordsPerHead = 256;
constexpr int kQprepFixedOffset = 128;
constexpr int kPartialStride = 132;   // o'[128], m, l, 2 pad (16-byte rows)
// RoPE table of the pre-RoPE decode: per channel pair i < 64 the frequency in
// revolutions per position as 64-bit fixed point (high, low word), then the
// cosine and sine (fp32 bits) of 16 positions' angle
constexpr size_t kRopeTableBytes = 64 * 4 * sizeof(uint32_t);

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream);

// Device address of this GPU's static scratch array (KVQ_NOALLOC_SCRATCH_BYTES
// bytes, 256-byte aligned), looked up on the first call per GPU; the current
// device is the GPU.
hipError_t noalloc_scratch(void **ptr);

}  // namespace kvq
