// Split planning of the decode: pure host arithmetic, shared by the
// workspace queries of the C ABI and the decode launches.
#include "kvq_launch.h"

namespace kvq {

// Enough waves to fill the chip once: 256 CUs x 4 SIMDs x 2 resident waves
// of the attention kernel (its register budget allows two per SIMD).  One
// round of resident waves, each streaming every S-th tile of its head,
// measured faster than more, shorter waves.
constexpr int64_t kTargetWaves = 2048;
// The one-query-head b-bit attention at 1-bit keys and values holds 144
// registers, so three of its waves fit per SIMD, and it is bound by issue
// rather than memory: a round of three waves per SIMD measured 6% faster
// there (at the other widths more waves were slower or did not fit).
constexpr int64_t kTargetWavesNarrow = 3072;

int64_t decode_target_waves(int64_t G, int kbits, int vbits) {
  return G == 1 && kbits == 1 && vbits == 1 ? kTargetWavesNarrow : kTargetWaves;
}

int64_t workspace_target_waves(int64_t G) { return G == 1 ? kTargetWavesNarrow : kTargetWaves; }

// Waves per split unit: one per query head for G = 1, one per four query
// heads of a KV head for G >= 2 (the matrix-core GQA kernel).
int64_t split_units(int64_t B, int64_t Hq, int64_t Hkv) {
  const int64_t G = Hq / Hkv;
  return G == 1 ? B * Hq : B * Hkv * ((G + 3) / 4);
}

SplitPlan plan_splits(int64_t B, int64_t Hq, int64_t Hkv, int64_t n_int2, int64_t target_waves) {
  SplitPlan p{0};
  if (n_int2 <= 0 || B <= 0 || Hq <= 0 || Hkv <= 0) return p;
  const int64_t units = split_units(B, Hq, Hkv);
  int64_t s = target_waves / units;              // stay within one round of resident waves
  const int64_t by_len = (n_int2 + 255) / 256;   // at least ~256 tokens per wave
  if (s > by_len) s = by_len;
  if (s > 4096) s = 4096;
  if (s < 1) s = 1;
  p.n_splits = s;
  return p;
}

}  // namespace kvq
