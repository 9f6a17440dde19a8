// Launch plan of the attention call, shared by its entry point and the
// workspace query.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include "lopa.h"

namespace lopa {

// Attention MFMA kernels (bf16, d = 128): workgroups of query rows of one KV
// head walk work units of 64 keys -- the committed prefix in blocks, then the
// own block of every branch their rows belong to.  k_attn_dma takes 64 rows
// per workgroup (four producer and four compute waves); k_attn_wide takes 128
// (eight compute waves, two per SIMD, in two groups one pipeline phase
// apart) and serves prefixes of at least kAttnWideMinKeys, where it measured
// faster (prefix 4096, 9 branches of 64: 73.7 against 84.8 us; at 2048 and
// below it is slower).  The units may be split over
// workgroups (at most one workgroup per compute unit, at least two units per
// split, at most kAttnMaxSplits), and a second kernel then merges the splits'
// unnormalised partials; that merge (with its launch) costs about
// kAttnSplitCost{Dma,Wide} units of one workgroup's time, so the split count
// minimises ceil(units / splits) + (splits > 1) * cost.
constexpr int kAttnRowsPerWG = 64;
constexpr int kAttnWideRows = 128;
constexpr int kAttnWideMinKeys = 4096;
constexpr int kAttnKeysPerBlock = 64;
constexpr int kAttnMaxSplits = 16;
constexpr int kAttnSplitCostDma = 5;
constexpr int kAttnSplitCostWide = 8;

struct AttnPlan {
  bool mfma;
  bool wide;       // k_attn_wide (128-row workgroups) instead of k_attn_dma
  int row_groups;  // workgroups per KV head and split
  int splits;
};

// Split count for `units` 64-key work units (own blocks included), wgs
// workgroups per split and a merge worth `cost` units.
inline int attn_splits(int units, int wgs, int cost) {
  int smax = 256 / wgs;
  if (smax > units / 2) smax = units / 2;
  if (smax > kAttnMaxSplits) smax = kAttnMaxSplits;
  int splits = 1;
  int best = units;
  for (int s = 2; s <= smax; ++s) {
    const int t = (units + s - 1) / s + cost;
    if (t < best) {
      best = t;
      splits = s;
    }
  }
  return splits;
}

inline int attn_units(const lopa_dims& d) {
  return (d.L + kAttnKeysPerBlock - 1) / kAttnKeysPerBlock +
         (d.B + kAttnKeysPerBlock - 1) / kAttnKeysPerBlock;
}

inline AttnPlan attn_plan(const lopa_dims& d) {
  AttnPlan p{};
  p.mfma = d.dtype == LOPA_BF16 && d.d == 128;
  p.splits = 1;
  if (!p.mfma) return p;
  p.wide = d.L >= kAttnWideMinKeys;
  const int rows = (d.k_max + 1) * d.B * (d.Hq / d.Hkv);
  const int per = p.wide ? kAttnWideRows : kAttnRowsPerWG;
  p.row_groups = (rows + per - 1) / per;
  p.splits = attn_splits(attn_units(d), p.row_groups * d.Hkv,
                         p.wide ? kAttnSplitCostWide : kAttnSplitCostDma);
  return p;
}

// Partials of the split prefix: per split, KV head and query row, the
// unnormalised output (d floats), the running max and the running sum.  The
// split count is not monotone in the prefix length, so the size returned is
// the largest over every prefix up to d.L: a buffer sized for a prefix also
// serves every shorter one (a sequence decoded block after block grows its
// prefix and keeps one workspace).
inline size_t attn_workspace_bytes(const lopa_dims& d) {
  if (!attn_plan(d).mfma) return 0;
  int smax = 1;
  for (int up = 0; up * kAttnKeysPerBlock < d.L + kAttnKeysPerBlock && smax < kAttnMaxSplits;
       ++up) {
    lopa_dims e = d;
    e.L = up * kAttnKeysPerBlock < d.L ? up * kAttnKeysPerBlock : d.L;
    const int s = attn_plan(e).splits;
    smax = s > smax ? s : smax;
  }
  if (smax <= 1) return 0;
  const size_t rows = static_cast<size_t>(d.k_max + 1) * d.B * (d.Hq / d.Hkv);
  return static_cast<size_t>(smax) * d.Hkv * rows * (d.d + 2) * 4u;
}

}  // namespace lopa
