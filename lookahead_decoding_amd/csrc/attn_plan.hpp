// Launch plan of the attention call, shared by its entry point and the
// workspace query.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include "lopa.h"

namespace lopa {

// Attention MFMA kernel (bf16, d = 128): workgroups of 64 query rows per KV
// head walk work units of 64 keys -- the committed prefix in blocks, then the
// own block of every branch their rows belong to.  The units may be split
// over grid.z (at most one workgroup per compute unit, at least two units per
// split, at most kAttnMaxSplits), and a second kernel then merges the splits'
// unnormalised partials; that merge (with its launch) costs about
// kAttnSplitCostUnits units of one workgroup's time, so the split count minimises
// ceil(units / splits) + (splits > 1) * kAttnSplitCostUnits.
constexpr int kAttnRowsPerWG = 64;
constexpr int kAttnKeysPerBlock = 64;
constexpr int kAttnMaxSplits = 16;
constexpr int kAttnSplitCostUnits = 5;

struct AttnPlan {
  bool mfma;
  int row_groups;  // grid.x
  int splits;      // grid.z
};

// Split count for a prefix of `units` 64-key work units (own blocks
// included) and wgs workgroups per split.
inline int attn_splits(int units, int wgs) {
  int smax = 256 / wgs;
  if (smax > units / 2) smax = units / 2;
  if (smax > kAttnMaxSplits) smax = kAttnMaxSplits;
  int splits = 1;
  int best = units;
  for (int s = 2; s <= smax; ++s) {
    const int t = (units + s - 1) / s + kAttnSplitCostUnits;
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
  const int rows = (d.k_max + 1) * d.B * (d.Hq / d.Hkv);
  p.row_groups = (rows + kAttnRowsPerWG - 1) / kAttnRowsPerWG;
  p.splits = attn_splits(attn_units(d), p.row_groups * d.Hkv);
  return p;
}

// Partials of the split prefix: per split, KV head and query row, the
// unnormalised output (d floats), the running max and the running sum.  The
// split count is not monotone in the prefix length, so the size returned is
// the largest over every prefix up to d.L: a buffer sized for a prefix also
// serves every shorter one (a sequence decoded block after block grows its
// prefix and keeps one workspace).
inline size_t attn_workspace_bytes(const lopa_dims& d) {
  const AttnPlan p = attn_plan(d);
  if (!p.mfma) return 0;
  const int wgs = p.row_groups * d.Hkv;
  const int u0 = (d.B + kAttnKeysPerBlock - 1) / kAttnKeysPerBlock;
  int cap = 256 / wgs;
  cap = cap < kAttnMaxSplits ? cap : kAttnMaxSplits;
  int smax = 1;
  for (int u = u0; u <= attn_units(d) && smax < cap; ++u) {
    const int s = attn_splits(u, wgs);
    smax = s > smax ? s : smax;
  }
  if (smax <= 1) return 0;
  const size_t rows = static_cast<size_t>(d.k_max + 1) * d.B * (d.Hq / d.Hkv);
  return static_cast<size_t>(smax) * d.Hkv * rows * (d.d + 2) * 4u;
}

}  // namespace lopa
