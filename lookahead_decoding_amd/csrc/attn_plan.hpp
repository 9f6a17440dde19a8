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

inline AttnPlan attn_plan(const lopa_dims& d) {
  AttnPlan p{};
  p.mfma = d.dtype == LOPA_BF16 && d.d == 128;
  p.splits = 1;
  if (!p.mfma) return p;
  const int rows = (d.k_max + 1) * d.B * (d.Hq / d.Hkv);
  p.row_groups = (rows + kAttnRowsPerWG - 1) / kAttnRowsPerWG;
  const int wgs = p.row_groups * d.Hkv;
  const int units = (d.L + kAttnKeysPerBlock - 1) / kAttnKeysPerBlock +
                    (d.B + kAttnKeysPerBlock - 1) / kAttnKeysPerBlock;
  int smax = 256 / wgs;
  if (smax > units / 2) smax = units / 2;
  if (smax > kAttnMaxSplits) smax = kAttnMaxSplits;
  p.splits = 1;
  int best = units;
  for (int s = 2; s <= smax; ++s) {
    const int t = (units + s - 1) / s + kAttnSplitCostUnits;
    if (t < best) {
      best = t;
      p.splits = s;
    }
  }
  return p;
}

// Partials of the split prefix: per split, KV head and query row, the
// unnormalised output (d floats), the running max and the running sum.
inline size_t attn_workspace_bytes(const lopa_dims& d) {
  const AttnPlan p = attn_plan(d);
  if (p.splits <= 1) return 0;
  const size_t rows = static_cast<size_t>(d.k_max + 1) * d.B * (d.Hq / d.Hkv);
  return static_cast<size_t>(p.splits) * d.Hkv * rows * (d.d + 2) * 4u;
}

}  // namespace lopa
