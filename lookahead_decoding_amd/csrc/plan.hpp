// Launch plans of the attention and LM-head calls, shared by the entry
// points and the workspace query so all three always agree.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include "lopa.h"

namespace lopa {

// MFMA kernel (bf16, hidden % 64 == 0): one launch of kHeadParts persistent
// workgroups, one per compute unit of an MI355X.  The device-side row count
// M picks the layout (head_groups): up to kHeadSmallRows rows, every
// workgroup owns a balanced contiguous vocabulary range and all rows; above
// that the rows are split into at most kHeadGroupTiles 32-row tiles per
// group, and the groups of one vocabulary range run side by side on the same
// XCD so the weight crosses HBM once.
constexpr int kHeadParts = 256;
constexpr int kHeadSmallRows = 128;
constexpr int kHeadGroupTiles = 8;
// Plain kernel (float32, or shapes outside the MFMA kernel): one vocabulary
// entry per thread, 256 per workgroup.
constexpr int kPlainVocabPerWG = 256;

struct HeadPlan {
  bool mfma;    // the MFMA kernel runs (else the plain one)
  int ntiles;   // upper bound on the partials per row (workspace stride)
  int m_max;    // nb_max * B
};

inline HeadPlan head_plan(const lopa_dims& d) {
  HeadPlan p{};
  const int hidden = d.Hq * d.d;
  p.m_max = (d.k_max + 1) * d.B;
  p.mfma = d.dtype == LOPA_BF16 && hidden % 64 == 0;
  p.ntiles = p.mfma ? kHeadParts : (d.V + kPlainVocabPerWG - 1) / kPlainVocabPerWG;
  return p;
}

// Row groups of the MFMA kernel for M rows.  wide: 2x2 compute-wave layout
// (vocabulary x rows) instead of 4x1; groups: row groups; nparts: vocabulary
// parts per group (a multiple of the 8 XCDs, nparts * groups <= kHeadParts);
// tpg: 32-row tiles per group.  m_max <= 1024 keeps groups <= 4.
struct HeadGroups {
  int wide, groups, nparts, tpg;
};

__host__ __device__ inline HeadGroups head_groups(int M) {
  const int tiles = (M + 31) / 32;
  if (M <= kHeadSmallRows) return HeadGroups{0, 1, kHeadParts, tiles};
  const int g = (tiles + kHeadGroupTiles - 1) / kHeadGroupTiles;
  return HeadGroups{1, g, 8 * (kHeadParts / 8 / g), (tiles + g - 1) / g};
}

// Per (row, vocabulary tile) partial: max logit (float), scaled sum (float),
// argmax (int32) -- three planes of m_max * ntiles.
inline size_t lmhead_workspace_bytes(const lopa_dims& d) {
  const HeadPlan p = head_plan(d);
  return static_cast<size_t>(p.m_max) * static_cast<size_t>(p.ntiles) * 12u;
}

// Attention MFMA kernel (bf16, d = 128): workgroups of 128 query rows per KV
// head walk work units of 64 keys -- the committed prefix in blocks, then the
// own block of every branch their rows belong to.  When one pass leaves most
// compute units idle the units are split over grid.z (at most one workgroup
// per compute unit, at least two units per split) and a second kernel merges
// the splits' unnormalised partials.
constexpr int kAttnRowsPerWG = 128;
constexpr int kAttnKeysPerBlock = 64;

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
  int s = 256 / wgs;
  if (s > units / 2) s = units / 2;
  p.splits = s < 1 ? 1 : s;
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

inline size_t workspace_bytes(const lopa_dims& d) {
  const size_t a = attn_workspace_bytes(d);
  const size_t h = lmhead_workspace_bytes(d);
  return a > h ? a : h;
}

}  // namespace lopa
