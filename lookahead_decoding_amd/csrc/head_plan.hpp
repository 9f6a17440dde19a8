// Launch plan of the LM-head call, shared by its entry point and the
// workspace query.
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

}  // namespace lopa
