// Launch plan of the LM-head call, shared by the entry point and the
// workspace query so both always agree.
#pragma once

#include <stddef.h>

#include "lopa.h"

namespace lopa {

// MFMA kernel (bf16): 128 vocabulary rows per workgroup.  Variants by the
// device-side row count M: small (M <= 160, 64-wide K chunks), mid
// (161..384, 64-wide), large (> 384, 32-wide K chunks, row groups of 576).
// Without hidden % 128 == 0 only the large variant (hidden % 64 == 0) runs,
// for every M.
constexpr int kHeadVocabPerWG = 128;
constexpr int kHeadSmallRows = 160;
constexpr int kHeadMidRows = 384;
constexpr int kHeadGroupRows = 576;
// Plain kernel (float32, or shapes outside the MFMA kernel): one vocabulary
// entry per thread, 256 per workgroup.
constexpr int kPlainVocabPerWG = 256;

struct HeadPlan {
  bool small, mid, large;  // which MFMA variants are enqueued
  int large_lo;            // the large variant serves M > large_lo
  int groups;              // row groups of the large variant (grid.y)
  int ntiles;              // vocabulary tiles = partials per row
  int m_max;               // nb_max * B
};

inline HeadPlan head_plan(const lopa_dims& d) {
  HeadPlan p{};
  const int hidden = d.Hq * d.d;
  p.m_max = (d.k_max + 1) * d.B;
  const bool bf16 = d.dtype == LOPA_BF16;
  const bool k128 = bf16 && hidden % 128 == 0;
  const bool k64 = bf16 && hidden % 64 == 0;
  p.small = k128;
  p.mid = k128 && p.m_max > kHeadSmallRows;
  p.large = k64 && (!k128 || p.m_max > kHeadMidRows);
  p.large_lo = k128 ? kHeadMidRows : 0;
  p.groups = (p.m_max + kHeadGroupRows - 1) / kHeadGroupRows;
  p.ntiles = k64 ? (d.V + kHeadVocabPerWG - 1) / kHeadVocabPerWG
                 : (d.V + kPlainVocabPerWG - 1) / kPlainVocabPerWG;
  return p;
}

// Per (row, vocabulary tile) partial: max logit (float), scaled sum (float),
// argmax (int32) -- three planes of m_max * ntiles.
inline size_t lmhead_workspace_bytes(const lopa_dims& d) {
  const HeadPlan p = head_plan(d);
  return static_cast<size_t>(p.m_max) * static_cast<size_t>(p.ntiles) * 12u;
}

}  // namespace lopa
