// Launch plans of the attention and LM-head calls, shared by the entry
// points and the workspace query so all three always agree.
#pragma once

#include <stddef.h>

#include "lopa.h"

namespace lopa {

// MFMA kernel (bf16): kHeadParts persistent workgroups, one per compute
// unit of an MI355X, each owning a balanced contiguous vocabulary range.
// Variants by the device-side row count M (64-wide K chunks): small
// (M <= 128, 256 vocabulary rows per pass), mid (129..256, 128 rows per
// pass), large (> 256, 128 rows per pass, balanced row groups of at most
// 320 rows, each group streaming the weight once).  hidden must be a
// multiple of 128.
constexpr int kHeadParts = 256;
constexpr int kHeadSmallRows = 128;
constexpr int kHeadMidRows = 256;
constexpr int kHeadGroupRows = 320;
// Plain kernel (float32, or shapes outside the MFMA kernel): one vocabulary
// entry per thread, 256 per workgroup.
constexpr int kPlainVocabPerWG = 256;

struct HeadPlan {
  bool small, mid, large;  // which MFMA variants are enqueued
  int large_lo;            // the large variant serves M > large_lo
  int groups;              // row groups of the large variant (grid.y)
  int ntiles;              // vocabulary parts = partials per row
  int m_max;               // nb_max * B
};

inline HeadPlan head_plan(const lopa_dims& d) {
  HeadPlan p{};
  const int hidden = d.Hq * d.d;
  p.m_max = (d.k_max + 1) * d.B;
  const bool bf16 = d.dtype == LOPA_BF16;
  const bool k128 = bf16 && hidden % 128 == 0;
  p.small = k128;
  p.mid = k128 && p.m_max > kHeadSmallRows;
  p.large = k128 && p.m_max > kHeadMidRows;
  p.large_lo = kHeadMidRows;
  p.groups = (p.m_max + kHeadGroupRows - 1) / kHeadGroupRows;
  p.ntiles = k128 ? kHeadParts : (d.V + kPlainVocabPerWG - 1) / kPlainVocabPerWG;
  return p;
}

// Per (row, vocabulary tile) partial: max logit (float), scaled sum (float),
// argmax (int32) -- three planes of m_max * ntiles.
inline size_t lmhead_workspace_bytes(const lopa_dims& d) {
  const HeadPlan p = head_plan(d);
  return static_cast<size_t>(p.m_max) * static_cast<size_t>(p.ntiles) * 12u;
}

// Attention MFMA kernel (bf16, d = 128, (B * Hq/Hkv) % 16 == 0): workgroups
// of 128 query rows per KV head; the committed prefix may be split over
// grid.z when that is the only way to occupy the chip, with the splits'
// unnormalised partials merged by a second kernel.
constexpr int kAttnRowsPerWG = 128;
constexpr int kAttnKeysPerBlock = 64;

struct AttnPlan {
  bool mfma;
  int row_groups;  // grid.x
  int splits;      // grid.z
};

inline AttnPlan attn_plan(const lopa_dims& d) {
  AttnPlan p{};
  const int G = d.Hq / d.Hkv;
  p.mfma = d.dtype == LOPA_BF16 && d.d == 128 && (d.B * G) % 16 == 0;
  p.splits = 1;
  if (!p.mfma) return p;
  const int rows = (d.k_max + 1) * d.B * G;
  p.row_groups = (rows + kAttnRowsPerWG - 1) / kAttnRowsPerWG;
  const int wgs = p.row_groups * d.Hkv;
  const int blocks = (d.L + kAttnKeysPerBlock - 1) / kAttnKeysPerBlock;
  // split only when one pass leaves most compute units idle and every split
  // keeps at least 8 key blocks
  if (wgs < 256 && blocks >= 16) {
    int s = 256 / wgs;
    if (s > blocks / 8) s = blocks / 8;
    p.splits = s < 1 ? 1 : s;
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

inline size_t workspace_bytes(const lopa_dims& d) {
  const size_t a = attn_workspace_bytes(d);
  const size_t h = lmhead_workspace_bytes(d);
  return a > h ? a : h;
}

}  // namespace lopa
