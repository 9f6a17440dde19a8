// Launch plan of the LM-head call, shared by the entry point and the
// workspace query so both always agree.
#pragma once

#include <stddef.h>

#include "lopa.h"

namespace lopa {

// MFMA path: bf16, hidden a multiple of 64.  A workgroup owns 128 vocabulary
// entries and up to 16*kMaxRowTiles LM-head rows; more rows use more row
// groups (grid.y).
constexpr int kHeadVocabPerWG = 128;
constexpr int kHeadMaxRowTiles = 36;
// Plain path (float32, or shapes the MFMA path does not cover): one vocab
// entry per thread, 256 per workgroup.
constexpr int kHeadVocabPerWGPlain = 256;

struct HeadPlan {
  bool mfma;
  int ntiles;      // vocabulary tiles (grid.x)
  int row_tiles;   // compile-time row tiles per group (MFMA path)
  int groups;      // row groups (grid.y, MFMA path)
  int m_max;       // nb_max * B
};

inline HeadPlan head_plan(const lopa_dims& d) {
  HeadPlan p{};
  const int hidden = d.Hq * d.d;
  p.m_max = (d.k_max + 1) * d.B;
  p.mfma = d.dtype == LOPA_BF16 && hidden % 64 == 0;
  if (p.mfma) {
    p.ntiles = (d.V + kHeadVocabPerWG - 1) / kHeadVocabPerWG;
    int tiles = (p.m_max + 15) / 16;
    int per = tiles < kHeadMaxRowTiles ? tiles : kHeadMaxRowTiles;
    per = (per + 3) / 4 * 4;                       // instantiated in steps of 4
    if (per > kHeadMaxRowTiles) per = kHeadMaxRowTiles;
    p.row_tiles = per;
    p.groups = (tiles + per - 1) / per;
  } else {
    p.ntiles = (d.V + kHeadVocabPerWGPlain - 1) / kHeadVocabPerWGPlain;
    p.row_tiles = 0;
    p.groups = 1;
  }
  return p;
}

// Per (row, vocab tile) partial: max logit (float), scaled sum (float),
// argmax (int32) -- three planes of m_max * ntiles.
inline size_t lmhead_workspace_bytes(const lopa_dims& d) {
  const HeadPlan p = head_plan(d);
  return static_cast<size_t>(p.m_max) * static_cast<size_t>(p.ntiles) * 12u;
}

}  // namespace lopa
