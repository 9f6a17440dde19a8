// Launch plan of the LM-head call, shared by its entry point and the
// workspace query.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include "lopa.h"

namespace lopa {

// MFMA kernel (bf16, hidden % 64 == 0): one launch of kHeadParts persistent
// workgroups, one per compute unit of an MI355X.  The device-side row count
// M picks the layout (head_groups): with few rows every workgroup owns a
// balanced contiguous vocabulary range and all rows; with many the rows are
// split into groups, and the groups of one vocabulary range run side by side
// on the same XCD so the weight crosses HBM once.
constexpr int kHeadParts = 256;
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

// Row groups of the MFMA kernel for M rows (in 32-row tiles).  wide: the
// 2 x 4 compute-wave layout (128 vocabulary rows x 256 rows per pass) instead
// of 4 x 2 (256 x 128); groups: row groups, whose workgroups stream the same
// vocabulary part side by side; nparts: vocabulary parts per group (a
// multiple of the 8 XCDs, nparts * groups <= kHeadParts); tpg: tiles per
// group.  Each choice below takes the fewest K chunks per workgroup (one
// chunk costs about the same in either layout), the fewer groups on a tie:
// <= 4 tiles: one group, 4 x 2; 5..8: one group, 2 x 4; 9..12: three groups
// of <= 4 tiles, 4 x 2; more: groups of <= 8 tiles, 2 x 4.  m_max <= 1024
// keeps groups <= 4.
struct HeadGroups {
  int wide, groups, nparts, tpg;
};

__host__ __device__ inline HeadGroups head_groups(int M) {
  const int tiles = (M + 31) / 32;
  int wide, g;
  if (tiles <= 4) {
    wide = 0;
    g = 1;
  } else if (tiles <= 8) {
    wide = 1;
    g = 1;
  } else if (tiles <= 12) {
    wide = 0;
    g = 3;
  } else {
    wide = 1;
    g = (tiles + kHeadGroupTiles - 1) / kHeadGroupTiles;
  }
  return HeadGroups{wide, g, 8 * (kHeadParts / 8 / g), (tiles + g - 1) / g};
}

// The wide kernel (k_lmhead_wide): four waves, one per SIMD, each of them
// both loading and computing, with large register tiles.  Its row groups
// hold at most kWideMaxTiles 32-row tiles; th = 4q + r tiles per group: each
// wave owns q tiles against every weight tile of a pass, and the r remaining
// tiles are shared out by weight tile (wave w takes weight tiles w, w + 4,
// ...), so every wave runs the same number of MFMAs.  tw: weight tiles per
// pass (8 up to 8 row tiles, else 4).  The weight streams through an LDS
// ring; the activation fragments go straight from an operand-ordered copy
// (made per call) into registers.  It serves the row-tile counts where it
// measured faster than the narrow kernel (k_lmhead_mfma) in a same-box
// comparison at the 7B shapes (6 and 9..32 tiles): 6, 9-20 and 23-26 tiles
// (by 3-20 %; 19, 23 and 25 by their layouts' neighbours); the narrow kernel
// serves every other count (at 7, 8, 22 and 27-32 tiles it measured equal or
// up to 12 % faster).  At 5 tiles the wide kernel measured
// 17 % faster as well, but the row count lives on the device, so a call that
// may reach the wide kernel launches both and the idle one costs about 5 us:
// a call of at most 5 tiles (block 32, 5 branches: m_max = 160) launches the
// narrow kernel alone.
constexpr int kWideMinTiles = 6;
constexpr int kWideMaxTiles = 13;

struct WideGroups {
  int tw, th, groups, nparts;
};

__host__ __device__ inline WideGroups wide_groups(int M) {
  const int tiles = (M + 31) / 32;
  const int g = (tiles + kWideMaxTiles - 1) / kWideMaxTiles;
  const int th = (tiles + g - 1) / g;
  return WideGroups{th <= 8 ? 8 : 4, th, g, 8 * (kHeadParts / 8 / g)};
}

__host__ __device__ inline bool wide_takes(int M) {
  const int t = (M + 31) / 32;
  return t == 6 || (t >= 9 && t <= 20) || t == 23 || t == 24 || t == 25 || t == 26;
}

// Whether a call with m_max rows may reach the wide kernel (its K loop takes
// 128 hidden values per round).
inline bool wide_possible(int m_max, int hidden) {
  return (m_max + 31) / 32 >= kWideMinTiles && hidden % 128 == 0;
}

// Vocabulary parts per row of whichever MFMA kernel serves M rows (wide:
// whether the wide kernel was launched beside the narrow one).
__host__ __device__ inline int head_nparts(int M, bool wide) {
  return wide && wide_takes(M) ? wide_groups(M).nparts : head_groups(M).nparts;
}

// Largest byte range of W one MFMA workgroup addresses: the rows of the
// widest vocabulary part over every row count the device may see (up to
// m_max) plus one pass of 256 rows read past its end.
inline long long head_part_bytes_max(const lopa_dims& d) {
  const HeadPlan p = head_plan(d);
  int nparts = kHeadParts;
  for (int m = 1; m <= p.m_max; m += 32) {
    const int n = head_nparts(m, true);
    nparts = n < nparts ? n : nparts;
  }
  const long long t16 = (d.V + 15) / 16;
  const long long rows = (t16 + nparts - 1) / nparts * 16 + 256;
  return rows * d.Hq * d.d * 2;
}

// Per (row, vocabulary tile) partial: max logit (float), scaled sum (float),
// argmax or sample (int32), entropy term or perturbed best score (float),
// scaled logit of the sample (float) -- five planes of m_max * ntiles.
// When the wide kernel may run, an operand-ordered copy of the activation
// rows follows (256-byte aligned): m_max rounded up to 32 rows x hidden bf16.
inline size_t lmhead_workspace_bytes(const lopa_dims& d) {
  const HeadPlan p = head_plan(d);
  const size_t partials = static_cast<size_t>(p.m_max) * static_cast<size_t>(p.ntiles) * 20u;
  if (!p.mfma || !wide_possible(p.m_max, d.Hq * d.d)) return partials;
  return (partials + 255) / 256 * 256 +
         static_cast<size_t>((p.m_max + 31) / 32) * 32 * static_cast<size_t>(d.Hq * d.d) * 2;
}

}  // namespace lopa
