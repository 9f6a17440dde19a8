// Building blocks of the weight-streaming MFMA kernels (the LM head and the
// projection GEMMs of the layer forward): a three-stage LDS ring filled by
// producer waves with buffer loads that write LDS directly, and 32x32x16 bf16
// MFMA tiles read from it by compute waves.
#pragma once

#include "lopa_common.hpp"

namespace lopa {

constexpr int kKC = 64;          // K chunk
constexpr int kRB = kKC * 2;     // bytes of one row per chunk (8 slots of 16 B)
constexpr int kStages = 3;       // LDS stages: S - 1 chunks in flight while one is computed
// Cache policy of the weight loads: non-temporal.  Measured faster than
// normal caching in every layout, also where row groups share the weight
// through L2 (LM head, prefix 512: 212 vs 232 us per call).
constexpr int kWeightAux = 2;
constexpr int kComputeWaves = 8; // two per SIMD, so one wave's LDS reads hide under the other's MFMAs
constexpr int kLoadWaves = 4;
constexpr int kStreamThreads = 64 * (kComputeWaves + kLoadWaves);

// Physical 16-byte slot of logical slot s in LDS row r.  Rows of a K chunk
// are KC*2 bytes; the XOR keeps 16-lane fragment reads (16 consecutive rows,
// one slot) and the staging writes free of bank conflicts.
template <int KC>
__device__ __forceinline__ int swz(int r, int s) {
  if constexpr (KC == 64) return s ^ ((r & 7) ^ ((r >> 3) & 1));
  else return s ^ (((r >> 1) ^ (r >> 2)) & 3);
}

// Shape of one body: WX x (kComputeWaves / WX) compute waves over
// (weight rows, activation rows); each wave holds NVW 32-row weight tiles
// against MTW 32-row activation tiles.
template <int WX, int NVW, int MTW>
struct StreamTile {
  static constexpr int WY = kComputeWaves / WX;
  static constexpr int WROWS = WX * NVW * 32;       // weight rows per pass
  static constexpr int HROWS = WY * MTW * 32;       // activation rows staged per chunk
  static constexpr int BUF = (WROWS + HROWS) * kRB; // bytes per LDS stage
  static constexpr int WP = WROWS / 32;             // W DMA loads per producer wave per chunk
  static constexpr int HP = HROWS / 32;             // activation DMA loads per producer wave per chunk
};

// s_waitcnt on the vector-memory counter only (lgkm and exp counts left open).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

#define LOPA_LDS(p) ((__attribute__((address_space(3))) void*)(p))

}  // namespace lopa
