// Philox4x32-10 counter-based generator (Salmon, Moraes, Dror and Shaw,
// "Parallel random numbers: as easy as 1, 2, 3", SC 2011): ten rounds of two
// 32 x 32 -> 64-bit multiplies, the high halves mixed into the other words
// with the round key, the key advanced by a Weyl increment between rounds.
// Used for the library's synthetic inputs (token-keyed projections, model
// weights), never inside the method's arithmetic.
#pragma once

#include "lopa_common.hpp"

namespace lopa {

struct U32x4 {
  unsigned x0, x1, x2, x3;
};

__device__ __forceinline__ U32x4 philox4x32_10(U32x4 c, unsigned k0, unsigned k1) {
  constexpr unsigned M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
  constexpr unsigned W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += W0;
      k1 += W1;
    }
    const unsigned long long p0 = static_cast<unsigned long long>(M0) * c.x0;
    const unsigned long long p1 = static_cast<unsigned long long>(M1) * c.x2;
    const unsigned hi0 = static_cast<unsigned>(p0 >> 32), lo0 = static_cast<unsigned>(p0);
    const unsigned hi1 = static_cast<unsigned>(p1 >> 32), lo1 = static_cast<unsigned>(p1);
    c = U32x4{hi1 ^ c.x1 ^ k0, lo1, hi0 ^ c.x3 ^ k1, lo0};
  }
  return c;
}

}  // namespace lopa
