/*
 * Fast path of the model oracle's weight generator (test infrastructure;
 * only the oracle loads it).  Philox4x32-10 as published by Salmon, Moraes,
 * Dror and Shaw ("Parallel random numbers: as easy as 1, 2, 3", SC 2011):
 * ten rounds; each multiplies words 0 and 2 by the round multipliers, mixes
 * the high halves into the other words with the round key, and the key
 * advances by the Weyl increments between rounds.
 *
 * oracle_philox_fill_rows writes, for rows r0 <= r < r1 and columns c < cols,
 * the values the oracle's numpy generator defines:
 *   x = word (c % 4) of Philox(counter (c / 4, r, tag, 0), key (k0, k1))
 *   rule 1 (norm):    1 + ((x >> 27) - 16) / 128
 *   rule 0 (uniform): ((x >> 8) - 2^23) * 2^(-24 - shift) rounded to bf16:
 *                     the integer (x >> 8) - 2^23 rounded to 8 significant
 *                     bits, nearest with ties to even, then scaled (exact)
 */
#include <math.h>
#include <stdint.h>

static void philox(uint32_t c[4], uint32_t k0, uint32_t k1) {
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = (uint64_t)0xD2511F53u * c[0];
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c[2];
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c[1] ^ k0;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c[3] ^ k1;
    c[1] = (uint32_t)p1;
    c[3] = (uint32_t)p0;
    c[0] = n0;
    c[2] = n2;
  }
}

/* m rounded to 8 significant bits, nearest, ties to even */
static int64_t round8(int64_t m) {
  const int64_t a = m < 0 ? -m : m;
  if (a < 256) return m;
  const int bits = 64 - __builtin_clzll((unsigned long long)a);
  const int sh = bits - 8;
  int64_t q = a >> sh;
  const int64_t rem = a & ((1LL << sh) - 1), half = 1LL << (sh - 1);
  if (rem > half || (rem == half && (q & 1))) ++q;
  const int64_t r = q << sh;
  return m < 0 ? -r : r;
}

/* rows r0 .. r1-1 of the tensor into out [r1 - r0][cols] */
void oracle_philox_fill_rows(uint32_t k0, uint32_t k1, uint32_t tag, int64_t r0, int64_t r1,
                             int64_t cols, int rule, int shift, double* out) {
  const double scale = ldexp(1.0, -24 - shift);
  out -= r0 * cols;
  for (int64_t r = r0; r < r1; ++r) {
    for (int64_t q = 0; q * 4 < cols; ++q) {
      uint32_t c[4] = {(uint32_t)q, (uint32_t)r, tag, 0u};
      philox(c, k0, k1);
      for (int j = 0; j < 4 && q * 4 + j < cols; ++j) {
        const uint32_t x = c[j];
        out[r * cols + q * 4 + j] =
            rule == 1 ? 1.0 + (double)((int64_t)(x >> 27) - 16) / 128.0
                      : (double)round8((int64_t)(x >> 8) - (1 << 23)) * scale;
      }
    }
  }
}
