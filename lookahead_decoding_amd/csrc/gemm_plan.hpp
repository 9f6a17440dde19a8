// Host-side plan of the weight-streaming GEMM Y[M][N] = X[M][K] W[N][K]^T
// (bf16 in, float32 out) used by the layer forward.  Pure host code; the
// same view is handed to the kernels that consume the partial sums.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace lopa {

constexpr int kGemmMaxWorkgroups = 256;   // one per compute unit

// The iteration space is (unit, K chunk) with unit = (weight block of WROWS
// rows, activation row group of HROWS rows), weight-block major.  It is cut
// into G equal contiguous ranges, one per workgroup ("stream-K"): a
// workgroup walks its range, and whenever its unit changes (or its range
// ends) it writes the unit's partial sum as one float32 tile into slot
// g - first_wg(unit) of that unit.  Summing a unit's slots gives its tile of
// Y; every slot of every unit is written exactly once.
struct GemmView {
  int M, N, K;
  int body;       // 0: 64 activation rows x 256 weight rows per pass; 1: 128 x 256; 2: 256 x 128
  int hrows, wrows;
  int groups;     // activation row groups
  int units;      // weight blocks x groups
  int nch;        // K / 64
  int G;          // workgroups
  int smax;       // most slots any unit has
  long long iters;

  // first / last workgroup whose range holds iteration x: the largest g
  // with floor(g * iters / G) <= x
  __host__ __device__ int owner(long long x) const {
    return static_cast<int>(((x + 1) * G + iters - 1) / iters) - 1;
  }
  __host__ __device__ int first_wg(int u) const { return owner(static_cast<long long>(u) * nch); }
  __host__ __device__ int last_wg(int u) const {
    return owner(static_cast<long long>(u + 1) * nch - 1);
  }
  __host__ __device__ long long range_begin(int g) const { return g * iters / G; }
  __host__ __device__ size_t tile_elems() const { return static_cast<size_t>(hrows) * wrows; }
  // element (row, col) of slot s of unit u
  __host__ __device__ size_t at(int u, int s, int row_local, int col_local) const {
    return (static_cast<size_t>(u) * smax + s) * tile_elems() +
           static_cast<size_t>(row_local) * wrows + col_local;
  }
  // Y[row][col] = sum over the slots of its unit
  __host__ __device__ float sum(const float* P, int row, int col) const {
    const int grp = row / hrows, wb = col / wrows;
    const int u = wb * groups + grp;
    const int s1 = last_wg(u) - first_wg(u);
    const int rl = row - grp * hrows, cl = col - wb * wrows;
    float y = 0.f;
    for (int s = 0; s <= s1; ++s) y += P[at(u, s, rl, cl)];
    return y;
  }
  size_t partial_bytes() const { return static_cast<size_t>(units) * smax * tile_elems() * 4; }
};

inline GemmView gemm_view(int M, int N, int K, int max_wgs = kGemmMaxWorkgroups) {
  GemmView v{};
  v.M = M;
  v.N = N;
  v.K = K;
  if (M <= 64) {
    v.body = 0; v.hrows = 64; v.wrows = 256;
  } else if (M <= 128) {
    v.body = 1; v.hrows = 128; v.wrows = 256;
  } else {
    v.body = 2; v.hrows = 256; v.wrows = 128;
  }
  v.groups = (M + v.hrows - 1) / v.hrows;
  v.units = ((N + v.wrows - 1) / v.wrows) * v.groups;
  v.nch = K / 64;
  v.iters = static_cast<long long>(v.units) * v.nch;
  v.G = static_cast<int>(v.iters < max_wgs ? v.iters : max_wgs);
  if (v.G < 1) v.G = 1;
  v.smax = 1;
  for (int u = 0; u < v.units; ++u) {
    const int s = v.last_wg(u) - v.first_wg(u) + 1;
    if (s > v.smax) v.smax = s;
  }
  return v;
}

}  // namespace lopa
