// Host-side plan of the weight-streaming GEMM Y[M][N] = X[M][K] W[N][K]^T
// (bf16 in, float32 out) used by the layer forward.  Pure host code; the
// same view is handed to the kernels that consume the partial sums.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lopa {

constexpr int kGemmMaxWorkgroups = 256;   // one per compute unit
constexpr int kSlotTableMax = 4096;       // units whose slot counts a consumer keeps in LDS

// The iteration space is (unit, K chunk) with unit = (weight block of WROWS
// rows, activation row group of HROWS rows), weight-block major.  It is cut
// into G contiguous ranges, one per workgroup ("stream-K"): the first r = I
// mod G ranges hold q + 1 iterations, the rest q = I / G.  A workgroup walks
// its range, and whenever its unit changes (or its range ends) it writes the
// unit's partial sum as one float32 tile into slot g - first_wg(unit) of
// that unit.  Summing a unit's slots gives its tile of Y; every slot of every
// unit is written exactly once.
struct GemmView {
  int M, N, K;
  // activation rows (staged per K chunk) x weight rows per pass, LDS stages:
  // 0: 64 x 256, 3; 1: 128 x 256, 3; 2: 256 x 128, 3; 3: 160 x 128, 4;
  // 4: 160 x 256, 3.  Bodies 3 and 4 stage only the 160 rows they serve.
  int body;
  int hrows, wrows;
  int hshift, wshift;   // log2 of hrows, wrows
  int groups;     // activation row groups
  int units;      // weight blocks x groups
  int nch;        // K / 64
  int G;          // workgroups
  int smax;       // most slots any unit has
  int iters;      // units * nch
  int q, r;       // iterations per range: q + 1 for the first r ranges, then q

  __host__ __device__ int range_begin(int g) const { return g * q + (g < r ? g : r); }
  // the workgroup whose range holds iteration x
  __host__ __device__ int owner(int x) const {
    const int big = r * (q + 1);
    return x < big ? x / (q + 1) : r + (x - big) / q;
  }
  __host__ __device__ int first_wg(int u) const { return owner(u * nch); }
  __host__ __device__ int last_wg(int u) const { return owner((u + 1) * nch - 1); }
  __host__ __device__ size_t tile_elems() const { return static_cast<size_t>(hrows) * wrows; }
  // element (row, col) of slot s of unit u
  __host__ __device__ size_t at(int u, int s, int row_local, int col_local) const {
    return (static_cast<size_t>(u) * smax + s) * tile_elems() +
           static_cast<size_t>(row_local) * wrows + col_local;
  }
  // Consumers first write every unit's slot count into an LDS table (units
  // <= kSlotTableMax), then sum a unit's slots in slot order.
  __device__ void load_slots(unsigned char* tab) const {
    for (int u = threadIdx.x; u < units; u += blockDim.x)
      tab[u] = static_cast<unsigned char>(last_wg(u) - first_wg(u) + 1);
  }
  // Y[row][col .. col+3] (col % 4 == 0; the four columns share a unit); the
  // slot loads are issued BATCH at a time before any is added, and the slots
  // are added in slot order whatever BATCH is.
  template <int BATCH = 4>
  __device__ float4 sum4(const float* __restrict__ P, const unsigned char* tab, int row,
                         int col) const {
    const int grp = row >> hshift, wb = col >> wshift;
    const int u = wb * groups + grp;
    const int ns = tab[u];
    const float4* p = reinterpret_cast<const float4*>(
        P + at(u, 0, row - (grp << hshift), col - (wb << wshift)));
    const size_t stride = tile_elems() / 4;
    float4 y = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s0 = 0; s0 < ns; s0 += BATCH) {
      // every load is issued (a slot past the last re-reads the last one),
      // so there is no branch around each; only the present slots are added
      float4 t[BATCH];
#pragma unroll
      for (int j = 0; j < BATCH; ++j) t[j] = p[min(s0 + j, ns - 1) * stride];
#pragma unroll
      for (int j = 0; j < BATCH; ++j) {
        const bool in = s0 + j < ns;
        y.x += in ? t[j].x : 0.f;
        y.y += in ? t[j].y : 0.f;
        y.z += in ? t[j].z : 0.f;
        y.w += in ? t[j].w : 0.f;
      }
    }
    return y;
  }
  size_t partial_bytes() const { return static_cast<size_t>(units) * smax * tile_elems() * 4; }
};

inline GemmView gemm_view(int M, int N, int K, int max_wgs = kGemmMaxWorkgroups) {
  GemmView v{};
  v.M = M;
  v.N = N;
  v.K = K;
  // hrows is the partial tile's row count (a power of two); bodies 3 and 4
  // hold a single row group (M <= the 160 rows they stage).  Above 128 rows a
  // wide weight (more than 64 blocks of 256 rows) takes the 256-row weight
  // tile; a narrow one keeps 128 rows, as wider blocks would split its K
  // range further and multiply the partial tiles.
  if (M <= 64) {
    v.body = 0; v.hrows = 64; v.wrows = 256;
  } else if (M <= 128) {
    v.body = 1; v.hrows = 128; v.wrows = 256;
  } else if (M <= 160) {
    if (N > 64 * 256) {
      v.body = 4; v.hrows = 256; v.wrows = 256;
    } else {
      v.body = 3; v.hrows = 256; v.wrows = 128;
    }
  } else {
    v.body = 2; v.hrows = 256; v.wrows = 128;
  }
  v.hshift = v.hrows == 64 ? 6 : (v.hrows == 128 ? 7 : 8);
  v.wshift = v.wrows == 128 ? 7 : 8;
  v.groups = (M + v.hrows - 1) / v.hrows;
  v.units = ((N + v.wrows - 1) / v.wrows) * v.groups;
  v.nch = K / 64;
  const long long iters = static_cast<long long>(v.units) * v.nch;
  v.iters = static_cast<int>(iters);   // callers keep units * nch below 2^31
  v.G = static_cast<int>(iters < max_wgs ? iters : max_wgs);
  if (v.G < 1) v.G = 1;
  v.q = v.iters / v.G;
  v.r = v.iters - v.q * v.G;
  v.smax = 1;
  for (int u = 0; u < v.units; ++u) {
    const int s = v.last_wg(u) - v.first_wg(u) + 1;
    if (s > v.smax) v.smax = s;
  }
  return v;
}

// Gate/up projection of the MLP with its SwiGLU finished in the same kernel
// (k_gemm_glu): workgroup g takes blocks [blk_begin(g), blk_begin(g + 1)) of
// 16 gate rows and the 16 up rows of the same indices, one 32-row weight
// tile per block, over the whole of K, so no partial tiles are written and
// no second kernel sums them.  At most kGluTiles blocks per workgroup and
// kGluRows activation rows (one 160-row group); other shapes take the
// stream-K GEMM and k_swiglu.
constexpr int kGluTiles = 5;
constexpr int kGluRows = 160;

struct GluView {
  int M, K, inter;
  int nblk;   // inter / 16
  int G;      // workgroups
  __host__ __device__ int blk_begin(int g) const {
    return static_cast<int>(static_cast<long long>(g) * nblk / G);
  }
};

inline bool glu_fits(int M, int K, int inter) {
  if (M < 1 || M > kGluRows || K % 64 != 0 || inter % 16 != 0 || inter < 16) return false;
  const int nblk = inter / 16;
  const int G = nblk < kGemmMaxWorkgroups ? nblk : kGemmMaxWorkgroups;
  // buffer offsets of the weight (2 inter rows of K bf16) stay below 2^31
  return (nblk + G - 1) / G <= kGluTiles && 4LL * inter * K < (1LL << 31);
}

inline GluView glu_view(int M, int K, int inter) {
  GluView v{};
  v.M = M;
  v.K = K;
  v.inter = inter;
  v.nblk = inter / 16;
  v.G = v.nblk < kGemmMaxWorkgroups ? v.nblk : kGemmMaxWorkgroups;
  return v;
}

}  // namespace lopa
