// Weight-streaming GEMM of the layer forward: Y[M][N] = X[M][K] W[N][K]^T,
// bf16 operands, float32 accumulation, for the short activation matrices of
// a verification pass (M = every branch's block rows, a few hundred at most)
// against long weights.
//
// Section 3.3 of "解码效率革命：LoPA如何突破扩散语言模型的并行瓶颈" has every
// branch's forward computed in one shared matrix multiply; here all branches'
// rows ride one stream of each weight, so a weight byte crosses HBM once per
// pass whatever the number of branches.
//
// The work is the iteration space (unit, 64-wide K chunk), cut into equal
// contiguous ranges, one per workgroup (see GemmView): every compute unit
// streams the same number of weight bytes however N and K fall, and each
// workgroup writes float32 partial tiles that the consumer kernels sum.
// Inside a workgroup the machinery is the LM head's: four producer waves move
// W and X chunks straight into a three- or four-stage XOR-swizzled LDS ring with
// buffer loads that write LDS, eight compute waves read
// v_mfma_f32_32x32x16_bf16 fragments from it.  The activation fragment is the
// MFMA's A operand, so a lane's outputs run along one weight row and the
// partial stores are 128-byte row segments.
#include <type_traits>

#include "gemm_plan.hpp"
#include "stream_tile.hpp"

namespace lopa {

constexpr int kGemmSmem = 3 * (256 + 160) * kRB;   // largest S x stage of the bodies

// S LDS stages of HS activation rows (HS <= HROWS: a body that stages fewer
// rows than its waves cover serves one row group of at most HS rows).
template <int WX, int NVW, int MTW, int S, int HS>
__device__ __forceinline__ void gemm_body(const GemmView& v, const unsigned short* __restrict__ X,
                                          const unsigned short* __restrict__ W,
                                          float* __restrict__ P, unsigned char* smem) {
  using T = StreamTile<WX, NVW, MTW>;
  constexpr int WROWS = T::WROWS, HROWS = T::HROWS, WP = T::WP;
  constexpr int BUF = (WROWS + HS) * kRB, HP = HS / 32;
  static_assert(HS % 32 == 0 && HS <= HROWS && S >= 3 && S * BUF <= kGemmSmem, "body shape");
  constexpr int KS = kKC / 16;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = blockIdx.x;
  const int row_bytes = v.K * 2;
  const int it0 = v.range_begin(g);
  const int cnt = v.range_begin(g + 1) - it0;
  if (cnt <= 0) return;

  if (w >= kComputeWaves) {
    // ---------------- producer waves ----------------
    const int pw = w - kComputeWaves;
    const int r8 = lane >> 3;
    const int ls = (lane & 7) ^ r8 ^ (pw & 1);
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<unsigned short*>(W), 0, v.N * row_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<unsigned short*>(X), 0, v.M * row_bytes, 0x00020000);
    const int wv = (8 * pw + r8) * row_bytes + ls * 16;
    // (weight block, row group, K chunk) of the next chunk to issue: chunks
    // are issued in order, so these step along instead of being divided out
    int nu = it0 / v.nch;
    int kc = it0 - nu * v.nch;
    int wb = nu / v.groups;
    int grp = nu - wb * v.groups;
    auto issue = [&](int j) __attribute__((always_inline)) {
      unsigned char* dst = smem + (j % S) * BUF;
      const int sw = wb * WROWS * row_bytes + kc * kRB;
#pragma unroll
      for (int p = 0; p < WP; ++p)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, LOPA_LDS(dst + (4 * p + pw) * 1024), 16, wv,
                                                 sw + 32 * p * row_bytes, 0, kWeightAux);
#pragma unroll
      for (int p = 0; p < HP; ++p) {
        const int row = min(grp * HROWS + 8 * (4 * p + pw) + r8, v.M - 1);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            xr, LOPA_LDS(dst + WROWS * kRB + (4 * p + pw) * 1024), 16,
            row * row_bytes + ls * 16, kc * kRB, 0, 0);
      }
      // past the range's last chunk, that chunk is loaded again
      if (j + 1 < cnt && ++kc == v.nch) {
        kc = 0;
        if (++grp == v.groups) {
          grp = 0;
          ++wb;
        }
      }
    };
#pragma unroll
    for (int u = 0; u < S - 1; ++u) issue(u);
    wait_vmcnt<(S - 2) * (WP + HP)>();
    __builtin_amdgcn_s_barrier();
    for (int i = 0; i + 1 < cnt; ++i) {
      issue(i + S - 1);
      wait_vmcnt<(S - 2) * (WP + HP)>();
      __builtin_amdgcn_s_barrier();
    }
    wait_vmcnt<0>();   // no load may still target LDS when the workgroup ends
  } else {
    // ---------------- compute waves ----------------
    const int wx = w % WX;
    const int wy = w / WX;
    const int ln = lane & 31;
    const int lh = lane >> 5;
    f32x16 acc[MTW][NVW];
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
      for (int n = 0; n < NVW; ++n) acc[mt][n] = f32x16{};
    auto frags = [&](const unsigned char* base, int j, u16x8 (&wf)[NVW], u16x8 (&hf)[MTW],
                     auto live) __attribute__((always_inline)) {
      constexpr int LIVE = decltype(live)::value;
      const int s = j * 2 + lh;
#pragma unroll
      for (int n = 0; n < NVW; ++n) {
        const int r = (wx * NVW + n) * 32 + ln;
        wf[n] = *reinterpret_cast<const u16x8*>(base + r * kRB + swz<kKC>(r, s) * 16);
      }
#pragma unroll
      for (int mt = 0; mt < LIVE; ++mt) {
        const int r = (wy * MTW + mt) * 32 + ln;
        hf[mt] = *reinterpret_cast<const u16x8*>(base + (WROWS + r) * kRB + swz<kKC>(r, s) * 16);
      }
    };
    // LIVE = how many of the wave's activation tiles hold rows below M (the
    // rest would only multiply padding)
    auto compute = [&](int b, auto live) __attribute__((always_inline)) {
      constexpr int LIVE = decltype(live)::value;
      const unsigned char* base = smem + b * BUF;
      u16x8 wf[2][NVW], hf[2][MTW];
      frags(base, 0, wf[0], hf[0], live);
#pragma unroll
      for (int j = 0; j < KS; ++j) {
        if (j + 1 < KS) frags(base, j + 1, wf[(j + 1) & 1], hf[(j + 1) & 1], live);
#pragma unroll
        for (int mt = 0; mt < LIVE; ++mt)
#pragma unroll
          for (int n = 0; n < NVW; ++n)
            acc[mt][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, hf[j & 1][mt]), __builtin_bit_cast(bf16x8, wf[j & 1][n]),
                acc[mt][n], 0, 0, 0);
      }
    };
    // acc[mt][n][q] = Y[row (wy*MTW + mt)*32 + 8(q/4) + 4lh + q%4 of the group]
    //                  [col (wx*NVW + n)*32 + ln of the weight block]
    auto flush = [&](int u, auto live) __attribute__((always_inline)) {
      constexpr int LIVE = decltype(live)::value;
      const int wb = u / v.groups;
      const int grp = u - wb * v.groups;
      const int slot = g - v.first_wg(u);
      const int mg = min(v.M - grp * HROWS, HROWS);
      const int ng = min(v.N - wb * WROWS, WROWS);
      float* tile = P + v.at(u, slot, 0, 0);
      // the lane's first row, opaque to the compiler so the 16 x MTW x NVW
      // store addresses are formed here and not kept live across the K loop
      int r0 = wy * MTW * 32 + 4 * lh;
      __asm__ volatile("" : "+v"(r0));
      // A wave whose rows and columns all lie inside the unit's tile (every
      // wave, unless M or N is ragged) stores without per-element tests:
      // straight-line stores, not a branch around each one.
      const bool inside = (wy * MTW + LIVE) * 32 <= mg && (wx * NVW + NVW) * 32 <= ng;
      if (inside) {
#pragma unroll
        for (int mt = 0; mt < LIVE; ++mt)
#pragma unroll
          for (int n = 0; n < NVW; ++n) {
            const int c = (wx * NVW + n) * 32 + ln;
#pragma unroll
            for (int q = 0; q < 16; ++q)
              tile[(r0 + mt * 32 + 8 * (q >> 2) + (q & 3)) * WROWS + c] = acc[mt][n][q];
            acc[mt][n] = f32x16{};
          }
      } else {
#pragma unroll
        for (int mt = 0; mt < LIVE; ++mt)
#pragma unroll
          for (int n = 0; n < NVW; ++n) {
            const int c = (wx * NVW + n) * 32 + ln;
#pragma unroll
            for (int q = 0; q < 16; ++q) {
              const int r = r0 + mt * 32 + 8 * (q >> 2) + (q & 3);
              if (r < mg && c < ng) tile[r * WROWS + c] = acc[mt][n][q];
            }
            acc[mt][n] = f32x16{};
          }
      }
    };
    auto run = [&](auto live) __attribute__((always_inline)) {
      // (unit, K chunk, row group) of iteration it0 + i, stepped along
      // rather than divided out every chunk
      int u = it0 / v.nch;
      int kc = it0 - u * v.nch;
      int grp = u % v.groups;
      for (int i = 0; i < cnt; ++i) {
        __syncthreads();
        // a wave whose activation tiles all lie past the last row only keeps step
        if (grp * HROWS + wy * MTW * 32 < v.M) {
          compute(i % S, live);
          if (kc == v.nch - 1 || i == cnt - 1) flush(u, live);
        }
        if (++kc == v.nch) {
          kc = 0;
          ++u;
          if (++grp == v.groups) grp = 0;
        }
      }
    };
    // with one row group, a wave whose later activation tiles hold only
    // padding (160 rows in 256: tile 5) skips them: two-tile waves multiply
    // their live tile alone, three-tile waves (rows 0..95 or 96..191, 160
    // staged) their first two, which always lie within the staged rows
    const int live = v.groups == 1 ? (v.M - wy * MTW * 32 + 31) >> 5 : MTW;
    if constexpr (MTW == 5) {
      run(std::integral_constant<int, 5>{});   // one group of more than 128 rows
    } else if constexpr (MTW == 3) {
      if (live <= 2) run(std::integral_constant<int, 2>{});
      else run(std::integral_constant<int, 3>{});
    } else if constexpr (MTW == 2) {
      if (live == 1) run(std::integral_constant<int, 1>{});
      else run(std::integral_constant<int, 2>{});
    } else {
      run(std::integral_constant<int, MTW>{});
    }
  }
}

template <int WX, int NVW, int MTW, int S, int HS>
__global__ void __launch_bounds__(kStreamThreads)
k_gemm_stream(GemmView v, const unsigned short* __restrict__ X,
              const unsigned short* __restrict__ W, float* __restrict__ P) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kGemmSmem];
  gemm_body<WX, NVW, MTW, S, HS>(v, X, W, P, smem);
}

// Enqueue Y = X W^T as partial tiles into P (v.partial_bytes() bytes).
int gemm_launch(const GemmView& v, const unsigned short* X, const unsigned short* W, float* P,
                hipStream_t stream) {
  const dim3 grid(v.G), block(kStreamThreads);
  switch (v.body) {
    case 0:
      hipLaunchKernelGGL((k_gemm_stream<4, 2, 1, 3, 64>), grid, block, 0, stream, v, X, W, P);
      break;
    case 1:
      hipLaunchKernelGGL((k_gemm_stream<4, 2, 2, 3, 128>), grid, block, 0, stream, v, X, W, P);
      break;
    case 3:
      hipLaunchKernelGGL((k_gemm_stream<4, 1, 3, 4, 160>), grid, block, 0, stream, v, X, W, P);
      break;
    case 4:
      hipLaunchKernelGGL((k_gemm_stream<8, 1, 5, 3, 160>), grid, block, 0, stream, v, X, W, P);
      break;
    default:
      hipLaunchKernelGGL((k_gemm_stream<2, 2, 2, 3, 256>), grid, block, 0, stream, v, X, W, P);
      break;
  }
  return hipGetLastError() == hipSuccess ? LOPA_OK : LOPA_ERR_HIP;
}

}  // namespace lopa
