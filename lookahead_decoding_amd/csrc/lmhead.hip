// Verify stage, LM-head part: per still-masked (branch, position) row, the
// largest softmax probability over the vocabulary and its argmax token.
//
// The news article "上交大 × 华为小艺推出LoPA：7B扩散语言模型单样例1000+ tokens/s！"
// (section "LoPA 的核心设计：前瞻并行与分支验证", stages 分支置信度验证 and
// 并行验证与复用) scores a branch by the confidence of the positions it leaves
// unfilled and reuses the verification logits for the next step; section 3.3
// of "解码效率革命：LoPA如何突破扩散语言模型的并行瓶颈" has all branches share one
// matrix multiply.  Here every branch's rows ride one stream of the weight:
// the weight W [V][hidden] is read from HBM exactly once per step, whatever
// the number of branches.
//
// Two kernels write per-(row, vocab tile) online-softmax partials
// (max, sum exp(l - max), argmax); a merge kernel folds the tiles of a row.
//   k_lmhead_mfma  bf16, hidden % 64 == 0: v_mfma_f32_16x16x32_bf16 tiles.
//                  A workgroup (4 waves) owns 128 vocabulary rows of W; each
//                  wave streams its 2x16 rows straight from HBM into MFMA
//                  A-operand registers (16 B per lane per K step, one chunk
//                  ahead), while the LM-head rows of H are staged through LDS
//                  (64-wide K chunks, double-buffered, XOR-swizzled 16-byte
//                  slots) and shared by the four waves.
//   k_lmhead_plain float32 (and shapes outside the MFMA path): one thread per
//                  vocabulary entry, FMA dot products.
#include "lopa_common.hpp"
#include "lmhead_plan.hpp"

namespace lopa {

// ---------------------------------------------------------------------------
// MFMA path
// ---------------------------------------------------------------------------

template <int MT>
__global__ void __launch_bounds__(256)
k_lmhead_mfma(int V, int hidden, int ntiles, int nb_max, int m_max,
              const unsigned short* __restrict__ H,
              const unsigned short* __restrict__ W, const int32_t* __restrict__ rows,
              const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ nb_ptr,
              float* __restrict__ ws_m, float* __restrict__ ws_s, int32_t* __restrict__ ws_i,
              float* __restrict__ logits_out) {
  constexpr int NW = 2;              // 16-row vocabulary tiles per wave
  constexpr int ROWS = MT * 16;      // LM-head rows per group
  constexpr int PASSES = ROWS / 32;  // H staging: 32 rows x 128 B per pass
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * ROWS * 128];

  const int M = listed_rows(row_ptr, nb_ptr, nb_max, m_max);
  const int row0 = blockIdx.y * ROWS;
  if (row0 >= M) return;
  const int Mg = min(M - row0, ROWS);
  const int Mt = (Mg + 15) >> 4;
  const int tile = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int ln = lane & 15;
  const int lg = lane >> 4;
  const int vbase = tile * kHeadVocabPerWG + w * 32;

  // W: this lane's two vocabulary rows; 32 B per 64-wide K chunk at byte
  // offset 32*lg (K values 16*lg .. 16*lg+15).  Rows past V read row V-1 and
  // are dropped in the epilogue.
  const u16x8* wp[NW];
#pragma unroll
  for (int n = 0; n < NW; ++n) {
    const int v = min(vbase + n * 16 + ln, V - 1);
    wp[n] = reinterpret_cast<const u16x8*>(W + static_cast<size_t>(v) * hidden) + lg * 2;
  }

  // H staging: thread owns physical 16-B slot (tid & 7) of rows (tid >> 3) + 32*j.
  const int slot = tid & 7;
  int hrow[PASSES];
#pragma unroll
  for (int j = 0; j < PASSES; ++j) {
    const int r = (tid >> 3) + 32 * j;
    hrow[j] = r < Mg ? rows[row0 + r] : -1;
  }
  const int npass = (Mt * 16 + 31) >> 5;

  auto load_h = [&](int c, u16x8* hv) {
#pragma unroll
    for (int j = 0; j < PASSES; ++j) {
      if (j < npass) {
        const int r = (tid >> 3) + 32 * j;
        const int seg = slot ^ (r & 7);     // logical 16-B segment of the K chunk
        if (hrow[j] >= 0) {
          hv[j] = *reinterpret_cast<const u16x8*>(H + static_cast<size_t>(hrow[j]) * hidden +
                                                  c * 64 + seg * 8);
        } else {
          hv[j] = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
        }
      }
    }
  };
  auto store_h = [&](int buf, const u16x8* hv) {
    unsigned char* base = smem + buf * (ROWS * 128);
#pragma unroll
    for (int j = 0; j < PASSES; ++j) {
      if (j < npass) {
        const int r = (tid >> 3) + 32 * j;
        *reinterpret_cast<u16x8*>(base + r * 128 + slot * 16) = hv[j];
      }
    }
  };

  f32x4 acc[NW][MT];
#pragma unroll
  for (int n = 0; n < NW; ++n)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[n][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nchunks = hidden >> 6;
  u16x8 hv[PASSES];
  load_h(0, hv);
  store_h(0, hv);
  u16x8 wa[NW][2];
#pragma unroll
  for (int n = 0; n < NW; ++n) {
    wa[n][0] = __builtin_nontemporal_load(wp[n] + 0);
    wa[n][1] = __builtin_nontemporal_load(wp[n] + 1);
  }
  __syncthreads();

  for (int c = 0; c < nchunks; ++c) {
    const bool more = c + 1 < nchunks;
    u16x8 wb[NW][2];
    if (more) {
      load_h(c + 1, hv);
#pragma unroll
      for (int n = 0; n < NW; ++n) {
        wb[n][0] = __builtin_nontemporal_load(wp[n] + (c + 1) * 8 + 0);
        wb[n][1] = __builtin_nontemporal_load(wp[n] + (c + 1) * 8 + 1);
      }
    }
    const unsigned char* hb = smem + (c & 1) * (ROWS * 128);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        if (mt < Mt) {
          const int r = mt * 16 + ln;
          const int phys = (lg * 2 + s) ^ (r & 7);
          const u16x8 hf = *reinterpret_cast<const u16x8*>(hb + r * 128 + phys * 16);
#pragma unroll
          for (int n = 0; n < NW; ++n) {
            acc[n][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, wa[n][s]), __builtin_bit_cast(bf16x8, hf),
                acc[n][mt], 0, 0, 0);
          }
        }
      }
    }
    if (more) store_h((c + 1) & 1, hv);
    __syncthreads();
    if (more) {
#pragma unroll
      for (int n = 0; n < NW; ++n) {
        wa[n][0] = wb[n][0];
        wa[n][1] = wb[n][1];
      }
    }
  }

  // Epilogue.  acc[n][mt][q] = logit of row mt*16 + ln and vocabulary entry
  // vbase + n*16 + 4*lg + q.
  Partial* red = reinterpret_cast<Partial*>(smem);   // [4 waves][ROWS]
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    if (mt < Mt) {
      const int r = mt * 16 + ln;
      Partial p = empty_partial();
#pragma unroll
      for (int n = 0; n < NW; ++n)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int v = vbase + n * 16 + 4 * lg + q;
          if (v < V && acc[n][mt][q] > p.m) {
            p.m = acc[n][mt][q];
            p.i = v;
          }
        }
      if (p.i != 0x7fffffff) {
        float s = 0.f;
#pragma unroll
        for (int n = 0; n < NW; ++n)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int v = vbase + n * 16 + 4 * lg + q;
            if (v < V) s += exp2f((acc[n][mt][q] - p.m) * kLog2e);
          }
        p.s = s;
      }
      p = merge(p, shfl_xor(p, 16));
      p = merge(p, shfl_xor(p, 32));
      if (lg == 0) red[w * ROWS + r] = p;
      if (logits_out && r < Mg) {
        const size_t base = static_cast<size_t>(rows[row0 + r]) * V;
#pragma unroll
        for (int n = 0; n < NW; ++n)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int v = vbase + n * 16 + 4 * lg + q;
            if (v < V) logits_out[base + v] = acc[n][mt][q];
          }
      }
    }
  }
  __syncthreads();
  for (int r = tid; r < Mg; r += 256) {
    Partial p = red[r];
    p = merge(p, red[ROWS + r]);
    p = merge(p, red[2 * ROWS + r]);
    p = merge(p, red[3 * ROWS + r]);
    const size_t o = static_cast<size_t>(row0 + r) * ntiles + tile;
    ws_m[o] = p.m;
    ws_s[o] = p.s;
    ws_i[o] = p.i;
  }
}

// ---------------------------------------------------------------------------
// Plain path
// ---------------------------------------------------------------------------

template <typename T>
__global__ void __launch_bounds__(256)
k_lmhead_plain(int V, int hidden, int ntiles, int nb_max, int m_max, const T* __restrict__ H,
               const T* __restrict__ W,
               const int32_t* __restrict__ rows, const int32_t* __restrict__ row_ptr,
               const int32_t* __restrict__ nb_ptr, float* __restrict__ ws_m,
               float* __restrict__ ws_s, int32_t* __restrict__ ws_i,
               float* __restrict__ logits_out) {
  __shared__ Partial red[4];
  const int m = blockIdx.y;
  const int M = listed_rows(row_ptr, nb_ptr, nb_max, m_max);
  if (m >= M) return;
  const int row = rows[m];
  const int v = blockIdx.x * kHeadVocabPerWGPlain + threadIdx.x;
  Partial p = empty_partial();
  if (v < V) {
    float l = 0.f;
    const size_t hb = static_cast<size_t>(row) * hidden;
    const size_t wb = static_cast<size_t>(v) * hidden;
    for (int k = 0; k < hidden; ++k) l = fmaf(Act<T>::load(H, hb + k), Act<T>::load(W, wb + k), l);
    p = Partial{l, 1.f, v};
    if (logits_out) logits_out[static_cast<size_t>(row) * V + v] = l;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) p = merge(p, shfl_xor(p, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = p;
  __syncthreads();
  if (threadIdx.x == 0) {
    p = merge(merge(red[0], red[1]), merge(red[2], red[3]));
    const size_t o = static_cast<size_t>(m) * ntiles + blockIdx.x;
    ws_m[o] = p.m;
    ws_s[o] = p.s;
    ws_i[o] = p.i;
  }
}

// ---------------------------------------------------------------------------
// Merge of the vocabulary tiles of each row: conf = 1 / sum, arg = argmax.
// ---------------------------------------------------------------------------

__global__ void __launch_bounds__(256)
k_lmhead_merge(int ntiles, int nb_max, int m_max, const int32_t* __restrict__ rows, const int32_t* __restrict__ row_ptr,
               const int32_t* __restrict__ nb_ptr, const float* __restrict__ ws_m,
               const float* __restrict__ ws_s, const int32_t* __restrict__ ws_i,
               float* __restrict__ conf, int32_t* __restrict__ arg) {
  __shared__ Partial red[4];
  const int m = blockIdx.x;
  const int M = listed_rows(row_ptr, nb_ptr, nb_max, m_max);
  if (m >= M) return;
  Partial p = empty_partial();
  const size_t base = static_cast<size_t>(m) * ntiles;
  for (int t = threadIdx.x; t < ntiles; t += 256)
    p = merge(p, Partial{ws_m[base + t], ws_s[base + t], ws_i[base + t]});
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) p = merge(p, shfl_xor(p, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = p;
  __syncthreads();
  if (threadIdx.x == 0) {
    p = merge(merge(red[0], red[1]), merge(red[2], red[3]));
    const int r = rows[m];
    conf[r] = 1.f / p.s;
    arg[r] = p.i;
  }
}

template <int MT>
static void launch_mfma(dim3 grid, hipStream_t st, int V, int hidden, int ntiles, int nb_max,
                        int m_max,
                        const void* H, const void* W, const int32_t* rows,
                        const int32_t* row_ptr, const int32_t* nb, float* wm, float* wsum,
                        int32_t* wi, float* logits) {
  hipLaunchKernelGGL(k_lmhead_mfma<MT>, grid, dim3(256), 0, st, V, hidden, ntiles, nb_max, m_max,
                     static_cast<const unsigned short*>(H), static_cast<const unsigned short*>(W),
                     rows, row_ptr, nb, wm, wsum, wi, logits);
}

}  // namespace lopa

extern "C" int lopa_lmhead_conf(const lopa_dims* dims, const void* H, const void* W,
                                const int32_t* rows, const int32_t* row_ptr,
                                const int32_t* nb, float* conf, int32_t* arg,
                                float* logits_out, void* ws, size_t ws_bytes,
                                hipStream_t stream) {
  using namespace lopa;
  int st = lopa_check_dims(dims);
  if (st != LOPA_OK) return st;
  if (!H || !W || !rows || !row_ptr || !nb || !conf || !arg) return LOPA_ERR_INVALID;
  const size_t need = lmhead_workspace_bytes(*dims);
  if (!ws || ws_bytes < need) return LOPA_ERR_WORKSPACE;
  const HeadPlan p = head_plan(*dims);
  const int hidden = dims->Hq * dims->d;
  const size_t plane = static_cast<size_t>(p.m_max) * p.ntiles;
  float* wm = static_cast<float*>(ws);
  float* wsum = wm + plane;
  int32_t* wi = reinterpret_cast<int32_t*>(wsum + plane);
  const int V = dims->V;
  const int nb_max = dims->k_max + 1;
  if (p.mfma) {
    const dim3 grid(p.ntiles, p.groups);
    switch (p.row_tiles) {
      case 4: launch_mfma<4>(grid, stream, V, hidden, p.ntiles, nb_max, p.m_max, H, W, rows, row_ptr, nb, wm, wsum, wi, logits_out); break;
      case 8: launch_mfma<8>(grid, stream, V, hidden, p.ntiles, nb_max, p.m_max, H, W, rows, row_ptr, nb, wm, wsum, wi, logits_out); break;
      case 12: launch_mfma<12>(grid, stream, V, hidden, p.ntiles, nb_max, p.m_max, H, W, rows, row_ptr, nb, wm, wsum, wi, logits_out); break;
      case 16: launch_mfma<16>(grid, stream, V, hidden, p.ntiles, nb_max, p.m_max, H, W, rows, row_ptr, nb, wm, wsum, wi, logits_out); break;
      case 20: launch_mfma<20>(grid, stream, V, hidden, p.ntiles, nb_max, p.m_max, H, W, rows, row_ptr, nb, wm, wsum, wi, logits_out); break;
      case 24: launch_mfma<24>(grid, stream, V, hidden, p.ntiles, nb_max, p.m_max, H, W, rows, row_ptr, nb, wm, wsum, wi, logits_out); break;
      case 28: launch_mfma<28>(grid, stream, V, hidden, p.ntiles, nb_max, p.m_max, H, W, rows, row_ptr, nb, wm, wsum, wi, logits_out); break;
      case 32: launch_mfma<32>(grid, stream, V, hidden, p.ntiles, nb_max, p.m_max, H, W, rows, row_ptr, nb, wm, wsum, wi, logits_out); break;
      case 36: launch_mfma<36>(grid, stream, V, hidden, p.ntiles, nb_max, p.m_max, H, W, rows, row_ptr, nb, wm, wsum, wi, logits_out); break;
      default: return LOPA_ERR_UNSUPPORTED;
    }
  } else {
    const dim3 grid(p.ntiles, p.m_max);
    if (dims->dtype == LOPA_F32) {
      hipLaunchKernelGGL(k_lmhead_plain<float>, grid, dim3(256), 0, stream, V, hidden, p.ntiles,
                         nb_max, p.m_max,
                         static_cast<const float*>(H), static_cast<const float*>(W), rows,
                         row_ptr, nb, wm, wsum, wi, logits_out);
    } else {
      hipLaunchKernelGGL(k_lmhead_plain<unsigned short>, grid, dim3(256), 0, stream, V, hidden,
                         p.ntiles, nb_max, p.m_max, static_cast<const unsigned short*>(H),
                         static_cast<const unsigned short*>(W), rows, row_ptr, nb, wm, wsum, wi,
                         logits_out);
    }
  }
  LOPA_LAUNCH_CHECK();
  hipLaunchKernelGGL(k_lmhead_merge, dim3(p.m_max), dim3(256), 0, stream, p.ntiles, nb_max,
                     p.m_max, rows,
                     row_ptr, nb, wm, wsum, wi, conf, arg);
  LOPA_LAUNCH_CHECK();
  return LOPA_OK;
}
