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
// Kernels write per-(row, 128-entry vocabulary tile) online-softmax partials
// (max, sum exp(l - max), argmax); a merge kernel folds the tiles of a row.
//   k_lmhead_mfma   bf16.  A workgroup (4 waves) owns 128 vocabulary rows of
//                   W and all LM-head rows of H (up to 576 per row group) and
//                   walks the full hidden dimension in K chunks.  Each chunk
//                   of W and of H is fetched with row-contiguous 16-byte loads
//                   two chunks ahead into registers, written to a
//                   double-buffered XOR-swizzled LDS tile and read back as
//                   v_mfma_f32_16x16x32_bf16 fragments (each wave: 2 x 16
//                   vocabulary rows against every 16-row tile of H).  W is
//                   read from HBM exactly once.  The row count M lives on the
//                   device: three variants are enqueued when M could fall in
//                   their range (M <= 160, 161..384, > 384), the others
//                   return at once, and inside a variant the tile count picks
//                   a body compiled for it.
//   k_lmhead_plain  float32 (and shapes outside the MFMA kernel): one thread
//                   per vocabulary entry, FMA dot products.
#include "lopa_common.hpp"
#include "plan.hpp"

namespace lopa {

// ---------------------------------------------------------------------------
// MFMA kernel
// ---------------------------------------------------------------------------

constexpr int kNV = 2;           // 16-row vocabulary tiles per wave
constexpr int kWR = 128;         // vocabulary rows per workgroup (4 waves x 2 x 16)

// Physical 16-byte slot of logical slot s in LDS row r.  Rows of a K chunk
// are KC*2 bytes; the XOR keeps 16-lane fragment reads (16 consecutive rows,
// one slot) and the staging writes free of bank conflicts.
template <int KC>
__device__ __forceinline__ int swz(int r, int s) {
  if constexpr (KC == 64) return s ^ ((r & 7) ^ ((r >> 3) & 1));
  else return s ^ (((r >> 1) ^ (r >> 2)) & 3);
}

// Online-softmax partial of one lane's logits a[n][q] (vocabulary entries
// vb + 16n + 4lg + q) for one row, merged over the 4 lane groups that hold
// the same row.
template <int NV>
__device__ __forceinline__ Partial row_partial(const f32x4 (&a)[NV], int vb, int lg, int V) {
  Partial p = empty_partial();
#pragma unroll
  for (int n = 0; n < NV; ++n)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int v = vb + n * 16 + 4 * lg + q;
      if (v < V && a[n][q] > p.m) {
        p.m = a[n][q];
        p.i = v;
      }
    }
  if (p.i != 0x7fffffff) {
    float s = 0.f;
#pragma unroll
    for (int n = 0; n < NV; ++n)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int v = vb + n * 16 + 4 * lg + q;
        if (v < V) s += exp2f((a[n][q] - p.m) * kLog2e);
      }
    p.s = s;
  }
  p = merge(p, shfl_xor(p, 16));
  p = merge(p, shfl_xor(p, 32));
  return p;
}

template <int KC, int HRMAX>
struct HeadSmem {
  static constexpr int RB = KC * 2;                      // bytes per row per chunk
  static constexpr int SPR = RB / 16;                    // 16-byte slots per row
  static constexpr int RPP = 256 / SPR;                  // rows per staging pass
  static constexpr int HRP = (HRMAX + RPP - 1) / RPP * RPP;
  static constexpr int BUF = (kWR + HRP) * RB;           // bytes per buffer
  static constexpr int BYTES = 2 * BUF > 4 * HRMAX * 12 ? 2 * BUF : 4 * HRMAX * 12;
};

// One workgroup: 128 vocabulary rows x MT*16 LM-head rows, full hidden.
// K advances in chunks of KC: every chunk of W (128 rows) and of H (the
// group's rows) is fetched with row-contiguous 16-byte buffer loads (SPR
// threads per row) into registers -- W two chunks ahead, H one -- written to
// a double-buffered swizzled LDS tile and read back as MFMA fragments; one
// barrier per chunk.  W is addressed through a buffer descriptor that starts
// at the tile's first row and ends at the last vocabulary row, so a ragged
// last tile reads zeros instead of running past the weight.
template <int KC, int MT, int HRMAX>
__device__ __forceinline__ void head_body(int V, int hidden, int ntiles, int Mg, int row0,
                                          int h_bytes, const unsigned short* __restrict__ H,
                                          const unsigned short* __restrict__ W,
                                          const int32_t* __restrict__ rows,
                                          unsigned char* smem, float* __restrict__ ws_m,
                                          float* __restrict__ ws_s, int32_t* __restrict__ ws_i,
                                          float* __restrict__ logits_out) {
  using SM = HeadSmem<KC, HRMAX>;
  constexpr int RB = SM::RB, SPR = SM::SPR, RPP = SM::RPP, BUF = SM::BUF;
  constexpr int WP = kWR / RPP;                   // W staging passes
  constexpr int HP = (MT * 16 + RPP - 1) / RPP;   // H staging passes
  constexpr int KS = KC / 32;                     // MFMA K steps per chunk
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int ln = lane & 15;
  const int lg = lane >> 4;
  const int tile = blockIdx.x;
  const int v0 = tile * kWR;
  const int slot = tid % SPR;
  const int rin = tid / SPR;
  const int row_bytes = hidden * 2;

  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<unsigned short*>(W) + static_cast<size_t>(v0) * hidden, 0,
      min(kWR, V - v0) * row_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t hr =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned short*>(H), 0, h_bytes, 0x00020000);
  const int wvoff = rin * row_bytes + slot * 16;          // + pass and chunk in soffset
  int hvoff[HP];
#pragma unroll
  for (int p = 0; p < HP; ++p)
    hvoff[p] = rows[row0 + min(p * RPP + rin, Mg - 1)] * row_bytes + slot * 16;
  // swz(r + RPP, s) == swz(r, s): every pass uses the same in-row slot
  const int dst0 = rin * RB + swz<KC>(rin, slot) * 16;

  auto load_w = [&](int c, u16x8 (&st)[WP]) {
    const int k = c * (KC * 2);
#pragma unroll
    for (int p = 0; p < WP; ++p)
      st[p] = __builtin_bit_cast(
          u16x8, __builtin_amdgcn_raw_buffer_load_b128(wr, wvoff, p * RPP * row_bytes + k, 2));
  };
  auto load_h = [&](int c, u16x8 (&st)[HP]) {
    const int k = c * (KC * 2);
#pragma unroll
    for (int p = 0; p < HP; ++p)
      st[p] = __builtin_bit_cast(u16x8, __builtin_amdgcn_raw_buffer_load_b128(hr, hvoff[p], k, 0));
  };
  auto store = [&](int b, const u16x8 (&sw)[WP], const u16x8 (&sh)[HP]) {
    unsigned char* base = smem + b * BUF + dst0;
#pragma unroll
    for (int p = 0; p < WP; ++p) *reinterpret_cast<u16x8*>(base + p * RPP * RB) = sw[p];
#pragma unroll
    for (int p = 0; p < HP; ++p)
      *reinterpret_cast<u16x8*>(base + (kWR + p * RPP) * RB) = sh[p];
  };

  f32x4 acc[MT][kNV];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int n = 0; n < kNV; ++n) acc[mt][n] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int b) {
    const unsigned char* base = smem + b * BUF;
#pragma unroll
    for (int j = 0; j < KS; ++j) {
      const int ls = j * 4 + lg;   // logical slot: K values 32j + 8lg .. +8
      u16x8 wf[kNV];
#pragma unroll
      for (int n = 0; n < kNV; ++n) {
        const int r = w * 32 + n * 16 + ln;
        wf[n] = *reinterpret_cast<const u16x8*>(base + r * RB + swz<KC>(r, ls) * 16);
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int r = mt * 16 + ln;
        const u16x8 hf =
            *reinterpret_cast<const u16x8*>(base + (kWR + r) * RB + swz<KC>(r, ls) * 16);
#pragma unroll
        for (int n = 0; n < kNV; ++n)
          acc[mt][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, wf[n]), __builtin_bit_cast(bf16x8, hf), acc[mt][n],
              0, 0, 0);
      }
    }
  };

  const int nch = hidden / KC;    // even
  u16x8 wa[WP], wb[WP], hs[HP];
  load_w(0, wa);
  load_h(0, hs);
  load_w(1, wb);
  store(0, wa, hs);
  __syncthreads();
  for (int c = 0; c < nch; c += 2) {
    // chunk c is in LDS buffer 0, W of chunk c+1 in flight in wb
    load_h(min(c + 1, nch - 1), hs);
    load_w(min(c + 2, nch - 1), wa);
    __builtin_amdgcn_sched_barrier(0);
    compute(0);
    __builtin_amdgcn_sched_barrier(0);
    store(1, wb, hs);
    __syncthreads();
    load_h(min(c + 2, nch - 1), hs);
    load_w(min(c + 3, nch - 1), wb);
    __builtin_amdgcn_sched_barrier(0);
    compute(1);
    __builtin_amdgcn_sched_barrier(0);
    store(0, wa, hs);
    __syncthreads();
  }

  // acc[mt][n][q] = logit of row mt*16 + ln, vocabulary entry
  // v0 + 32w + 16n + 4lg + q.
  Partial* red = reinterpret_cast<Partial*>(smem);   // [4 waves][HRMAX]
  const int vbw = v0 + w * 32;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const Partial p = row_partial<kNV>(acc[mt], vbw, lg, V);
    const int r = mt * 16 + ln;
    if (lg == 0) red[w * HRMAX + r] = p;
    if (logits_out && r < Mg) {
      const size_t base = static_cast<size_t>(rows[row0 + r]) * V;
#pragma unroll
      for (int n = 0; n < kNV; ++n)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int v = vbw + n * 16 + 4 * lg + q;
          if (v < V) logits_out[base + v] = acc[mt][n][q];
        }
    }
  }
  __syncthreads();
  for (int r = tid; r < Mg; r += 256) {
    Partial p = red[r];
    p = merge(p, red[HRMAX + r]);
    p = merge(p, red[2 * HRMAX + r]);
    p = merge(p, red[3 * HRMAX + r]);
    const size_t o = static_cast<size_t>(row0 + r) * ntiles + tile;
    ws_m[o] = p.m;
    ws_s[o] = p.s;
    ws_i[o] = p.i;
  }
}

// Variant serving total row counts M in (m_lo, m_hi]: row groups of up to
// 16*MTHI rows (grid.y); the group's tile count picks a body compiled for
// exactly that many tiles (in steps of STEP tiles).
template <int KC, int MTLO, int MTHI, int STEP>
__global__ void __launch_bounds__(256)
k_lmhead_mfma(int V, int hidden, int ntiles, int nb_max, int m_max, int m_lo, int m_hi,
              int h_bytes, const unsigned short* __restrict__ H, const unsigned short* __restrict__ W,
              const int32_t* __restrict__ rows, const int32_t* __restrict__ row_ptr,
              const int32_t* __restrict__ nb_ptr, float* __restrict__ ws_m,
              float* __restrict__ ws_s, int32_t* __restrict__ ws_i,
              float* __restrict__ logits_out) {
  constexpr int HRMAX = MTHI * 16;
  __shared__ __attribute__((aligned(16))) unsigned char smem[HeadSmem<KC, HRMAX>::BYTES];
  const int M = listed_rows(row_ptr, nb_ptr, nb_max, m_max);
  if (M <= m_lo || M > m_hi) return;
  const int row0 = blockIdx.y * HRMAX;
  if (row0 >= M) return;
  const int Mg = min(M - row0, HRMAX);
  int Mt = (Mg + 15) >> 4;
  Mt = (Mt + STEP - 1) / STEP * STEP;
  Mt = Mt < MTLO ? MTLO : Mt;
  switch (Mt) {
#define LOPA_BODY(T)                                                                         \
  case T:                                                                                    \
    if constexpr (T >= MTLO && T <= MTHI && T % STEP == 0)                                   \
      head_body<KC, T, HRMAX>(V, hidden, ntiles, Mg, row0, h_bytes, H, W, rows, smem, ws_m,  \
                              ws_s, ws_i, logits_out);                                       \
    break;
    LOPA_BODY(1) LOPA_BODY(2) LOPA_BODY(3) LOPA_BODY(4) LOPA_BODY(5) LOPA_BODY(6)
    LOPA_BODY(7) LOPA_BODY(8) LOPA_BODY(9) LOPA_BODY(10) LOPA_BODY(11) LOPA_BODY(12)
    LOPA_BODY(13) LOPA_BODY(14) LOPA_BODY(15) LOPA_BODY(16) LOPA_BODY(17) LOPA_BODY(18)
    LOPA_BODY(19) LOPA_BODY(20) LOPA_BODY(21) LOPA_BODY(22) LOPA_BODY(23) LOPA_BODY(24)
    LOPA_BODY(28) LOPA_BODY(32) LOPA_BODY(36)
#undef LOPA_BODY
    default: break;
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
  const int v = blockIdx.x * kPlainVocabPerWG + threadIdx.x;
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
k_lmhead_merge(int ntiles, int nb_max, int m_max,
               const int32_t* __restrict__ rows, const int32_t* __restrict__ row_ptr,
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
  const unsigned short* Hb = static_cast<const unsigned short*>(H);
  const unsigned short* Wb = static_cast<const unsigned short*>(W);
  const int h_bytes = p.m_max * hidden * 2;   // H is [nb_max][B][hidden]
  if (p.small) {
    hipLaunchKernelGGL((k_lmhead_mfma<64, 1, 10, 1>), dim3(p.ntiles), dim3(256), 0, stream, V,
                       hidden, p.ntiles, nb_max, p.m_max, 0, kHeadSmallRows, h_bytes, Hb, Wb, rows,
                       row_ptr, nb, wm, wsum, wi, logits_out);
    LOPA_LAUNCH_CHECK();
  }
  if (p.mid) {
    hipLaunchKernelGGL((k_lmhead_mfma<64, 11, 24, 1>), dim3(p.ntiles), dim3(256), 0, stream, V,
                       hidden, p.ntiles, nb_max, p.m_max, kHeadSmallRows, kHeadMidRows, h_bytes, Hb, Wb,
                       rows, row_ptr, nb, wm, wsum, wi, logits_out);
    LOPA_LAUNCH_CHECK();
  }
  if (p.large) {
    hipLaunchKernelGGL((k_lmhead_mfma<32, 4, 36, 4>), dim3(p.ntiles, p.groups), dim3(256), 0,
                       stream, V, hidden, p.ntiles, nb_max, p.m_max, p.large_lo, 1 << 30, h_bytes, Hb, Wb,
                       rows, row_ptr, nb, wm, wsum, wi, logits_out);
    LOPA_LAUNCH_CHECK();
  }
  if (!p.small && !p.mid && !p.large) {
    const dim3 grid(p.ntiles, p.m_max);
    if (dims->dtype == LOPA_F32) {
      hipLaunchKernelGGL(k_lmhead_plain<float>, grid, dim3(256), 0, stream, V, hidden, p.ntiles,
                         nb_max, p.m_max, static_cast<const float*>(H),
                         static_cast<const float*>(W), rows, row_ptr, nb, wm, wsum, wi,
                         logits_out);
    } else {
      hipLaunchKernelGGL(k_lmhead_plain<unsigned short>, grid, dim3(256), 0, stream, V, hidden,
                         p.ntiles, nb_max, p.m_max, Hb, Wb, rows, row_ptr, nb, wm, wsum, wi,
                         logits_out);
    }
    LOPA_LAUNCH_CHECK();
  }
  hipLaunchKernelGGL(k_lmhead_merge, dim3(p.m_max), dim3(256), 0, stream, p.ntiles, nb_max,
                     p.m_max, rows,
                     row_ptr, nb, wm, wsum, wi, conf, arg);
  LOPA_LAUNCH_CHECK();
  return LOPA_OK;
}
