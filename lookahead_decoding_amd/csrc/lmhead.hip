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
// Kernels write per-(row, vocabulary part) online-softmax partials
// (max, sum exp(l - max), argmax); a merge kernel folds the parts of a row.
//   k_lmhead_mfma   bf16.  One persistent workgroup per compute unit owns a
//                   balanced contiguous vocabulary range and every LM-head
//                   row of its row group.  Four producer waves fetch 64-wide
//                   K chunks of W and H with row-contiguous 16-byte buffer
//                   loads into a register ring several chunks deep and write
//                   them to a double-buffered XOR-swizzled LDS tile; four
//                   compute waves read v_mfma_f32_32x32x16_bf16 fragments
//                   from it.  W is read from HBM exactly once.  The row count
//                   M lives on the device: each variant is enqueued when M
//                   could fall in its range and returns at once otherwise;
//                   inside a variant the 32-row tile count picks a body
//                   compiled for it.
//   k_lmhead_plain  float32 (and shapes outside the MFMA kernel): one thread
//                   per vocabulary entry, FMA dot products.
#include "lopa_common.hpp"
#include "plan.hpp"

namespace lopa {

// ---------------------------------------------------------------------------
// MFMA kernel
// ---------------------------------------------------------------------------


// Physical 16-byte slot of logical slot s in LDS row r.  Rows of a K chunk
// are KC*2 bytes; the XOR keeps 16-lane fragment reads (16 consecutive rows,
// one slot) and the staging writes free of bank conflicts.
template <int KC>
__device__ __forceinline__ int swz(int r, int s) {
  if constexpr (KC == 64) return s ^ ((r & 7) ^ ((r >> 3) & 1));
  else return s ^ (((r >> 1) ^ (r >> 2)) & 3);
}

// Online-softmax partial of one lane's logits for one LM-head row:
// a[n][r] = logit of vocabulary entry vb + 32n + 8(r/4) + 4h + r%4 (the
// 32x32 MFMA output layout, h = lane / 32), merged with the other lane half
// that holds the same row.
template <int NV>
__device__ __forceinline__ Partial row_partial(const f32x16 (&a)[NV], int vb, int h, int vend) {
  Partial p = empty_partial();
#pragma unroll
  for (int n = 0; n < NV; ++n)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int v = vb + n * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
      if (v < vend && a[n][r] > p.m) {
        p.m = a[n][r];
        p.i = v;
      }
    }
  if (p.i != 0x7fffffff) {
    float s = 0.f;
#pragma unroll
    for (int n = 0; n < NV; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int v = vb + n * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        if (v < vend) s += exp2f((a[n][r] - p.m) * kLog2e);
      }
    p.s = s;
  }
  return merge(p, shfl_xor(p, 32));
}

constexpr int kKC = 64;          // K chunk
constexpr int kRB = kKC * 2;     // bytes of one row per chunk (8 slots of 16 B)
constexpr int kRPP = 32;         // rows per staging load (256 producer threads / 8 slots)

template <int NVW, int HRMAX>
struct HeadSmem {
  static constexpr int WROWS = 128 * NVW;                // vocabulary rows per pass
  static constexpr int HRP = (HRMAX + kRPP - 1) / kRPP * kRPP;
  static constexpr int BUF = (WROWS + HRP) * kRB;        // bytes per staging buffer
  static constexpr int RUN = 4 * HRMAX * 12;             // running partials [4 waves][rows]
  static constexpr int BYTES = 2 * BUF + RUN;
};

// One persistent workgroup per compute unit owns a contiguous, balanced
// range of the vocabulary (a multiple of 16 rows) and every LM-head row of
// its row group; it walks the range in passes of 128*NVW vocabulary rows and
// each pass walks the full hidden dimension in 64-wide K chunks.
//
// The workgroup is warp-specialised (512 threads).  Waves 4..7 only move
// data: they fetch each chunk of W and of H with row-contiguous 16-byte
// buffer loads (8 threads per 128-byte row segment) into a register ring D
// chunks deep -- so D-1 chunks (tens of KB per compute unit) stay in flight
// -- and write it to a double-buffered, XOR-swizzled LDS tile.  Waves 0..3
// only compute: each takes NVW 32-row tiles of W against every 32-row tile
// of H with v_mfma_f32_32x32x16_bf16 straight from LDS.  One barrier per
// chunk.  After each pass the compute waves fold their logits into a running
// (max, sum, argmax) per row in LDS; at the end the four are merged and one
// partial per row is written.  W is addressed through a buffer descriptor
// covering exactly the workgroup's range: loads past it return zeros
// without touching memory, so a ragged range needs no clamping.
template <int NVW, int MT, int HRMAX, int D>
__device__ __forceinline__ void head_body(int V, int hidden, int nparts, int Mg, int row0,
                                          int h_bytes, const unsigned short* __restrict__ H,
                                          const unsigned short* __restrict__ W,
                                          const int32_t* __restrict__ rows,
                                          unsigned char* smem, float* __restrict__ ws_m,
                                          float* __restrict__ ws_s, int32_t* __restrict__ ws_i,
                                          float* __restrict__ logits_out) {
  using SM = HeadSmem<NVW, HRMAX>;
  constexpr int BUF = SM::BUF, WROWS = SM::WROWS;
  constexpr int WP = WROWS / kRPP;                 // W loads per producer thread per chunk
  constexpr int HP = (MT * 32 + kRPP - 1) / kRPP;  // H loads per producer thread per chunk
  constexpr int NS = WP + HP;
  constexpr int KS = kKC / 16;                     // MFMA K steps per chunk
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int row_bytes = hidden * 2;

  // this workgroup's vocabulary range [v_lo, v_hi)
  const int t16 = (V + 15) >> 4;
  const int part = blockIdx.x;
  const int v_lo = static_cast<int>(static_cast<long long>(part) * t16 / nparts) * 16;
  const int v_hi = min(static_cast<int>(static_cast<long long>(part + 1) * t16 / nparts) * 16, V);
  const int npass = (v_hi - v_lo + WROWS - 1) / WROWS;
  const int nch = hidden / kKC;
  const int total = npass * nch;

  Partial* run = reinterpret_cast<Partial*>(smem + 2 * BUF);   // [4][HRMAX]
  for (int r = tid; r < 4 * HRMAX; r += 512) run[r] = empty_partial();

  if (w >= 4) {
    // ---------------- producer waves ----------------
    const int ptid = tid - 256;
    const int slot = ptid & 7;
    const int rin = ptid >> 3;
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<unsigned short*>(W) + static_cast<size_t>(v_lo) * hidden, 0,
        max(v_hi - v_lo, 0) * row_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t hr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned short*>(H), 0, h_bytes, 0x00020000);
    const int wvoff = rin * row_bytes + slot * 16;
    int hvoff[HP];
#pragma unroll
    for (int p = 0; p < HP; ++p)
      hvoff[p] = rows[row0 + min(p * kRPP + rin, Mg - 1)] * row_bytes + slot * 16;
    // swz(r + 32, s) == swz(r, s): every load of a thread uses the same slot
    const int dst0 = rin * kRB + swz<kKC>(rin, slot) * 16;
    u16x8 ring[D][NS];
    // chunk i = pass * nch + k-chunk, clamped to the last one
    auto load = [&](int i, u16x8 (&st)[NS]) {
      i = min(i, total - 1);
      const int k = (i % nch) * kRB;
      const int wbase = (i / nch) * WROWS * row_bytes + k;
#pragma unroll
      for (int p = 0; p < WP; ++p)
        st[p] = __builtin_bit_cast(u16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                              wr, wvoff, wbase + p * kRPP * row_bytes, 2));
#pragma unroll
      for (int p = 0; p < HP; ++p)
        st[WP + p] = __builtin_bit_cast(
            u16x8, __builtin_amdgcn_raw_buffer_load_b128(hr, hvoff[p], k, 0));
    };
    auto store = [&](int b, const u16x8 (&st)[NS]) {
      unsigned char* base = smem + b * BUF + dst0;
#pragma unroll
      for (int p = 0; p < WP; ++p) *reinterpret_cast<u16x8*>(base + p * kRPP * kRB) = st[p];
#pragma unroll
      for (int p = 0; p < HP; ++p)
        *reinterpret_cast<u16x8*>(base + (WROWS + p * kRPP) * kRB) = st[WP + p];
    };
    if (total > 0) {
#pragma unroll
      for (int u = 0; u < D; ++u) load(u, ring[u]);
      store(0, ring[0]);
      load(D, ring[0]);
    }
    __syncthreads();
    // iteration i: the compute waves read buffer i%2; here chunk i+1 goes to
    // buffer (i+1)%2 and its ring slot is refilled with chunk i+1+D
    // full groups of 2*D iterations without conditions (so the compiler's
    // wait counts stay exact and D-1 chunks remain in flight), then a tail
    int i0 = 0;
    for (; i0 + 2 * D <= total; i0 += 2 * D) {
#pragma unroll
      for (int u = 0; u < 2 * D; ++u) {
        store((u + 1) & 1, ring[(u + 1) % D]);
        load(i0 + u + 1 + D, ring[(u + 1) % D]);
        __syncthreads();
      }
    }
#pragma unroll
    for (int u = 0; u < 2 * D; ++u) {
      if (i0 + u < total) {
        store((u + 1) & 1, ring[(u + 1) % D]);
        load(i0 + u + 1 + D, ring[(u + 1) % D]);
      }
      if (i0 < total) __syncthreads();
    }
  } else {
    // ---------------- compute waves ----------------
    const int ln = lane & 31;     // MFMA row / column within a 32-tile
    const int lh = lane >> 5;     // which 8 of the 16 K values of a step
    f32x16 acc[MT][NVW];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int n = 0; n < NVW; ++n) acc[mt][n] = f32x16{};
    auto compute = [&](int b) {
      const unsigned char* base = smem + b * BUF;
#pragma unroll
      for (int j = 0; j < KS; ++j) {
        const int ls = j * 2 + lh;   // logical slot: K values 16j + 8lh .. +8
        u16x8 wf[NVW];
#pragma unroll
        for (int n = 0; n < NVW; ++n) {
          const int r = w * (32 * NVW) + n * 32 + ln;
          wf[n] = *reinterpret_cast<const u16x8*>(base + r * kRB + swz<kKC>(r, ls) * 16);
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const int r = mt * 32 + ln;
          const u16x8 hf =
              *reinterpret_cast<const u16x8*>(base + (WROWS + r) * kRB + swz<kKC>(r, ls) * 16);
#pragma unroll
          for (int n = 0; n < NVW; ++n)
            acc[mt][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, wf[n]), __builtin_bit_cast(bf16x8, hf), acc[mt][n],
                0, 0, 0);
        }
      }
    };
    // acc[mt][n][r] = logit of row 32mt + ln, vocabulary entry
    // vbw + 32n + 8(r/4) + 4lh + r%4
    auto finish_pass = [&](int pass) {
      const int vbw = v_lo + pass * WROWS + w * (32 * NVW);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const Partial p = row_partial<NVW>(acc[mt], vbw, lh, v_hi);
        const int r = mt * 32 + ln;
        if (lh == 0) run[w * HRMAX + r] = merge(run[w * HRMAX + r], p);
        if (logits_out && r < Mg) {
          const size_t lb = static_cast<size_t>(rows[row0 + r]) * V;
#pragma unroll
          for (int n = 0; n < NVW; ++n)
#pragma unroll
            for (int q = 0; q < 16; ++q) {
              const int v = vbw + n * 32 + 8 * (q >> 2) + 4 * lh + (q & 3);
              if (v < v_hi) logits_out[lb + v] = acc[mt][n][q];
            }
        }
#pragma unroll
        for (int n = 0; n < NVW; ++n) acc[mt][n] = f32x16{};
      }
    };
    __syncthreads();
    int i0 = 0;
    for (; i0 + 2 * D <= total; i0 += 2 * D) {
#pragma unroll
      for (int u = 0; u < 2 * D; ++u) {
        compute(u & 1);
        if ((i0 + u) % nch == nch - 1) finish_pass((i0 + u) / nch);
        __syncthreads();
      }
    }
#pragma unroll
    for (int u = 0; u < 2 * D; ++u) {
      if (i0 + u < total) {
        compute(u & 1);
        if ((i0 + u) % nch == nch - 1) finish_pass((i0 + u) / nch);
      }
      if (i0 < total) __syncthreads();
    }
  }
  __syncthreads();
  for (int r = tid; r < Mg; r += 512) {
    Partial p = run[r];
    p = merge(p, run[HRMAX + r]);
    p = merge(p, run[2 * HRMAX + r]);
    p = merge(p, run[3 * HRMAX + r]);
    const size_t o = static_cast<size_t>(row0 + r) * nparts + part;
    ws_m[o] = p.m;
    ws_s[o] = p.s;
    ws_i[o] = p.i;
  }
}

// Variant serving total row counts M in (m_lo, m_hi]: balanced row groups of
// at most 32*MTHI rows (grid.y); the group's 32-row tile count picks a body
// compiled for exactly that many tiles.
template <int NVW, int MTLO, int MTHI, int D>
__global__ void __launch_bounds__(512)
k_lmhead_mfma(int V, int hidden, int nparts, int nb_max, int m_max, int m_lo, int m_hi,
              int h_bytes, const unsigned short* __restrict__ H, const unsigned short* __restrict__ W,
              const int32_t* __restrict__ rows, const int32_t* __restrict__ row_ptr,
              const int32_t* __restrict__ nb_ptr, float* __restrict__ ws_m,
              float* __restrict__ ws_s, int32_t* __restrict__ ws_i,
              float* __restrict__ logits_out) {
  constexpr int HRMAX = MTHI * 32;
  __shared__ __attribute__((aligned(16))) unsigned char smem[HeadSmem<NVW, HRMAX>::BYTES];
  const int M = listed_rows(row_ptr, nb_ptr, nb_max, m_max);
  if (M <= m_lo || M > m_hi) return;
  // balanced row groups of at most MTHI tiles
  const int mt_all = (M + 31) >> 5;
  const int ngroups = (mt_all + MTHI - 1) / MTHI;
  const int tpg = (mt_all + ngroups - 1) / ngroups;
  const int row0 = blockIdx.y * tpg * 32;
  if (static_cast<int>(blockIdx.y) >= ngroups || row0 >= M) return;
  const int Mg = min(M - row0, tpg * 32);
  int Mt = (Mg + 31) >> 5;
  Mt = Mt < MTLO ? MTLO : Mt;
  switch (Mt) {
#define LOPA_BODY(T)                                                                           \
  case T:                                                                                      \
    if constexpr (T >= MTLO && T <= MTHI)                                                      \
      head_body<NVW, T, HRMAX, D>(V, hidden, nparts, Mg, row0, h_bytes, H, W, rows, smem,     \
                                  ws_m, ws_s, ws_i, logits_out);                               \
    break;
    LOPA_BODY(1) LOPA_BODY(2) LOPA_BODY(3) LOPA_BODY(4) LOPA_BODY(5) LOPA_BODY(6)
    LOPA_BODY(7) LOPA_BODY(8) LOPA_BODY(9) LOPA_BODY(10)
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
    hipLaunchKernelGGL((k_lmhead_mfma<2, 1, 4, 4>), dim3(p.ntiles), dim3(512), 0, stream, V,
                       hidden, p.ntiles, nb_max, p.m_max, 0, kHeadSmallRows, h_bytes, Hb, Wb, rows,
                       row_ptr, nb, wm, wsum, wi, logits_out);
    LOPA_LAUNCH_CHECK();
  }
  if (p.mid) {
    hipLaunchKernelGGL((k_lmhead_mfma<1, 5, 8, 3>), dim3(p.ntiles), dim3(512), 0, stream, V,
                       hidden, p.ntiles, nb_max, p.m_max, kHeadSmallRows, kHeadMidRows, h_bytes, Hb, Wb,
                       rows, row_ptr, nb, wm, wsum, wi, logits_out);
    LOPA_LAUNCH_CHECK();
  }
  if (p.large) {
    hipLaunchKernelGGL((k_lmhead_mfma<1, 1, 10, 3>), dim3(p.ntiles, p.groups), dim3(512), 0,
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
