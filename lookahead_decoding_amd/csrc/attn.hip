// Verify stage, attention part: every branch's block attends to the shared
// committed prefix and to its own block, never to another branch's block.
//
// Section 3.3 of "解码效率革命：LoPA如何突破扩散语言模型的并行瓶颈" isolates the
// branches through the attention mask and runs all of them in one pass;
// section 6 of the same article needs full-sequence (bidirectional)
// attention; the news article "上交大 × 华为小艺推出LoPA：7B扩散语言模型单样例
// 1000+ tokens/s！" (section "LoPA 的核心设计：前瞻并行与分支验证", stage
// 并行验证与复用) verifies all branches in one forward pass.  The mask is never
// stored: a query row's branch follows from its index, and the kernel only
// ever visits the prefix keys and that branch's block keys.
//
//   k_attn_mfma   bf16, d = 128, (B * Hq/Hkv) % 16 == 0.  A workgroup (4
//                 waves) takes 64 query rows of one KV head -- rows are
//                 (branch, position, q-head of the group), so the 64 rows span
//                 several positions and at most a few branches -- and streams
//                 the prefix K/V of that head through LDS once for all of
//                 them.  S^T = K Q^T and O^T = V^T P^T are
//                 v_mfma_f32_16x16x32_bf16 tiles; online softmax in float32;
//                 P enters the PV product as a bf16 hi + lo pair so the
//                 probabilities keep ~16 significant bits.
//   k_attn_plain  any dtype / d <= 256: one wave per query row, keys in
//                 chunks of 1024 with online softmax, float32 throughout.
#include <type_traits>

#include "lopa_common.hpp"
#include "plan.hpp"

namespace lopa {

// ---------------------------------------------------------------------------
// MFMA path
// ---------------------------------------------------------------------------

constexpr int kAD = 128;          // head dim
constexpr int kAKB = 64;          // keys per LDS block
constexpr int kAKRow = kAD + 8;   // K row in LDS (bf16): 272 B, conflict-free 16-B reads
constexpr int kAVRow = kAKB + 8;  // V^T row in LDS (bf16): 144 B, conflict-free 16-B reads
constexpr int kARows = 128;       // query rows per workgroup (4 waves x 2 groups of 16)

// K is staged so that the QK^T tile t, MFMA row i reads key
// 32(t/2) + 8(i/4) + 4(t%2) + i%4: the S^T accumulator of lane (i, g) then
// holds, for the two tiles of a 32-key PV step, 8 consecutive keys
// 32s + 8g .. 32s + 8g + 7 -- exactly the contraction slice the P^T operand
// of that lane needs, so V^T fragments are single contiguous 16-byte reads.
__device__ __forceinline__ int key_slot(int k) {
  return (k & 32) | ((k & 4) << 2) | ((k & 24) >> 1) | (k & 3);
}

struct AttnStage {
  u16x8 k[4];   // 4 keys' 16-byte segments
  u16x8 v[4];   // 4 consecutive keys x 8 dims
};

// One workgroup: 128 query rows (branch, position, q-head of the group) of
// KV head g, split s of the prefix keys.  Each wave owns two 16-row groups.
// Prefix blocks are double-buffered in LDS (next block's loads in flight
// during the current block's MFMAs); the last split also visits every
// branch's own block, each seen only by that branch's rows.  With one split
// the output is normalised and rounded to bf16 here; otherwise the
// unnormalised partial (O, max, sum) goes to `part` for k_attn_combine.
__global__ void __launch_bounds__(256)
k_attn_mfma(int L, int B, int Hq, int Hkv, int nb_max, int splits,
            const int32_t* __restrict__ nb_ptr, const unsigned short* __restrict__ Kp,
            const unsigned short* __restrict__ Vp, const unsigned short* __restrict__ Qb,
            const unsigned short* __restrict__ Kb, const unsigned short* __restrict__ Vb,
            unsigned short* __restrict__ H, float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) unsigned short Ks[2][kAKB * kAKRow];
  __shared__ __attribute__((aligned(16))) unsigned short Vt[2][kAD * kAVRow];

  const int G = Hq / Hkv;
  const int g = blockIdx.y;
  const int split = blockIdx.z;
  const int RB = B * G;                 // query rows per branch for this KV head
  const int nb = min(max(*nb_ptr, 0), nb_max);
  const int R = nb * RB;
  const int r0 = blockIdx.x * kARows;
  if (r0 >= R) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int ln = lane & 15;
  const int lg = lane >> 4;

  // two 16-row groups per wave; rows of a group share one branch
  int grow[2], gbr[2], qoff[2];
  bool act[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    // wave-uniform: keep it in scalar registers so branches on it are scalar
    grow[q] = __builtin_amdgcn_readfirstlane(r0 + 32 * w + 16 * q);
    act[q] = grow[q] < R;
    gbr[q] = act[q] ? grow[q] / RB : -1;
    qoff[q] = 0;
    if (act[q]) {
      const int rem = grow[q] + ln - gbr[q] * RB;
      qoff[q] = ((gbr[q] * B + rem / G) * Hq + g * G + rem % G) * kAD;
    }
  }
  u16x8 qf[2][4];
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int s = 0; s < 4; ++s)
      qf[q][s] = act[q] ? *reinterpret_cast<const u16x8*>(Qb + qoff[q] + 32 * s + 8 * lg)
                        : u16x8{0, 0, 0, 0, 0, 0, 0, 0};

  const float scale2 = kLog2e * 0.08838834764831845f;   // log2(e) / sqrt(128)
  float m_run[2] = {-INFINITY, -INFINITY};
  float l_run[2] = {0.f, 0.f};
  f32x4 o[2][8];
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int u = 0; u < 8; ++u) o[q][u] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- staging: kn (<= 64) keys of KV head g from key-major sources ----
  const int kseg = tid & 15;            // K: 16-byte segment of a key row
  const int kq = tid & 15;              // V: keys 4kq .. 4kq+3
  const int dq = tid >> 4;              // V: dims 8dq .. 8dq+7
  auto load_stage = [&](const unsigned short* ks, const unsigned short* vs, int kn,
                        AttnStage& st) {
    // keys past kn repeat key kn-1: their scores are masked to -inf, so
    // they weigh 0 in the value product
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int key = min((tid >> 4) + 16 * p, kn - 1);
      st.k[p] = *reinterpret_cast<const u16x8*>(
          ks + (static_cast<size_t>(key) * Hkv + g) * kAD + kseg * 8);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = min(4 * kq + i, kn - 1);
      st.v[i] = *reinterpret_cast<const u16x8*>(
          vs + (static_cast<size_t>(key) * Hkv + g) * kAD + dq * 8);
    }
  };
  auto store_stage = [&](int b, const AttnStage& st) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int key = (tid >> 4) + 16 * p;
      *reinterpret_cast<u16x8*>(&Ks[b][key_slot(key) * kAKRow + kseg * 8]) = st.k[p];
    }
    // 4 keys x 8 dims -> 8 dims x 4 consecutive keys
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const unsigned lo = static_cast<unsigned>(st.v[0][e]) | (static_cast<unsigned>(st.v[1][e]) << 16);
      const unsigned hi = static_cast<unsigned>(st.v[2][e]) | (static_cast<unsigned>(st.v[3][e]) << 16);
      *reinterpret_cast<uint2*>(&Vt[b][(dq * 8 + e) * kAVRow + 4 * kq]) = make_uint2(lo, hi);
    }
  };

  // ---- one 64-key block for the groups in GM (bit q = group q) ----
  // LDS fragments are read one MFMA group ahead into alternating registers
  // (scheduling barriers keep the reads ahead of the MFMAs that hide them).
  auto process = [&](auto gmc, int b, int kn) __attribute__((always_inline)) {
    constexpr int gm = decltype(gmc)::value;
    const unsigned short* kbase = &Ks[b][ln * kAKRow + 8 * lg];
    const unsigned short* vbase = &Vt[b][ln * kAVRow + 8 * lg];
    f32x4 st[2][4];
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int t = 0; t < 4; ++t) st[q][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    u16x8 kf[2][4];
#pragma unroll
    for (int s = 0; s < 4; ++s) kf[0][s] = *reinterpret_cast<const u16x8*>(kbase + 32 * s);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (t < 3) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
          kf[(t + 1) & 1][s] =
              *reinterpret_cast<const u16x8*>(kbase + 16 * (t + 1) * kAKRow + 32 * s);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int q = 0; q < 2; ++q)
          if ((gm >> q) & 1)   // compile-time
            st[q][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, kf[t & 1][s]), __builtin_bit_cast(bf16x8, qf[q][s]),
                st[q][t], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    // first V fragments go out before the softmax arithmetic
    u16x8 vf[2][2];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) vf[0][s2] = *reinterpret_cast<const u16x8*>(vbase + 32 * s2);
    // st[q][t][r] = q_row(ln) . k(32(t/2) + 8lg + 4(t%2) + r)
    bf16x8 phi[2][2], plo[2][2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      if (!((gm >> q) & 1)) continue;   // compile-time
      float bmax = -INFINITY;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = 32 * (t >> 1) + 8 * lg + 4 * (t & 1) + r;
          st[q][t][r] = key < kn ? st[q][t][r] * scale2 : -INFINITY;
          bmax = fmaxf(bmax, st[q][t][r]);
        }
      bmax = fmaxf(bmax, __shfl_xor(bmax, 16, kWave));
      bmax = fmaxf(bmax, __shfl_xor(bmax, 32, kWave));
      const float m_new = fmaxf(m_run[q], bmax);
      const float alpha = __builtin_amdgcn_exp2f(m_run[q] - m_new);
      m_run[q] = m_new;
      l_run[q] *= alpha;
#pragma unroll
      for (int u = 0; u < 8; ++u) o[q][u] *= alpha;
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float pv = __builtin_amdgcn_exp2f(st[q][2 * s2 + (j >> 2)][j & 3] - m_new);
          l_run[q] += pv;
          const bf16 hi = static_cast<bf16>(pv);
          phi[q][s2][j] = hi;
          plo[q][s2][j] = static_cast<bf16>(pv - static_cast<float>(hi));
        }
    }
    // O^T += V^T P^T (P as bf16 hi + lo)
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (u < 7) {
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
          vf[(u + 1) & 1][s2] =
              *reinterpret_cast<const u16x8*>(vbase + 16 * (u + 1) * kAVRow + 32 * s2);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          if (!((gm >> q) & 1)) continue;   // compile-time
          const bf16x8 v8 = __builtin_bit_cast(bf16x8, vf[u & 1][s2]);
          o[q][u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v8, phi[q][s2], o[q][u], 0, 0, 0);
          o[q][u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v8, plo[q][s2], o[q][u], 0, 0, 0);
        }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  const int gm_all = (act[0] ? 1 : 0) | (act[1] ? 2 : 0);
  using G1 = std::integral_constant<int, 1>;
  using G2 = std::integral_constant<int, 2>;
  using G3 = std::integral_constant<int, 3>;
#define LOPA_PROCESS_GM(GMV, BUF, KN)       \
  do {                                       \
    if ((GMV) == 3) process(G3{}, BUF, KN);  \
    else if ((GMV) == 1) process(G1{}, BUF, KN); \
    else if ((GMV) == 2) process(G2{}, BUF, KN); \
  } while (0)

  // ---- phase 1: this split's share of the committed prefix ----
  const int nbp = (L + kAKB - 1) / kAKB;
  const int kb_lo = split * nbp / splits;
  const int kb_hi = (split + 1) * nbp / splits;
  if (kb_lo < kb_hi) {
    AttnStage st;
    {
      const size_t off = static_cast<size_t>(kb_lo) * kAKB * Hkv * kAD;
      load_stage(Kp + off, Vp + off, min(kAKB, L - kb_lo * kAKB), st);
      store_stage(0, st);
    }
    __syncthreads();
    for (int kb = kb_lo; kb < kb_hi; ++kb) {
      const int cur = (kb - kb_lo) & 1;
      // the next block's loads stay in flight during this block's MFMAs;
      // unconditional (the last iteration reloads its own block into the
      // idle buffer) so the wait lands at the LDS store, not the branch
      const int nx = min(kb + 1, kb_hi - 1);
      const size_t off = static_cast<size_t>(nx) * kAKB * Hkv * kAD;
      load_stage(Kp + off, Vp + off, min(kAKB, L - nx * kAKB), st);
      __builtin_amdgcn_sched_barrier(0);
      LOPA_PROCESS_GM(gm_all, cur, min(kAKB, L - kb * kAKB));
      __builtin_amdgcn_sched_barrier(0);
      store_stage(cur ^ 1, st);
      __syncthreads();
    }
  }
  // ---- phase 2: every branch's own block, seen only by its own rows ----
  if (split == splits - 1) {
    const int b_lo = r0 / RB;
    const int b_hi = min(r0 + kARows - 1, R - 1) / RB;
    for (int bb = b_lo; bb <= b_hi; ++bb) {
      const int gm = (gbr[0] == bb ? 1 : 0) | (gbr[1] == bb ? 2 : 0);
      for (int j0 = 0; j0 < B; j0 += kAKB) {
        AttnStage st;
        const size_t off = (static_cast<size_t>(bb) * B + j0) * Hkv * kAD;
        load_stage(Kb + off, Vb + off, min(kAKB, B - j0), st);
        store_stage(0, st);
        __syncthreads();
        LOPA_PROCESS_GM(gm, 0, min(kAKB, B - j0));
        __syncthreads();
      }
    }
  }

#undef LOPA_PROCESS_GM

  // ---- output: o[q][u][r] = O[row ln of group q][dim 16u + 4lg + r] ----
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    if (!act[q]) continue;
    float l_tot = l_run[q] + __shfl_xor(l_run[q], 16, kWave);
    l_tot += __shfl_xor(l_tot, 32, kWave);
    if (splits == 1) {
      const float inv = 1.f / l_tot;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const unsigned a = f32_to_bf16_bits(o[q][u][0] * inv) |
                           (static_cast<unsigned>(f32_to_bf16_bits(o[q][u][1] * inv)) << 16);
        const unsigned c = f32_to_bf16_bits(o[q][u][2] * inv) |
                           (static_cast<unsigned>(f32_to_bf16_bits(o[q][u][3] * inv)) << 16);
        *reinterpret_cast<uint2*>(H + qoff[q] + 16 * u + 4 * lg) = make_uint2(a, c);
      }
    } else {
      // partial of row (g, grow + ln): [split][Hkv][rows][128] O, then max, sum
      const size_t rmax = static_cast<size_t>(nb_max) * RB;
      const size_t row = (static_cast<size_t>(split) * Hkv + g) * rmax + grow[q] + ln;
      float* po = part + row * kAD;
#pragma unroll
      for (int u = 0; u < 8; ++u) *reinterpret_cast<f32x4*>(po + 16 * u + 4 * lg) = o[q][u];
      float* pm = part + static_cast<size_t>(splits) * Hkv * rmax * kAD;
      if (lg == 0) {
        pm[row] = m_run[q];
        pm[static_cast<size_t>(splits) * Hkv * rmax + row] = l_tot;
      }
    }
  }
}

// Merge of the prefix splits: O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s,
// rounded to bf16.  One wave per row (2 dims per lane).
__global__ void __launch_bounds__(256)
k_attn_combine(int B, int Hq, int Hkv, int nb_max, int splits, const int32_t* __restrict__ nb_ptr,
               const float* __restrict__ part, unsigned short* __restrict__ H) {
  const int G = Hq / Hkv;
  const int RB = B * G;
  const int nb = min(max(*nb_ptr, 0), nb_max);
  const int g = blockIdx.y;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= nb * RB) return;
  const int lane = threadIdx.x & 63;
  const size_t rmax = static_cast<size_t>(nb_max) * RB;
  const float* pm = part + static_cast<size_t>(splits) * Hkv * rmax * kAD;
  const float* pl = pm + static_cast<size_t>(splits) * Hkv * rmax;
  float M = -INFINITY;
  for (int s = 0; s < splits; ++s) M = fmaxf(M, pm[(static_cast<size_t>(s) * Hkv + g) * rmax + r]);
  float lsum = 0.f, o0 = 0.f, o1 = 0.f;
  for (int s = 0; s < splits; ++s) {
    const size_t row = (static_cast<size_t>(s) * Hkv + g) * rmax + r;
    const float wgt = exp2f(pm[row] - M);   // 0 for a split that saw no key
    lsum += wgt * pl[row];
    const float2 ov = *reinterpret_cast<const float2*>(part + row * kAD + 2 * lane);
    o0 += wgt * ov.x;
    o1 += wgt * ov.y;
  }
  const float inv = 1.f / lsum;
  const int b = r / RB, rem = r % RB;
  const size_t hoff = (static_cast<size_t>(b * B + rem / G) * Hq + g * G + rem % G) * kAD;
  const unsigned v = f32_to_bf16_bits(o0 * inv) | (static_cast<unsigned>(f32_to_bf16_bits(o1 * inv)) << 16);
  *reinterpret_cast<unsigned*>(H + hoff + 2 * lane) = v;
}

// ---------------------------------------------------------------------------
// Plain path
// ---------------------------------------------------------------------------

template <typename T>
__global__ void __launch_bounds__(64)
k_attn_plain(int L, int B, int Hq, int Hkv, int d, int nb_max, const int32_t* __restrict__ nb_ptr,
             const T* __restrict__ Kp, const T* __restrict__ Vp, const T* __restrict__ Qb,
             const T* __restrict__ Kb, const T* __restrict__ Vb, T* __restrict__ H) {
  constexpr int CH = 1024;
  __shared__ float sc[CH];
  const int rid = blockIdx.x;          // (b*B + i)*Hq + h
  const int h = rid % Hq;
  const int bi = rid / Hq;
  const int b = bi / B;
  if (b >= min(*nb_ptr, nb_max)) return;
  const int g = h / (Hq / Hkv);
  const int lane = threadIdx.x;
  const int nu = (d + 63) / 64;
  const float scale = 1.f / sqrtf(static_cast<float>(d));
  const size_t qoff = static_cast<size_t>(rid) * d;
  float o[4] = {0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const int n = L + B;
  for (int j0 = 0; j0 < n; j0 += CH) {
    const int cn = min(CH, n - j0);
    float cmax = -INFINITY;
    for (int jj = lane; jj < cn; jj += 64) {
      const int j = j0 + jj;
      const T* kr = j < L ? Kp + (static_cast<size_t>(j) * Hkv + g) * d
                          : Kb + ((static_cast<size_t>(b) * B + (j - L)) * Hkv + g) * d;
      float s = 0.f;
      for (int e = 0; e < d; ++e) s = fmaf(Act<T>::load(Qb, qoff + e), Act<T>::load(kr, e), s);
      s *= scale;
      sc[jj] = s;
      cmax = fmaxf(cmax, s);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) cmax = fmaxf(cmax, __shfl_xor(cmax, off, kWave));
    __syncthreads();
    const float m_new = fmaxf(m_run, cmax);
    const float alpha = expf(m_run - m_new);
    l_run *= alpha;
    for (int u = 0; u < nu; ++u) o[u] *= alpha;
    for (int jj = 0; jj < cn; ++jj) {
      const int j = j0 + jj;
      const float p = expf(sc[jj] - m_new);
      l_run += p;
      const T* vr = j < L ? Vp + (static_cast<size_t>(j) * Hkv + g) * d
                          : Vb + ((static_cast<size_t>(b) * B + (j - L)) * Hkv + g) * d;
      for (int u = 0; u < nu; ++u) {
        const int e = lane + 64 * u;
        if (e < d) o[u] = fmaf(p, Act<T>::load(vr, e), o[u]);
      }
    }
    m_run = m_new;
    __syncthreads();
  }
  const float inv = 1.f / l_run;
  const size_t hoff = (static_cast<size_t>(bi) * Hq + h) * d;
  for (int u = 0; u < nu; ++u) {
    const int e = lane + 64 * u;
    if (e < d) Act<T>::store(H, hoff + e, o[u] * inv);
  }
}

}  // namespace lopa

extern "C" int lopa_branch_attn(const lopa_dims* dims, const void* Kp, const void* Vp,
                                const void* Qb, const void* Kb, const void* Vb,
                                const int32_t* nb, void* H, void* ws, size_t ws_bytes,
                                hipStream_t stream) {
  using namespace lopa;
  int st = lopa_check_dims(dims);
  if (st != LOPA_OK) return st;
  if ((dims->L > 0 && (!Kp || !Vp)) || !Qb || !Kb || !Vb || !nb || !H) return LOPA_ERR_INVALID;
  const AttnPlan p = attn_plan(*dims);
  const size_t need = attn_workspace_bytes(*dims);
  if (need > 0 && (!ws || ws_bytes < need)) return LOPA_ERR_WORKSPACE;
  const int nb_max = dims->k_max + 1;
  if (p.mfma) {
    const dim3 grid(p.row_groups, dims->Hkv, p.splits);
    hipLaunchKernelGGL(k_attn_mfma, grid, dim3(256), 0, stream, dims->L, dims->B, dims->Hq,
                       dims->Hkv, nb_max, p.splits, nb, static_cast<const unsigned short*>(Kp),
                       static_cast<const unsigned short*>(Vp),
                       static_cast<const unsigned short*>(Qb),
                       static_cast<const unsigned short*>(Kb),
                       static_cast<const unsigned short*>(Vb), static_cast<unsigned short*>(H),
                       static_cast<float*>(ws));
    LOPA_LAUNCH_CHECK();
    if (p.splits > 1) {
      const int rows = nb_max * dims->B * (dims->Hq / dims->Hkv);
      hipLaunchKernelGGL(k_attn_combine, dim3((rows + 3) / 4, dims->Hkv), dim3(256), 0, stream,
                         dims->B, dims->Hq, dims->Hkv, nb_max, p.splits, nb,
                         static_cast<const float*>(ws), static_cast<unsigned short*>(H));
      LOPA_LAUNCH_CHECK();
    }
    return LOPA_OK;
  }
  const dim3 grid(nb_max * dims->B * dims->Hq);
  if (dims->dtype == LOPA_F32) {
    hipLaunchKernelGGL(k_attn_plain<float>, grid, dim3(64), 0, stream, dims->L, dims->B,
                       dims->Hq, dims->Hkv, dims->d, nb_max, nb, static_cast<const float*>(Kp),
                       static_cast<const float*>(Vp), static_cast<const float*>(Qb),
                       static_cast<const float*>(Kb), static_cast<const float*>(Vb),
                       static_cast<float*>(H));
  } else {
    hipLaunchKernelGGL(k_attn_plain<unsigned short>, grid, dim3(64), 0, stream, dims->L,
                       dims->B, dims->Hq, dims->Hkv, dims->d, nb_max, nb,
                       static_cast<const unsigned short*>(Kp),
                       static_cast<const unsigned short*>(Vp),
                       static_cast<const unsigned short*>(Qb),
                       static_cast<const unsigned short*>(Kb),
                       static_cast<const unsigned short*>(Vb), static_cast<unsigned short*>(H));
  }
  LOPA_LAUNCH_CHECK();
  return LOPA_OK;
}
