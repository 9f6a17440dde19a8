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
#include "lopa_common.hpp"

namespace lopa {

// ---------------------------------------------------------------------------
// MFMA path
// ---------------------------------------------------------------------------

constexpr int kAD = 128;          // head dim
constexpr int kAKB = 64;          // keys per LDS block
constexpr int kAKRow = kAD + 8;   // K row in LDS (bf16), 272 B: conflict-free 16-B reads
constexpr int kAVRow = kAKB + 4;  // V^T row in LDS (bf16), 136 B

__global__ void __launch_bounds__(256)
k_attn_mfma(int L, int B, int Hq, int Hkv, int nb_max, const int32_t* __restrict__ nb_ptr,
            const unsigned short* __restrict__ Kp, const unsigned short* __restrict__ Vp,
            const unsigned short* __restrict__ Qb, const unsigned short* __restrict__ Kb,
            const unsigned short* __restrict__ Vb, unsigned short* __restrict__ H) {
  __shared__ __attribute__((aligned(16))) unsigned short Ks[kAKB * kAKRow];
  __shared__ __attribute__((aligned(16))) unsigned short Vt[kAD * kAVRow];

  const int G = Hq / Hkv;
  const int g = blockIdx.y;
  const int RB = B * G;                 // query rows per branch for this KV head
  const int nb = min(max(*nb_ptr, 0), nb_max);
  const int R = nb * RB;
  const int r0 = blockIdx.x * 64;
  if (r0 >= R) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int ln = lane & 15;
  const int lg = lane >> 4;
  const int rw = r0 + 16 * w;
  const bool active = rw < R;
  const int bw = active ? rw / RB : -1;

  // this lane's query row (as the MFMA N index): rw + ln
  int qoff = 0;   // element offset of the row in Qb / H
  if (active) {
    const int rem = rw + ln - bw * RB;
    const int i = rem / G;
    const int h = g * G + rem % G;
    qoff = ((bw * B + i) * Hq + h) * kAD;
  }
  u16x8 qf[4];
#pragma unroll
  for (int s = 0; s < 4; ++s)
    qf[s] = active ? *reinterpret_cast<const u16x8*>(Qb + qoff + 32 * s + 8 * lg)
                   : u16x8{0, 0, 0, 0, 0, 0, 0, 0};

  const float scale2 = kLog2e * 0.08838834764831845f;   // log2(e) / sqrt(128)
  float m_run = -INFINITY;
  float l_run = 0.f;
  f32x4 o[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) o[u] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Stage kn (<= 64) keys of KV head g into LDS: K row-major, V transposed.
  // src points at key 0, head 0; consecutive keys are Hkv*128 elements apart.
  auto stage = [&](const unsigned short* ksrc, const unsigned short* vsrc, int kn) {
    const int seg = tid & 15;
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
      const int key = (tid >> 4) + 16 * pass;
      u16x8 kv = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
      u16x8 vv = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
      if (key < kn) {
        const size_t off = (static_cast<size_t>(key) * Hkv + g) * kAD + seg * 8;
        kv = *reinterpret_cast<const u16x8*>(ksrc + off);
        vv = *reinterpret_cast<const u16x8*>(vsrc + off);
      }
      *reinterpret_cast<u16x8*>(Ks + key * kAKRow + seg * 8) = kv;
#pragma unroll
      for (int e = 0; e < 8; ++e) Vt[(seg * 8 + e) * kAVRow + key] = vv[e];
    }
  };

  auto process = [&](int kn) {
    f32x4 st[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      st[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const u16x8 kf = *reinterpret_cast<const u16x8*>(Ks + (16 * t + ln) * kAKRow + 32 * s + 8 * lg);
        st[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kf),
                                                         __builtin_bit_cast(bf16x8, qf[s]), st[t],
                                                         0, 0, 0);
      }
    }
    // st[t][q] = q_row(ln) . k(16t + 4lg + q)
    float bmax = -INFINITY;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int key = 16 * t + 4 * lg + q;
        st[t][q] = key < kn ? st[t][q] * scale2 : -INFINITY;
        bmax = fmaxf(bmax, st[t][q]);
      }
    bmax = fmaxf(bmax, __shfl_xor(bmax, 16, kWave));
    bmax = fmaxf(bmax, __shfl_xor(bmax, 32, kWave));
    const float m_new = fmaxf(m_run, bmax);
    const float alpha = exp2f(m_run - m_new);
    l_run *= alpha;
#pragma unroll
    for (int u = 0; u < 8; ++u) o[u] *= alpha;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        st[t][q] = exp2f(st[t][q] - m_new);
        l_run += st[t][q];
      }
    m_run = m_new;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      // MFMA K index 8*lg + j  <->  key 32*s2 + 16*(j >= 4) + 4*lg + (j & 3)
      bf16x8 phi, plo;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float pv = st[2 * s2 + (j >> 2)][j & 3];
        const bf16 hi = static_cast<bf16>(pv);
        phi[j] = hi;
        plo[j] = static_cast<bf16>(pv - static_cast<float>(hi));
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const unsigned short* vr = Vt + (16 * u + ln) * kAVRow + 32 * s2 + 4 * lg;
        const uint2 lo4 = *reinterpret_cast<const uint2*>(vr);
        const uint2 hi4 = *reinterpret_cast<const uint2*>(vr + 16);
        const uint4 packed = make_uint4(lo4.x, lo4.y, hi4.x, hi4.y);
        const bf16x8 vf = __builtin_bit_cast(bf16x8, packed);
        o[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, phi, o[u], 0, 0, 0);
        o[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, plo, o[u], 0, 0, 0);
      }
    }
  };

  // Phase 1: the committed prefix, shared by every row of the workgroup.
  for (int j0 = 0; j0 < L; j0 += kAKB) {
    const int kn = min(kAKB, L - j0);
    const size_t off = static_cast<size_t>(j0) * Hkv * kAD;
    stage(Kp + off, Vp + off, kn);
    __syncthreads();
    if (active) process(kn);
    __syncthreads();
  }
  // Phase 2: each branch's own block, visible to that branch's rows only.
  const int b_lo = r0 / RB;
  const int b_hi = (min(r0 + 63, R - 1)) / RB;
  for (int bb = b_lo; bb <= b_hi; ++bb) {
    for (int j0 = 0; j0 < B; j0 += kAKB) {
      const int kn = min(kAKB, B - j0);
      const size_t off = (static_cast<size_t>(bb) * B + j0) * Hkv * kAD;
      stage(Kb + off, Vb + off, kn);
      __syncthreads();
      if (active && bw == bb) process(kn);
      __syncthreads();
    }
  }

  if (active) {
    float l_tot = l_run + __shfl_xor(l_run, 16, kWave);
    l_tot += __shfl_xor(l_tot, 32, kWave);
    const float inv = 1.f / l_tot;
    // o[u][q] = O[row ln][dim 16u + 4lg + q]
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const unsigned a = f32_to_bf16_bits(o[u][0] * inv) | (static_cast<unsigned>(f32_to_bf16_bits(o[u][1] * inv)) << 16);
      const unsigned b = f32_to_bf16_bits(o[u][2] * inv) | (static_cast<unsigned>(f32_to_bf16_bits(o[u][3] * inv)) << 16);
      *reinterpret_cast<uint2*>(H + qoff + 16 * u + 4 * lg) = make_uint2(a, b);
    }
  }
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
                                const int32_t* nb, void* H, hipStream_t stream) {
  using namespace lopa;
  int st = lopa_check_dims(dims);
  if (st != LOPA_OK) return st;
  if ((dims->L > 0 && (!Kp || !Vp)) || !Qb || !Kb || !Vb || !nb || !H) return LOPA_ERR_INVALID;
  const int nb_max = dims->k_max + 1;
  const int G = dims->Hq / dims->Hkv;
  const bool mfma = dims->dtype == LOPA_BF16 && dims->d == kAD && (dims->B * G) % 16 == 0;
  if (mfma) {
    const int rows = nb_max * dims->B * G;
    const dim3 grid((rows + 63) / 64, dims->Hkv);
    hipLaunchKernelGGL(k_attn_mfma, grid, dim3(256), 0, stream, dims->L, dims->B, dims->Hq,
                       dims->Hkv, nb_max, nb, static_cast<const unsigned short*>(Kp),
                       static_cast<const unsigned short*>(Vp),
                       static_cast<const unsigned short*>(Qb),
                       static_cast<const unsigned short*>(Kb),
                       static_cast<const unsigned short*>(Vb), static_cast<unsigned short*>(H));
  } else {
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
                         static_cast<const unsigned short*>(Vb),
                         static_cast<unsigned short*>(H));
    }
  }
  LOPA_LAUNCH_CHECK();
  return LOPA_OK;
}
