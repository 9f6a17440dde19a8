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
//   k_attn_dma    bf16, d = 128.  A workgroup takes 64 query rows of one KV
//                 head -- rows are (branch, position, q-head of the group), so
//                 they span several positions and at most a few branches --
//                 and walks 64-key work units: the committed prefix, then the
//                 own block of each branch its rows belong to.  Four producer
//                 waves move K and V rows into a three-stage LDS ring with
//                 buffer-to-LDS loads; four compute waves take 32 rows and
//                 one 32-key half of every unit each, and the two halves of
//                 a row tile are merged through LDS at the end:
//                 S^T = K Q^T and O^T = V^T P^T as v_mfma_f32_32x32x16_bf16
//                 (V^T through transposing LDS reads), online softmax in
//                 float32, P entering PV as a bf16 hi + lo pair so the
//                 probabilities keep ~16 significant bits.  Units may be split
//                 over workgroups; k_attn_combine merges the splits.
//   k_attn_wide   bf16, d = 128, prefixes of 4096 keys and more.  128 query
//                 rows per workgroup and eight compute waves (two per SIMD)
//                 that issue the buffer-to-LDS loads themselves into a
//                 four-stage ring; each wave pipelines its units into matrix
//                 phases (scores of the next unit, P V of this one) and
//                 vector phases (softmax), and the two waves of a SIMD run one
//                 phase apart.
//   k_attn_plain  any dtype / d <= 256: one wave per query row, keys in
//                 chunks of 1024 with online softmax, float32 throughout.
#include <type_traits>

#include "lopa_common.hpp"
#include "attn_plan.hpp"

namespace lopa {

// ---------------------------------------------------------------------------
// MFMA path
// ---------------------------------------------------------------------------

constexpr int kAD = 128;          // head dim
constexpr int kARows = 64;        // query rows per workgroup (2 row tiles x 2 key halves)
// ---------------------------------------------------------------------------
// MFMA path with buffer-to-LDS staging
// ---------------------------------------------------------------------------

constexpr int kAUnitKeys = 64;                 // keys per work unit
constexpr int kARowBytes = kAD * 2;            // one key row of K or V in LDS: 256 B
constexpr int kAHalf = kAUnitKeys * kARowBytes;  // K (or V) part of a stage: 16 KB
constexpr int kAStages = 3;
constexpr int kADmaPerUnit = 8;                // 16-byte LDS loads per producer wave per unit

// XOR of the 16-byte slot of key row r in LDS: conflict-free for the K
// fragment reads (16 rows, one slot) and the transposed V reads (4 rows x 32 B).
__device__ __forceinline__ int aswz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// Key row read by MFMA row i of a 32-key S^T tile: with this order the 16
// scores lane (j, h) holds are keys 16(r/8) + 8h + r%8, r = 0..15 -- the two
// 8-key slices of P^T that lane feeds to the two 16-key PV steps of the tile.
__device__ __forceinline__ int kperm(int i) {
  const int a = i >> 3, h = (i >> 2) & 1, c = i & 3;
  return ((a >> 1) << 4) | (h << 3) | ((a & 1) << 2) | c;
}

template <int N>
__device__ __forceinline__ void attn_wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

#define LOPA_LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

// One workgroup: 64 query rows (branch, position, q-head of the group) of
// KV head g, and the work units [u_lo, u_hi) of its split -- units are the
// 64-key blocks of the committed prefix followed by the own blocks of every
// branch its rows belong to (a row only scores its own branch's block).
// Waves 4..7 move K and V rows of a unit straight into an XOR-swizzled
// three-stage LDS ring with buffer-to-LDS loads; wave w < 4 owns 32 query
// rows (w & 1) and 32 keys of every unit (w >> 1): S^T = K Q^T and
// O^T = V^T P^T as v_mfma_f32_32x32x16_bf16, K fragments read in the kperm
// order, V^T fragments with transposing LDS reads, online softmax in
// float32, P entering PV as a bf16 hi + lo pair; the two key halves of a
// row tile keep separate softmax states, merged through LDS at the end.
__global__ void __launch_bounds__(512)
k_attn_dma(int L, int B, int Hq, int Hkv, int nb_max, int splits,
           const int32_t* __restrict__ nb_ptr, const unsigned short* __restrict__ Kp,
           const unsigned short* __restrict__ Vp, const unsigned short* __restrict__ Qb,
           const unsigned short* __restrict__ Kb, const unsigned short* __restrict__ Vb,
           unsigned short* __restrict__ H, float* __restrict__ part) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kAStages * 2 * kAHalf];
  const int G = Hq / Hkv;
  const int g = blockIdx.y;
  const int split = blockIdx.z;
  const int RB = B * G;
  const int nb = __builtin_amdgcn_readfirstlane(min(max(*nb_ptr, 0), nb_max));
  const int R = nb * RB;
  const int r0 = blockIdx.x * kARows;
  if (r0 >= R) return;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;

  // work units of this workgroup
  const int nbp = (L + kAUnitKeys - 1) / kAUnitKeys;
  const int obp = (B + kAUnitKeys - 1) / kAUnitKeys;
  const int b_lo = r0 / RB;
  const int b_hi = (min(r0 + kARows, R) - 1) / RB;
  const int units = nbp + (b_hi - b_lo + 1) * obp;
  const int u_lo = static_cast<int>(static_cast<long long>(split) * units / splits);
  const int u_hi = static_cast<int>(static_cast<long long>(split + 1) * units / splits);
  const int n = u_hi - u_lo;

  if (w >= 4) {
    // ---------------- producer waves ----------------
    const int pw = w - 4;
    const int kq = lane >> 4;                    // key within a 4-key load
    const int ps = lane & 15;                    // physical 16-byte slot
    const __amdgpu_buffer_rsrc_t kpr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<unsigned short*>(Kp), 0, L * Hkv * kARowBytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t vpr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<unsigned short*>(Vp), 0, L * Hkv * kARowBytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t kbr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<unsigned short*>(Kb), 0, nb_max * B * Hkv * kARowBytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t vbr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<unsigned short*>(Vb), 0, nb_max * B * Hkv * kARowBytes, 0x00020000);
    // unit number i of this workgroup -> stage i % kAStages; past the end the
    // last unit is loaded again into the free stage so every iteration issues
    // the same number of loads
    auto issue = [&](int i) __attribute__((always_inline)) {
      unsigned char* st = smem + (i % kAStages) * 2 * kAHalf;
      const int u = u_lo + min(i, n - 1);
      const bool own = u >= nbp;
      const int v = u - nbp;
      const int kn = own ? min(kAUnitKeys, B - (v % obp) * kAUnitKeys)
                         : min(kAUnitKeys, L - u * kAUnitKeys);
      const int key0 = own ? (b_lo + v / obp) * B + (v % obp) * kAUnitKeys : u * kAUnitKeys;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int kr = 4 * (pw + 4 * p) + kq;    // key row of the unit
        const int key = key0 + min(kr, kn - 1);
        const int off = ((key * Hkv + g) * kAD + ((ps ^ aswz(kr)) << 3)) * 2;
        unsigned char* dk = st + (pw + 4 * p) * 1024;
        if (own) {
          __builtin_amdgcn_raw_ptr_buffer_load_lds(kbr, LOPA_LDS_PTR(dk), 16, off, 0, 0, 0);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(vbr, LOPA_LDS_PTR(dk + kAHalf), 16, off, 0, 0, 0);
        } else {
          __builtin_amdgcn_raw_ptr_buffer_load_lds(kpr, LOPA_LDS_PTR(dk), 16, off, 0, 0, 0);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(vpr, LOPA_LDS_PTR(dk + kAHalf), 16, off, 0, 0, 0);
        }
      }
    };
    if (n > 0) {
#pragma unroll
      for (int u = 0; u < kAStages - 1; ++u) issue(u);
      attn_wait_vmcnt<(kAStages - 2) * kADmaPerUnit>();
      __builtin_amdgcn_s_barrier();
      for (int i = 0; i + 1 < n; ++i) {
        issue(i + kAStages - 1);
        attn_wait_vmcnt<(kAStages - 2) * kADmaPerUnit>();
        __builtin_amdgcn_s_barrier();
      }
    }
    attn_wait_vmcnt<0>();   // no load may still target LDS when the ring is reused
    // the two barriers of the key-half merge below
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_s_barrier();
    return;
  }

  // ---------------- compute waves ----------------
  // wave w: row tile rt = w & 1 (32 query rows), key half kh = w >> 1 (keys
  // 32 kh .. 32 kh + 31 of every unit); the two halves of a row tile keep
  // their own online softmax and are merged through LDS at the end
  const int rt = w & 1, kh = w >> 1;
  const int ln = lane & 31;     // this lane's query row within the wave's 32
  const int lh = lane >> 5;
  const int grow = r0 + 32 * rt + ln;
  const bool row_ok = grow < R;
  const int row = min(grow, R - 1);
  const int rbr = row / RB;                    // branch of the row
  const int rem = row - rbr * RB;
  const int qoff = ((rbr * B + rem / G) * Hq + g * G + rem % G) * kAD;
  // Q^T as the B operand: lane (j, h) holds Q[row j][16s + 8h .. +8]
  u16x8 qf[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) qf[s] = *reinterpret_cast<const u16x8*>(Qb + qoff + 16 * s + 8 * lh);

  const float scale2 = kLog2e * 0.08838834764831845f;   // log2(e) / sqrt(128)
  float m_ref = -INFINITY;   // exponent reference of the row, log2 units
  float l_run = 0.f;
  f32x16 o[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) o[u] = f32x16{};

  // transposed V reads: lane (q = lane/16, i = lane%16) supplies the address of
  // key k0 + i/4, dims n0 + 4(i%4) .. +4 and receives 4 keys of dim n0 + i
  const int tq = lane >> 4, ti = lane & 15;
  const int vkey = 8 * (tq >> 1) + (ti >> 2);          // + 16 t' + 4 hh
  const int vdim = 16 * (tq & 1) + 4 * (ti & 3);       // + 32 u
  for (int i = 0; i < n; ++i) {
    __syncthreads();
    const unsigned char* Ks = smem + (i % kAStages) * 2 * kAHalf;
    const unsigned char* Vs = Ks + kAHalf;
    const int u = u_lo + i;
    const bool own = u >= nbp;
    const int v = u - nbp;
    const int kn = own ? min(kAUnitKeys, B - (v % obp) * kAUnitKeys)
                       : min(kAUnitKeys, L - u * kAUnitKeys);
    // rows of another branch see nothing of this branch's own block
    const bool see = !own || rbr == b_lo + v / obp;
    // whether any score of this half needs masking (keys past kn, another
    // branch's block); decided before the MFMAs so that no branch sits
    // between them and the first use of their results
    const bool need_mask = __builtin_amdgcn_readfirstlane(kn) < 32 * kh + 32 ||
                           __builtin_amdgcn_ballot_w64(!see) != 0;
    // S^T = K Q^T over this wave's 32 keys: all 8 K fragments go out first,
    // and the K = 128 sum runs as two interleaved chains added at the end
    u16x8 kf[8];
    {
      const int kr = 32 * kh + kperm(ln);
      const unsigned char* kb = Ks + kr * kARowBytes;
      const int sw = aswz(kr);
#pragma unroll
      for (int s = 0; s < 8; ++s)
        kf[s] = *reinterpret_cast<const u16x8*>(kb + (((2 * s + lh) ^ sw) << 4));
    }
    f32x16 sa = f32x16{}, sb = f32x16{};
#pragma unroll
    for (int s = 0; s < 8; s += 2) {
      sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kf[s]),
                                                   __builtin_bit_cast(bf16x8, qf[s]), sa, 0, 0, 0);
      sb = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kf[s + 1]),
                                                   __builtin_bit_cast(bf16x8, qf[s + 1]), sb, 0, 0,
                                                   0);
    }
    const f32x16 sc = sa + sb;
    // V^T fragments of one 16-key PV step: [u2][half]
    auto vload = [&](int tp, bf16x4 (&va)[4][2]) __attribute__((always_inline)) {
#pragma unroll
      for (int u2 = 0; u2 < 4; ++u2)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int key = 16 * tp + 4 * hh + vkey;
          const int dim = 32 * u2 + vdim;
          const int byte = key * kARowBytes + (((dim >> 3) ^ aswz(key)) << 4) + ((dim & 7) << 1);
          va[u2][hh] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
              reinterpret_cast<__attribute__((address_space(3))) bf16x4*>(
                  reinterpret_cast<uintptr_t>(Vs + byte)));
        }
    };
    bf16x4 va[2][4][2];
    vload(2 * kh, va[0]);   // in flight during the softmax arithmetic
    // sc[r] = raw score of key 32kh + 16(r/8) + 8lh + r%8; keys past kn and
    // other branches' own blocks are masked (wave-uniform test first)
    float scm[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) scm[r] = sc[r];
    if (need_mask) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 32 * kh + 16 * (r >> 3) + 8 * lh + (r & 7);
        if (!(see && key < kn)) scm[r] = -INFINITY;
      }
    }
    float bmax = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) bmax = fmaxf(bmax, scm[r]);
    bmax = fmaxf(bmax, __shfl_xor(bmax, 32, kWave)) * scale2;
    // The exponent reference m_ref (log2 units) only moves when a row's block
    // maximum exceeds it by more than 8, so p <= 2^8 and the rescale of O and
    // l is skipped for most blocks; O / l is the same for any reference.
    const bool grow_ref = bmax > m_ref + 8.f;
    if (__builtin_amdgcn_ballot_w64(grow_ref)) {
      const float m_new = grow_ref ? bmax : m_ref;
      const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);   // 0 when m_ref = -inf
      m_ref = m_new;
      l_run *= alpha;
#pragma unroll
      for (int u2 = 0; u2 < 4; ++u2) o[u2] *= alpha;
    }
    // a row that has seen no key yet keeps m_ref = -inf and all p = 0
    const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
    // P^T operands of this half's two 16-key PV steps, as bf16 hi + lo
    bf16x8 phi[2], plo[2];
#pragma unroll
    for (int tp = 0; tp < 2; ++tp)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = __builtin_amdgcn_exp2f(fmaf(scm[8 * tp + e], scale2, -m_use));
        l_run += p;
        const bf16 hi = static_cast<bf16>(p);
        phi[tp][e] = hi;
        plo[tp][e] = static_cast<bf16>(p - static_cast<float>(hi));
      }
    // O^T += V^T P^T; the next step's V^T fragments are read during this one's MFMAs
#pragma unroll
    for (int tp = 0; tp < 2; ++tp) {
      if (tp < 1) vload(2 * kh + tp + 1, va[(tp + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u2 = 0; u2 < 4; ++u2) {
        const bf16x8 vf =
            __builtin_shufflevector(va[tp & 1][u2][0], va[tp & 1][u2][1], 0, 1, 2, 3, 4, 5, 6, 7);
        o[u2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, phi[tp], o[u2], 0, 0, 0);
        o[u2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, plo[tp], o[u2], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ---- merge of the two key halves of each row tile, through the ring ----
  // (the producers' last loads have landed before the first barrier)
  float* xo = reinterpret_cast<float*>(smem) + rt * (64 * 64);        // [j][lane]
  float* xm = reinterpret_cast<float*>(smem) + 2 * (64 * 64) + rt * 128;  // m, then l
  __syncthreads();
  if (kh == 1) {
#pragma unroll
    for (int u2 = 0; u2 < 4; ++u2)
#pragma unroll
      for (int r = 0; r < 16; ++r) xo[(16 * u2 + r) * 64 + lane] = o[u2][r];
    xm[lane] = m_ref;
    xm[64 + lane] = l_run;
  }
  __syncthreads();
  if (kh == 1) return;
  {
    const float m1 = xm[lane], l1 = xm[64 + lane];
    const float M = fmaxf(m_ref, m1);
    const float a0 = m_ref == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_ref - M);
    const float a1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - M);
#pragma unroll
    for (int u2 = 0; u2 < 4; ++u2)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[u2][r] = o[u2][r] * a0 + xo[(16 * u2 + r) * 64 + lane] * a1;
    l_run = l_run * a0 + l1 * a1;
    m_ref = M;
  }

  // ---- output: o[u][r] = O[row ln][dim 32u + 8(r/4) + 4lh + r%4] ----
  if (!row_ok) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32, kWave);
  if (splits == 1) {
    const float inv = 1.f / l_tot;
#pragma unroll
    for (int u2 = 0; u2 < 4; ++u2)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const unsigned lo = f32_to_bf16_bits(o[u2][4 * a] * inv) |
                            (static_cast<unsigned>(f32_to_bf16_bits(o[u2][4 * a + 1] * inv)) << 16);
        const unsigned hi = f32_to_bf16_bits(o[u2][4 * a + 2] * inv) |
                            (static_cast<unsigned>(f32_to_bf16_bits(o[u2][4 * a + 3] * inv)) << 16);
        *reinterpret_cast<uint2*>(H + qoff + 32 * u2 + 8 * a + 4 * lh) = make_uint2(lo, hi);
      }
  } else {
    // partial of row (g, grow): [split][Hkv][rows][128] O, then max, then sum
    const size_t rmax = static_cast<size_t>(nb_max) * RB;
    const size_t prow = (static_cast<size_t>(split) * Hkv + g) * rmax + grow;
    float* po = part + prow * kAD;
#pragma unroll
    for (int u2 = 0; u2 < 4; ++u2)
#pragma unroll
      for (int a = 0; a < 4; ++a)
        *reinterpret_cast<f32x4*>(po + 32 * u2 + 8 * a + 4 * lh) =
            f32x4{o[u2][4 * a], o[u2][4 * a + 1], o[u2][4 * a + 2], o[u2][4 * a + 3]};
    if (lh == 0) {
      float* pm = part + static_cast<size_t>(splits) * Hkv * rmax * kAD;
      pm[prow] = m_ref;
      pm[static_cast<size_t>(splits) * Hkv * rmax + prow] = l_tot;
    }
  }
}

// ---------------------------------------------------------------------------
// MFMA path, 128-row workgroups of eight compute waves (long prefixes)
// ---------------------------------------------------------------------------
//
// k_attn_wide: eight waves, all of them computing and each issuing an equal
// share of every unit's buffer-to-LDS loads into a four-stage ring.  Wave w
// owns 32 query rows (w & 3) and one 32-key half of every unit (w >> 2).
// Per unit and wave: S^T = K Q^T as one chain of 8 MFMAs, the probabilities
// split into a truncated bf16 high part and the bf16-rounded exact
// remainder, O^T += V^T P^T as 16 MFMAs.  Each wave pipelines its units into
// matrix phases (the next unit's scores and this unit's products) and vector
// phases (the next unit's softmax), and waves 4..7 run one phase behind
// waves 0..3 -- waves w and w + 4 share a SIMD, so while one issues MFMAs the
// other runs its softmax.  Measured against k_attn_dma (prefix 4096, 9
// branches of block 64, 28 q-heads over 4 KV heads): 73.7 against 84.8 us;
// the per-phase timing shows the matrix phase at about twice its MFMA time
// and the vector phase slowed about twofold by the other wave's MFMAs, so
// the two waves' work still overlaps only in part.

constexpr int kWRows = 128;
constexpr int kWThreads = 512;
constexpr int kWStages = 4;       // LDS ring depth (units of 32 KB)
constexpr int kWDmaPerUnit = 4;   // 16-byte LDS loads per wave per unit

// s_waitcnt vmcnt(VM) lgkmcnt(0)
template <int VM>
__device__ __forceinline__ void attn_wait_vm_lgkm0() {
  static_assert(VM >= 0 && VM < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4));
}

__device__ __forceinline__ void attn_raw_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__global__ void __launch_bounds__(kWThreads)
k_attn_wide(int L, int B, int Hq, int Hkv, int nb_max, int row_groups, int splits,
            const int32_t* __restrict__ nb_ptr, const unsigned short* __restrict__ Kp,
            const unsigned short* __restrict__ Vp, const unsigned short* __restrict__ Qb,
            const unsigned short* __restrict__ Kb, const unsigned short* __restrict__ Vb,
            unsigned short* __restrict__ H, float* __restrict__ part) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kWStages * 2 * kAHalf];
  // Consecutive workgroup ids go to consecutive XCDs (eight of them): id i
  // takes slot (i % 8) * (grid / 8) + i / 8 of the (KV head, split, row
  // group) order, so each XCD works through a contiguous stretch of it --
  // one or two KV heads, whose prefix its own L2 then serves.
  const int per = gridDim.x >> 3;
  const int slot = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (slot >= row_groups * splits * Hkv) return;
  const int rg = slot % row_groups;
  const int split = (slot / row_groups) % splits;
  const int g = slot / (row_groups * splits);
  const int G = Hq / Hkv;
  const int RB = B * G;
  const int nb = __builtin_amdgcn_readfirstlane(min(max(*nb_ptr, 0), nb_max));
  const int R = nb * RB;
  const int r0 = rg * kWRows;
  if (r0 >= R) return;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;

  const int nbp = (L + kAUnitKeys - 1) / kAUnitKeys;
  const int obp = (B + kAUnitKeys - 1) / kAUnitKeys;
  const int b_lo = r0 / RB;
  const int b_hi = (min(r0 + kWRows, R) - 1) / RB;
  const int units = nbp + (b_hi - b_lo + 1) * obp;
  const int u_lo = static_cast<int>(static_cast<long long>(split) * units / splits);
  const int u_hi = static_cast<int>(static_cast<long long>(split + 1) * units / splits);
  const int n = u_hi - u_lo;

  // ---- loads: wave w moves key rows 4(w + 8p) .. +3, p = 0, 1, of K and V ----
  const int kq = lane >> 4;
  const int ps = lane & 15;
  const __amdgpu_buffer_rsrc_t kpr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<unsigned short*>(Kp), 0, L * Hkv * kARowBytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t vpr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<unsigned short*>(Vp), 0, L * Hkv * kARowBytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t kbr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<unsigned short*>(Kb), 0, nb_max * B * Hkv * kARowBytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t vbr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<unsigned short*>(Vb), 0, nb_max * B * Hkv * kARowBytes, 0x00020000);
  // unit number i -> stage i % kWStages; past the end the last unit is loaded
  // again, so every iteration sees the same number of loads in flight
  auto issue = [&](int i) __attribute__((always_inline)) {
    unsigned char* st = smem + (i % kWStages) * 2 * kAHalf;
    const int u = u_lo + min(i, n - 1);
    const bool own = u >= nbp;
    const int v = u - nbp;
    const int kn = own ? min(kAUnitKeys, B - (v % obp) * kAUnitKeys)
                       : min(kAUnitKeys, L - u * kAUnitKeys);
    const int key0 = own ? (b_lo + v / obp) * B + (v % obp) * kAUnitKeys : u * kAUnitKeys;
    const __amdgpu_buffer_rsrc_t kr_ = own ? kbr : kpr;
    const __amdgpu_buffer_rsrc_t vr_ = own ? vbr : vpr;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int kr = 4 * (w + 8 * p) + kq;
      const int key = key0 + min(kr, kn - 1);
      const int off = ((key * Hkv + g) * kAD + ((ps ^ aswz(kr)) << 3)) * 2;
      unsigned char* dk = st + (w + 8 * p) * 1024;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kr_, LOPA_LDS_PTR(dk), 16, off, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vr_, LOPA_LDS_PTR(dk + kAHalf), 16, off, 0, 0, 0);
    }
  };

  // ---- the wave's rows: tile rt, keys 32 kh .. +31 of every unit ----
  const int rt = w & 3, kh = w >> 2;
  const int ln = lane & 31;
  const int lh = lane >> 5;
  const int grow = r0 + 32 * rt + ln;
  const int row = min(grow, R - 1);
  const int rbr = row / RB;
  const int rem = row - rbr * RB;
  const int qoff = ((rbr * B + rem / G) * Hq + g * G + rem % G) * kAD;
  u16x8 qf[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) qf[s] = *reinterpret_cast<const u16x8*>(Qb + qoff + 16 * s + 8 * lh);

  const float scale2 = kLog2e * 0.08838834764831845f;   // log2(e) / sqrt(128)
  float m_ref = -INFINITY;
  float l_run = 0.f;
  f32x16 o[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) o[u] = f32x16{};

  // transposed V reads: lane (q = lane/16, i = lane%16) supplies the address
  // of key 16 tp + 4 hh + 8(q/2) + i/4 of the wave's half, dims 32 u + 16(q%2)
  // + 4(i%4) .. +4.  The row swizzle aswz(key) has high bits i/4 (the same for
  // every read of a lane) and low bits that depend on hh only, so a read's
  // byte offset is vbase[hh] + ((64 u) ^ a64) + 4096 tp.
  const int tq = lane >> 4, ti = lane & 15;
  const int vkey = 8 * (tq >> 1) + (ti >> 2);
  const int vdim = 16 * (tq & 1) + 4 * (ti & 3);
  const int a64 = (ti >> 2) << 6;
  int vbase[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int key = 32 * kh + 4 * hh + vkey;
    vbase[hh] = key * kARowBytes + (((vdim >> 3) ^ (aswz(key) & 3)) << 4) + ((vdim & 7) << 1);
  }
  const int kr_s = 32 * kh + kperm(ln);
  const int sw_s = aswz(kr_s);

  // S^T = K Q^T of unit i over the wave's 32 keys: one chain of 8 MFMAs
  auto s_part = [&](int i) __attribute__((always_inline)) {
    const unsigned char* Ks = smem + (i % kWStages) * 2 * kAHalf;
    u16x8 kf[8];
#pragma unroll
    for (int s = 0; s < 8; ++s)
      kf[s] = *reinterpret_cast<const u16x8*>(Ks + kr_s * kARowBytes + (((2 * s + lh) ^ sw_s) << 4));
    f32x16 sc = f32x16{};
#pragma unroll
    for (int s = 0; s < 8; ++s)
      sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kf[s]),
                                                   __builtin_bit_cast(bf16x8, qf[s]), sc, 0, 0, 0);
    return sc;
  };
  // O^T += V^T P^T of unit i: 16 MFMAs, the same accumulator's two products
  // 4 apart; each 16-key step's V^T fragments are read just before it
  auto pv_part = [&](int i, const bf16x8 (&phi)[2], const bf16x8 (&plo)[2])
      __attribute__((always_inline)) {
    const unsigned char* Vs = smem + (i % kWStages) * 2 * kAHalf + kAHalf;
#pragma unroll
    for (int tp = 0; tp < 2; ++tp) {
      bf16x4 va[4][2];
#pragma unroll
      for (int u2 = 0; u2 < 4; ++u2)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int byte = vbase[hh] + ((64 * u2) ^ a64) + 16 * kARowBytes * tp;
          va[u2][hh] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
              reinterpret_cast<__attribute__((address_space(3))) bf16x4*>(
                  reinterpret_cast<uintptr_t>(Vs + byte)));
        }
#pragma unroll
      for (int hl = 0; hl < 2; ++hl)
#pragma unroll
        for (int u2 = 0; u2 < 4; ++u2) {
          const bf16x8 vf = __builtin_shufflevector(va[u2][0], va[u2][1], 0, 1, 2, 3, 4, 5, 6, 7);
          o[u2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, hl ? plo[tp] : phi[tp], o[u2], 0,
                                                          0, 0);
        }
    }
  };
  // P^T operands of scores sc under exponent reference m: the bf16 high part
  // (truncated) and the bf16-rounded exact remainder; returns their sum
  auto probs = [&](const float (&scm)[16], float m, bf16x8 (&phi)[2], bf16x8 (&plo)[2])
      __attribute__((always_inline)) {
    float lsum = 0.f;
#pragma unroll
    for (int tp = 0; tp < 2; ++tp) {
      u16x8 h;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = __builtin_amdgcn_exp2f(fmaf(scm[8 * tp + e], scale2, -m));
        lsum += p;
        const unsigned pb = __float_as_uint(p);
        h[e] = static_cast<unsigned short>(pb >> 16);
        plo[tp][e] = static_cast<bf16>(p - __uint_as_float(pb & 0xffff0000u));
      }
      phi[tp] = __builtin_bit_cast(bf16x8, h);
    }
    return lsum;
  };
  // block maximum of the scores (log2 units), both halves of the wave
  auto block_max = [&](const float (&scm)[16]) __attribute__((always_inline)) {
    float mx = scm[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, scm[r]);
    return fmaxf(mx, __shfl_xor(mx, 32, kWave)) * scale2;
  };
  // Softmax of unit i's scores sc into the P^T operands, with masking for
  // partial and own-block units; the exponent reference of a row moves only
  // when a block maximum exceeds it by more than 8 (log2 units), rescaling O
  // and l (O / l is the same for any reference), so p <= 2^8.
  auto soft = [&](int i, const f32x16& sc, bf16x8 (&phi)[2], bf16x8 (&plo)[2])
      __attribute__((always_inline)) {
    const int u = u_lo + i;
    float scm[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) scm[r] = sc[r];
    if (u >= L / kAUnitKeys) {   // not a full prefix unit
      const bool own = u >= nbp;
      const int v = u - nbp;
      const int kn = own ? min(kAUnitKeys, B - (v % obp) * kAUnitKeys)
                         : min(kAUnitKeys, L - u * kAUnitKeys);
      const bool see = !own || rbr == b_lo + v / obp;
      // sc[r] = raw score of key 32kh + 16(r/8) + 8lh + r%8
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 32 * kh + 16 * (r >> 3) + 8 * lh + (r & 7);
        if (!(see && key < kn)) scm[r] = -INFINITY;
      }
    }
    const float bmax = block_max(scm);
    const bool grow_ref = bmax > m_ref + 8.f;
    if (__builtin_amdgcn_ballot_w64(grow_ref)) {
      const float m_new = grow_ref ? bmax : m_ref;
      const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);   // 0 from -inf
      m_ref = m_new;
      l_run *= alpha;
#pragma unroll
      for (int u2 = 0; u2 < 4; ++u2) o[u2] *= alpha;
    }
    // a row that has seen no key yet keeps m_ref = -inf and all p = 0
    l_run += probs(scm, m_ref == -INFINITY ? 0.f : m_ref, phi, plo);
  };

  // Schedule.  A wave takes each unit u through S_u (scores), soft_u and
  // PV_u, pipelined into phases: M(-1) = S_0, V(-1) = soft_0, then
  // M(j) = {S_(j+1), PV_j} and V(j) = soft_(j+1) for j < n - 1, and last
  // M(n-1) = PV_(n-1): 2n + 1 phases of matrix (M) or vector (V) work.
  // Waves 0-3 run phase p in slot p, waves 4-7 in slot p + 1, and every slot
  // ends at a workgroup barrier: each SIMD holds one wave of each group, so
  // one wave's softmax runs while the other's MFMAs do.
  // Ring: unit v is loaded at the start of slot 2v - 4 (units 0, 1 before
  // slot 0) into stage v % 4, whose previous unit v - 4 was last read in slot
  // 2v - 5; unit u is first read in slot 2u, and at the end of slot 2u - 1
  // each wave waits for its loads of unit u (those of u + 1 may be in flight).
  f32x16 sc = f32x16{};
  bf16x8 phi[2], plo[2];
  // end of slot s: this wave's loads of unit (s + 1) / 2 have landed when s
  // is odd; then the workgroup barrier
  auto end_slot = [&](bool odd) __attribute__((always_inline)) {
    if (odd) attn_wait_vm_lgkm0<kWDmaPerUnit>();
    else attn_wait_vm_lgkm0<2 * kWDmaPerUnit>();
    attn_raw_barrier();
  };
  if (n > 0) {
    issue(0);
    issue(1);
    attn_wait_vm_lgkm0<kWDmaPerUnit>();
    attn_raw_barrier();
    if (w < 4) {
      // phase p in slot p; slot 2n + 1 idle
      issue(2);
      sc = s_part(0);                       // slot 0: S_0
      end_slot(false);
      for (int j = 0; j + 1 < n; ++j) {
        soft(j, sc, phi, plo);              // slot 2j + 1: soft_j
        end_slot(true);
        issue(j + 3);                       // slot 2j + 2: S_(j+1), PV_j
        sc = s_part(j + 1);
        pv_part(j, phi, plo);
        end_slot(false);
      }
      soft(n - 1, sc, phi, plo);            // slot 2n - 1
      end_slot(true);
      issue(n + 2);                         // slot 2n: PV_(n-1)
      pv_part(n - 1, phi, plo);
      end_slot(false);
    } else {
      // phase p in slot p + 1; slot 0 idle
      issue(2);
      end_slot(false);
      sc = s_part(0);                       // slot 1: S_0
      end_slot(true);
      for (int j = 0; j + 1 < n; ++j) {
        issue(j + 3);                       // slot 2j + 2: soft_j
        soft(j, sc, phi, plo);
        end_slot(false);
        sc = s_part(j + 1);                 // slot 2j + 3: S_(j+1), PV_j
        pv_part(j, phi, plo);
        end_slot(true);
      }
      issue(n + 2);                         // slot 2n: soft_(n-1)
      soft(n - 1, sc, phi, plo);
      end_slot(false);
      pv_part(n - 1, phi, plo);             // slot 2n + 1: PV_(n-1)
    }
  }
  attn_wait_vm_lgkm0<0>();   // no load may still target the ring
  attn_raw_barrier();

  // ---- merge of the two key halves of each row tile, through the ring ----
  float* xo = reinterpret_cast<float*>(smem) + rt * (64 * 64);             // [u2][r][lane]
  float* xm = reinterpret_cast<float*>(smem) + 4 * (64 * 64) + rt * 128;   // m, then l
  if (kh == 1) {
#pragma unroll
    for (int u2 = 0; u2 < 4; ++u2)
#pragma unroll
      for (int r = 0; r < 16; ++r) xo[(16 * u2 + r) * 64 + lane] = o[u2][r];
    xm[lane] = m_ref;
    xm[64 + lane] = l_run;
  }
  __syncthreads();
  if (kh == 1) return;
  {
    const float m1 = xm[lane], l1 = xm[64 + lane];
    const float M = fmaxf(m_ref, m1);
    const float a0 = m_ref == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_ref - M);
    const float a1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - M);
#pragma unroll
    for (int u2 = 0; u2 < 4; ++u2)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[u2][r] = o[u2][r] * a0 + xo[(16 * u2 + r) * 64 + lane] * a1;
    l_run = l_run * a0 + l1 * a1;
    m_ref = M;
  }

  // ---- output: o[u][r] = O[row][dim 32u + 8(r/4) + 4lh + r%4] ----
  if (grow >= R) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32, kWave);
  if (splits == 1) {
    const float inv = 1.f / l_tot;
#pragma unroll
    for (int u2 = 0; u2 < 4; ++u2)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const unsigned lo = f32_to_bf16_bits(o[u2][4 * a] * inv) |
                            (static_cast<unsigned>(f32_to_bf16_bits(o[u2][4 * a + 1] * inv)) << 16);
        const unsigned hi = f32_to_bf16_bits(o[u2][4 * a + 2] * inv) |
                            (static_cast<unsigned>(f32_to_bf16_bits(o[u2][4 * a + 3] * inv)) << 16);
        *reinterpret_cast<uint2*>(H + qoff + 32 * u2 + 8 * a + 4 * lh) = make_uint2(lo, hi);
      }
  } else {
    const size_t rmax = static_cast<size_t>(nb_max) * RB;
    const size_t prow = (static_cast<size_t>(split) * Hkv + g) * rmax + grow;
    float* po = part + prow * kAD;
#pragma unroll
    for (int u2 = 0; u2 < 4; ++u2)
#pragma unroll
      for (int a = 0; a < 4; ++a)
        *reinterpret_cast<f32x4*>(po + 32 * u2 + 8 * a + 4 * lh) =
            f32x4{o[u2][4 * a], o[u2][4 * a + 1], o[u2][4 * a + 2], o[u2][4 * a + 3]};
    if (lh == 0) {
      float* pm = part + static_cast<size_t>(splits) * Hkv * rmax * kAD;
      pm[prow] = m_ref;
      pm[static_cast<size_t>(splits) * Hkv * rmax + prow] = l_tot;
    }
  }
}

// Merge of the splits: O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s,
// rounded to bf16.  Half a wave per row (4 dims per lane, 16-byte loads),
// eight rows per workgroup; every split's loads are issued before any is
// used, so the merge costs one memory round trip.
template <int S>
__global__ void __launch_bounds__(256)
k_attn_combine(int B, int Hq, int Hkv, int nb_max, const int32_t* __restrict__ nb_ptr,
               const float* __restrict__ part, unsigned short* __restrict__ H) {
  constexpr int splits = S;
  const int G = Hq / Hkv;
  const int RB = B * G;
  const int nb = min(max(*nb_ptr, 0), nb_max);
  const int g = blockIdx.y;
  const int r = blockIdx.x * 8 + (threadIdx.x >> 5);
  if (r >= nb * RB) return;   // whole half-waves: a row's 32 lanes leave together
  const int l = threadIdx.x & 31;
  const int half = threadIdx.x & 32;   // lane offset of this row's half of the wave
  const size_t rmax = static_cast<size_t>(nb_max) * RB;
  const float* pm = part + static_cast<size_t>(splits) * Hkv * rmax * kAD;
  const float* pl = pm + static_cast<size_t>(splits) * Hkv * rmax;
  // lane s < splits of the half holds split s's (max, sum)
  const size_t lrow = (static_cast<size_t>(min(l, splits - 1)) * Hkv + g) * rmax + r;
  const float ms = l < splits ? pm[lrow] : -INFINITY;
  const float ls = l < splits ? pl[lrow] : 0.f;
  f32x4 ov[S];
#pragma unroll
  for (int s = 0; s < S; ++s)
    ov[s] = *reinterpret_cast<const f32x4*>(
        part + ((static_cast<size_t>(s) * Hkv + g) * rmax + r) * kAD + 4 * l);
  float M = ms;
#pragma unroll
  for (int o = 16; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, kWave));
  const float wgt = l < splits ? exp2f(ms - M) : 0.f;   // 0 for a split that saw no key
  float lsum = wgt * ls;
#pragma unroll
  for (int o = 16; o > 0; o >>= 1) lsum += __shfl_xor(lsum, o, kWave);
  f32x4 acc = f32x4{};
#pragma unroll
  for (int s = 0; s < S; ++s) acc += __shfl(wgt, half + s, kWave) * ov[s];
  const float inv = 1.f / lsum;
  const int b = r / RB, rem = r % RB;
  const size_t hoff = (static_cast<size_t>(b * B + rem / G) * Hq + g * G + rem % G) * kAD;
  const unsigned lo = f32_to_bf16_bits(acc[0] * inv) |
                      (static_cast<unsigned>(f32_to_bf16_bits(acc[1] * inv)) << 16);
  const unsigned hi = f32_to_bf16_bits(acc[2] * inv) |
                      (static_cast<unsigned>(f32_to_bf16_bits(acc[3] * inv)) << 16);
  *reinterpret_cast<uint2*>(H + hoff + 4 * l) = make_uint2(lo, hi);
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
    // the MFMA kernel addresses K/V through buffer descriptors with 32-bit
    // byte offsets
    if (static_cast<long long>(dims->L) * dims->Hkv * dims->d * 2 >= (1LL << 31))
      return LOPA_ERR_UNSUPPORTED;
    const auto* kp = static_cast<const unsigned short*>(Kp);
    const auto* vp = static_cast<const unsigned short*>(Vp);
    const auto* qb = static_cast<const unsigned short*>(Qb);
    const auto* kb = static_cast<const unsigned short*>(Kb);
    const auto* vb = static_cast<const unsigned short*>(Vb);
    if (p.wide) {
      const int wgs = p.row_groups * dims->Hkv * p.splits;
      hipLaunchKernelGGL(k_attn_wide, dim3((wgs + 7) / 8 * 8), dim3(kWThreads), 0, stream,
                         dims->L, dims->B, dims->Hq, dims->Hkv, nb_max, p.row_groups, p.splits,
                         nb, kp, vp, qb, kb, vb, static_cast<unsigned short*>(H),
                         static_cast<float*>(ws));
    } else {
      const dim3 grid(p.row_groups, dims->Hkv, p.splits);
      hipLaunchKernelGGL(k_attn_dma, grid, dim3(512), 0, stream, dims->L, dims->B, dims->Hq,
                         dims->Hkv, nb_max, p.splits, nb, kp, vp, qb, kb, vb,
                         static_cast<unsigned short*>(H), static_cast<float*>(ws));
    }
    LOPA_LAUNCH_CHECK();
    if (p.splits > 1) {
      const int rows = nb_max * dims->B * (dims->Hq / dims->Hkv);
      const dim3 cg((rows + 7) / 8, dims->Hkv);
      const float* pw = static_cast<const float*>(ws);
      unsigned short* Hw = static_cast<unsigned short*>(H);
      switch (p.splits) {
#define LOPA_COMBINE(S)                                                                      \
  case S:                                                                                    \
    hipLaunchKernelGGL(k_attn_combine<S>, cg, dim3(256), 0, stream, dims->B, dims->Hq,       \
                       dims->Hkv, nb_max, nb, pw, Hw);                                       \
    break;
        LOPA_COMBINE(2) LOPA_COMBINE(3) LOPA_COMBINE(4) LOPA_COMBINE(5) LOPA_COMBINE(6)
        LOPA_COMBINE(7) LOPA_COMBINE(8) LOPA_COMBINE(9) LOPA_COMBINE(10) LOPA_COMBINE(11)
        LOPA_COMBINE(12) LOPA_COMBINE(13) LOPA_COMBINE(14) LOPA_COMBINE(15) LOPA_COMBINE(16)
#undef LOPA_COMBINE
        default: return LOPA_ERR_UNSUPPORTED;
      }
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
