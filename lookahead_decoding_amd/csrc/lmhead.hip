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
// Two more modes ride the same pass: the entropy term sum exp(l - max)(l - max)
// (lopa_lmhead_conf_ent) and temperature sampling by Gumbel-max
// (lopa_lmhead_sample: partials over l / T plus the best perturbed score).
//   k_lmhead_mfma   bf16.  One persistent workgroup per compute unit owns a
//                   balanced contiguous vocabulary range and every LM-head
//                   row of its row group.  Four producer waves move 64-wide
//                   K chunks of W and H straight from HBM/L2 into a
//                   three-stage XOR-swizzled LDS ring with buffer loads that
//                   write LDS; eight compute waves (two per SIMD) read
//                   v_mfma_f32_32x32x16_bf16 fragments from it.  W is read
//                   from HBM exactly once.  The row count M lives on the
//                   device and picks the body and the row groups; the
//                   groups of one vocabulary range share the weight stream
//                   through L2.
//   k_lmhead_wide   bf16, 6 or more row tiles (the counts wide_takes()
//                   names): four waves that load and compute, register
//                   tiles of up to 13 row tiles, the weight through an LDS
//                   ring, the activation fragments straight into registers
//                   from an operand-ordered copy that the narrow kernel's
//                   launch makes first (it serves no rows then).
//   k_lmhead_f32    float32: v_mfma_f32_32x32x2_f32 tiles of 256 vocabulary
//                   entries x 32 rows, staged through LDS.
//   k_lmhead_plain  bf16 shapes outside the MFMA kernels (hidden not a
//                   multiple of 64): one thread per vocabulary entry, FMA
//                   dot products.
#include <mutex>
#include <type_traits>
#include <utility>

#include "lopa_common.hpp"
#include "head_plan.hpp"
#include "stream_tile.hpp"
#include "philox.hpp"

namespace lopa {

// ---------------------------------------------------------------------------
// MFMA kernel
// ---------------------------------------------------------------------------


// Calls f(integral_constant<int, i>) for i = 0 .. N-1.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// What the LM head folds per row: the confidence and argmax; also the
// entropy term; or, for temperature sampling, the scaled-logit softmax and a
// Gumbel-max sample.
constexpr int kModeConf = 0, kModeEnt = 1, kModeSample = 2;

// Temperature sampling: scaled logits z = l / T, Gumbel noise from Philox4x32-10
// with key (seed low, seed high) and counter (v / 4, block position, kSampleTag,
// 0), word v % 4 -> u = (2 (x >> 9) + 1) 2^-24 (exact, in (0, 1)),
// G = -ln(-ln u).  The sample is the argmax of z + G (Gumbel-max: a draw
// from softmax(z)); the noise depends on the position, not the branch, so
// branches holding the same logits at a position draw the same token.
constexpr unsigned kSampleTag = 0x5AB1Eu;
struct Sampling {
  float inv_t;
  unsigned k0, k1;
  int B;
};

// Both logarithms take the hardware log2 (times ln 2): u >= 2^-24 and
// -ln u >= 2^-24 are normal numbers, so no denormal scaling is needed, and
// the result stays within a few ulp of the library logf's.
constexpr float kLn2 = 0.6931471805599453f;
__device__ __forceinline__ float gumbel(unsigned x) {
  const float u = static_cast<float>(2u * (x >> 9) + 1u) * (1.f / 16777216.f);
  return -kLn2 * __builtin_amdgcn_logf(-kLn2 * __builtin_amdgcn_logf(u));
}

// Sampling partial of one lane's logits for one LM-head row at block
// position pos (layout as row_partial below), merged with the other lane
// half that holds the same row.
template <int NV, int VS = 32, int NL = NV>
__device__ __forceinline__ SPartial row_partial_sample(const f32x16 (&a)[NV], int vb, int h,
                                                       int vend, const Sampling& smp,
                                                       unsigned pos) {
  static_assert(NL <= NV, "tiles");
  SPartial p = empty_spartial();
#pragma unroll
  for (int n = 0; n < NL; ++n)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int v0 = vb + n * VS + 8 * q4 + 4 * h;   // a multiple of 4
      unsigned key0 = smp.k0, key1 = smp.k1;
      // the key schedule in vector registers: hoisted into scalar registers
      // for every call at once, it spills
      __asm__ volatile("" : "+v"(key0), "+v"(key1));
      const U32x4 w = philox4x32_10(
          U32x4{static_cast<unsigned>(v0) >> 2, pos, kSampleTag, 0u}, key0, key1);
      const unsigned xs[4] = {w.x0, w.x1, w.x2, w.x3};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int v = v0 + j;
        if (v < vend) {
          const float z = a[n][4 * q4 + j] * smp.inv_t;
          p.m = fmaxf(p.m, z);
          const float gv = z + gumbel(xs[j]);
          if (gv > p.g) {   // v ascends within the lane: the lowest v keeps a tie
            p.g = gv;
            p.i = v;
            p.z = z;
          }
        }
      }
    }
  if (p.i != 0x7fffffff) {
    float s = 0.f;
#pragma unroll
    for (int n = 0; n < NL; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int v = vb + n * VS + 8 * (r >> 2) + 4 * h + (r & 3);
        if (v < vend) s += exp2f((a[n][r] * smp.inv_t - p.m) * kLog2e);
      }
    p.s = s;
  }
  return merge(p, shfl_xor(p, 32));
}

// Online-softmax partial of one lane's logits for one LM-head row:
// a[n][r] = logit of vocabulary entry vb + VS n + 8(r/4) + 4h + r%4 (the
// 32x32 MFMA output layout, h = lane / 32; VS = 32 for adjacent weight
// tiles), merged with the other lane half that holds the same row.  ENT:
// also the entropy term t (else t = 0).
//
// Straight-line code: the max and its index move together by selects when
// an entry is strictly larger (the entries ascend in this order, so the
// lowest index keeps a tie).  MASKED: some entries may lie at or past vend
// and are skipped; without it (every pass but a part's last) there is no
// test at all.  exp2 is the hardware instruction: its argument
// (l - max) log2 e is <= 0, and a term below 2^-126, which the hardware
// flushes to zero, is far below half an ulp of a sum that holds the max's
// own term 1.
template <int NV, bool ENT, bool MASKED, int VS = 32, int NL = NV>
__device__ __forceinline__ Partial row_partial(const f32x16 (&a)[NV], int vb, int h, int vend) {
  static_assert(NL <= NV, "tiles");
  Partial p = empty_partial();
  const int v0 = vb + 4 * h;
#pragma unroll
  for (int n = 0; n < NL; ++n)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int v = v0 + n * VS + 8 * (r >> 2) + (r & 3);
      const bool c = MASKED ? (v < vend) & (a[n][r] > p.m) : a[n][r] > p.m;
      p.m = c ? a[n][r] : p.m;
      p.i = c ? v : p.i;
    }
  if (!MASKED || p.i != 0x7fffffff) {
    float s = 0.f, t = 0.f;
#pragma unroll
    for (int n = 0; n < NL; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float dl = a[n][r] - p.m;
        const float e = __builtin_amdgcn_exp2f(dl * kLog2e);
        if constexpr (MASKED) {
          const bool ok = v0 + n * VS + 8 * (r >> 2) + (r & 3) < vend;
          s += ok ? e : 0.f;
          if constexpr (ENT) t = ok ? fmaf(e, dl, t) : t;
        } else {
          s += e;
          if constexpr (ENT) t = fmaf(e, dl, t);
        }
      }
    p.s = s;
    p.t = t;
  }
  return merge(p, shfl_xor(p, 32));
}

constexpr int kRunRows = 512;    // running partials: compute-wave columns x rows
constexpr int kHeadThreads = kStreamThreads;
constexpr int kHeadStage = (256 + 128) * kRB;        // largest BUF of the bodies below
constexpr int kTailStages = 4;   // stages of a short last pass (half-width weight rows)
constexpr int kHeadSmem = kStages * kHeadStage + kRunRows * static_cast<int>(sizeof(SPartial));

// One persistent workgroup owns a contiguous, balanced vocabulary range
// (multiples of 16 rows) of its part and the Mg rows of its row group; it
// walks the range in passes of WROWS vocabulary rows, each pass the full
// hidden dimension in 64-wide K chunks.
//
// Warp-specialised, 768 threads.  Waves 8..11 only issue loads: each 128-byte
// row segment of a chunk is fetched by 8 lanes with 16-byte buffer loads
// that write straight into LDS (no registers on the way), 8 rows per
// instruction, in the XOR-swizzled order the fragment reads expect.  Three
// LDS stages: while the compute waves work on chunk i, chunks i+1 and i+2 are
// in flight; the producers issue chunk i+2 once the barrier that ends chunk
// i-1 shows its stage is free, and wait for chunk i+1 to land before the
// next barrier.  Waves 0..7 only compute, two per SIMD:
// v_mfma_f32_32x32x16_bf16 with the A operand from W and the B operand from
// H, fragments read from LDS.  After
// each pass a wave folds its logits into a running (max, sum, argmax) per
// row in LDS; at the end the wave columns are merged and one partial per row
// is written.  W is addressed through a buffer descriptor covering exactly
// the workgroup's range, so loads past it return zeros without touching
// memory.  Chunks are visited in an order rotated by the part, so the
// compute units of one XCD do not all ask for the same H lines at once.
template <int WX, int NVW, int MTW, int MODE>
__device__ __forceinline__ void head_body(int V, int hidden, int nparts, int part, int Mg,
                                          int row0, int h_bytes,
                                          const unsigned short* __restrict__ H,
                                          const unsigned short* __restrict__ W,
                                          const int32_t* __restrict__ rows, unsigned char* smem,
                                          float* __restrict__ ws_m, float* __restrict__ ws_s,
                                          int32_t* __restrict__ ws_i, float* __restrict__ ws_t,
                                          float* __restrict__ ws_z, const Sampling smp,
                                          float* __restrict__ logits_out) {
  constexpr bool ENT = MODE == kModeEnt;
  using RP = typename std::conditional<MODE == kModeSample, SPartial, Partial>::type;
  using T = StreamTile<WX, NVW, MTW>;
  constexpr int WROWS = T::WROWS, BUF = T::BUF, WP = T::WP, HP = T::HP;
  constexpr int RUNS = kRunRows / WX;   // running-partial stride per wave column
  static_assert(T::HROWS <= RUNS, "running partials");
  constexpr int KS = kKC / 16;   // MFMA K steps per chunk
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int row_bytes = hidden * 2;

  const int t16 = (V + 15) >> 4;
  const int v_lo = static_cast<int>(static_cast<long long>(part) * t16 / nparts) * 16;
  const int v_hi = min(static_cast<int>(static_cast<long long>(part + 1) * t16 / nparts) * 16, V);
  const int npass = (v_hi - v_lo + WROWS - 1) / WROWS;
  const int nch = hidden / kKC;
  const int rot = ((part >> 3) * nch / 32) % nch;
  // A last pass of at most WROWS / 2 vocabulary rows (82 of 256 at V = 152064
  // over 256 parts) runs as a second pipeline (the tail) whose kTailStages
  // stages hold only WROWS / 2 weight rows: with its few rows a chunk is
  // latency-bound, and the smaller stages keep one more chunk in flight.
  // Only the four-column layout has such a tail; its upper two columns idle.
  constexpr bool HAS_TAIL = WX == 4;
  constexpr int TROWS = WROWS / 2, TBUF = (TROWS + T::HROWS) * kRB, TWP = WP / 2;
  static_assert(!HAS_TAIL || kTailStages * TBUF <= kStages * BUF, "tail stages");
  const int rem = v_hi - v_lo - (npass - 1) * WROWS;   // rows of the last pass
  const bool tail = HAS_TAIL && npass > 0 && rem <= TROWS;
  const int total_a = (tail ? npass - 1 : npass) * nch;   // chunks of the full-width pipeline
  const int total_b = tail ? nch : 0;                     // chunks of the tail

  RP* run = reinterpret_cast<RP*>(smem + kStages * kHeadStage);
  for (int r = tid; r < kRunRows; r += kHeadThreads) {
    if constexpr (MODE == kModeSample) run[r] = empty_spartial();
    else run[r] = empty_partial();
  }
  __syncthreads();

  if (w >= kComputeWaves) {
    // ---------------- producer waves ----------------
    const int pw = w - kComputeWaves;
    const int r8 = lane >> 3;                    // row within an 8-row load
    const int ls = (lane & 7) ^ r8 ^ (pw & 1);   // logical slot landing in physical slot lane & 7
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<unsigned short*>(W) + static_cast<size_t>(v_lo) * hidden, 0,
        max(v_hi - v_lo, 0) * row_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t hr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned short*>(H), 0, h_bytes, 0x00020000);
    // load p of this wave covers rows 8 * (4p + pw) .. +8 of the chunk
    const int wv = (8 * pw + r8) * row_bytes + ls * 16;
    int hv[HP];
#pragma unroll
    for (int p = 0; p < HP; ++p)
      hv[p] = rows[row0 + min(8 * (4 * p + pw) + r8, Mg - 1)] * row_bytes + ls * 16;
    // One pipeline over chunks c0 .. c0 + cnt - 1: chunk c0 + i -> stage i % S
    // of BUFX bytes (WPX * 32 weight rows, then the activation rows); past the
    // end the last chunk is loaded again into the free stage so every
    // iteration issues the same count.  One barrier per chunk.
    auto pipeline = [&](auto s_c, auto wp_c, int c0, int cnt) __attribute__((always_inline)) {
      constexpr int S = decltype(s_c)::value, WPX = decltype(wp_c)::value;
      constexpr int BUFX = (WPX * 32 + T::HROWS) * kRB;
      auto issue = [&](int i) __attribute__((always_inline)) {
        unsigned char* dst = smem + (i % S) * BUFX;
        const int c = c0 + min(i, cnt - 1);
        const int pass = c / nch;
        int kc = c - pass * nch + rot;
        kc = kc >= nch ? kc - nch : kc;
        const int sw = pass * WROWS * row_bytes + kc * kRB;
#pragma unroll
        for (int p = 0; p < WPX; ++p)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, LOPA_LDS(dst + (4 * p + pw) * 1024), 16, wv,
                                                   sw + 32 * p * row_bytes, 0, kWeightAux);
#pragma unroll
        for (int p = 0; p < HP; ++p)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              hr, LOPA_LDS(dst + WPX * 32 * kRB + (4 * p + pw) * 1024), 16, hv[p], kc * kRB, 0, 0);
      };
#pragma unroll
      for (int u = 0; u < S - 1; ++u) issue(u);
      wait_vmcnt<(S - 2) * (WPX + HP)>();
      __builtin_amdgcn_s_barrier();
      for (int i = 0; i + 1 < cnt; ++i) {
        issue(i + S - 1);
        wait_vmcnt<(S - 2) * (WPX + HP)>();
        __builtin_amdgcn_s_barrier();
      }
      wait_vmcnt<0>();   // the next pipeline reuses the stages
    };
    if (total_a > 0)
      pipeline(std::integral_constant<int, kStages>{}, std::integral_constant<int, WP>{}, 0,
               total_a);
    if constexpr (HAS_TAIL) {
      if (total_b > 0) {
        // the compute waves leave the full-width stages before the tail's
        // first loads overwrite them
        if (total_a > 0) __builtin_amdgcn_s_barrier();
        pipeline(std::integral_constant<int, kTailStages>{}, std::integral_constant<int, TWP>{},
                 total_a, total_b);
      }
    }
    wait_vmcnt<0>();   // no load may still target LDS when the workgroup ends
  } else {
    // ---------------- compute waves ----------------
    // wave -> (vocabulary column, row group).  Wave w runs on SIMD w mod 4;
    // with four columns SIMD s holds columns s/2 and s/2 + 2, so the live
    // columns of a partial last pass are spread over all four SIMDs.
    const int wx = WX == 4 ? w >> 1 : w % WX;
    const int wy = WX == 4 ? w & 1 : w / WX;
    const int ln = lane & 31;     // MFMA row / column within a 32-tile
    const int lh = lane >> 5;     // which 8 of the 16 K values of a step
    f32x16 acc[MTW][NVW];
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
      for (int n = 0; n < NVW; ++n) acc[mt][n] = f32x16{};
    auto frags = [&](const unsigned char* base, const unsigned char* hb, int j, u16x8 (&wf)[NVW],
                     u16x8 (&hf)[MTW]) __attribute__((always_inline)) {
      const int s = j * 2 + lh;   // logical slot: K values 16j + 8lh .. +8
#pragma unroll
      for (int n = 0; n < NVW; ++n) {
        const int r = (wx * NVW + n) * 32 + ln;
        wf[n] = *reinterpret_cast<const u16x8*>(base + r * kRB + swz<kKC>(r, s) * 16);
      }
#pragma unroll
      for (int mt = 0; mt < MTW; ++mt) {
        const int r = (wy * MTW + mt) * 32 + ln;
        hf[mt] = *reinterpret_cast<const u16x8*>(hb + r * kRB + swz<kKC>(r, s) * 16);
      }
    };
    // base: the stage; hb: its activation rows (after the stage's weight rows)
    auto compute = [&](const unsigned char* base, const unsigned char* hb)
        __attribute__((always_inline)) {
      u16x8 wf[2][NVW], hf[2][MTW];
      frags(base, hb, 0, wf[0], hf[0]);
#pragma unroll
      for (int j = 0; j < KS; ++j) {
        if (j + 1 < KS) frags(base, hb, j + 1, wf[(j + 1) & 1], hf[(j + 1) & 1]);
#pragma unroll
        for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
          for (int n = 0; n < NVW; ++n)
            acc[mt][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, wf[j & 1][n]), __builtin_bit_cast(bf16x8, hf[j & 1][mt]),
                acc[mt][n], 0, 0, 0);
      }
    };
    // Fold the logits of one activation row tile -- tiles a[0 .. NV) of 32
    // vocabulary entries from vb on, row r -- into the running partial of
    // vocabulary column col, and clear the tiles.
    auto fold = [&](auto masked, auto& a, int vb, int col, int r) __attribute__((always_inline)) {
      constexpr int NV = static_cast<int>(sizeof(a) / sizeof(a[0]));
      constexpr bool MASKED = decltype(masked)::value;
      RP p;
      if constexpr (MODE == kModeSample) {
        const unsigned pos = static_cast<unsigned>(rows[row0 + min(r, Mg - 1)] % smp.B);
        p = row_partial_sample<NV>(a, vb, lh, v_hi, smp, pos);
      } else {
        p = row_partial<NV, ENT, MASKED>(a, vb, lh, v_hi);
      }
      if (lh == 0) {
        RP q = merge(run[col * RUNS + r], p);
        if constexpr (MODE == kModeConf) q.t = 0.f;   // keeps the entropy arithmetic out
        run[col * RUNS + r] = q;
      }
      if (logits_out && r < Mg) {
        const size_t lb = static_cast<size_t>(rows[row0 + r]) * V;
#pragma unroll
        for (int n = 0; n < NV; ++n)
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            const int v = vb + n * 32 + 8 * (q >> 2) + 4 * lh + (q & 3);
            if (v < v_hi) logits_out[lb + v] = a[n][q];
          }
      }
#pragma unroll
      for (int n = 0; n < NV; ++n) a[n] = f32x16{};
    };
    // acc[mt][n][q] = logit of row (wy*MTW + mt)*32 + ln, vocabulary entry
    // vbw + 32n + 8(q/4) + 4lh + q%4
    // A pass wholly inside the part folds without bound tests.
    auto finish_pass = [&](int pass) {
      const int vb = v_lo + pass * WROWS + wx * (32 * NVW);
      if (v_lo + (pass + 1) * WROWS <= v_hi) {
#pragma unroll
        for (int mt = 0; mt < MTW; ++mt)
          fold(std::false_type{}, acc[mt], vb, wx, (wy * MTW + mt) * 32 + ln);
      } else {
#pragma unroll
        for (int mt = 0; mt < MTW; ++mt)
          fold(std::true_type{}, acc[mt], vb, wx, (wy * MTW + mt) * 32 + ln);
      }
    };
    // One pass = nch chunks, then the fold.  The fold sits outside the
    // chunk loop so the loop body holds nothing but the MFMA step.
    for (int pass = 0, i = 0; pass * nch < total_a; ++pass) {
      // in a partial last pass a wave column whose vocabulary tiles all lie
      // past the range only keeps step (its logits would all be dropped).
      // Only the 4-column bodies have such columns; the 2-column ones run
      // unconditionally.
      const bool live = WX != 4 || v_lo + pass * WROWS + wx * (32 * NVW) < v_hi;
      for (int c = 0; c < nch; ++c, ++i) {
        __syncthreads();
        const unsigned char* base = smem + (i % kStages) * BUF;
        if (live) compute(base, base + WROWS * kRB);
      }
      finish_pass(pass);
    }
    if constexpr (HAS_TAIL) {
      if (total_b > 0) {
        if (total_a > 0) __syncthreads();   // done with the full-width stages
        // In the tail every wave takes one 32-row weight tile tw = w / 2
        // against the activation tiles of row group ty = w mod 2, so the
        // live tiles (rem <= 128 rows) are spread over all eight waves; the
        // accumulators acc[mt][0] hold them (acc[mt][1] stays zero).
        static_assert(NVW == 2 && T::WY == 2, "tail layout");
        const int tw = w >> 1, ty = w & 1;
        const bool live = tw * 32 < rem;
        const int wr = tw * 32 + ln;
        for (int i = 0; i < total_b; ++i) {
          __syncthreads();
          if (!live) continue;
          const unsigned char* base = smem + (i % kTailStages) * TBUF;
          const unsigned char* hb = base + TROWS * kRB;
          u16x8 wf[2], hf[2][MTW];
          auto tfrags = [&](int j, u16x8& wv, u16x8 (&hv)[MTW]) __attribute__((always_inline)) {
            const int sl = j * 2 + lh;
            wv = *reinterpret_cast<const u16x8*>(base + wr * kRB + swz<kKC>(wr, sl) * 16);
#pragma unroll
            for (int mt = 0; mt < MTW; ++mt) {
              const int r = (ty * MTW + mt) * 32 + ln;
              hv[mt] = *reinterpret_cast<const u16x8*>(hb + r * kRB + swz<kKC>(r, sl) * 16);
            }
          };
          tfrags(0, wf[0], hf[0]);
#pragma unroll
          for (int j = 0; j < KS; ++j) {
            if (j + 1 < KS) tfrags(j + 1, wf[(j + 1) & 1], hf[(j + 1) & 1]);
#pragma unroll
            for (int mt = 0; mt < MTW; ++mt)
              acc[mt][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                  __builtin_bit_cast(bf16x8, wf[j & 1]), __builtin_bit_cast(bf16x8, hf[j & 1][mt]),
                  acc[mt][0], 0, 0, 0);
          }
        }
#pragma unroll
        for (int mt = 0; mt < MTW; ++mt)
          fold(std::true_type{}, *reinterpret_cast<f32x16(*)[1]>(&acc[mt][0]),
               v_lo + (npass - 1) * WROWS + tw * 32, tw, (ty * MTW + mt) * 32 + ln);
      }
    }
  }
  __syncthreads();
  for (int r = tid; r < Mg; r += kHeadThreads) {
    RP p = run[r];
#pragma unroll
    for (int x = 1; x < WX; ++x) p = merge(p, run[x * RUNS + r]);
    const size_t o = static_cast<size_t>(row0 + r) * nparts + part;
    ws_m[o] = p.m;
    ws_s[o] = p.s;
    ws_i[o] = p.i;
    if constexpr (ENT) ws_t[o] = p.t;
    if constexpr (MODE == kModeSample) {
      ws_t[o] = p.g;
      ws_z[o] = p.z;
    }
  }
}

// The activation rows in MFMA operand order, for the wide kernel: fragment
// f = tile * (hidden / 16) + s holds, for lane l, the eight values
// 16 s + 8 (l / 32) .. +8 of listed row 32 tile + l % 32 (rows past the
// listed count repeat the last one), 16 bytes per lane, 1 KB per fragment.
// A wave of the wide kernel then loads its activation fragments straight into
// registers, each one 1 KB contiguous read from L2.  Wave `wave` of `waves`
// writes fragments wave, wave + waves, ...
__device__ __forceinline__ void operand_copy(int M, int hidden, int h_bytes,
                                             const unsigned short* __restrict__ H,
                                             const int32_t* __restrict__ rows,
                                             u32x4* __restrict__ Hf, int wave, int waves) {
  const int nks = hidden >> 4;
  const int nfrag = (M + 31) / 32 * nks;
  const int lane = threadIdx.x & 63;
  const __amdgpu_buffer_rsrc_t hr =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned short*>(H), 0, h_bytes, 0x00020000);
  for (int f = wave; f < nfrag; f += waves) {
    const int tile = f / nks;
    const int s = f - tile * nks;
    const int r = rows[min(tile * 32 + (lane & 31), M - 1)];
    Hf[static_cast<size_t>(f) * 64 + lane] =
        __builtin_amdgcn_raw_buffer_load_b128(hr, r * hidden * 2 + s * 32 + (lane >> 5) * 16, 0, 0);
  }
}

// kHeadParts workgroups of 768 threads, one per compute unit.  Block b sits
// on XCD b % 8; the row groups of one vocabulary part take consecutive
// blocks of the same XCD, so they stream the same weight lines together and
// the second reader is served from that XCD's L2 (or the MALL behind it).
// MODE: conf only, + entropy term, or temperature sampling (ws_t then
// holds the perturbed best score, ws_z the scaled logit of the sample).
// wide: the wide kernel is launched after this one and serves the row counts
// wide_takes() names; for those this launch only writes the wide kernel's
// operand-ordered copy of the rows (hf).
template <int MODE>
__global__ void __launch_bounds__(kHeadThreads)
k_lmhead_mfma(int V, int hidden, int nb_max, int m_max, int wide, int h_bytes,
              const unsigned short* __restrict__ H, const unsigned short* __restrict__ W,
              const int32_t* __restrict__ rows, const int32_t* __restrict__ row_ptr,
              const int32_t* __restrict__ nb_ptr, float* __restrict__ ws_m,
              float* __restrict__ ws_s, int32_t* __restrict__ ws_i, float* __restrict__ ws_t,
              float* __restrict__ ws_z, const Sampling smp, float* __restrict__ logits_out,
              u32x4* __restrict__ hf) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kHeadSmem];
  const int M = __builtin_amdgcn_readfirstlane(listed_rows(row_ptr, nb_ptr, nb_max, m_max));
  if (M <= 0) return;
  if (wide && wide_takes(M)) {
    operand_copy(M, hidden, h_bytes, H, rows, hf,
                 blockIdx.x * (kHeadThreads / 64) + (threadIdx.x >> 6),
                 gridDim.x * (kHeadThreads / 64));
    return;
  }
  const HeadGroups g = head_groups(M);
  const int b = blockIdx.x;
  const int q = b >> 3;
  const int group = q % g.groups;
  const int part = (q / g.groups) * 8 + (b & 7);
  const int row0 = group * g.tpg * 32;
  if (part >= g.nparts || row0 >= M) return;
  const int Mg = min(M - row0, g.tpg * 32);
#define LOPA_ARGS V, hidden, g.nparts, part, Mg, row0, h_bytes, H, W, rows, smem, ws_m, ws_s, ws_i, \
                  ws_t, ws_z, smp, logits_out
  // up to 4 tiles: 4 x 2 compute waves (256 vocabulary rows per pass);
  // 5..8 tiles: 2 x 4 compute waves (128 vocabulary rows per pass)
  if (!g.wide) {
    if (g.tpg <= 2) head_body<4, 2, 1, MODE>(LOPA_ARGS);
    else head_body<4, 2, 2, MODE>(LOPA_ARGS);
  } else {
    head_body<2, 2, 2, MODE>(LOPA_ARGS);
  }
#undef LOPA_ARGS
}

// ---------------------------------------------------------------------------
// Wide MFMA kernel (the row counts wide_takes() names)
// ---------------------------------------------------------------------------
//
// Four waves (one per SIMD, up to 512 registers each) hold large register
// tiles: wave w owns q activation tiles against all tw weight tiles of a
// pass (q tw MFMAs per 16-wide K step), plus its share of the r remaining
// activation tiles (their pairs with weight tiles w, w + 4, ...): at 13 tiles
// every wave runs 13 MFMAs per step.  The accumulators live in the matrix
// (AGPR) registers.  The weight streams through an LDS ring (4 to 7 stages,
// as many as the LDS and the vector-memory counter allow), every wave
// issuing its share of the buffer loads that write LDS; each weight fragment
// read from LDS feeds q MFMAs.  The activation rows do not pass through LDS:
// the narrow kernel's launch (which serves no rows then) first lays the
// listed rows out in MFMA operand order (one 1 KB block per 32-row tile and
// 16-wide K step), and each wave loads its own fragments from there straight
// into registers, one contiguous 1 KB read per fragment, four to seven K
// steps ahead in a ring of eight register sets.  Staging them through LDS as
// well (the layout before this one: two activation stages, each wave reading
// 9 fragments per 13 MFMAs) took 460-475 us per call at 13 tiles against
// 420-430 us here (same box).
//
// One barrier per K chunk, taken in the chunk's last K step after its first
// few MFMAs: by then this wave's weight reads of the chunk are done (they run
// one step ahead), and the step's remaining MFMAs carry the loads into the
// freed stage and the reads of the next chunk's first step.  With one wave
// per SIMD nothing else hides a wait, so each MFMA is followed by at most one
// fragment read and one load and the order is pinned with scheduling
// barriers (the compiler's own order put reads next to their MFMAs and
// waited on them).  The barrier waits for this wave's own loads of the next
// chunk (vmcnt) and its LDS reads (lgkmcnt), and neither it nor the compiler
// lets memory accesses move across it (a __syncthreads() would wait for
// every load in flight).
//
// What still bounds it (timing-only copies at 13 tiles, same box): the MFMAs
// with their reads, barriers and folds alone take about 268 us; with the
// weight stream but no activation loads 318 us; with both 420 us.  The
// vector-memory counter completes in issue order, so waiting for an
// activation fragment also waits for every older weight load: the weight's
// HBM latency is covered only by the activation loads' one-chunk lead.

// Entry r of a lane's 16 (the 32x32 MFMA output layout) lies at vocabulary
// vb + 4h + kTileOff(r).  The folds below compare these compile-time offsets
// against one per-lane limit and keep the winning entry's r, so no per-entry
// index is ever held in a register.
__device__ __forceinline__ constexpr int kTileOff(int r) { return 8 * (r >> 2) + (r & 3); }

// Online fold of one 32x32 output tile into a lane's running partial: the
// lane holds 16 logits of its row.  A lane folds its entries in ascending
// vocabulary order, so a strictly larger value is needed to move the argmax
// (the lowest index keeps a tie).  Only 16 values are live at a time.  The
// two lane halves of a row are merged once, after the last fold.
template <bool ENT, bool MASKED>
__device__ __forceinline__ void fold_tile(Partial& p, const f32x16& a, int vb, int h, int vend) {
  const int lim = vend - vb - 4 * h;   // entries with kTileOff(r) < lim are live
  float m = -INFINITY;
  int ri = -1;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const bool c = MASKED ? (kTileOff(r) < lim) & (a[r] > m) : a[r] > m;
    m = c ? a[r] : m;
    ri = c ? r : ri;
  }
  if (MASKED && ri < 0) return;   // no live entry in this tile
  const int i = vb + 4 * h + 8 * (ri >> 2) + (ri & 3);
  const bool take = m > p.m;
  const float M = take ? m : p.m;
  p.i = take ? i : p.i;
  // the running sums rescaled to the new maximum (none yet: s = 0)
  const float d = p.s > 0.f ? p.m - M : 0.f;
  const float cs = p.s > 0.f ? __builtin_amdgcn_exp2f(d * kLog2e) : 0.f;
  float s = 0.f, t = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const float dl = a[r] - M;
    const float e = __builtin_amdgcn_exp2f(dl * kLog2e);
    if constexpr (MASKED) {
      const bool ok = kTileOff(r) < lim;
      s += ok ? e : 0.f;
      if constexpr (ENT) t = ok ? fmaf(e, dl, t) : t;
    } else {
      s += e;
      if constexpr (ENT) t = fmaf(e, dl, t);
    }
  }
  if constexpr (ENT) p.t = fmaf(cs, fmaf(d, p.s, p.t), t);
  p.s = fmaf(cs, p.s, s);
  p.m = M;
}

// The same for temperature sampling: (max, sum) over z = l / T and the best
// perturbed score z + G with its index and z.  Noise of entry v: word v % 4
// of Philox4x32-10 at counter (v / 4, pos, kSampleTag, 0).
__device__ __forceinline__ void fold_tile_sample(SPartial& p, const f32x16& a, int vb, int h,
                                                 int vend, const Sampling& smp, unsigned pos) {
  const int lim = vend - vb - 4 * h;
  const unsigned q0 = static_cast<unsigned>(vb + 4 * h) >> 2;   // vb + 4h is a multiple of 4
  float m = -INFINITY;
  int ri = -1;
  float g = p.g, zb = 0.f;
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {
    unsigned key0 = smp.k0, key1 = smp.k1;
    __asm__ volatile("" : "+v"(key0), "+v"(key1));
    const U32x4 wd = philox4x32_10(U32x4{q0 + 2u * q4, pos, kSampleTag, 0u}, key0, key1);
    const unsigned xs[4] = {wd.x0, wd.x1, wd.x2, wd.x3};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 4 * q4 + j;
      const bool live = kTileOff(r) < lim;
      const float z = a[r] * smp.inv_t;
      m = live ? fmaxf(m, z) : m;
      const float gv = z + gumbel(xs[j]);
      const bool c = live & (gv > g);
      g = c ? gv : g;
      zb = c ? z : zb;
      ri = c ? r : ri;
    }
  }
  if (m == -INFINITY) return;
  if (ri >= 0) {
    p.g = g;
    p.z = zb;
    p.i = vb + 4 * h + 8 * (ri >> 2) + (ri & 3);
  }
  const float M = fmaxf(m, p.m);
  const float cs = p.s > 0.f ? __builtin_amdgcn_exp2f((p.m - M) * kLog2e) : 0.f;
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const float e = __builtin_amdgcn_exp2f((a[r] * smp.inv_t - M) * kLog2e);
    s += kTileOff(r) < lim ? e : 0.f;
  }
  p.s = fmaf(cs, p.s, s);
  p.m = M;
}

template <int MODE, bool MASKED, typename RP>
__device__ __forceinline__ void fold_tile_mode(RP& p, const f32x16& a, int vb, int h, int vend,
                                               const Sampling& smp, unsigned pos) {
  if constexpr (MODE == kModeSample) fold_tile_sample(p, a, vb, h, vend, smp, pos);
  else fold_tile<MODE == kModeEnt, MASKED>(p, a, vb, h, vend);
}

constexpr int kWideThreads = 256;
constexpr int kWideSmem = 128 * 1024;      // the weight ring
constexpr int kWideFoldSlot = 2048;        // bytes of LDS per wave for the fold's round trip

// Stages of the weight ring: as many as the LDS and the vector-memory
// counter allow (4..8).  A wave may have (S - 3) TW weight loads and
// (S - 2) NH activation loads in flight when it waits for a weight chunk
// (the loop's issue order), and the counter holds at most 63.
template <int TW, int NH>
constexpr int wide_stages() {
  int s = 8;
  while (s > 4 && ((s - 3) * TW + (s - 2) * NH > 63 || s * TW * 32 * kRB > kWideSmem)) --s;
  return s;
}

// s_waitcnt vmcnt(VM) lgkmcnt(0)
template <int VM>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(VM >= 0 && VM < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4));
}

__device__ __forceinline__ void raw_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Sequence position of the loads: load number i goes to stage i % S and
// fetches chunk min(i, total - 1) (past the end the last chunk again, so
// every barrier sees the same number of loads in flight).
template <int S>
struct LoadCursor {
  int i, stage, pass, kci;
  __device__ __forceinline__ void step(int total, int nch) {
    stage = stage + 1 == S ? 0 : stage + 1;
    if (i + 1 < total) {
      ++i;
      if (++kci == nch) {
        kci = 0;
        ++pass;
      }
    }
  }
};

// Bytes of the operand-ordered activation copy for m_max rows.
__host__ __device__ inline size_t hfrag_bytes(int m_max, int hidden) {
  return static_cast<size_t>((m_max + 31) / 32) * 32 * hidden * 2;
}

template <int TW, int Q, int R, int MODE>
__device__ __forceinline__ void wide_body(int V, int hidden, int nparts, int part, int Mg,
                                          int row0, int hf_bytes,
                                          const unsigned short* __restrict__ Hf,
                                          const unsigned short* __restrict__ W,
                                          const int32_t* __restrict__ rows, unsigned char* smem,
                                          float* __restrict__ ws_m, float* __restrict__ ws_s,
                                          int32_t* __restrict__ ws_i, float* __restrict__ ws_t,
                                          float* __restrict__ ws_z, const Sampling smp) {
  using RP = typename std::conditional<MODE == kModeSample, SPartial, Partial>::type;
  constexpr int TH = 4 * Q + R;          // activation tiles of the group
  constexpr int QR = Q + R;              // activation tiles this wave multiplies
  constexpr int WROWS = TW * 32;         // weight rows per pass
  constexpr int WBUF = WROWS * kRB;
  constexpr int XP = R > 0 ? TW / 4 : 0; // weight tiles per remaining activation tile per wave
  constexpr int XA = XP > 0 ? XP : 1;
  constexpr int KS = kKC / 16;           // MFMA K steps per chunk
  constexpr int NH = QR * KS;            // activation fragment loads per chunk
  constexpr int NR = TW + XP;            // weight fragment reads per K step
  constexpr int S = wide_stages<TW, NH>();
  // loads a wave may have in flight at a chunk's barrier: after the weight
  // chunk it waits for come the activation loads of S - 2 chunks and S - 3
  // weight chunks (the issue order of the loop below)
  constexpr int VM_BAR = (S - 3) * TW + (S - 2) * NH;
  // activation loads run LA K steps ahead, in a ring of eight register sets
  // (LA + 1 of them live: as many as keep the layout free of scratch spills)
  constexpr int LA = QR * 4 + NR * 2 <= 22 ? 7 : QR * 4 + NR * 2 <= 26 ? 5 : 4;
  static_assert(TW % 4 == 0 && Q >= 1 && R >= 0 && R < 4 && TH <= kWideMaxTiles, "wide layout");
  static_assert(S >= 4 && S * WBUF <= kWideSmem, "wide LDS");
  static_assert(VM_BAR < 64 && 2 * TW + LA * QR < 64, "vmcnt range");
  static_assert(LA >= 4 && LA <= 7, "activation ring");
  static_assert(R * 4 * 32 * static_cast<int>(sizeof(RP)) <= kWideSmem, "merge area");
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int ln = lane & 31, lh = lane >> 5;
  const int row_bytes = hidden * 2;
  const int t16 = (V + 15) >> 4;
  const int v_lo = static_cast<int>(static_cast<long long>(part) * t16 / nparts) * 16;
  const int v_hi = min(static_cast<int>(static_cast<long long>(part + 1) * t16 / nparts) * 16, V);
  const int npass = max(v_hi - v_lo, 0) / WROWS + ((max(v_hi - v_lo, 0) % WROWS) != 0);
  const int nch = hidden / kKC;          // even: the kernel is served only when hidden % 128 == 0
  const int total = npass * nch;
  const int rot = ((part >> 3) * nch / 32) % nch;

  // running partials: own tiles (complete over the part) and the remaining
  // tiles (this wave's weight tiles only; merged across waves at the end)
  RP run[Q], runx[R > 0 ? R : 1];
#pragma unroll
  for (int t = 0; t < Q; ++t) {
    if constexpr (MODE == kModeSample) run[t] = empty_spartial();
    else run[t] = empty_partial();
  }
#pragma unroll
  for (int t = 0; t < (R > 0 ? R : 1); ++t) {
    if constexpr (MODE == kModeSample) runx[t] = empty_spartial();
    else runx[t] = empty_partial();
  }
  // activation tile of each tile slot of this wave (own, then the remaining
  // ones), and its lanes' block positions (temperature sampling only)
  int htile[QR];
#pragma unroll
  for (int t = 0; t < QR; ++t) htile[t] = t < Q ? w * Q + t : 4 * Q + t - Q;
  unsigned pos[QR];
  if constexpr (MODE == kModeSample) {
#pragma unroll
    for (int t = 0; t < QR; ++t)
      pos[t] = static_cast<unsigned>(rows[row0 + min(htile[t] * 32 + ln, Mg - 1)] % smp.B);
  }

  if (total > 0) {
    // ---- the weight: 16-byte pieces straight into LDS, 8 rows per
    // instruction; instruction p of wave w fills rows 8 (4p + w) .. +8 of a
    // stage, lane l the XOR-swizzled slot of row 8 (4p + w) + l / 8
    const int r8 = lane >> 3;
    const int ls = (lane & 7) ^ r8 ^ (w & 1);
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<unsigned short*>(W) + static_cast<size_t>(v_lo) * hidden, 0,
        (v_hi - v_lo) * row_bytes, 0x00020000);
    const int wv = (8 * w + r8) * row_bytes + ls * 16;
    // ---- the activation fragments: one 1 KB read each from the
    // operand-ordered copy (bounds-checked descriptor)
    const __amdgpu_buffer_rsrc_t hr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<unsigned short*>(Hf), 0, hf_bytes, 0x00020000);
    int hoff[QR];
#pragma unroll
    for (int t = 0; t < QR; ++t) hoff[t] = ((row0 >> 5) + htile[t]) * (hidden >> 4) * 1024 + lane * 16;
    LoadCursor<S> lw{0, 0, 0, 0};
    auto kc_of = [&](int kci) __attribute__((always_inline)) {
      const int kc = kci + rot;
      return kc >= nch ? kc - nch : kc;
    };
    auto issue_w = [&]() __attribute__((always_inline)) {
      unsigned char* dst = smem + lw.stage * WBUF;
      const int so = lw.pass * WROWS * row_bytes + kc_of(lw.kci) * kRB;
#pragma unroll
      for (int p = 0; p < TW; ++p)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, LOPA_LDS(dst + (4 * p + w) * 1024), 16, wv,
                                                 so + 32 * p * row_bytes, 0, kWeightAux);
      lw.step(total, nch);
    };
    // activation fragments of one K step, by tile slot; the registers hold
    // a ring of eight K steps (step j of the first or second chunk of a pair
    // in set j or 4 + j)
    using HStep = u32x4[QR];
    auto load_h = [&](auto t_c, HStep& dst, int kc, int j) __attribute__((always_inline)) {
      constexpr int t = decltype(t_c)::value;
      dst[t] = __builtin_amdgcn_raw_buffer_load_b128(hr, hoff[t] + j * 1024, kc * 4096, 0);
    };

    // ---- weight fragments of one K step, read one at a time in the order
    // the step's MFMAs first use them: w0 .. w(TW-1), then the tiles w + 4k
    // paired with the remaining activation tiles
    struct Frags {
      u16x8 w[TW], xw[XA];
    };
    auto read_one = [&](auto k_c, int sw, int j, Frags& f) __attribute__((always_inline)) {
      constexpr int k = decltype(k_c)::value;
      const int sl = 2 * j + lh;   // logical slot: K values 16j + 8lh .. +8
      if constexpr (k < TW) {
        const int r = k * 32 + ln;
        f.w[k] = *reinterpret_cast<const u16x8*>(smem + sw * WBUF + r * kRB + swz<kKC>(r, sl) * 16);
      } else {
        const int r = (w + 4 * (k - TW)) * 32 + ln;
        f.xw[k - TW] =
            *reinterpret_cast<const u16x8*>(smem + sw * WBUF + r * kRB + swz<kKC>(r, sl) * 16);
      }
    };

    f32x16 acc[Q][TW], accx[R > 0 ? R : 1][XA];
#pragma unroll
    for (int t = 0; t < Q; ++t)
#pragma unroll
      for (int n = 0; n < TW; ++n) acc[t][n] = f32x16{};
#pragma unroll
    for (int t = 0; t < (R > 0 ? R : 1); ++t)
#pragma unroll
      for (int k = 0; k < XA; ++k) accx[t][k] = f32x16{};

    // NL: live weight tiles of the pass (the others are neither multiplied
    // nor folded); the remaining tiles' pairs always run (a pair past the
    // part reads zeros and its entries are dropped by the masked fold)
    auto mfma_one = [&](auto nl_c, auto i_c, const Frags& f, const HStep& hc)
        __attribute__((always_inline)) {
      constexpr int NL = decltype(nl_c)::value, i = decltype(i_c)::value;
      if constexpr (i < Q * NL) {
        constexpr int t = i / NL, n = i % NL;
        acc[t][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8, f.w[n]), __builtin_bit_cast(bf16x8, hc[t]), acc[t][n],
            0, 0, 0);
      } else {
        constexpr int k = (i - Q * NL) / R, t = (i - Q * NL) % R;
        accx[t][k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8, f.xw[k]), __builtin_bit_cast(bf16x8, hc[Q + t]),
            accx[t][k], 0, 0, 0);
      }
    };

    // An accumulator tile on its way to the fold passes through this wave's
    // slot of LDS (volatile, so the round trip stays): the matrix registers
    // that hold the accumulators are stored as they are, and the fold reads
    // ordinary registers back, one tile at a time.
    // (an LDS-typed pointer: through a generic one the round trip became
    // flat accesses, each waited on in full)
    using lds_f32x4 = __attribute__((address_space(3))) f32x4;
    volatile lds_f32x4* fslot =
        reinterpret_cast<volatile lds_f32x4*>(static_cast<unsigned>(
            reinterpret_cast<uintptr_t>(smem + kWideSmem + w * kWideFoldSlot))) + lane;
    auto through_lds = [&](const f32x16& a) __attribute__((always_inline)) {
      f32x16 r;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        fslot[64 * (q & 1)] = f32x4{a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]};
        if (q & 1) {
          const f32x4 u = fslot[0], v = fslot[64];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            r[4 * (q - 1) + e] = u[e];
            r[4 * q + e] = v[e];
          }
        }
      }
      return r;
    };
    // fold a pass's logits into the running partials (one tile at a time)
    // and clear them
    auto fold = [&](auto nl_c, auto masked_c, int pass) __attribute__((always_inline)) {
      constexpr int NL = decltype(nl_c)::value;
      constexpr bool MASKED = decltype(masked_c)::value;
      const int vb = v_lo + pass * WROWS;
#pragma unroll
      for (int t = 0; t < Q; ++t) {
#pragma unroll
        for (int n = 0; n < NL; ++n) {
          fold_tile_mode<MODE, MASKED>(run[t], through_lds(acc[t][n]), vb + n * 32, lh, v_hi, smp,
                                       MODE == kModeSample ? pos[t] : 0u);
          acc[t][n] = f32x16{};
          // one tile at a time: interleaving the tiles' folds would move
          // every accumulator out of the matrix registers at once
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if constexpr (R > 0) {
#pragma unroll
        for (int t = 0; t < R; ++t) {
#pragma unroll
          for (int k = 0; k < XP; ++k) {
            const int vt = vb + 32 * (w + 4 * k);
            fold_tile_mode<MODE, MASKED>(runx[t], through_lds(accx[t][k]), vt, lh, v_hi, smp,
                                         MODE == kModeSample ? pos[Q + t] : 0u);
            accx[t][k] = f32x16{};
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
    };

    // ---- prologue: W(0) .. W(S - 2), then the activation fragments of K
    // steps 0 .. LA - 1; W(0) .. W(S - 4) landed and the barrier; the first
    // K step's weight fragments.  Steady state: during K step s the
    // activation fragments of step s + LA are loaded into a free set of the
    // ring (steps 0..2 of a chunk: spread over their MFMAs; step 3: before its
    // barrier), and after the barrier in the chunk's last step W(c + S - 1)
    // goes into the stage chunk c - 1 left.  At that barrier W(c + 1) must
    // have landed, with VM_BAR loads after it still allowed in flight (from
    // chunk S - 3 on; the earlier chunks' weight has landed in the prologue).
    // The counter completes in issue order, so an activation load waits for
    // every weight load issued before it: issued before the chunk's own
    // weight loads, each one follows weight loads at least LA + 1 K steps
    // older than its use.  The compiler waits for each activation register
    // itself before its first MFMA.
    static_assert(KS == 4, "one chunk is four K steps");
    HStep hs[8];
    static_for<S - 1>([&](auto) { issue_w(); });
    int hci = 0;   // chunk index (within the pass) of the chunk being computed
    {
      const int kc0 = kc_of(0), kc1 = kc_of(1);   // nch >= 2
      static_for<LA>([&](auto s_c) {
        constexpr int st = decltype(s_c)::value;
        static_for<QR>([&](auto t) { load_h(t, hs[st], st < 4 ? kc0 : kc1, st & 3); });
      });
    }
    wait_vm_lgkm0<2 * TW + LA * QR>();
    raw_barrier();
    Frags f0, f1;
    int cw = 0;   // stage of the chunk being computed
    static_for<NR>([&](auto k) { read_one(k, cw, 0, f0); });
    // K step j (0..2) of the chunk: its MFMAs from fc and hc, step j + 1's
    // weight reads into fn, and the activation loads of K step s + LA (step
    // jl of the chunk with K chunk kcl) into hn, spread over the slots
    auto step = [&](auto nl_c, const Frags& fc, Frags& fn, const HStep& hc, HStep& hn, int kcl,
                    int jl, auto j_c) __attribute__((always_inline)) {
      constexpr int NM = Q * decltype(nl_c)::value + R * XP;
      constexpr int NSL = NM > NR ? NM : NR;
      constexpr int J = decltype(j_c)::value;
      static_for<NSL>([&](auto i) {
        constexpr int I = decltype(i)::value;
        if constexpr (I < NM) mfma_one(nl_c, i, fc, hc);
        if constexpr (I < NR) read_one(i, cw, J + 1, fn);
        // loads ceil(I QR / NSL) .. ceil((I + 1) QR / NSL) - 1 in slot I
        constexpr int t_lo = (I * QR + NSL - 1) / NSL, t_hi = ((I + 1) * QR + NSL - 1) / NSL;
        static_for<(QR + NSL - 1) / NSL>([&](auto q) {
          constexpr int t = t_lo + decltype(q)::value;
          if constexpr (t < t_hi) load_h(std::integral_constant<int, t>{}, hn, kcl, jl);
        });
        __builtin_amdgcn_sched_barrier(0);
      });
    };
    // chunk P (0 or 1) of a pair: K steps 4P .. 4P + 3 of the ring
    auto chunk = [&](auto nl_c, auto p_c) __attribute__((always_inline)) {
      constexpr int NM = Q * decltype(nl_c)::value + R * XP;
      constexpr int PRE = NM - NR > 2 ? NM - NR : (NM < 2 ? NM : 2);
      constexpr int B0 = 4 * decltype(p_c)::value;
      // the chunk 1 and 2 ahead: K chunks of the activation loads
      const int kca[2] = {kc_of(hci + 1 == nch ? 0 : hci + 1),
                          kc_of(hci + 2 >= nch ? hci + 2 - nch : hci + 2)};
      // K step j's load: step (j + LA) % 4 of chunk c + (j + LA) / 4, set (B0 + j + LA) % 8
      step(nl_c, f0, f1, hs[B0], hs[(B0 + LA) & 7], kca[LA / 4 - 1], LA & 3,
           std::integral_constant<int, 0>{});
      step(nl_c, f1, f0, hs[B0 + 1], hs[(B0 + 1 + LA) & 7], kca[(1 + LA) / 4 - 1], (1 + LA) & 3,
           std::integral_constant<int, 1>{});
      step(nl_c, f0, f1, hs[B0 + 2], hs[(B0 + 2 + LA) & 7], kca[(2 + LA) / 4 - 1], (2 + LA) & 3,
           std::integral_constant<int, 2>{});
      // step 3: its first PRE MFMAs with the activation loads of step s + LA
      // (before this chunk's weight loads), the barrier, the rest
      static_for<PRE>([&](auto i) {
        constexpr int I = decltype(i)::value;
        mfma_one(nl_c, i, f1, hs[B0 + 3]);
        constexpr int t_lo = (I * QR + PRE - 1) / PRE, t_hi = ((I + 1) * QR + PRE - 1) / PRE;
        static_for<(QR + PRE - 1) / PRE>([&](auto q) {
          constexpr int t = t_lo + decltype(q)::value;
          if constexpr (t < t_hi)
            load_h(std::integral_constant<int, t>{}, hs[(B0 + 3 + LA) & 7], kca[(3 + LA) / 4 - 1],
                   (3 + LA) & 3);
        });
        __builtin_amdgcn_sched_barrier(0);
      });
      asm volatile("" ::: "memory");
      wait_vm_lgkm0<VM_BAR>();
      raw_barrier();
      // W(c + S - 1) into the stage chunk c - 1 left, spread over the step's
      // remaining MFMAs, with the reads of the next chunk's first step
      unsigned char* const wdst = smem + lw.stage * WBUF;
      const int wso = lw.pass * WROWS * row_bytes + kc_of(lw.kci) * kRB;
      lw.step(total, nch);
      cw = cw + 1 == S ? 0 : cw + 1;
      hci = hci + 1 == nch ? 0 : hci + 1;
      __builtin_amdgcn_sched_barrier(0);
      constexpr int NSLOT = NM - PRE > NR ? NM - PRE : NR;
      constexpr int LPS = (TW + NSLOT - 1) / NSLOT;   // loads per slot
      static_for<NSLOT>([&](auto i) {
        constexpr int I = decltype(i)::value;
        if constexpr (I < NM - PRE)
          mfma_one(nl_c, std::integral_constant<int, PRE + I>{}, f1, hs[B0 + 3]);
        static_for<LPS>([&](auto q) {
          constexpr int p = I * LPS + decltype(q)::value;
          if constexpr (p < TW)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, LOPA_LDS(wdst + (4 * p + w) * 1024), 16,
                                                     wv, wso + 32 * p * row_bytes, 0, kWeightAux);
        });
        if constexpr (I < NR) read_one(i, cw, 0, f0);
        __builtin_amdgcn_sched_barrier(0);
      });
    };
    auto run_pass = [&](auto nl_c, auto masked_c, int pass) __attribute__((always_inline)) {
      for (int kk = 0; kk < nch; kk += 2) {
        chunk(nl_c, std::integral_constant<int, 0>{});
        chunk(nl_c, std::integral_constant<int, 1>{});
      }
      fold(nl_c, masked_c, pass);
    };
    for (int pass = 0; pass + 1 < npass; ++pass)
      run_pass(std::integral_constant<int, TW>{}, std::false_type{}, pass);
    {
      const int rem = v_hi - v_lo - (npass - 1) * WROWS;   // rows of the last pass, 1..WROWS
      const int nl = (rem + 31) / 32;
      static_assert(TW == 4 || TW == 8, "last-pass dispatch");
#define LOPA_LAST(N)                                                                   \
  case N:                                                                              \
    run_pass(std::integral_constant<int, N>{}, std::true_type{}, npass - 1);           \
    break;
      if constexpr (TW == 4) {
        switch (nl) { LOPA_LAST(1) LOPA_LAST(2) LOPA_LAST(3) default: LOPA_LAST(4) }
      } else {
        switch (nl) {
          LOPA_LAST(1) LOPA_LAST(2) LOPA_LAST(3) LOPA_LAST(4) LOPA_LAST(5) LOPA_LAST(6)
          LOPA_LAST(7) default: LOPA_LAST(8)
        }
      }
#undef LOPA_LAST
    }
    wait_vmcnt<0>();   // no load may still target LDS when it is reused below
  }
  __syncthreads();
  // the two lane halves of every row
#pragma unroll
  for (int t = 0; t < Q; ++t) run[t] = merge(run[t], shfl_xor(run[t], 32));
#pragma unroll
  for (int t = 0; t < R; ++t) runx[t] = merge(runx[t], shfl_xor(runx[t], 32));
  // own rows: complete partials; remaining rows: merged over the four waves
  if (lh == 0) {
#pragma unroll
    for (int t = 0; t < Q; ++t) {
      const int r = (w * Q + t) * 32 + ln;
      if (r < Mg) {
        const size_t o = static_cast<size_t>(row0 + r) * nparts + part;
        ws_m[o] = run[t].m;
        ws_s[o] = run[t].s;
        ws_i[o] = run[t].i;
        if constexpr (MODE == kModeEnt) ws_t[o] = run[t].t;
        if constexpr (MODE == kModeSample) {
          ws_t[o] = run[t].g;
          ws_z[o] = run[t].z;
        }
      }
    }
  }
  if constexpr (R > 0) {
    RP* xm = reinterpret_cast<RP*>(smem);   // [R][4 waves][32 rows]
    if (lh == 0) {
#pragma unroll
      for (int t = 0; t < R; ++t) xm[(t * 4 + w) * 32 + ln] = runx[t];
    }
    __syncthreads();
    for (int i = threadIdx.x; i < R * 32; i += kWideThreads) {
      const int t = i >> 5, l = i & 31;
      const int r = (4 * Q + t) * 32 + l;
      if (r < Mg) {
        RP p = xm[(t * 4) * 32 + l];
#pragma unroll
        for (int x = 1; x < 4; ++x) p = merge(p, xm[(t * 4 + x) * 32 + l]);
        const size_t o = static_cast<size_t>(row0 + r) * nparts + part;
        ws_m[o] = p.m;
        ws_s[o] = p.s;
        ws_i[o] = p.i;
        if constexpr (MODE == kModeEnt) ws_t[o] = p.t;
        if constexpr (MODE == kModeSample) {
          ws_t[o] = p.g;
          ws_z[o] = p.z;
        }
      }
    }
  }
}

// kHeadParts workgroups of 256 threads, one per compute unit.  Row groups as
// in k_lmhead_mfma: the groups of one vocabulary part take consecutive blocks
// of the same XCD (block b runs on XCD b mod 8).  Returns at once when the
// narrow kernel serves the row count.
template <int MODE>
__global__ void __launch_bounds__(kWideThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
k_lmhead_wide(int V, int hidden, int nb_max, int m_max, int hf_bytes,
              const unsigned short* __restrict__ Hf, const unsigned short* __restrict__ W,
              const int32_t* __restrict__ rows, const int32_t* __restrict__ row_ptr,
              const int32_t* __restrict__ nb_ptr, float* __restrict__ ws_m,
              float* __restrict__ ws_s, int32_t* __restrict__ ws_i, float* __restrict__ ws_t,
              float* __restrict__ ws_z, const Sampling smp) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kWideSmem + 4 * kWideFoldSlot];
  const int M = __builtin_amdgcn_readfirstlane(listed_rows(row_ptr, nb_ptr, nb_max, m_max));
  if (!wide_takes(M)) return;
  const WideGroups g = wide_groups(M);
  const int b = blockIdx.x;
  const int q = b >> 3;
  const int group = q % g.groups;
  const int part = (q / g.groups) * 8 + (b & 7);
  const int row0 = group * g.th * 32;
  if (part >= g.nparts || row0 >= M) return;
  const int Mg = min(M - row0, g.th * 32);
#define LOPA_ARGS V, hidden, g.nparts, part, Mg, row0, hf_bytes, Hf, W, rows, smem, ws_m, ws_s, \
                  ws_i, ws_t, ws_z, smp
  switch (g.th) {   // the layouts wide_takes() can reach
    case 6: wide_body<8, 1, 2, MODE>(LOPA_ARGS); break;
    case 7: wide_body<8, 1, 3, MODE>(LOPA_ARGS); break;
    case 8: wide_body<8, 2, 0, MODE>(LOPA_ARGS); break;
    case 9: wide_body<4, 2, 1, MODE>(LOPA_ARGS); break;
    case 10: wide_body<4, 2, 2, MODE>(LOPA_ARGS); break;
    case 11: wide_body<4, 2, 3, MODE>(LOPA_ARGS); break;
    case 12: wide_body<4, 3, 0, MODE>(LOPA_ARGS); break;
    default: wide_body<4, 3, 1, MODE>(LOPA_ARGS); break;
  }
#undef LOPA_ARGS
}

// ---------------------------------------------------------------------------
// float32 MFMA kernel
// ---------------------------------------------------------------------------
//
// A workgroup takes one tile of 256 vocabulary entries against one tile of
// 32 listed rows; wave w multiplies entries 64w .. 64w + 63 (two 32 x 32
// output tiles) with v_mfma_f32_32x32x2_f32 (A: weight rows, B: activation
// rows, so a lane holds 16 logits of one row, laid out as in the bf16
// kernels).  K runs in chunks of 32: the workgroup stages the chunk of its
// weight and activation rows in LDS with coalesced loads (zeros past V, the
// listed rows and hidden; rows padded to 33 floats against bank conflicts),
// then every wave reads its fragments from there.  The fold and the partials
// are the bf16 kernels': one partial per (row, 256-entry tile), merged by
// k_lmhead_merge.
constexpr int kF32KC = 32;
constexpr int kF32Stride = kF32KC + 1;

template <int MODE>
__global__ void __launch_bounds__(256)
k_lmhead_f32(int V, int hidden, int ntiles, int nb_max, int m_max, const float* __restrict__ H,
             const float* __restrict__ W, const int32_t* __restrict__ rows,
             const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ nb_ptr,
             float* __restrict__ ws_m, float* __restrict__ ws_s, int32_t* __restrict__ ws_i,
             float* __restrict__ ws_t, float* __restrict__ ws_z, const Sampling smp,
             float* __restrict__ logits_out) {
  using RP = typename std::conditional<MODE == kModeSample, SPartial, Partial>::type;
  __shared__ float wl[kPlainVocabPerWG * kF32Stride];
  __shared__ float hl[32 * kF32Stride];
  __shared__ RP red[4][32];
  const int M = listed_rows(row_ptr, nb_ptr, nb_max, m_max);
  const int t0 = blockIdx.y * 32;
  if (t0 >= M) return;
  const int v0 = blockIdx.x * kPlainVocabPerWG;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int ln = lane & 31, lh = lane >> 5;
  f32x16 acc[2] = {f32x16{}, f32x16{}};
  for (int k0 = 0; k0 < hidden; k0 += kF32KC) {
    __syncthreads();   // the previous chunk's reads are done
    for (int e = tid; e < kPlainVocabPerWG * kF32KC; e += 256) {
      const int r = e / kF32KC, kk = e % kF32KC;
      const int v = v0 + r, k = k0 + kk;
      wl[r * kF32Stride + kk] = v < V && k < hidden ? W[static_cast<size_t>(v) * hidden + k] : 0.f;
    }
    for (int e = tid; e < 32 * kF32KC; e += 256) {
      const int r = e / kF32KC, kk = e % kF32KC;
      const int m = t0 + r, k = k0 + kk;
      hl[r * kF32Stride + kk] =
          m < M && k < hidden ? H[static_cast<size_t>(rows[m]) * hidden + k] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kF32KC; kk += 2) {
      const float b = hl[ln * kF32Stride + kk + lh];
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        const float a = wl[(w * 64 + n * 32 + ln) * kF32Stride + kk + lh];
        acc[n] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc[n], 0, 0, 0);
      }
    }
  }
  // acc[n][q]: logit of listed row t0 + ln, vocabulary entry
  // v0 + 64w + 32n + 4lh + kTileOff(q)
  const int m = t0 + ln;
  RP p;
  if constexpr (MODE == kModeSample) p = empty_spartial();
  else p = empty_partial();
  const unsigned pos =
      MODE == kModeSample ? static_cast<unsigned>(rows[min(m, M - 1)] % smp.B) : 0u;
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int vb = v0 + w * 64 + n * 32;
    fold_tile_mode<MODE, true>(p, acc[n], vb, lh, V, smp, pos);
    if (logits_out && m < M) {
      const size_t lb = static_cast<size_t>(rows[m]) * V;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int v = vb + 4 * lh + kTileOff(q);
        if (v < V) logits_out[lb + v] = acc[n][q];
      }
    }
  }
  p = merge(p, shfl_xor(p, 32));
  if (lh == 0) red[w][ln] = p;
  __syncthreads();
  if (tid < 32 && t0 + tid < M) {
    RP q = merge(merge(red[0][tid], red[1][tid]), merge(red[2][tid], red[3][tid]));
    const size_t o = static_cast<size_t>(t0 + tid) * ntiles + blockIdx.x;
    ws_m[o] = q.m;
    ws_s[o] = q.s;
    ws_i[o] = q.i;
    if constexpr (MODE == kModeEnt) ws_t[o] = q.t;
    if constexpr (MODE == kModeSample) {
      ws_t[o] = q.g;
      ws_z[o] = q.z;
    }
  }
}

// ---------------------------------------------------------------------------
// Plain path
// ---------------------------------------------------------------------------

template <typename T, int MODE>
__global__ void __launch_bounds__(256)
k_lmhead_plain(int V, int hidden, int ntiles, int nb_max, int m_max, const T* __restrict__ H,
               const T* __restrict__ W,
               const int32_t* __restrict__ rows, const int32_t* __restrict__ row_ptr,
               const int32_t* __restrict__ nb_ptr, float* __restrict__ ws_m,
               float* __restrict__ ws_s, int32_t* __restrict__ ws_i, float* __restrict__ ws_t,
               float* __restrict__ ws_z, const Sampling smp, float* __restrict__ logits_out) {
  using RP = typename std::conditional<MODE == kModeSample, SPartial, Partial>::type;
  __shared__ RP red[4];
  const int m = blockIdx.y;
  const int M = listed_rows(row_ptr, nb_ptr, nb_max, m_max);
  if (m >= M) return;
  const int row = rows[m];
  const int v = blockIdx.x * kPlainVocabPerWG + threadIdx.x;
  RP p;
  if constexpr (MODE == kModeSample) p = empty_spartial();
  else p = empty_partial();
  if (v < V) {
    float l = 0.f;
    const size_t hb = static_cast<size_t>(row) * hidden;
    const size_t wb = static_cast<size_t>(v) * hidden;
    for (int k = 0; k < hidden; ++k) l = fmaf(Act<T>::load(H, hb + k), Act<T>::load(W, wb + k), l);
    if constexpr (MODE == kModeSample) {
      const U32x4 w = philox4x32_10(
          U32x4{static_cast<unsigned>(v) >> 2, static_cast<unsigned>(row % smp.B), kSampleTag, 0u},
          smp.k0, smp.k1);
      const unsigned xs[4] = {w.x0, w.x1, w.x2, w.x3};
      const float z = l * smp.inv_t;
      p = SPartial{z, 1.f, v, z + gumbel(xs[v & 3]), z};
    } else {
      p = Partial{l, 1.f, v, 0.f};
    }
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
    if constexpr (MODE == kModeEnt) ws_t[o] = p.t;
    if constexpr (MODE == kModeSample) {
      ws_t[o] = p.g;
      ws_z[o] = p.z;
    }
  }
}

// ---------------------------------------------------------------------------
// Merge of the vocabulary tiles of each row: conf = 1 / sum, arg = argmax;
// with the entropy, ent = the entropy of the row's softmax divided by ln V
// (0 when V == 1); when sampling, conf = the sampled token's probability
// under softmax(l / T) and arg = the sample.
// ---------------------------------------------------------------------------

template <int MODE>
__global__ void __launch_bounds__(256)
k_lmhead_merge(int V, int ntiles, int mfma, int nb_max, int m_max,
               const int32_t* __restrict__ rows, const int32_t* __restrict__ row_ptr,
               const int32_t* __restrict__ nb_ptr, const float* __restrict__ ws_m,
               const float* __restrict__ ws_s, const int32_t* __restrict__ ws_i,
               const float* __restrict__ ws_t, const float* __restrict__ ws_z,
               float* __restrict__ conf, int32_t* __restrict__ arg, float* __restrict__ ent) {
  using RP = typename std::conditional<MODE == kModeSample, SPartial, Partial>::type;
  __shared__ RP red[4];
  const int m = blockIdx.x;
  const int M = listed_rows(row_ptr, nb_ptr, nb_max, m_max);
  if (m >= M) return;
  // mfma: 0 the plain kernel ran, 1 the narrow kernel alone, 2 both MFMA
  // kernels (the wide one serving the row counts wide_takes() names)
  if (mfma) ntiles = head_nparts(M, mfma == 2);
  RP p;
  if constexpr (MODE == kModeSample) p = empty_spartial();
  else p = empty_partial();
  const size_t base = static_cast<size_t>(m) * ntiles;
  for (int t = threadIdx.x; t < ntiles; t += 256) {
    if constexpr (MODE == kModeSample)
      p = merge(p, SPartial{ws_m[base + t], ws_s[base + t], ws_i[base + t], ws_t[base + t],
                            ws_z[base + t]});
    else
      p = merge(p, Partial{ws_m[base + t], ws_s[base + t], ws_i[base + t],
                           MODE == kModeEnt ? ws_t[base + t] : 0.f});
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) p = merge(p, shfl_xor(p, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = p;
  __syncthreads();
  if (threadIdx.x == 0) {
    p = merge(merge(red[0], red[1]), merge(red[2], red[3]));
    const int r = rows[m];
    arg[r] = p.i;
    if constexpr (MODE == kModeSample) {
      conf[r] = exp2f((p.z - p.m) * kLog2e) / p.s;
    } else {
      conf[r] = 1.f / p.s;
      if constexpr (MODE == kModeEnt)
        ent[r] = V > 1 ? (logf(p.s) - p.t / p.s) / logf(static_cast<float>(V)) : 0.f;
    }
  }
}

}  // namespace lopa

// The wide kernel is launched beside the narrow one when the device-side row
// count may reach one it serves (m_max of kWideMinTiles 32-row tiles or more;
// confidence and entropy modes, no full logits requested).
template <int MODE>
static bool wide_serves(const lopa::HeadPlan& p, int hidden, const float* logits_out) {
  return MODE != lopa::kModeSample && p.mfma && lopa::wide_possible(p.m_max, hidden) &&
         logits_out == nullptr;
}

// All three entry points.  Workspace planes of m_max x ntiles: max, sum,
// index, then the entropy term or the perturbed best score, then the scaled
// logit of the sample.
template <int MODE>
static int lmhead_launch(const lopa_dims* dims, const void* H, const void* W,
                         const int32_t* rows, const int32_t* row_ptr, const int32_t* nb,
                         float* conf, int32_t* arg, float* ent, const lopa::Sampling& smp,
                         float* logits_out, void* ws, size_t ws_bytes, hipStream_t stream) {
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
  float* wt = reinterpret_cast<float*>(wi + plane);
  float* wz = wt + plane;
  const int V = dims->V;
  const int nb_max = dims->k_max + 1;
  const unsigned short* Hb = static_cast<const unsigned short*>(H);
  const unsigned short* Wb = static_cast<const unsigned short*>(W);
  const int h_bytes = p.m_max * hidden * 2;   // H is [nb_max][B][hidden]
  if (p.mfma) {
    // the weight range of one vocabulary part (plus one pass of overrun) is
    // addressed with 32-bit byte offsets
    if (head_part_bytes_max(*dims) >= (1LL << 31)) return LOPA_ERR_UNSUPPORTED;
    // the row count lives on the device: when it may exceed what the narrow
    // kernel serves, both kernels are launched and the one not needed
    // returns at once.  Full logits and temperature sampling are served by
    // the narrow kernel only (it takes any row count).
    const bool wide = wide_serves<MODE>(p, hidden, logits_out);
    // the wide kernel's operand-ordered copy of the rows, after the partial
    // planes
    const size_t hf_off = (5 * plane * 4 + 255) / 256 * 256;
    u32x4* hf = wide ? reinterpret_cast<u32x4*>(static_cast<char*>(ws) + hf_off) : nullptr;
    hipLaunchKernelGGL(k_lmhead_mfma<MODE>, dim3(kHeadParts), dim3(kHeadThreads), 0, stream, V,
                       hidden, nb_max, p.m_max, wide ? 1 : 0, h_bytes, Hb, Wb, rows, row_ptr, nb,
                       wm, wsum, wi, wt, wz, smp, logits_out, hf);
    LOPA_LAUNCH_CHECK();
    if constexpr (MODE != kModeSample) {
      if (wide)
        hipLaunchKernelGGL(k_lmhead_wide<MODE>, dim3(kHeadParts), dim3(kWideThreads), 0, stream,
                           V, hidden, nb_max, p.m_max,
                           static_cast<int>(hfrag_bytes(p.m_max, hidden)),
                           reinterpret_cast<const unsigned short*>(hf), Wb, rows, row_ptr, nb, wm,
                           wsum, wi, wt, wz, smp);
    }
  } else {
    const dim3 grid(p.ntiles, p.m_max);
    if (dims->dtype == LOPA_F32) {
      hipLaunchKernelGGL(k_lmhead_f32<MODE>, dim3(p.ntiles, (p.m_max + 31) / 32), dim3(256), 0,
                         stream, V, hidden, p.ntiles, nb_max, p.m_max,
                         static_cast<const float*>(H), static_cast<const float*>(W), rows,
                         row_ptr, nb, wm, wsum, wi, wt, wz, smp, logits_out);
    } else {
      hipLaunchKernelGGL((k_lmhead_plain<unsigned short, MODE>), grid, dim3(256), 0, stream, V,
                         hidden, p.ntiles, nb_max, p.m_max, Hb, Wb, rows, row_ptr, nb, wm, wsum,
                         wi, wt, wz, smp, logits_out);
    }
  }
  LOPA_LAUNCH_CHECK();
  const int served = !p.mfma ? 0 : (wide_serves<MODE>(p, hidden, logits_out) ? 2 : 1);
  hipLaunchKernelGGL(k_lmhead_merge<MODE>, dim3(p.m_max), dim3(256), 0, stream, V, p.ntiles,
                     served, nb_max, p.m_max, rows, row_ptr, nb, wm, wsum, wi, wt, wz,
                     conf, arg, ent);
  LOPA_LAUNCH_CHECK();
  return LOPA_OK;
}

extern "C" int lopa_lmhead_conf(const lopa_dims* dims, const void* H, const void* W,
                                const int32_t* rows, const int32_t* row_ptr,
                                const int32_t* nb, float* conf, int32_t* arg,
                                float* logits_out, void* ws, size_t ws_bytes,
                                hipStream_t stream) {
  return lmhead_launch<lopa::kModeConf>(dims, H, W, rows, row_ptr, nb, conf, arg, nullptr,
                                        lopa::Sampling{}, logits_out, ws, ws_bytes, stream);
}

extern "C" int lopa_lmhead_conf_ent(const lopa_dims* dims, const void* H, const void* W,
                                    const int32_t* rows, const int32_t* row_ptr,
                                    const int32_t* nb, float* conf, int32_t* arg, float* ent,
                                    float* logits_out, void* ws, size_t ws_bytes,
                                    hipStream_t stream) {
  if (!ent) return LOPA_ERR_INVALID;
  return lmhead_launch<lopa::kModeEnt>(dims, H, W, rows, row_ptr, nb, conf, arg, ent,
                                       lopa::Sampling{}, logits_out, ws, ws_bytes, stream);
}

extern "C" int lopa_lmhead_sample(const lopa_dims* dims, float temperature, uint64_t seed,
                                  const void* H, const void* W, const int32_t* rows,
                                  const int32_t* row_ptr, const int32_t* nb, float* conf,
                                  int32_t* arg, float* logits_out, void* ws, size_t ws_bytes,
                                  hipStream_t stream) {
  if (!(temperature > 0.f) || !(temperature < INFINITY)) return LOPA_ERR_INVALID;
  const lopa::Sampling smp{1.f / temperature, static_cast<unsigned>(seed),
                           static_cast<unsigned>(seed >> 32), dims ? dims->B : 1};
  return lmhead_launch<lopa::kModeSample>(dims, H, W, rows, row_ptr, nb, conf, arg, nullptr, smp,
                                          logits_out, ws, ws_bytes, stream);
}

// ---------------------------------------------------------------------------
// Allocation-free LM head (for callers that cannot allocate): the partials
// live in a fixed device array instead of a caller workspace.
// ---------------------------------------------------------------------------

// 16 MiB: the partials of every bfloat16 MFMA shape (m_max <= 1024 rows x 256
// vocabulary parts x 20 bytes = 5 MiB) plus the wide kernel's operand-ordered
// activation copy while m_max (rounded up to 32) x hidden x 2 bytes <= 11 MiB
// (1024 rows at hidden 5632); the float32 path fits while
// m_max x ceil(V / 256) <= 838860.
constexpr size_t kScratchBytes = static_cast<size_t>(16) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kScratchDevices];   // device address of `scratch` on each device, once looked up
}  // namespace

extern "C" int lopa_lmhead_conf_noalloc(const lopa_dims* dims, const void* H, const void* W,
                                        const int32_t* rows, const int32_t* row_ptr,
                                        const int32_t* nb, float* conf, int32_t* arg,
                                        float* logits_out, hipStream_t stream) {
  int st = lopa_check_dims(dims);
  if (st != LOPA_OK) return st;
  if (!H || !W || !rows || !row_ptr || !nb || !conf || !arg) return LOPA_ERR_INVALID;
  if (lopa::lmhead_workspace_bytes(*dims) > kScratchBytes) return LOPA_ERR_TOO_LARGE;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchDevices) return LOPA_ERR_HIP;
  void* ws = nullptr;
  {
    // the array's address on the current device, looked up once per device
    // (in host code `scratch` names a host-side stand-in, not device memory)
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
      void* ptr = nullptr;
      if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr)
        return LOPA_ERR_HIP;
      g_scratch[dev] = ptr;
    }
    ws = g_scratch[dev];
  }
  return lmhead_launch<lopa::kModeConf>(dims, H, W, rows, row_ptr, nb, conf, arg, nullptr,
                                        lopa::Sampling{}, logits_out, ws, kScratchBytes, stream);
}
