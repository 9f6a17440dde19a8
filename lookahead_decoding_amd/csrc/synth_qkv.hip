// Token-keyed synthetic projections for decoding a block over several steps.
//
// The news article "上交大 × 华为小艺推出LoPA：7B扩散语言模型单样例1000+ tokens/s！"
// (section "LoPA 的核心设计：前瞻并行与分支验证") iterates explore, verify and
// select until the block is decoded; each iteration's verification pass sees
// every branch's own tokens.  Without trained weights, the per-branch
// projections Q, K, V of a block are stood in for by values drawn from a
// counter-based generator keyed by (seed, tensor, head, position, token,
// dimension): two branches holding the same token at a position get the same
// vectors there, so branches differ exactly where they fill differently.
//
// Generator: Philox4x32-10 as published by Salmon, Moraes, Dror and Shaw
// ("Parallel random numbers: as easy as 1, 2, 3", SC 2011): ten rounds of two
// 32 x 32 -> 64-bit multiplies, the high halves mixed into the other words
// with the round key, the key advanced by a Weyl increment between rounds.
// Value: an Irwin-Hall sum of twelve 16-bit uniforms (the 8 halves of draw 0
// and the low and high halves of words 0 and 1 of draw 1) minus 6 -- mean 0,
// variance 1, an integer multiple of 2^-16 and therefore exact in float32
// before the single rounding to bf16 (nearest, ties to even).
//
// Counters of element (slot b, position p, head h, dimension e) of tensor
// kind (0 Q, 1 K, 2 V): (p | kind << 8 | h << 16, token as uint32, e, draw);
// key (seed low 32 bits, seed high 32 bits).
#include "philox.hpp"

namespace lopa {

__device__ __forceinline__ unsigned halves_sum(unsigned w) { return (w & 0xFFFFu) + (w >> 16); }

// One thread per element of Q, K and V of slots b < nb.  Layout of the
// flattened index: [slot][position][Hq + 2 Hkv heads][d]; heads 0..Hq-1 are
// Q's, then K's, then V's.
template <typename T>
__global__ void __launch_bounds__(256)
k_synth_qkv(int B, int Hq, int Hkv, int d, int nb_max, unsigned k0, unsigned k1,
            const int32_t* __restrict__ br_tok, const int32_t* __restrict__ nb_ptr,
            T* __restrict__ Qb, T* __restrict__ Kb, T* __restrict__ Vb) {
  const int nb = min(max(*nb_ptr, 0), nb_max);
  const int heads = Hq + 2 * Hkv;
  const long long n = static_cast<long long>(nb) * B * heads * d;
  const long long i = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int e = static_cast<int>(i % d);
  const long long r = i / d;
  const int hh = static_cast<int>(r % heads);
  const long long bp = r / heads;            // slot * B + position
  const int p = static_cast<int>(bp % B);
  int kind, h;
  if (hh < Hq) {
    kind = 0;
    h = hh;
  } else if (hh < Hq + Hkv) {
    kind = 1;
    h = hh - Hq;
  } else {
    kind = 2;
    h = hh - Hq - Hkv;
  }
  const unsigned c0 = static_cast<unsigned>(p) | (static_cast<unsigned>(kind) << 8) |
                      (static_cast<unsigned>(h) << 16);
  const unsigned tok = static_cast<unsigned>(br_tok[bp]);
  const U32x4 d0 = philox4x32_10(U32x4{c0, tok, static_cast<unsigned>(e), 0u}, k0, k1);
  const U32x4 d1 = philox4x32_10(U32x4{c0, tok, static_cast<unsigned>(e), 1u}, k0, k1);
  const int s = static_cast<int>(halves_sum(d0.x0) + halves_sum(d0.x1) + halves_sum(d0.x2) +
                                 halves_sum(d0.x3) + halves_sum(d1.x0) + halves_sum(d1.x1)) -
                6 * 65536;
  const float v = static_cast<float>(s) * (1.0f / 65536.0f);   // exact
  const int nh = kind == 0 ? Hq : Hkv;
  T* dst = kind == 0 ? Qb : (kind == 1 ? Kb : Vb);
  Act<T>::store(dst, (bp * nh + h) * d + e, v);
}

}  // namespace lopa

extern "C" int lopa_synth_qkv(const lopa_dims* dims, uint64_t seed, const int32_t* br_tok,
                              const int32_t* nb, void* Qb, void* Kb, void* Vb,
                              hipStream_t stream) {
  using namespace lopa;
  int st = lopa_check_dims(dims);
  if (st != LOPA_OK) return st;
  if (!br_tok || !nb || !Qb || !Kb || !Vb) return LOPA_ERR_INVALID;
  const int nb_max = dims->k_max + 1;
  const long long n =
      static_cast<long long>(nb_max) * dims->B * (dims->Hq + 2 * dims->Hkv) * dims->d;
  const dim3 grid(static_cast<unsigned>((n + 255) / 256));
  const unsigned k0 = static_cast<unsigned>(seed), k1 = static_cast<unsigned>(seed >> 32);
  if (dims->dtype == LOPA_F32) {
    hipLaunchKernelGGL(k_synth_qkv<float>, grid, dim3(256), 0, stream, dims->B, dims->Hq,
                       dims->Hkv, dims->d, nb_max, k0, k1, br_tok, nb, static_cast<float*>(Qb),
                       static_cast<float*>(Kb), static_cast<float*>(Vb));
  } else {
    hipLaunchKernelGGL(k_synth_qkv<unsigned short>, grid, dim3(256), 0, stream, dims->B,
                       dims->Hq, dims->Hkv, dims->d, nb_max, k0, k1, br_tok, nb,
                       static_cast<unsigned short*>(Qb), static_cast<unsigned short*>(Kb),
                       static_cast<unsigned short*>(Vb));
  }
  LOPA_LAUNCH_CHECK();
  return LOPA_OK;
}

// ---------------------------------------------------------------------------
// Commit of a decoded block's K and V to the committed prefix.
//
// Every branch slot already holds its block's K and V (written for the last
// verification pass); once the block is decoded, the winner's slot is kept by
// index and appended to the prefix, not recomputed -- the pre-write and
// commit-winner cache of the news article's section
// "系统级创新：LoPA-Dist 分布式推理", in its one-GPU form.
// ---------------------------------------------------------------------------

namespace lopa {

template <typename T>
__global__ void __launch_bounds__(256)
k_commit_block(int n, int nb_max, const int32_t* __restrict__ winner, const T* __restrict__ Kb,
               const T* __restrict__ Vb, T* __restrict__ Kp, T* __restrict__ Vp) {
  const int w = min(max(*winner, 0), nb_max - 1);
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const size_t src = static_cast<size_t>(w) * n + i;
  Kp[i] = Kb[src];
  Vp[i] = Vb[src];
}

}  // namespace lopa

extern "C" int lopa_commit_block(const lopa_dims* dims, const int32_t* winner, const void* Kb,
                                 const void* Vb, void* Kp, void* Vp, int32_t at,
                                 hipStream_t stream) {
  using namespace lopa;
  int st = lopa_check_dims(dims);
  if (st != LOPA_OK) return st;
  if (!winner || !Kb || !Vb || !Kp || !Vp || at < 0) return LOPA_ERR_INVALID;
  const int n = dims->B * dims->Hkv * dims->d;   // one slot of Kb / Vb
  const size_t row0 = static_cast<size_t>(at) * dims->Hkv * dims->d;
  const int nb_max = dims->k_max + 1;
  const dim3 grid((n + 255) / 256);
  if (dims->dtype == LOPA_F32) {
    hipLaunchKernelGGL(k_commit_block<float>, grid, dim3(256), 0, stream, n, nb_max, winner,
                       static_cast<const float*>(Kb), static_cast<const float*>(Vb),
                       static_cast<float*>(Kp) + row0, static_cast<float*>(Vp) + row0);
  } else {
    hipLaunchKernelGGL(k_commit_block<unsigned short>, grid, dim3(256), 0, stream, n, nb_max,
                       winner, static_cast<const unsigned short*>(Kb),
                       static_cast<const unsigned short*>(Vb),
                       static_cast<unsigned short*>(Kp) + row0,
                       static_cast<unsigned short*>(Vp) + row0);
  }
  LOPA_LAUNCH_CHECK();
  return LOPA_OK;
}
