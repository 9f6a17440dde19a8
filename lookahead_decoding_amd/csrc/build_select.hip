// Explore and select stages of one LoPA step.  Each is one wavefront: lane p
// owns block position p (B <= 64), so the whole stage is ballots, shuffles
// and one coalesced store per array.
//
// Explore follows the news article "上交大 × 华为小艺推出LoPA：7B扩散语言模型单样例
// 1000+ tokens/s！", section "LoPA 的核心设计：前瞻并行与分支验证", stage
// 多分支并行探索 (anchor = ordinary greedy fill, plus k branches that each also
// fill one of the currently most confident positions), and section 3.1 of
// "解码效率革命：LoPA如何突破扩散语言模型的并行瓶颈".
// Select follows the same news section, stages 分支置信度验证 (branch
// confidence = mean confidence of the positions a branch leaves unfilled) and
// 并行验证与复用 (the best branch is kept and its verification outputs seed
// the next step).
#include "lopa_common.hpp"

namespace lopa {

__global__ void __launch_bounds__(64)
k_branch_build(int B, int nb_max, int k, float tau, float gamma,
               const int32_t* __restrict__ tok, const float* __restrict__ conf,
               const int32_t* __restrict__ arg, int32_t* __restrict__ nb_out,
               int32_t* __restrict__ br_tok, uint8_t* __restrict__ br_mask,
               int32_t* __restrict__ rows, int32_t* __restrict__ row_ptr) {
  const int p = threadIdx.x;
  const bool live = p < B;
  const int t = live ? tok[p] : 0;
  const float c = live ? conf[p] : 0.f;
  const int a = live ? arg[p] : 0;
  const bool masked = live && t == LOPA_MASK_TOKEN;
  const unsigned long long mask_bits = __ballot(masked);
  // rank of each masked position among all masked positions by (confidence
  // desc, position asc); the position index is wave-uniform, so the other
  // lanes' confidences come through v_readlane, not LDS
  const int cbits = __float_as_int(c);
  int rank = 0;
  for (int q = 0; q < B; ++q) {
    const float cq = __int_as_float(__builtin_amdgcn_readlane(cbits, q));
    if (((mask_bits >> q) & 1ull) && (cq > c || (cq == c && q < p))) ++rank;
  }
  // Anchor: every masked position strictly above tau, else the single most
  // confident masked position (rank 0, lowest p on a tie).
  bool fill = masked && c > tau;
  if (__ballot(fill) == 0ull) fill = masked && rank == 0;
  const int n_fill = __popcll(__ballot(fill));
  const bool remaining = masked && !fill;
  const unsigned long long rem_bits = __ballot(remaining);
  const int n_rem = __popcll(rem_bits);
  // every filled position is more confident than every remaining one (above
  // tau against at most tau, or the overall first), so among the remaining
  // positions the rank drops by the fill count
  rank -= n_fill;
  // lookahead candidates: the remaining positions whose confidence reaches
  // the floor gamma (all of them for the plain call) -- a prefix of the
  // remaining positions in rank order
  const int n_cand = __popcll(__ballot(remaining && c >= gamma));
  const int k_eff = k < n_cand ? k : n_cand;
  const int nb = 1 + k_eff;
  const int my_branch = (remaining && rank < k_eff) ? rank + 1 : 0;  // 0: not a lookahead pos

  const int anchor_tok = fill ? a : t;
  // index of p among the remaining positions (ascending p)
  const unsigned long long below = (p == 0) ? 0ull : (~0ull >> (64 - p));
  const int idx_rem = __popcll(rem_bits & below);

  for (int b = 0; b < nb_max; ++b) {
    const bool in_use = b < nb;
    const int tb = (in_use && b >= 1 && my_branch == b) ? a : anchor_tok;
    const bool mb = in_use && tb == LOPA_MASK_TOKEN;
    // lookahead position of this branch, to drop it from the row list
    int qb = -1;
    if (b >= 1 && in_use) {
      const unsigned long long qbits = __ballot(my_branch == b);
      qb = __ffsll(static_cast<long long>(qbits)) - 1;
    }
    if (live) {
      br_tok[b * B + p] = tb;
      br_mask[b * B + p] = mb ? 1 : 0;
    }
    const int start = (b == 0) ? 0 : (b <= nb ? n_rem + (b - 1) * (n_rem - 1)
                                              : n_rem + (nb - 1) * (n_rem - 1));
    if (mb) rows[start + idx_rem - ((qb >= 0 && p > qb) ? 1 : 0)] = b * B + p;
    if (p == 0) row_ptr[b] = start;
  }
  if (p == 0) {
    row_ptr[nb_max] = n_rem == 0 ? 0 : n_rem + (nb - 1) * (n_rem - 1);
    nb_out[0] = nb;
  }
}

// ALPHA: the alternative branch score (alpha * the state confidences of the
// positions branch b fills + (1 - alpha) * the sum of 1 - ent over the
// positions it leaves masked) in place of the mean confidence.
template <bool ALPHA>
__global__ void __launch_bounds__(64)
k_branch_select(int B, int nb_max, const int32_t* __restrict__ nb_ptr,
                const uint8_t* __restrict__ br_mask, const int32_t* __restrict__ br_tok,
                const float* __restrict__ conf, const int32_t* __restrict__ arg,
                float alpha, const int32_t* __restrict__ tok_state,
                const float* __restrict__ conf_state, const float* __restrict__ ent,
                float* __restrict__ bconf, int32_t* __restrict__ winner,
                int32_t* __restrict__ tok_next, float* __restrict__ conf_next,
                int32_t* __restrict__ arg_next) {
  const int p = threadIdx.x;
  const bool live = p < B;
  const int pc = live ? p : B - 1;   // in-bounds index for idle lanes
  const int nb = *nb_ptr;
  bool was_masked = false;
  float cs = 0.f;
  if constexpr (ALPHA) {
    was_masked = live && tok_state[pc] == LOPA_MASK_TOKEN;
    cs = conf_state[pc];
  }
  // every slot's flag and confidence is fetched before any is used
  uint8_t mk[LOPA_MAX_BRANCHES];
  float cf[LOPA_MAX_BRANCHES];
  int32_t tk[LOPA_MAX_BRANCHES], ag[LOPA_MAX_BRANCHES];
#pragma unroll
  for (int b = 0; b < LOPA_MAX_BRANCHES; ++b) {
    const int bb = b < nb_max ? b : nb_max - 1;
    mk[b] = br_mask[bb * B + pc];
    cf[b] = conf[bb * B + pc];
    tk[b] = br_tok[bb * B + pc];
    ag[b] = arg[bb * B + pc];
  }
  // every slot's sum over its still-masked positions, all reduced together
  // (one butterfly: six cross-lane steps in total, not six per slot)
  float sm[LOPA_MAX_BRANCHES];
  int cnt[LOPA_MAX_BRANCHES];
#pragma unroll
  for (int b = 0; b < LOPA_MAX_BRANCHES; ++b) {
    const bool m = live && mk[b] != 0;
    if constexpr (ALPHA) {
      const int bb = b < nb_max ? b : nb_max - 1;
      const float keep = m ? 1.f - ent[bb * B + pc] : 0.f;
      const float fill = was_masked && !m ? cs : 0.f;
      sm[b] = alpha * fill + (1.f - alpha) * keep;
    } else {
      sm[b] = m ? cf[b] : 0.f;
    }
    cnt[b] = __popcll(__ballot(m));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    float x[LOPA_MAX_BRANCHES];
#pragma unroll
    for (int b = 0; b < LOPA_MAX_BRANCHES; ++b) x[b] = __shfl_xor(sm[b], o, kWave);
#pragma unroll
    for (int b = 0; b < LOPA_MAX_BRANCHES; ++b) sm[b] += x[b];
  }
  float best = 0.f;
  int w = 0;
#pragma unroll
  for (int b = 0; b < LOPA_MAX_BRANCHES; ++b) {
    if (b >= nb_max) break;
    float bc = -1.f;
    if (b < nb) {
      if constexpr (ALPHA) bc = sm[b];
      else bc = cnt[b] ? sm[b] / static_cast<float>(cnt[b]) : 1.f;
      if (b == 0 || bc > best) {
        best = bc;
        w = b;
      }
    }
    if (p == 0) bconf[b] = bc;
  }
  // the winner's slot, picked from registers (w is wave-uniform)
  bool m = false;
  float cw = 0.f;
  int32_t tw = 0, aw = 0;
#pragma unroll
  for (int b = 0; b < LOPA_MAX_BRANCHES; ++b)
    if (b == w) {
      m = mk[b] != 0;
      cw = cf[b];
      tw = tk[b];
      aw = ag[b];
    }
  if (live) {
    tok_next[p] = tw;
    conf_next[p] = m ? cw : 0.f;
    arg_next[p] = m ? aw : -1;
  }
  if (p == 0) winner[0] = w;
}

}  // namespace lopa

namespace lopa {

// Initial pass of a block: slot 0 alone, every masked position listed.  Lane
// p owns position p; the rows are a ballot compaction (ascending p).  The
// other slots' rows and the LM head's outputs are cleared, so a position
// that is not listed reads as filled (conf 0, arg -1).
__global__ void __launch_bounds__(64)
k_block_rows(int B, int nb_max, const int32_t* __restrict__ tok, int32_t* __restrict__ nb_out,
             int32_t* __restrict__ rows, int32_t* __restrict__ row_ptr,
             float* __restrict__ conf, int32_t* __restrict__ arg) {
  __shared__ int pos[64];
  const int p = threadIdx.x;
  const bool masked = p < B && tok[p] == LOPA_MASK_TOKEN;
  const unsigned long long bits = __ballot(masked);
  const int m = __popcll(bits);
  const int rank = __popcll(bits & ((1ull << p) - 1ull));
  if (masked) pos[rank] = p;
  __syncthreads();
  const int n = nb_max * B;
  for (int i = p; i < n; i += 64) rows[i] = i < m ? pos[i] : 0;
  for (int i = p; i <= nb_max; i += 64) row_ptr[i] = i == 0 ? 0 : m;
  if (p == 0) nb_out[0] = 1;
  if (conf)
    for (int i = p; i < n; i += 64) conf[i] = 0.f;
  if (arg)
    for (int i = p; i < n; i += 64) arg[i] = -1;
}

}  // namespace lopa

extern "C" int lopa_block_rows(const lopa_dims* dims, const int32_t* tok, int32_t* nb,
                               int32_t* rows, int32_t* row_ptr, float* conf, int32_t* arg,
                               hipStream_t stream) {
  int st = lopa_check_dims(dims);
  if (st != LOPA_OK) return st;
  if (!tok || !nb || !rows || !row_ptr) return LOPA_ERR_INVALID;
  hipLaunchKernelGGL(lopa::k_block_rows, dim3(1), dim3(64), 0, stream, dims->B, dims->k_max + 1,
                     tok, nb, rows, row_ptr, conf, arg);
  LOPA_LAUNCH_CHECK();
  return LOPA_OK;
}

extern "C" int lopa_branch_build(const lopa_dims* dims, int32_t k, float tau,
                                 const int32_t* tok, const float* conf, const int32_t* arg,
                                 int32_t* nb, int32_t* br_tok, uint8_t* br_mask,
                                 int32_t* rows, int32_t* row_ptr, hipStream_t stream) {
  int st = lopa_check_dims(dims);
  if (st != LOPA_OK) return st;
  if (k < 0 || k > dims->k_max) return LOPA_ERR_INVALID;
  if (!tok || !conf || !arg || !nb || !br_tok || !br_mask || !rows || !row_ptr)
    return LOPA_ERR_INVALID;
  hipLaunchKernelGGL(lopa::k_branch_build, dim3(1), dim3(64), 0, stream, dims->B,
                     dims->k_max + 1, k, tau, -INFINITY, tok, conf, arg, nb, br_tok, br_mask,
                     rows, row_ptr);
  LOPA_LAUNCH_CHECK();
  return LOPA_OK;
}

extern "C" int lopa_branch_build_floor(const lopa_dims* dims, int32_t k, float tau, float gamma,
                                       const int32_t* tok, const float* conf, const int32_t* arg,
                                       int32_t* nb, int32_t* br_tok, uint8_t* br_mask,
                                       int32_t* rows, int32_t* row_ptr, hipStream_t stream) {
  int st = lopa_check_dims(dims);
  if (st != LOPA_OK) return st;
  if (k < 0 || k > dims->k_max || gamma != gamma) return LOPA_ERR_INVALID;
  if (!tok || !conf || !arg || !nb || !br_tok || !br_mask || !rows || !row_ptr)
    return LOPA_ERR_INVALID;
  hipLaunchKernelGGL(lopa::k_branch_build, dim3(1), dim3(64), 0, stream, dims->B,
                     dims->k_max + 1, k, tau, gamma, tok, conf, arg, nb, br_tok, br_mask, rows,
                     row_ptr);
  LOPA_LAUNCH_CHECK();
  return LOPA_OK;
}

extern "C" int lopa_branch_select(const lopa_dims* dims, const int32_t* nb,
                                  const uint8_t* br_mask, const int32_t* br_tok,
                                  const float* conf, const int32_t* arg, float* bconf,
                                  int32_t* winner, int32_t* tok_next, float* conf_next,
                                  int32_t* arg_next, hipStream_t stream) {
  int st = lopa_check_dims(dims);
  if (st != LOPA_OK) return st;
  if (!nb || !br_mask || !br_tok || !conf || !arg || !bconf || !winner || !tok_next ||
      !conf_next || !arg_next)
    return LOPA_ERR_INVALID;
  hipLaunchKernelGGL(lopa::k_branch_select<false>, dim3(1), dim3(64), 0, stream, dims->B,
                     dims->k_max + 1, nb, br_mask, br_tok, conf, arg, 0.f, nullptr, nullptr,
                     nullptr, bconf, winner, tok_next, conf_next, arg_next);
  LOPA_LAUNCH_CHECK();
  return LOPA_OK;
}

extern "C" int lopa_branch_select_alpha(const lopa_dims* dims, float alpha,
                                        const int32_t* tok, const float* conf_state,
                                        const int32_t* nb, const uint8_t* br_mask,
                                        const int32_t* br_tok, const float* conf,
                                        const int32_t* arg, const float* ent, float* score,
                                        int32_t* winner, int32_t* tok_next, float* conf_next,
                                        int32_t* arg_next, hipStream_t stream) {
  int st = lopa_check_dims(dims);
  if (st != LOPA_OK) return st;
  if (!(alpha >= 0.f && alpha <= 1.f)) return LOPA_ERR_INVALID;
  if (!tok || !conf_state || !nb || !br_mask || !br_tok || !conf || !arg || !ent || !score ||
      !winner || !tok_next || !conf_next || !arg_next)
    return LOPA_ERR_INVALID;
  hipLaunchKernelGGL(lopa::k_branch_select<true>, dim3(1), dim3(64), 0, stream, dims->B,
                     dims->k_max + 1, nb, br_mask, br_tok, conf, arg, alpha, tok, conf_state, ent,
                     score, winner, tok_next, conf_next, arg_next);
  LOPA_LAUNCH_CHECK();
  return LOPA_OK;
}
