/*
 * lopa.h -- C ABI of liblopa, the MI355X (gfx950) library for one LoPA
 * branch-verification step (Lookahead Parallel Decoding for diffusion LLMs).
 *
 * One step, in the order the method states it:
 *   1. lopa_branch_build  -- explore: the anchor branch (confidence-driven
 *      fill) plus k lookahead branches, each filling one more of the most
 *      confident positions the anchor left masked.
 *      ["上交大 × 华为小艺推出LoPA：7B扩散语言模型单样例1000+ tokens/s！",
 *       section "LoPA 的核心设计：前瞻并行与分支验证", stage 多分支并行探索;
 *       "解码效率革命：LoPA如何突破扩散语言模型的并行瓶颈", section 3.1]
 *   2. lopa_branch_attn   -- verify, attention part: every branch attends to
 *      the shared committed prefix and to its own block only; all branches in
 *      one pass.  ["解码效率革命…", section 3.3; same article section 6 for
 *      full-sequence (bidirectional) attention; news article, stage 并行验证与复用]
 *   3. lopa_lmhead_conf   -- verify, LM-head part: per still-masked (branch,
 *      position) the largest softmax probability over the vocabulary (the
 *      position's confidence) and its argmax token, without storing logits.
 *      [news article, stages 分支置信度验证 and 并行验证与复用]
 *   4. lopa_branch_select -- branch confidence = mean confidence over the
 *      branch's still-masked positions; the highest wins and its per-position
 *      (confidence, token) become the next step's state (reuse).
 *      [news article, stages 分支置信度验证 and 并行验证与复用;
 *       "LoPA：上海交大與華為聯手破解AI推理新困境", third stage]
 *
 * Conventions shared by every call:
 *   - Every array pointer is a DEVICE pointer owned by the caller; the library
 *     never allocates, frees or keeps one.  `dims` is a HOST pointer read
 *     during the call only.
 *   - Calls are asynchronous on `stream` (0 = the null stream) and never
 *     synchronise with the host.  The live branch count nb and the LM-head row
 *     count M stay on the device; launch grids are sized for nb_max = 1+k_max.
 *   - Arguments are validated on the host before anything is enqueued; a
 *     negative lopa_status is returned and nothing is launched.  A failed
 *     launch returns LOPA_ERR_HIP.  No C++ exception crosses the ABI.
 *   - Stateless and thread-safe; calls that share a workspace must be ordered
 *     (the same stream orders them).
 *   - Layouts are dense row-major as annotated.  Activations (Q, K, V, H, W)
 *     are all of dims->dtype: IEEE float32, or bfloat16 (raw 16-bit patterns).
 *   - Per-position arrays of all branches are indexed b*B + p (branch b,
 *     block position p).  The mask token id is LOPA_MASK_TOKEN.
 */
#ifndef LOPA_H
#define LOPA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LOPA_ABI_VERSION 2
#define LOPA_MASK_TOKEN (-1)
#define LOPA_MAX_BLOCK 64        /* B <= 64: one block fits one wavefront      */
#define LOPA_MAX_BRANCHES 16     /* nb_max = 1 + k_max <= 16                   */

typedef enum {
  LOPA_OK = 0,
  LOPA_ERR_INVALID = -1,      /* null pointer, bad size, k > k_max, ...        */
  LOPA_ERR_UNSUPPORTED = -2,  /* valid but outside what the kernels handle     */
  LOPA_ERR_WORKSPACE = -3,    /* workspace missing or smaller than required    */
  LOPA_ERR_HIP = -4,          /* the HIP runtime rejected a launch             */
  LOPA_ERR_TOO_LARGE = -5     /* more scratch than the fixed array holds
                                 (lopa_lmhead_conf_noalloc)                    */
} lopa_status;

typedef enum { LOPA_F32 = 0, LOPA_BF16 = 1 } lopa_dtype;

/* Shape of a step.  hidden = Hq * d is the LM-head contraction length. */
typedef struct lopa_dims {
  int32_t L;      /* committed prefix length shared by all branches, >= 0     */
  int32_t B;      /* block length, 1..64                                      */
  int32_t Hq;     /* query heads                                              */
  int32_t Hkv;    /* key/value heads, Hq % Hkv == 0 (grouped-query attention) */
  int32_t d;      /* head dimension, 1..256                                   */
  int32_t V;      /* vocabulary size, >= 1                                    */
  int32_t k_max;  /* largest lookahead count any call will use, 0..15         */
  int32_t dtype;  /* lopa_dtype of all activations                            */
} lopa_dims;

/* LOPA_ABI_VERSION of the built library. */
int lopa_abi_version(void);

/* Static English text for a lopa_status value (never NULL). */
const char* lopa_status_string(int status);

/* Bytes of device workspace that lopa_branch_attn and lopa_lmhead_conf need
 * for these dims (written to *bytes; the larger of the two, so one buffer
 * serves both calls of a step when they are ordered on one stream).  The
 * size never decreases as dims->L grows, so a buffer sized for the longest
 * prefix of a sequence serves every shorter one.  Returns LOPA_OK or
 * LOPA_ERR_INVALID.  Pure host computation. */
int lopa_workspace_bytes(const lopa_dims* dims, size_t* bytes);

/*
 * Initial pass of a block: the LM-head rows of the block as it stands, with
 * no branch yet -- slot 0 alone, every masked position listed.  Its LM head
 * gives the confidences and tokens the first explore step starts from (the
 * news article above, section "LoPA 的核心设计：前瞻并行与分支验证": each step
 * explores from the confidences the previous verification produced; for a
 * new block that is one plain forward of the block).
 *
 * In  tok[B]  int32  block tokens, LOPA_MASK_TOKEN where masked
 * Out nb[1]                 int32  1
 *     rows[nb_max*B]        int32  the masked positions p, ascending, in
 *                                  rows[0 .. m); 0 in the rest
 *     row_ptr[nb_max+1]     int32  {0, m, m, ..., m}
 *     conf[nb_max*B], arg[nb_max*B]  (optional, NULL to skip) the LM head's
 *                                  outputs, cleared to 0 / -1 so unlisted
 *                                  rows read as filled
 * Bit-exact; one wavefront; no host synchronisation.
 */
int lopa_block_rows(const lopa_dims* dims, const int32_t* tok, int32_t* nb, int32_t* rows,
                    int32_t* row_ptr, float* conf, int32_t* arg, hipStream_t stream);

/*
 * Explore: build the anchor branch and up to k lookahead branches.
 *
 * In  tok[B]  int32  block tokens, LOPA_MASK_TOKEN where masked
 *     conf[B] float  confidence of each masked position (previous step)
 *     arg[B]  int32  predicted token of each masked position
 *     k       lookahead count, 0 <= k <= dims->k_max
 *     tau     fill threshold: the anchor fills every masked p with conf > tau
 *             (strict); if there is none, the single most confident masked p
 *             (lowest p on a tie).  The lookahead positions are the
 *             k_eff = min(k, #left masked) most confident positions the anchor
 *             left masked (confidence descending, position ascending); branch
 *             j fills the anchor's positions plus the j-th of them.  A filled
 *             position takes arg[p].
 * Out nb[1]                 int32  1 + k_eff
 *     br_tok[nb_max*B]      int32  tokens of each branch
 *     br_mask[nb_max*B]     uint8  1 where the branch leaves p masked
 *     rows[nb_max*B]        int32  b*B+p of every still-masked pair, branch-
 *                                  major, p ascending; M = row_ptr[nb] entries
 *     row_ptr[nb_max+1]     int32  rows of branch b are [row_ptr[b], row_ptr[b+1])
 *     Slots b >= nb get the anchor's tokens, an all-zero mask and no rows.
 * Bit-exact integer/compare logic; one wavefront.
 */
int lopa_branch_build(const lopa_dims* dims, int32_t k, float tau,
                      const int32_t* tok, const float* conf, const int32_t* arg,
                      int32_t* nb, int32_t* br_tok, uint8_t* br_mask,
                      int32_t* rows, int32_t* row_ptr, hipStream_t stream);

/*
 * Explore with a branch count that follows the state: as lopa_branch_build,
 * but only remaining positions with conf >= gamma are lookahead candidates,
 * so k_eff = min(k, #{remaining p : conf[p] >= gamma}) and nb = 1 + k_eff.
 * The blog's section 6 ("解码效率革命：LoPA如何突破扩散语言模型的并行瓶颈")
 * names branch counts that adapt to how hard the context is as a next step;
 * this is one plain form of it: where the model is unsure of every other
 * position, fewer speculative fills are verified.  gamma <= 0 gives
 * lopa_branch_build exactly; NaN is rejected (LOPA_ERR_INVALID).
 */
int lopa_branch_build_floor(const lopa_dims* dims, int32_t k, float tau, float gamma,
                            const int32_t* tok, const float* conf, const int32_t* arg,
                            int32_t* nb, int32_t* br_tok, uint8_t* br_mask,
                            int32_t* rows, int32_t* row_ptr, hipStream_t stream);

/*
 * Verify, attention: for branch b < nb, position i < B, query head h with
 * key/value head g = h / (Hq/Hkv):
 *   H[b][i][h*d : h*d+d] = sum_j softmax_j(Q_b,i,h . K_j / sqrt(d)) V_j
 * over keys j = the L prefix keys (Kp/Vp, shared) followed by branch b's own
 * B block keys (Kb/Vb[b]); bidirectional inside the block, other branches'
 * blocks never visible.  The isolation is computed from indices; no mask is
 * stored.
 * In  Kp, Vp [L][Hkv][d];  Qb [nb_max][B][Hq][d];  Kb, Vb [nb_max][B][Hkv][d]
 *     nb[1] (device)
 * Out H [nb_max][B][Hq*d], rounded once to dtype (bf16: nearest-even).
 *     Slots b >= nb are not written.
 *     ws, ws_bytes  device workspace of at least lopa_workspace_bytes() (may
 *                   be NULL/0 when that is 0): partials when the prefix is
 *                   split across workgroups.
 * Accumulation and softmax in float32 (bf16: MFMA products, the softmax
 * weights enter the value product as a bf16 high + low pair).
 */
int lopa_branch_attn(const lopa_dims* dims, const void* Kp, const void* Vp,
                     const void* Qb, const void* Kb, const void* Vb,
                     const int32_t* nb, void* H, void* ws, size_t ws_bytes,
                     hipStream_t stream);

/*
 * Verify, LM head: for every listed row r = rows[m] (m < M = row_ptr[nb]),
 * logits l_v = sum_k H[r][k] * W[v][k] (v < V), and
 *   arg[r]  = lowest v attaining max_v l_v
 *   conf[r] = 1 / sum_v exp(l_v - max l)   (the largest softmax probability)
 * computed in one streaming pass over W with an online (max, sum, argmax)
 * merge; logits are not stored unless logits_out is given.
 * In  H [nb_max][B][Hq*d];  W [V][Hq*d] (vocabulary-major);  rows, row_ptr, nb
 *     as written by lopa_branch_build
 * Out conf[nb_max*B] float, arg[nb_max*B] int32 -- only listed entries written
 *     logits_out  NULL, or float [nb_max*B][V] indexed like H rows (b*B+p);
 *                 only listed rows written
 *     ws, ws_bytes  device workspace of at least lopa_workspace_bytes()
 * bf16: MFMA products with float32 accumulation (FMA when Hq*d is not a
 * multiple of 64); float32: float32 MFMA products.
 */
int lopa_lmhead_conf(const lopa_dims* dims, const void* H, const void* W,
                     const int32_t* rows, const int32_t* row_ptr,
                     const int32_t* nb, float* conf, int32_t* arg,
                     float* logits_out, void* ws, size_t ws_bytes,
                     hipStream_t stream);

/*
 * lopa_lmhead_conf without a workspace, for callers that cannot allocate
 * device memory (code being captured into a HIP graph, tight serving loops,
 * harnesses that forbid hipMalloc): the same kernels and results as
 * lopa_lmhead_conf, bit for bit, with its partials in a fixed array inside
 * the library (16 MiB per device, held by every device the library runs on
 * until the process ends).  The call itself allocates nothing; on its first
 * call on a device it looks up that device's copy of the array.
 *   Returns LOPA_ERR_TOO_LARGE (nothing launched) when what lopa_lmhead_conf
 *   would take from its workspace does not fit: for bfloat16 shapes the MFMA
 *   kernels take, only when the wide kernel's operand-ordered copy of the
 *   rows (nb_max*B rounded up to 32, x Hq*d x 2 bytes, taken when
 *   nb_max*B >= 161 and Hq*d % 128 == 0) passes 11 MiB (1024 rows at
 *   Hq*d = 5632 still fit); for the float32 path when
 *   nb_max*B x ceil(V / 256) > 838860.
 *   Every call on a device uses that device's one array and leaves it
 *   holding its partials: calls that overlap on one device (different
 *   streams, or host threads without ordering) race.  Calls ordered on one
 *   stream are safe; nothing has to be cleared between them (each call writes
 *   every partial it reads).
 */
int lopa_lmhead_conf_noalloc(const lopa_dims* dims, const void* H, const void* W,
                             const int32_t* rows, const int32_t* row_ptr,
                             const int32_t* nb, float* conf, int32_t* arg,
                             float* logits_out, hipStream_t stream);

/*
 * lopa_lmhead_conf plus, for every listed row, the normalised entropy of the
 * row's softmax distribution:
 *   ent[r] = -(sum_v p_v ln p_v) / ln V,  p = softmax(l)   (0 when V == 1)
 * gathered in the same streaming pass (each partial also carries
 * t = sum exp(l - max) (l - max); entropy = ln s - t / s).  The input to the
 * alternative branch score of lopa_branch_select_alpha.
 * ["解码效率革命：LoPA如何突破扩散语言模型的并行瓶颈", section 3.2]
 * Out ent[nb_max*B] float -- only listed entries written (non-NULL, else
 *     LOPA_ERR_INVALID); everything else as lopa_lmhead_conf.
 */
int lopa_lmhead_conf_ent(const lopa_dims* dims, const void* H, const void* W,
                         const int32_t* rows, const int32_t* row_ptr,
                         const int32_t* nb, float* conf, int32_t* arg, float* ent,
                         float* logits_out, void* ws, size_t ws_bytes,
                         hipStream_t stream);

/*
 * lopa_lmhead_conf with temperature sampling in place of the argmax
 * ("解码效率革命：LoPA如何突破扩散语言模型的并行瓶颈", section 5: a temperature of
 * 0.7-1.1 rather than greedy decoding).  For every listed row r at block
 * position p = r mod B:
 *   arg[r]  = argmax_v ( l_v / T + G_v ),  G_v = -ln(-ln u_v)  (Gumbel-max: a
 *             draw from softmax(l / T); lowest v on a tie)
 *   conf[r] = softmax(l / T)[arg[r]]
 * with u_v = (2 (x >> 9) + 1) 2^-24, x = word v % 4 of Philox4x32-10 (Salmon
 * et al., SC 2011) under key (seed low 32 bits, seed high 32 bits) and
 * counter (v / 4, p, 0x5AB1E, 0): the noise depends on the position, not the
 * branch.  Same single streaming pass as lopa_lmhead_conf.
 * In  temperature > 0 and finite (else LOPA_ERR_INVALID); seed (a new one
 *     per pass for independent draws); the rest as lopa_lmhead_conf.
 */
int lopa_lmhead_sample(const lopa_dims* dims, float temperature, uint64_t seed,
                       const void* H, const void* W, const int32_t* rows,
                       const int32_t* row_ptr, const int32_t* nb, float* conf, int32_t* arg,
                       float* logits_out, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Select and reuse: branch confidence bconf[b] = mean of conf[b*B+p] over
 * the p with br_mask[b*B+p] = 1 (1.0 when there is none), for b < nb;
 * bconf[b] = -1 for b >= nb.  winner = the first b with the largest bconf
 * (the anchor wins ties).  Next state: tok_next = br_tok[winner]; where the
 * winner is still masked conf_next/arg_next = its conf/arg, elsewhere 0 / -1.
 * In  nb[1], br_mask, br_tok, conf, arg  (as written by the calls above)
 * Out bconf[nb_max] float, winner[1] int32, tok_next[B], conf_next[B],
 *     arg_next[B].  float32 sums; one wavefront.
 */
int lopa_branch_select(const lopa_dims* dims, const int32_t* nb,
                       const uint8_t* br_mask, const int32_t* br_tok,
                       const float* conf, const int32_t* arg,
                       float* bconf, int32_t* winner, int32_t* tok_next,
                       float* conf_next, int32_t* arg_next, hipStream_t stream);

/*
 * Select and reuse with the alternative branch score of
 * ["解码效率革命：LoPA如何突破扩散语言模型的并行瓶颈", section 3.2], which weighs
 * the confidence of what a branch fills now against the certainty it leaves
 * for the positions still masked:
 *   score[b] = alpha * sum of conf_state[p] over the p that branch b fills
 *              (tok[p] == LOPA_MASK_TOKEN, br_mask[b*B+p] == 0)
 *            + (1 - alpha) * sum of (1 - ent[b*B+p]) over the p with
 *              br_mask[b*B+p] == 1
 * for b < nb; score[b] = -1 for b >= nb.  The sums are taken as written (not
 * averaged); the probability of a filled token is the confidence it was
 * filled on.  Winner and next state as in lopa_branch_select.
 * In  alpha in [0, 1] (else LOPA_ERR_INVALID); tok[B], conf_state[B]: the
 *     state the step started from (the arrays given to lopa_branch_build);
 *     nb, br_mask, br_tok, conf, arg, ent (lopa_lmhead_conf_ent)
 * Out score[nb_max] float, winner[1], tok_next[B], conf_next[B], arg_next[B].
 *     float32 sums; one wavefront.
 */
int lopa_branch_select_alpha(const lopa_dims* dims, float alpha, const int32_t* tok,
                             const float* conf_state, const int32_t* nb,
                             const uint8_t* br_mask, const int32_t* br_tok,
                             const float* conf, const int32_t* arg, const float* ent,
                             float* score, int32_t* winner, int32_t* tok_next,
                             float* conf_next, int32_t* arg_next, hipStream_t stream);

/*
 * Token-keyed synthetic projections, for decoding a whole block over several
 * steps without a model: the news article above (section "LoPA 的核心设计：
 * 前瞻并行与分支验证") repeats explore / verify / select until the block is
 * decoded, and each verification pass sees every branch's own tokens.  This
 * call stands in for the projections a model would compute from them.
 * For every slot b < nb, position p, head h and dimension e:
 *   value = (sum of twelve 16-bit uniforms) / 2^16 - 6
 * with the uniforms taken from two Philox4x32-10 draws (Salmon, Moraes, Dror,
 * Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC 2011) under key
 * (seed low 32 bits, seed high 32 bits) and counters
 * (p | kind << 8 | h << 16, br_tok[b*B+p] as uint32, e, draw), kind 0/1/2 for
 * Q/K/V: all 8 halves of draw 0's words, then the low and high halves of
 * draw 1's words 0 and 1.  Values are exact in float32; bf16 output rounds
 * them to nearest, ties to even.  Two slots holding the same token at p get
 * the same vectors there.
 * In  seed; br_tok[nb_max*B] (e.g. as written by lopa_branch_build); nb[1]
 * Out Qb [nb_max][B][Hq][d], Kb and Vb [nb_max][B][Hkv][d] in dims->dtype;
 *     slots b >= nb are not written.
 */
int lopa_synth_qkv(const lopa_dims* dims, uint64_t seed, const int32_t* br_tok,
                   const int32_t* nb, void* Qb, void* Kb, void* Vb, hipStream_t stream);

/*
 * Commit of a decoded block: once a block is decoded, the winner's branch
 * slot of Kb and Vb -- every slot holds its block's K and V from the last
 * verification pass -- is appended to the committed prefix by index, not
 * recomputed (the pre-write / commit-winner cache of the news article's
 * section "系统级创新：LoPA-Dist 分布式推理"; the two-phase KV commit of
 * "LoPA：上海交大與華為聯手破解AI推理新困境"), so the next block attends to it.
 * Copies Kb[w], Vb[w] ([B][Hkv][d], w = *winner clamped to 0..nb_max-1) to
 * rows at .. at+B-1 of Kp, Vp ([rows][Hkv][d]).
 * In  winner[1] (e.g. as written by lopa_branch_select); Kb, Vb
 *     [nb_max][B][Hkv][d]; at >= 0
 * Out Kp, Vp rows at .. at+B-1; the caller's buffers must hold at+B rows.
 */
int lopa_commit_block(const lopa_dims* dims, const int32_t* winner, const void* Kb,
                      const void* Vb, void* Kp, void* Vp, int32_t at, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Layer forward of the verification pass (bf16 only).
 *
 * The verify stage runs every branch through the model in one pass (news
 * article, stage 并行验证与复用; "解码效率革命…", section 3.3: one shared matrix
 * multiply, each branch attending to the original input and its own tokens;
 * section 6: full-sequence attention).  The model here is a decoder of the
 * Qwen2.5/Dream-7B family: per layer
 *   h = RMSNorm(x) g1;  q, k, v = h Wqkv^T + b, q and k rotated;
 *   x += Attn(q, [prefix K/V of the layer; the branch's own k, v]) Wo^T;
 *   h = RMSNorm(x) g2;  x += (silu(h Wg^T) * (h Wu^T)) Wd^T
 * with the embedding of each token (the mask_id row where masked) as x of
 * the first layer and a final RMSNorm.  Rotary embedding: pairs (i, i+d/2)
 * of each q/k head turned by (L + p) theta^(-2i/d) for block position p.
 * RMSNorm: x / sqrt(mean(x^2) + eps) * g.  Attention is lopa_branch_attn's.
 * Rounding points: the normed rows, q/k/v, the attention output and the
 * MLP activation are rounded once to bf16 (nearest even); projections
 * accumulate in float32 into a float32 residual stream.
 * Rows: all nb_max*B rows (every branch slot) go through the projections;
 * attention is computed for the live slots b < nb.
 * ---------------------------------------------------------------------- */
typedef struct lopa_model_dims {
  int32_t n_layers;   /* decoder layers, >= 1                                */
  int32_t inter;      /* MLP intermediate size, multiple of 64               */
  int32_t mask_id;    /* embedding row of the mask token, 0 <= mask_id < V   */
  float rope_theta;   /* rotary base, > 1                                    */
  float rms_eps;      /* RMSNorm epsilon, >= 0                               */
} lopa_model_dims;

/* Byte offsets in the weight buffer (all tensors bf16, row-major, each
 * 256-byte aligned).  Layer l's tensor t sits at layer0 + l*layer_stride + t:
 *   attn_norm [hidden]; wqkv [(Hq+2Hkv)d][hidden] (q rows, then k, then v);
 *   bqkv [(Hq+2Hkv)d]; wo [hidden][Hq d]; mlp_norm [hidden];
 *   wgu [2 inter][hidden] (gate rows, then up rows); wd [hidden][inter];
 * then final_norm [hidden], embed [V][hidden], lm_head [V][hidden]
 * (lopa_lmhead_conf's W).  total = bytes of the whole buffer. */
typedef struct lopa_model_layout {
  size_t attn_norm, wqkv, bqkv, wo, mlp_norm, wgu, wd;
  size_t layer0, layer_stride;
  size_t final_norm, embed, lm_head;
  size_t total;
} lopa_model_layout;

/* Host only.  LOPA_ERR_INVALID for bad sizes, LOPA_ERR_UNSUPPORTED for f32,
 * hidden or inter not a multiple of 64, d not a multiple of 8, or a projection too large for
 * 32-bit offsets. */
int lopa_model_layout_of(const lopa_dims* dims, const lopa_model_dims* md,
                         lopa_model_layout* out);

/* Host only: device workspace bytes lopa_branch_forward needs (residual
 * stream, activations, GEMM partial tiles, attention workspace). */
int lopa_model_workspace_bytes(const lopa_dims* dims, const lopa_model_dims* md,
                               size_t* bytes);

/*
 * Synthetic weights and prefix cache (no trained weights exist here).  Every
 * element comes from Philox4x32-10 (key = seed low / high 32 bits, counter =
 * (col/4, row, id | layer << 8, 0); word col%4), with id 0 attn_norm,
 * 1 wqkv, 2 bqkv, 3 wo, 4 mlp_norm, 5 wgu, 6 wd, 7 final_norm, 8 embed,
 * 9 lm_head, 10 prefix K, 11 prefix V (rows = prefix positions, columns =
 * Hkv*d).  Norm weights: 1 + ((x >> 27) - 16) / 128.  Other tensors:
 * ((x >> 8) - 2^23) * 2^(-24-s) rounded to bf16, with s = round(log2(sqrt(
 * fan_in / 12))) for the projections, that minus 2 for the LM head (logits
 * of spread ~4), 2 for the biases, 1 for the embedding and -1 for the prefix
 * keys and values.
 * Out weights (lopa_model_layout_of().total bytes); Kp, Vp
 *     [n_layers][kv_layer_rows][Hkv][d]: rows 0..L-1 of every layer.
 */
int lopa_model_synth(const lopa_dims* dims, const lopa_model_dims* md, uint64_t seed,
                     void* weights, void* Kp, void* Vp, size_t kv_layer_rows,
                     hipStream_t stream);

/*
 * One verification forward of every branch's block.
 * In  weights (layout above); Kp, Vp [n_layers][kv_layer_rows][Hkv][d]
 *     holding the committed prefix in rows 0..L-1 of each layer;
 *     br_tok [nb_max*B] (as written by lopa_branch_build), nb[1] (device)
 * Out Kb, Vb [n_layers][nb_max][B][Hkv][d]: every layer's block keys and
 *     values of every slot (rotated keys), kept for the commit;
 *     H [nb_max][B][hidden]: final-normed rows, lopa_lmhead_conf's input.
 *     ws, ws_bytes: at least lopa_model_workspace_bytes().
 * Projections stream each weight once for all rows (MFMA, float32
 * accumulation, split into partial tiles summed by the consumer kernels).
 * Up to 160 rows (and gate/up weights of at most 5 * 16 gate rows per compute
 * unit) the gate/up projection instead accumulates over the whole hidden
 * width per workgroup and writes the SwiGLU activation itself.
 */
int lopa_branch_forward(const lopa_dims* dims, const lopa_model_dims* md,
                        const void* weights, const void* Kp, const void* Vp,
                        size_t kv_layer_rows, const int32_t* br_tok, const int32_t* nb,
                        void* Kb, void* Vb, void* H, void* ws, size_t ws_bytes,
                        hipStream_t stream);

/*
 * lopa_commit_block for every layer: the winner's slot of Kb, Vb
 * ([n_layers][nb_max][B][Hkv][d]) copied to rows at .. at+B-1 of each
 * layer of Kp, Vp ([n_layers][kv_layer_rows][Hkv][d]; at + B <= kv_layer_rows).
 */
int lopa_model_commit(const lopa_dims* dims, const lopa_model_dims* md, const int32_t* winner,
                      const void* Kb, const void* Vb, void* Kp, void* Vp,
                      size_t kv_layer_rows, int32_t at, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* LOPA_H */
