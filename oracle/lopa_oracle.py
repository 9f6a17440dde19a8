"""CPU oracle for one LoPA branch-verification step -- TEST INFRASTRUCTURE.

This module is the reference that the GPU library is checked against.  Only
the tests, the smoke check and the benchmark's CPU-baseline leg may import
it; the product path (``lookahead_decoding_amd``) never does, and this file
imports nothing from it.  It is deliberately plain and slow: numpy in
float64, Python loops over block positions and branches, a library matmul
as the only large step.

Sources (cited by page title and section):
  [news]  "上交大 × 华为小艺推出LoPA：7B扩散语言模型单样例1000+ tokens/s！"
          -- section "LoPA 的核心设计：前瞻并行与分支验证" with its three
          stages (multi-branch exploration / branch-confidence verification /
          parallel verification and reuse), and figure 3 (algorithm flow).
  [blog]  "解码效率革命：LoPA如何突破扩散语言模型的并行瓶颈"
          -- section 3.1 (anchor + k lookahead branches sharing parameters),
          section 3.3 (attention isolation, one pass for all branches,
          logits cached for the next step), section 6 (full-sequence
          attention is required).
  [pop]   "LoPA：上海交大與華為聯手破解AI推理新困境" -- its three-stage
          description (prepare branches, verify in parallel, pick the branch
          with the highest future parallelism).

Readings taken where the pages are silent (each is repeated at the function
that uses it):
  * confidence of a masked position = the largest softmax probability of
    the model's distribution there; the predicted token = its argmax
    (lowest vocabulary id on an exact tie);
  * the anchor fills every masked position whose confidence is strictly
    above the threshold; if none is, it fills the single most confident one
    (lowest position on a tie), so every step makes progress;
  * lookahead branch j = the anchor plus one more fill, at the j-th most
    confident position the anchor left masked (confidence descending,
    position ascending); k_eff = min(k, #left masked), nb = 1 + k_eff;
  * branch confidence = mean confidence over the branch's still-masked
    positions, 1.0 if it has none; winner = highest, lowest branch on a tie
    (so the anchor wins ties);
  * attention of a branch row sees the whole committed prefix plus the
    whole of its own block (masked positions included), no causal mask,
    scale 1/sqrt(d), no rotary step (inputs count as already rotated);
  * the attention output H (hidden = Hq*d) feeds the LM head directly and is
    rounded to the activation dtype first (bf16 round-to-nearest-even, or
    fp32); the LM head is only evaluated on still-masked rows;
  * "reuse" = the winner's per-position (confidence, argmax) become the next
    step's state, with no further forward pass.

Parity pins: every public function here is pinned by CPU tests against
closed forms, brute force, library routines or invariants (see the tests
named ``test_oracle_*``).  No function is left unpinned.

Array conventions (identical to the C-ABI library's):
  tok [B] int32 (-1 = masked); conf [B] float32; arg [B] int32;
  Kp, Vp [L][Hkv][d]; Qb [nb_max][B][Hq][d]; Kb, Vb [nb_max][B][Hkv][d];
  W [V][hidden] (vocabulary-major); H [nb_max][B][hidden];
  per-position LM-head outputs are indexed b*B + p.
bf16 data is held as uint16 bit patterns; fp32 data as float32.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

MASK = -1


# ---------------------------------------------------------------------------
# Number formats
# ---------------------------------------------------------------------------

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns (uint16): a bf16 is the upper half of
    an IEEE float32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values straight to bf16 (8 significant bits, exponent
    range of float32), nearest with ties to even; return uint16 bits.

    Rounding is done once, from the exact float64 value (no intermediate
    float32).  Overflow past the largest finite bf16 gives +-inf; values
    below the normal range round on the subnormal grid (spacing 2**-133).
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.float64)
    finite = np.isfinite(x)
    ax = np.abs(np.where(finite, x, 0.0))
    # exponent e with 2**e <= |x| < 2**(e+1); grid spacing 2**(e-7),
    # but never finer than the subnormal spacing 2**-133.
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    # log2 can be off by one ulp near powers of two: fix e exactly
    e = np.where(np.ldexp(1.0, e.astype(np.int64)) > ax, e - 1, e)
    e = np.where(np.ldexp(1.0, (e + 1).astype(np.int64)) <= ax, e + 1, e)
    e = np.maximum(e, -126.0)
    q = np.ldexp(1.0, (e - 7).astype(np.int64))
    r = np.round(ax / q) * q            # numpy rounds halves to even
    largest = float(np.ldexp(255.0 / 128.0, 127))   # (2 - 2**-7) * 2**127
    r = np.where(r > largest, np.inf, r)
    out = np.where(finite, np.copysign(r, x), x)
    f32 = out.astype(np.float32)        # exact: every bf16 value is a float32
    bits = f32.view(np.uint32) >> np.uint32(16)
    # NaN keeps a quiet-NaN pattern
    bits = np.where(np.isnan(f32), np.uint32(0x7FC0), bits)
    return bits.astype(np.uint16)


def to_f64(a: np.ndarray) -> np.ndarray:
    """Activation tensor (float32 or bf16 bits) -> exact float64."""
    if a.dtype == np.uint16:
        return bf16_to_f64(a)
    if a.dtype == np.float32:
        return a.astype(np.float64)
    raise TypeError(f"unsupported activation dtype {a.dtype}")


def round_like(x64: np.ndarray, like_dtype) -> np.ndarray:
    """Round float64 values to the activation dtype (bf16 bits or float32)
    and return them back as exact float64 -- the one rounding point of H."""
    if like_dtype == np.uint16:
        return bf16_to_f64(f64_to_bf16(x64))
    if like_dtype == np.float32:
        return x64.astype(np.float32).astype(np.float64)
    raise TypeError(f"unsupported activation dtype {like_dtype}")


# ---------------------------------------------------------------------------
# Stage 1: explore -- anchor branch and k lookahead branches
# [news] core design, stage "多分支并行探索"; [blog] 3.1; [pop] stage 1.
# ---------------------------------------------------------------------------

@dataclass
class Branches:
    nb: int                 # number of live branches, 1 + k_eff
    br_tok: np.ndarray      # [nb_max][B] int32: block tokens of each branch
    br_mask: np.ndarray     # [nb_max][B] uint8: 1 where still masked
    rows: np.ndarray        # [M] int32: b*B + p of still-masked pairs
    row_ptr: np.ndarray     # [nb_max + 1] int32: rows of branch b
    anchor_fill: list       # positions the anchor fills
    lookahead: list         # q_1..q_k_eff


def anchor_fill_set(tok, conf, tau) -> list:
    """Positions the anchor (plain confidence-driven sampling) fills.

    Every masked position with confidence strictly above ``tau``; when none
    qualifies, the single most confident masked position (lowest position on
    a tie), so a step always makes progress.  Empty when nothing is masked.
    """
    masked = [p for p in range(len(tok)) if tok[p] == MASK]
    if not masked:
        return []
    fill = [p for p in masked if float(conf[p]) > float(tau)]
    if fill:
        return fill
    best = masked[0]
    for p in masked[1:]:
        if float(conf[p]) > float(conf[best]):
            best = p
    return [best]


def branch_build(tok, conf, arg, k: int, tau: float, nb_max: int,
                 gamma: float | None = None) -> Branches:
    """Anchor plus k lookahead branches, and the LM-head row list.

    Branch 0 (anchor) fills ``anchor_fill_set``.  The lookahead positions
    are the top ``k_eff = min(k, #remaining)`` of the positions the anchor
    leaves masked, ranked by confidence descending then position ascending;
    branch j fills the anchor's set plus the j-th of them.  A filled
    position takes the previous step's argmax token ``arg[p]``.

    Branches b >= nb are written as copies of the anchor's tokens with no
    masked positions, and ``row_ptr[b+1] = M`` for them.

    ``gamma`` (the branch count that follows the state, [blog] section 6's
    adaptive branch count in one plain form): only remaining positions with
    confidence >= gamma are lookahead candidates, k_eff = min(k, their
    number); None keeps every remaining position.
    """
    tok = np.asarray(tok, dtype=np.int32)
    B = len(tok)
    if k < 0 or 1 + k > nb_max:
        raise ValueError("need 0 <= k <= nb_max - 1")
    fill = anchor_fill_set(tok, conf, tau)
    masked = [p for p in range(B) if tok[p] == MASK]
    remaining = [p for p in masked if p not in fill]
    ranked = sorted(remaining, key=lambda p: (-float(conf[p]), p))
    if gamma is not None:
        ranked = [p for p in ranked if float(conf[p]) >= float(gamma)]
    k_eff = min(k, len(ranked))
    look = ranked[:k_eff]
    nb = 1 + k_eff

    anchor = tok.copy()
    for p in fill:
        anchor[p] = arg[p]
    br_tok = np.empty((nb_max, B), dtype=np.int32)
    for b in range(nb_max):
        br_tok[b] = anchor
    for j, q in enumerate(look, start=1):
        br_tok[j, q] = arg[q]
    br_mask = np.zeros((nb_max, B), dtype=np.uint8)
    for b in range(nb):
        br_mask[b] = (br_tok[b] == MASK)

    rows = []
    row_ptr = np.zeros(nb_max + 1, dtype=np.int32)
    for b in range(nb_max):
        row_ptr[b] = len(rows)
        if b < nb:
            for p in range(B):
                if br_mask[b, p]:
                    rows.append(b * B + p)
    row_ptr[nb_max] = len(rows)
    return Branches(nb, br_tok, br_mask, np.asarray(rows, dtype=np.int32),
                    row_ptr, fill, look)


# ---------------------------------------------------------------------------
# Stage 2a: verify -- attention with branch isolation
# [blog] 3.3: a branch attends to the original input and its own tokens,
# never to another branch's predictions; [blog] 6: full-sequence attention;
# [news] stage "并行验证与复用": all branches verified in one forward pass.
# ---------------------------------------------------------------------------

def softmax_rows(S: np.ndarray) -> np.ndarray:
    """Textbook row softmax: exp(s - max) / sum."""
    e = np.exp(S - S.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def attention_one_branch(Kp, Vp, Qb_b, Kb_b, Vb_b, Hq: int, Hkv: int) -> np.ndarray:
    """Attention output of one branch run on its own.

    Keys/values are the committed prefix followed by the branch's own block
    (length L + B).  Query head h reads key/value head h // (Hq // Hkv).
    Returns H_b [B][Hq*d] in float64.
    """
    L, _, d = Kp.shape
    B = Qb_b.shape[0]
    G = Hq // Hkv
    H = np.zeros((B, Hq * d), dtype=np.float64)
    for h in range(Hq):
        g = h // G
        K = np.concatenate([Kp[:, g, :], Kb_b[:, g, :]], axis=0)   # [L+B][d]
        Vv = np.concatenate([Vp[:, g, :], Vb_b[:, g, :]], axis=0)
        Q = Qb_b[:, h, :]                                         # [B][d]
        P = softmax_rows(Q @ K.T / math.sqrt(d))
        H[:, h * d:(h + 1) * d] = P @ Vv
    return H


def branch_attn(Kp, Vp, Qb, Kb, Vb, nb: int, Hq: int, Hkv: int) -> np.ndarray:
    """H [nb_max][B][Hq*d] (float64, unrounded); rows of branches b >= nb are
    zero.  Each branch is computed alone, which is what isolation means."""
    Kp64, Vp64 = to_f64(Kp), to_f64(Vp)
    Qb64, Kb64, Vb64 = to_f64(Qb), to_f64(Kb), to_f64(Vb)
    nb_max, B, _, d = Qb64.shape
    H = np.zeros((nb_max, B, Hq * d), dtype=np.float64)
    for b in range(nb):
        H[b] = attention_one_branch(Kp64, Vp64, Qb64[b], Kb64[b], Vb64[b], Hq, Hkv)
    return H


# ---------------------------------------------------------------------------
# Stage 2b: verify -- LM head, per-position confidence and argmax
# [news] stage "分支置信度验证" (confidence of the remaining positions) and
# "并行验证与复用" (the verification logits are reused next step).
# ---------------------------------------------------------------------------

@dataclass
class HeadOut:
    conf: np.ndarray      # [M] float64: max softmax probability
    arg: np.ndarray       # [M] int64: argmax token (lowest id on a tie)
    margin: np.ndarray    # [M] float64: top-1 minus top-2 logit
    logits: np.ndarray | None = None   # [M][V] float64 when asked for
    ent: np.ndarray | None = None      # [M] float64: entropy of softmax(l) / ln V
    top_tok: np.ndarray | None = None    # [M][T] int64: the T largest logits' tokens
    top_logit: np.ndarray | None = None  # [M][T] float64: their logits, descending


def top_logits(logits: np.ndarray, T: int) -> tuple[np.ndarray, np.ndarray]:
    """Per row, the T largest logits in descending order and their tokens
    (the lower token first among equal logits)."""
    M, V = logits.shape
    T = min(T, V)
    tok = np.zeros((M, T), dtype=np.int64)
    val = np.zeros((M, T))
    for r in range(M):
        # every token at or above the T-th largest value (ties at the cut
        # included), then the order and the cut by (logit desc, token asc)
        thr = np.partition(logits[r], V - T)[V - T] if T else np.inf
        cand = np.flatnonzero(logits[r] >= thr)
        order = sorted(cand.tolist(), key=lambda v: (-logits[r, v], v))[:T]
        tok[r] = order
        val[r] = logits[r, order]
    return tok, val


def lmhead_conf(Hrows64: np.ndarray, W, keep_logits: bool = False, top: int = 16) -> HeadOut:
    """Logits l = H_r . W_v for every row r and vocabulary entry v, in
    float64; confidence = max_v softmax(l)_v; token = argmax_v l_v;
    ent = -sum_v p_v ln p_v / ln V, the entropy of the position's
    distribution normalised to [0, 1] (0 when V = 1) -- the H of the
    alternative branch score of [blog] section 3.2.  ``top``: also the
    ``top`` largest logits of each row and their tokens (which tokens a
    near-tied row may validly predict)."""
    W64 = to_f64(W)
    M = Hrows64.shape[0]
    V = W64.shape[0]
    if M == 0:
        e = np.zeros(0)
        T = min(top, V)
        return HeadOut(e, np.zeros(0, dtype=np.int64), e,
                       np.zeros((0, V)) if keep_logits else None, e,
                       np.zeros((0, T), dtype=np.int64), np.zeros((0, T)))
    logits = Hrows64 @ W64.T
    P = softmax_rows(logits)
    conf = P.max(axis=1)
    arg = np.argmax(logits, axis=1)          # first (lowest) index on a tie
    if V > 1:
        top2 = np.sort(logits, axis=1)[:, -2:]
        margin = top2[:, 1] - top2[:, 0]
    else:
        margin = np.full(M, np.inf)
    with np.errstate(divide="ignore", invalid="ignore"):
        plogp = np.where(P > 0, P * np.log(P), 0.0)
    ent = -plogp.sum(axis=1) / math.log(V) if V > 1 else np.zeros(M)
    top_tok, top_val = top_logits(logits, top)
    return HeadOut(conf, arg, margin, logits if keep_logits else None, ent, top_tok, top_val)


# ---------------------------------------------------------------------------
# Stage 3: select and reuse
# [news] stage "分支置信度验证": branch confidence = mean predicted
# confidence over the branch's remaining unfilled positions; "并行验证与复用":
# the branch with the greatest future potential wins and its logits seed the
# next iteration; [pop] stage 3.
# ---------------------------------------------------------------------------

@dataclass
class Selection:
    bconf: np.ndarray     # [nb_max] float64, -1 for b >= nb
    winner: int
    margin: float         # best minus second-best branch confidence
    tok_next: np.ndarray  # [B] int32
    conf_next: np.ndarray  # [B] float64 (0 where filled)
    arg_next: np.ndarray  # [B] int32 (-1 where filled)


def branch_select(nb: int, br_mask, br_tok, conf_pos, arg_pos) -> Selection:
    """``conf_pos``/``arg_pos`` are indexed b*B + p (only still-masked
    entries are read)."""
    nb_max, B = br_mask.shape
    bconf = np.full(nb_max, -1.0)
    for b in range(nb):
        vals = [float(conf_pos[b * B + p]) for p in range(B) if br_mask[b, p]]
        bconf[b] = sum(vals) / len(vals) if vals else 1.0
    winner = 0
    for b in range(1, nb):
        if bconf[b] > bconf[winner]:
            winner = b
    others = [bconf[b] for b in range(nb) if b != winner]
    margin = bconf[winner] - max(others) if others else math.inf
    tok_next = br_tok[winner].astype(np.int32).copy()
    conf_next = np.zeros(B)
    arg_next = np.full(B, -1, dtype=np.int32)
    for p in range(B):
        if br_mask[winner, p]:
            conf_next[p] = float(conf_pos[winner * B + p])
            arg_next[p] = int(arg_pos[winner * B + p])
    return Selection(bconf, winner, margin, tok_next, conf_next, arg_next)


def branch_select_alpha(nb: int, br_mask, br_tok, conf_pos, arg_pos, ent_pos, tok_state,
                        conf_state, alpha: float) -> Selection:
    """The alternative branch score of [blog] section 3.2:
    score_b = alpha * sum of the probabilities of the tokens branch b fills
    this step + (1 - alpha) * sum over the positions b leaves masked of
    (1 - H), H the normalised entropy of the position's distribution in b's
    verification pass.  Readings: the sums are taken as written (not
    averaged); a fill's probability is the confidence it was filled on (the
    state's); H is normalised by ln V so 1 - H lies in [0, 1].  Winner and
    next state as in ``branch_select`` (the first best branch wins ties)."""
    nb_max, B = br_mask.shape
    score = np.full(nb_max, -1.0)
    for b in range(nb):
        fill = sum(float(conf_state[p]) for p in range(B)
                   if tok_state[p] == MASK and not br_mask[b, p])
        rest = sum(1.0 - float(ent_pos[b * B + p]) for p in range(B) if br_mask[b, p])
        score[b] = alpha * fill + (1.0 - alpha) * rest
    winner = 0
    for b in range(1, nb):
        if score[b] > score[winner]:
            winner = b
    others = [score[b] for b in range(nb) if b != winner]
    margin = score[winner] - max(others) if others else math.inf
    tok_next = br_tok[winner].astype(np.int32).copy()
    conf_next = np.zeros(B)
    arg_next = np.full(B, -1, dtype=np.int32)
    for p in range(B):
        if br_mask[winner, p]:
            conf_next[p] = float(conf_pos[winner * B + p])
            arg_next[p] = int(arg_pos[winner * B + p])
    return Selection(score, winner, margin, tok_next, conf_next, arg_next)


# ---------------------------------------------------------------------------
# Whole step and the pass that produces the state a step starts from
# ---------------------------------------------------------------------------

@dataclass
class StepOut:
    br: Branches
    H: np.ndarray          # [nb_max][B][hidden] float64 after rounding
    head: HeadOut          # per listed row
    conf_pos: np.ndarray   # [nb_max*B] float64 (0 where not listed)
    arg_pos: np.ndarray    # [nb_max*B] int64 (-1 where not listed)
    margin_pos: np.ndarray  # [nb_max*B] float64 (inf where not listed)
    sel: Selection
    ent_pos: np.ndarray | None = None   # [nb_max*B] float64 (0 where not listed)
    top_tok_pos: np.ndarray | None = None    # [nb_max*B][T] int64 (-1 where not listed)
    top_logit_pos: np.ndarray | None = None  # [nb_max*B][T] float64 (-inf where not listed)


def initial_state(inp) -> tuple[np.ndarray, np.ndarray, HeadOut]:
    """Confidence and argmax of the block's masked positions from one pass of
    branch slot 0 alone (the verification outputs a previous step would have
    left behind).  Returns conf [B] float32 (0 where filled), arg [B] int32
    (-1 where filled) and the head output of the masked rows."""
    cfg = inp.cfg
    H = branch_attn(inp.Kp, inp.Vp, inp.Qb, inp.Kb, inp.Vb, 1, cfg.Hq, cfg.Hkv)
    H = round_like(H, inp.Qb.dtype)
    masked = [p for p in range(cfg.B) if inp.tok[p] == MASK]
    head = lmhead_conf(H[0, masked, :], inp.W)
    conf = np.zeros(cfg.B, dtype=np.float32)
    arg = np.full(cfg.B, -1, dtype=np.int32)
    for i, p in enumerate(masked):
        conf[p] = np.float32(head.conf[i])
        arg[p] = head.arg[i]
    return conf, arg, head


def verification_step(inp, conf, arg, k: int | None = None,
                      tau: float | None = None, alpha: float | None = None,
                      gamma: float | None = None, temperature: float | None = None,
                      sample_seed: int = 0) -> StepOut:
    """One LoPA iteration: explore, verify (attention + LM head) and select.

    ``conf`` must be float32 (the library's input precision).  ``alpha``
    selects with ``branch_select_alpha`` instead of the mean confidence;
    ``gamma`` is branch_build's confidence floor for lookahead candidates;
    ``temperature`` draws each row's token from softmax(l / T)
    (sample_oracle.lmhead_sample, noise keyed by ``sample_seed``) instead of
    the argmax, its confidence being the drawn token's probability."""
    cfg = inp.cfg
    k = cfg.k if k is None else k
    tau = cfg.tau if tau is None else tau
    br = branch_build(inp.tok, conf, arg, k, np.float32(tau), cfg.nb_max,
                      None if gamma is None else np.float32(gamma))
    H = branch_attn(inp.Kp, inp.Vp, inp.Qb, inp.Kb, inp.Vb, br.nb, cfg.Hq, cfg.Hkv)
    H = round_like(H, inp.Qb.dtype)
    Hrows = np.stack([H[r // cfg.B, r % cfg.B] for r in br.rows]) if len(br.rows) \
        else np.zeros((0, cfg.hidden))
    head = lmhead_conf(Hrows, inp.W)
    if temperature is not None:
        from .sample_oracle import lmhead_sample
        smp = lmhead_sample(Hrows, inp.W, temperature, sample_seed, np.asarray(br.rows) % cfg.B)
        head = HeadOut(smp.conf, smp.arg, smp.margin, None, head.ent)
    n = cfg.nb_max * cfg.B
    conf_pos = np.zeros(n)
    arg_pos = np.full(n, -1, dtype=np.int64)
    margin_pos = np.full(n, np.inf)
    ent_pos = np.zeros(n)
    T = head.top_tok.shape[1] if head.top_tok is not None else 0
    top_tok_pos = np.full((n, T), -1, dtype=np.int64)
    top_logit_pos = np.full((n, T), -np.inf)
    for i, r in enumerate(br.rows):
        conf_pos[r] = head.conf[i]
        arg_pos[r] = head.arg[i]
        margin_pos[r] = head.margin[i]
        ent_pos[r] = head.ent[i]
        if T:
            top_tok_pos[r] = head.top_tok[i]
            top_logit_pos[r] = head.top_logit[i]
    if alpha is None:
        sel = branch_select(br.nb, br.br_mask, br.br_tok, conf_pos, arg_pos)
    else:
        sel = branch_select_alpha(br.nb, br.br_mask, br.br_tok, conf_pos, arg_pos, ent_pos,
                                  inp.tok, conf, alpha)
    return StepOut(br, H, head, conf_pos, arg_pos, margin_pos, sel, ent_pos, top_tok_pos,
                   top_logit_pos)
