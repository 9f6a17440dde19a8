"""CPU oracle for LoPA decoding of one block over several steps -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this module; the GPU library never does.

What it follows (page titles as in ``lopa_oracle``):
  [news]  "上交大 × 华为小艺推出LoPA：7B扩散语言模型单样例1000+ tokens/s！",
          section "LoPA 的核心设计：前瞻并行与分支验证": each iteration explores,
          verifies and selects, and the winner's verification outputs seed
          the next iteration, until the block is decoded; tokens per forward
          pass (TPF) is the figure of merit.
  [blog]  "解码效率革命：LoPA如何突破扩散语言模型的并行瓶颈", section 3.3
          (the winning branch's logits are reused by the next step).

Synthetic model.  There are no trained weights, so the projections a model
would compute for a branch's block are stood in for by vectors drawn from a
counter-based generator keyed by (seed, tensor, head, position, token,
dimension): branches agree wherever they hold the same token and differ only
where they fill differently, and every step's inputs follow from the tokens
alone.  The generator is Philox4x32-10 as published by Salmon, Moraes, Dror
and Shaw ("Parallel random numbers: as easy as 1, 2, 3", SC 2011; the
Random123 library), and each value is an Irwin-Hall sum of twelve 16-bit
uniforms minus 6 -- mean 0, variance 1, an integer multiple of 2^-16, so it
is exact in any float format before the one bf16 rounding.  The GPU library
implements the same published definition independently.

Readings (where the pages are silent):
  * the block is done when no position is masked; the number of steps is the
    number of verification passes after the initial one;
  * the state a block starts from comes from one pass of the initial tokens
    (branch slot 0 alone), as in ``lopa_oracle.initial_state``;
  * TPF = tokens decoded in the block / steps;
  * several blocks: once a block is decoded, the K and V of its final tokens
    -- the projections every branch slot already holds, so the winner's slot
    is kept by index rather than recomputed ([news] section
    "系统级创新：LoPA-Dist 分布式推理", its pre-write and commit-winner cache;
    [pop] the two-phase KV commit) -- are appended to the committed prefix,
    and the next block attends to the longer prefix.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np

from .lopa_oracle import MASK, branch_attn, branch_build, f64_to_bf16, lmhead_conf, \
    round_like, verification_step

# ---------------------------------------------------------------------------
# Philox4x32-10 (Salmon et al., SC 2011)
# ---------------------------------------------------------------------------

PHILOX_M0 = np.uint64(0xD2511F53)   # round multipliers
PHILOX_M1 = np.uint64(0xCD9E8D57)
PHILOX_W0 = np.uint32(0x9E3779B9)   # key increments (Weyl sequence)
PHILOX_W1 = np.uint32(0xBB67AE85)
_LO = np.uint64(0xFFFFFFFF)


def _mulhilo(m: np.uint64, x: np.ndarray):
    p = m * x.astype(np.uint64)
    return (p >> np.uint64(32)).astype(np.uint32), (p & _LO).astype(np.uint32)


def philox4x32_10(ctr: np.ndarray, key: np.ndarray) -> np.ndarray:
    """ctr [..., 4] uint32, key [..., 2] uint32 (broadcast) -> [..., 4] uint32.

    Ten rounds; each multiplies words 0 and 2 by the round multipliers, mixes
    the high halves with the other words and the round key, and the key
    advances by the Weyl increments between rounds."""
    x0, x1, x2, x3 = (ctr[..., i].astype(np.uint32) for i in range(4))
    k0 = np.broadcast_to(key[..., 0], x0.shape).astype(np.uint32)
    k1 = np.broadcast_to(key[..., 1], x0.shape).astype(np.uint32)
    for r in range(10):
        if r:   # 32-bit wrap-around
            k0 = ((k0.astype(np.uint64) + np.uint64(PHILOX_W0)) & _LO).astype(np.uint32)
            k1 = ((k1.astype(np.uint64) + np.uint64(PHILOX_W1)) & _LO).astype(np.uint32)
        hi0, lo0 = _mulhilo(PHILOX_M0, x0)
        hi1, lo1 = _mulhilo(PHILOX_M1, x2)
        x0, x1, x2, x3 = hi1 ^ x1 ^ k0, lo1, hi0 ^ x3 ^ k1, lo0
    return np.stack([x0, x1, x2, x3], axis=-1)


# ---------------------------------------------------------------------------
# Token-keyed synthetic projections
# ---------------------------------------------------------------------------

KIND_Q, KIND_K, KIND_V = 0, 1, 2


def irwin_hall(d0: np.ndarray, d1: np.ndarray) -> np.ndarray:
    """Twelve 16-bit uniforms -- the 8 halves of draw d0's four words and
    the 4 halves of draw d1's words 0 and 1 -- summed, minus 6, in float64
    (exact: an integer multiple of 2^-16 in [-6, 6))."""
    halves = [d0[..., i] & 0xFFFF for i in range(4)] + [d0[..., i] >> 16 for i in range(4)] + \
             [d1[..., i] & 0xFFFF for i in range(2)] + [d1[..., i] >> 16 for i in range(2)]
    s = np.zeros(d0.shape[:-1], dtype=np.int64)
    for h in halves:
        s += h.astype(np.int64)
    return (s - 6 * 65536).astype(np.float64) / 65536.0


def synth_values(seed: int, kind: int, heads: int, tokens: np.ndarray, d: int,
                 dtype=np.uint16) -> np.ndarray:
    """[nb][B][heads][d] values for branch tokens [nb][B], as bf16 bits
    (dtype uint16, rounded to nearest even) or float32 (exact).

    Element (b, p, h, e) uses key (seed low 32 bits, seed high 32 bits) and
    counters (p | kind << 8 | h << 16, token as uint32, e, draw) for draw 0
    and 1; only the position p within the block and the token enter, so two
    branches holding the same token at p get the same vectors there."""
    tokens = np.asarray(tokens, dtype=np.int64)
    nb, B = tokens.shape
    p = np.arange(B, dtype=np.uint32)[None, :, None, None]
    h = np.arange(heads, dtype=np.uint32)[None, None, :, None]
    e = np.arange(d, dtype=np.uint32)[None, None, None, :]
    t = (tokens & 0xFFFFFFFF).astype(np.uint32)[:, :, None, None]
    shape = (nb, B, heads, d)
    c0 = np.broadcast_to(p | np.uint32(kind << 8) | (h << np.uint32(16)), shape)
    c1 = np.broadcast_to(t, shape)
    c2 = np.broadcast_to(e, shape)
    key = np.array([seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF], dtype=np.uint32)
    draws = [philox4x32_10(np.stack([c0, c1, c2, np.full(shape, j, np.uint32)], -1), key)
             for j in (0, 1)]
    x = irwin_hall(*draws)
    return f64_to_bf16(x) if dtype == np.uint16 else x.astype(np.float32)


def token_qkv(seed: int, tokens: np.ndarray, Hq: int, Hkv: int, d: int, dtype=np.uint16):
    """Q [nb][B][Hq][d], K and V [nb][B][Hkv][d] for branch tokens [nb][B]."""
    return tuple(synth_values(seed, kind, heads, tokens, d, dtype)
                 for kind, heads in ((KIND_Q, Hq), (KIND_K, Hkv), (KIND_V, Hkv)))


# ---------------------------------------------------------------------------
# Block decoding
# ---------------------------------------------------------------------------

@dataclass
class DecodeStep:
    nb: int
    winner: int
    tok: np.ndarray          # [B] after the step
    filled: int              # positions filled by the step
    # how clear-cut the step's decisions were (for comparing with an
    # implementation that rounds differently):
    fill_margin: float       # smallest top-2 logit gap behind a token the step filled
    rank_gap: float          # smallest confidence gap the explore stage's choices hinged on
    tau_gap: float           # smallest |confidence - tau| over masked positions
    win_margin: float        # best minus second-best branch confidence


@dataclass
class DecodeTrace:
    tok0: np.ndarray
    conf0: np.ndarray
    arg0: np.ndarray
    init_margin: float
    steps: list = field(default_factory=list)

    @property
    def tpf(self) -> float:
        n = int(np.sum(self.tok0 == MASK))
        return n / max(len(self.steps), 1)


def _pad(a: np.ndarray, nb_max: int) -> np.ndarray:
    out = np.zeros((nb_max,) + a.shape[1:], dtype=a.dtype)
    out[:a.shape[0]] = a
    return out


def block_inputs(inp, seed: int, tokens: np.ndarray):
    """``inp`` with the per-branch projections replaced by the token-keyed ones."""
    cfg = inp.cfg
    Q, K, V = token_qkv(seed, tokens, cfg.Hq, cfg.Hkv, cfg.d, inp.Qb.dtype)
    return replace(inp, tok=np.asarray(tokens[0], np.int32), Qb=_pad(Q, cfg.nb_max),
                   Kb=_pad(K, cfg.nb_max), Vb=_pad(V, cfg.nb_max))


def _explore_gaps(tok, conf, tau, k, gamma=None):
    """Confidence gaps the explore stage's choices depend on: the threshold
    test of every masked position (and the candidate floor gamma, when
    given), the fallback's top-1 against top-2 when nothing passes it, and
    the order of the k+1 most confident positions the anchor leaves (which
    of them the lookahead branches fill)."""
    m = np.flatnonzero(tok == MASK)
    if m.size == 0:
        return np.inf, np.inf
    c = conf.astype(np.float64)
    tau_gap = float(np.min(np.abs(c[m] - tau)))
    if gamma is not None:
        tau_gap = min(tau_gap, float(np.min(np.abs(c[m] - gamma))))
    above = [p for p in m if c[p] > tau]
    gaps = []
    order = sorted(m, key=lambda p: (-c[p], p))
    if not above:
        if len(order) > 1:
            gaps.append(c[order[0]] - c[order[1]])
        fill = [order[0]]
    else:
        fill = above
    rest = [p for p in order if p not in fill][:k + 1]
    gaps += [c[a] - c[b] for a, b in zip(rest, rest[1:])]
    return (float(min(gaps)) if gaps else np.inf), tau_gap


def decode_block(inp, seed: int, k: int, tau: float, max_steps: int | None = None,
                 alpha: float | None = None, gamma: float | None = None,
                 temperature: float | None = None, sample_seed: int = 0) -> DecodeTrace:
    """Decode inp.tok's masked positions: the initial pass, then verification
    steps (explore, verify, select and reuse) until none is masked.  The
    committed prefix Kp, Vp and the weight W come from ``inp``; every
    branch's Q, K, V come from ``token_qkv`` of that branch's tokens.
    ``alpha`` selects with the alternative branch score
    (``lopa_oracle.branch_select_alpha``) instead of the mean confidence."""
    cfg = inp.cfg
    tok = np.asarray(inp.tok, np.int32).copy()
    # initial pass: branch slot 0 holds the block as it stands
    st = block_inputs(inp, seed, tok[None, :])
    H = round_like(branch_attn(st.Kp, st.Vp, st.Qb, st.Kb, st.Vb, 1, cfg.Hq, cfg.Hkv), st.Qb.dtype)
    masked = np.flatnonzero(tok == MASK)
    head = lmhead_conf(H[0, masked, :], inp.W)
    if temperature is not None:   # pass s draws with seed sample_seed + s (0: the initial pass)
        from .sample_oracle import lmhead_sample
        smp = lmhead_sample(H[0, masked, :], inp.W, temperature, sample_seed, masked)
        head = replace(head, conf=smp.conf, arg=smp.arg, margin=smp.margin)
    conf = np.zeros(cfg.B, np.float32)
    arg = np.full(cfg.B, -1, np.int32)
    conf[masked] = head.conf.astype(np.float32)
    arg[masked] = head.arg
    margin = np.full(cfg.B, np.inf)       # top-2 logit gap behind arg[p]
    margin[masked] = head.margin
    tr = DecodeTrace(tok.copy(), conf.copy(), arg.copy(),
                     float(head.margin.min()) if head.margin.size else np.inf)
    limit = int(masked.size) if max_steps is None else max_steps
    for _ in range(limit):
        if not np.any(tok == MASK):
            break
        g32 = None if gamma is None else np.float32(gamma)
        rank_gap, tau_gap = _explore_gaps(tok, conf, np.float64(np.float32(tau)), k,
                                          None if gamma is None else np.float64(g32))
        # explore with the state, then the projections of every branch's tokens
        br = branch_build(tok, conf, arg, k, np.float32(tau), cfg.nb_max, g32)
        st = block_inputs(inp, seed, br.br_tok.reshape(cfg.nb_max, cfg.B)[:br.nb])
        out = verification_step(replace(st, tok=tok), conf, arg, k, tau, alpha, gamma,
                                temperature, sample_seed + len(tr.steps) + 1)
        sel = out.sel
        bc = np.sort(np.asarray(sel.bconf[:out.br.nb], np.float64))[::-1]
        win_margin = float(bc[0] - bc[1]) if bc.size > 1 else np.inf
        new_tok = np.asarray(sel.tok_next, np.int32)
        filled = (tok == MASK) & (new_tok != MASK)
        tr.steps.append(DecodeStep(out.br.nb, int(sel.winner), new_tok.copy(), int(filled.sum()),
                                   float(margin[filled].min()) if filled.any() else np.inf,
                                   rank_gap, tau_gap, win_margin))
        w = int(sel.winner)
        margin = np.where(new_tok == MASK, out.margin_pos[w * cfg.B:(w + 1) * cfg.B], np.inf)
        tok = new_tok
        conf = np.asarray(sel.conf_next, np.float32)
        arg = np.asarray(sel.arg_next, np.int32)
    return tr


@dataclass
class SequenceTrace:
    blocks: list             # DecodeTrace per block
    Kp: np.ndarray           # committed prefix after the last block [L0 + n*B][Hkv][d]
    Vp: np.ndarray


def decode_sequence(inp, seed: int, k: int, tau: float, blocks) -> SequenceTrace:
    """Decode the blocks ``blocks`` (each an int32 [B] token array, MASK where
    masked) one after another.  Block j attends to inp's prefix plus the
    committed K, V of blocks 0..j-1: after a block is decoded, the K and V its
    final tokens map to (``token_qkv``) are appended to the prefix."""
    cfg = inp.cfg
    Kp, Vp = inp.Kp, inp.Vp
    traces = []
    for tok0 in blocks:
        cur = replace(inp, tok=np.asarray(tok0, np.int32), Kp=Kp, Vp=Vp,
                      cfg=replace(cfg, L=Kp.shape[0]))
        tr = decode_block(cur, seed, k, tau)
        traces.append(tr)
        final = tr.steps[-1].tok if tr.steps else np.asarray(tok0, np.int32)
        _, K, V = token_qkv(seed, final[None, :], cfg.Hq, cfg.Hkv, cfg.d, inp.Qb.dtype)
        Kp = np.concatenate([Kp, K[0]], axis=0)
        Vp = np.concatenate([Vp, V[0]], axis=0)
    return SequenceTrace(traces, Kp, Vp)
