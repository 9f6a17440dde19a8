"""Oracle of the verification pass's layer forward (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this module; the GPU library never does.  Plain numpy in
float64, one branch at a time, with bf16 rounding (nearest even) at the
points the forward defines.  Shares nothing with the HIP path: the weight
generator is this module's own implementation of the published Philox
definition (``decode_oracle.philox4x32_10``).

What it computes (citations by page and section):

* The verify stage runs every branch through the model in one pass: news
  article "上交大 × 华为小艺推出LoPA：7B扩散语言模型单样例1000+ tokens/s！",
  section "LoPA 的核心设计：前瞻并行与分支验证", stage 并行验证与复用.  Each
  branch attends to the original input (the committed prefix) and its own
  tokens only ("解码效率革命：LoPA如何突破扩散语言模型的并行瓶颈", section 3.3);
  attention is full-sequence, not causal (same article, section 6).
* The pages name the model (D2F-Dream, 7B) but not its layers.  Reading:
  the Qwen2.5-7B decoder that Dream-7B is built on -- per layer
  RMSNorm -> q/k/v projections with bias -> rotary embedding -> attention
  -> output projection (residual) -> RMSNorm -> SwiGLU MLP (residual); token
  embedding in, final RMSNorm out (the LM head's input).
* Rotary embedding: pairs (i, i + d/2) of each q/k head turned by
  (L + p) * theta^(-2i/d) at block position p; cos and sin evaluated in
  double and rounded to float32 (the library's definition).
* Rounding points: normed rows, q/k/v, the attention output and the MLP
  activation are rounded to bf16; everything else is float64 here (float32
  accumulation on the GPU).
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

from .decode_oracle import philox4x32_10
from .lopa_oracle import MASK, attention_one_branch, bf16_to_f64, f64_to_bf16

TENSOR_ID = dict(attn_norm=0, wqkv=1, bqkv=2, wo=3, mlp_norm=4, wgu=5, wd=6, final_norm=7,
                 embed=8, lm_head=9, kp=10, vp=11)


def rnd(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bf16 (nearest even), returned as float64."""
    return bf16_to_f64(f64_to_bf16(np.asarray(x, np.float64)))


def fan_in_shift(K: int) -> int:
    """The integer nearest log2(sqrt(K / 12)): uniform weights of range
    2^-s have standard deviation 2^-s / sqrt(12), about 1 / sqrt(K)."""
    return int(math.floor(0.5 * math.log2(K / 12.0) + 0.5))


_FILL = None


def _fill_lib():
    """The C fast path of synth_tensor (oracle/philox_fill.c: the same
    generator with the bf16 rounding done on the integer), or None when it
    has not been built; both paths give identical values (a CPU test
    checks)."""
    global _FILL
    if _FILL is None:
        import ctypes
        import os
        path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_philox_fill.so")
        _FILL = False
        if os.path.exists(path):
            lib = ctypes.CDLL(path)
            lib.oracle_philox_fill_rows.argtypes = [
                ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_int64, ctypes.c_int64,
                ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
            lib.oracle_philox_fill_rows.restype = None
            _FILL = lib
    return _FILL or None


def synth_tensor(seed: int, tid: int, layer: int, rows: int, cols: int, rule: str,
                 shift: int = 0, use_c: bool = True) -> np.ndarray:
    """[rows][cols] float64 values (exact bf16 values).

    Word j of Philox4x32-10(counter (q, row, tid | layer << 8, 0), key (seed
    low, seed high)) gives column 4q + j.  rule "norm": 1 + ((x >> 27) - 16)
    / 128 (exact in bf16); rule "uniform": ((x >> 8) - 2^23) * 2^(-24 - shift), rounded to
    bf16."""
    lib = _fill_lib() if use_c else None
    if lib is not None:
        out = np.empty((rows, cols), np.float64)
        lib.oracle_philox_fill_rows(seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF,
                                    tid | (layer << 8), 0, rows, cols, 1 if rule == "norm" else 0,
                                    shift, out.ctypes.data)
        return out
    return _synth_rows_np(seed, tid, layer, 0, rows, cols, rule, shift)


def _synth_rows_np(seed: int, tid: int, layer: int, r0: int, r1: int, cols: int, rule: str,
                   shift: int) -> np.ndarray:
    """Rows r0..r1-1 of synth_tensor, numpy only (the definition)."""
    quads = (cols + 3) // 4
    key = np.array([seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF], np.uint32)
    out = np.empty((r1 - r0, cols), np.float64)
    step = max(1, (1 << 22) // max(quads, 1))
    for a in range(r0, r1, step):
        b = min(r1, a + step)
        q = np.broadcast_to(np.arange(quads, dtype=np.uint32)[None, :], (b - a, quads))
        rr = np.broadcast_to(np.arange(a, b, dtype=np.uint32)[:, None], (b - a, quads))
        ctr = np.stack([q, rr, np.full(q.shape, tid | (layer << 8), np.uint32),
                        np.zeros(q.shape, np.uint32)], axis=-1)
        x = philox4x32_10(ctr, key).reshape(b - a, quads * 4)[:, :cols].astype(np.int64)
        if rule == "norm":
            out[a - r0:b - r0] = 1.0 + ((x >> 27) - 16) / 128.0
        else:
            out[a - r0:b - r0] = rnd(((x >> 8) - (1 << 23)) * 2.0 ** (-24 - shift))
    return out


@dataclass
class ModelCfg:
    """Geometry of the decoder (Qwen2.5/Dream-7B: hidden 3584, 28 layers,
    Hq 28, Hkv 4, d 128, inter 18944, V 152064, theta 1e6, eps 1e-6)."""
    n_layers: int
    Hq: int
    Hkv: int
    d: int
    inter: int
    V: int
    mask_id: int
    rope_theta: float = 1e6
    rms_eps: float = 1e-6

    @property
    def hidden(self) -> int:
        return self.Hq * self.d

    @property
    def qkv(self) -> int:
        return (self.Hq + 2 * self.Hkv) * self.d


class Proj:
    """A projection weight W [N][K] of the synthetic model, applied as
    x @ W^T.  W is drawn in blocks of rows into a reused buffer (the
    generator is counter-based, so a block of rows is the same whether drawn
    alone or with the rest); each output column is still one dot product of
    x with one weight row."""
    BLOCK = 1024
    _buf = None

    def __init__(self, seed: int, tid: int, layer: int, N: int, K: int, shift: int):
        self.seed, self.tid, self.layer, self.N, self.K, self.shift = seed, tid, layer, N, K, shift

    def rows(self, r0: int, r1: int) -> np.ndarray:
        lib = _fill_lib()
        if lib is None:
            return _synth_rows_np(self.seed, self.tid, self.layer, r0, r1, self.K, "uniform",
                                  self.shift)
        need = (r1 - r0) * self.K
        if Proj._buf is None or Proj._buf.size < need:
            Proj._buf = np.empty(max(need, self.BLOCK * 4096), np.float64)
        out = Proj._buf[:need].reshape(r1 - r0, self.K)
        lib.oracle_philox_fill_rows(self.seed & 0xFFFFFFFF, (self.seed >> 32) & 0xFFFFFFFF,
                                    self.tid | (self.layer << 8), r0, r1, self.K, 0, self.shift,
                                    out.ctypes.data)
        return out

    def full(self) -> np.ndarray:
        return np.concatenate([self.rows(r, min(self.N, r + self.BLOCK)).copy()
                               for r in range(0, self.N, self.BLOCK)])

    def __call__(self, x: np.ndarray) -> np.ndarray:
        y = np.empty((x.shape[0], self.N))
        for r in range(0, self.N, self.BLOCK):
            r1 = min(self.N, r + self.BLOCK)
            y[:, r:r1] = x @ self.rows(r, r1).T
        return y


@dataclass
class Layer:
    attn_norm: np.ndarray   # [hidden]
    wqkv: Proj              # [qkv][hidden]: q rows, then k, then v
    bqkv: np.ndarray        # [qkv]
    wo: Proj                # [hidden][Hq d]
    mlp_norm: np.ndarray    # [hidden]
    wgu: Proj               # [2 inter][hidden]: gate rows, then up rows
    wd: Proj                # [hidden][inter]


def synth_layer(seed: int, cfg: ModelCfg, l: int) -> Layer:
    h = cfg.hidden
    return Layer(
        synth_tensor(seed, 0, l, 1, h, "norm")[0],
        Proj(seed, 1, l, cfg.qkv, h, fan_in_shift(h)),
        synth_tensor(seed, 2, l, 1, cfg.qkv, "uniform", 2)[0],
        Proj(seed, 3, l, h, cfg.Hq * cfg.d, fan_in_shift(cfg.Hq * cfg.d)),
        synth_tensor(seed, 4, l, 1, h, "norm")[0],
        Proj(seed, 5, l, 2 * cfg.inter, h, fan_in_shift(h)),
        Proj(seed, 6, l, h, cfg.inter, fan_in_shift(cfg.inter)))


def synth_prefix(seed: int, cfg: ModelCfg, l: int, L: int):
    """Prefix keys and values of layer l: [L][Hkv][d], uniform on (-1, 1)."""
    c = cfg.Hkv * cfg.d
    K = synth_tensor(seed, 10, l, L, c, "uniform", -1).reshape(L, cfg.Hkv, cfg.d)
    V = synth_tensor(seed, 11, l, L, c, "uniform", -1).reshape(L, cfg.Hkv, cfg.d)
    return K, V


def synth_rows(seed: int, cfg: ModelCfg, tid: int, rows) -> np.ndarray:
    """Selected rows [len(rows)][hidden] of the embedding (tid 8) or the LM
    head (tid 9); the generator is counter-based, so a row can be drawn
    alone."""
    # the LM head is four times wider than fan-in scaling (logit spread ~4)
    shift = 1 if tid == TENSOR_ID["embed"] else fan_in_shift(cfg.hidden) - 2
    quads = (cfg.hidden + 3) // 4
    key = np.array([seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF], np.uint32)
    rows = np.asarray(rows, np.uint32)
    ctr = np.stack(np.broadcast_arrays(np.arange(quads, dtype=np.uint32)[None, :],
                                       rows[:, None], np.uint32(tid), np.uint32(0)), axis=-1)
    x = philox4x32_10(ctr, key).reshape(len(rows), quads * 4)[:, :cfg.hidden].astype(np.int64)
    return rnd(((x >> 8) - (1 << 23)) * 2.0 ** (-24 - shift))


# ---------------------------------------------------------------------------
# The forward
# ---------------------------------------------------------------------------

def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * g, row-wise."""
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * g


def rope_cos_sin(positions: np.ndarray, d: int, theta: float):
    """cos, sin [len(positions)][d/2] of the angles pos * theta^(-2i/d),
    evaluated in double and rounded to float32 (the library's definition)."""
    i = np.arange(d // 2, dtype=np.float64)
    ang = positions[:, None].astype(np.float64) * np.exp2(-2.0 * i / d * math.log2(theta))
    return np.cos(ang).astype(np.float32).astype(np.float64), \
        np.sin(ang).astype(np.float32).astype(np.float64)


def rope(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """x [B][heads][d]: pair (i, i + d/2) turned by the position's angle i."""
    h = x.shape[-1] // 2
    a, b = x[..., :h], x[..., h:]
    c, s = cos[:, None, :], sin[:, None, :]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


@dataclass
class ForwardOut:
    H: np.ndarray        # [nb][B][hidden] final-normed rows (bf16 values)
    Kb: np.ndarray       # [n_layers][nb][B][Hkv][d] block keys (rotated, bf16 values)
    Vb: np.ndarray       # [n_layers][nb][B][Hkv][d]


def layer_forward(cfg: ModelCfg, w: Layer, x: np.ndarray, Kp: np.ndarray, Vp: np.ndarray,
                  L: int, round_points: bool = True):
    """One decoder layer on the rows x [nb][B][hidden] of nb branches (float64,
    the residual stream).  Projections act on each row alone; attention runs
    each branch on its own (prefix + its own block).  Returns (x after the
    layer, k, v) with k, v [nb][B][Hkv][d] the blocks' rotated keys and
    values."""
    R = rnd if round_points else (lambda a: a)
    nb, B, hid = x.shape
    rows = x.reshape(nb * B, hid)
    h = R(rmsnorm(rows, w.attn_norm, cfg.rms_eps))
    y = w.wqkv(h) + w.bqkv
    qd, kd = cfg.Hq * cfg.d, cfg.Hkv * cfg.d
    q = y[:, :qd].reshape(nb, B, cfg.Hq, cfg.d)
    k = y[:, qd:qd + kd].reshape(nb, B, cfg.Hkv, cfg.d)
    v = y[:, qd + kd:].reshape(nb, B, cfg.Hkv, cfg.d)
    cos, sin = rope_cos_sin(L + np.arange(B), cfg.d, cfg.rope_theta)
    q = R(np.stack([rope(q[b], cos, sin) for b in range(nb)]))
    k = R(np.stack([rope(k[b], cos, sin) for b in range(nb)]))
    v = R(v)
    o = R(np.concatenate([attention_one_branch(Kp, Vp, q[b], k[b], v[b], cfg.Hq, cfg.Hkv)
                          for b in range(nb)]))
    rows = rows + w.wo(o)
    h = R(rmsnorm(rows, w.mlp_norm, cfg.rms_eps))
    gu = w.wgu(h)
    a = R(silu(gu[:, :cfg.inter]) * gu[:, cfg.inter:])
    rows = rows + w.wd(a)
    return rows.reshape(nb, B, hid), k, v


def embed_rows(seed: int, cfg: ModelCfg, tok: np.ndarray) -> np.ndarray:
    """x [B][hidden]: each token's embedding row, the mask_id row where masked."""
    ids = np.where(np.asarray(tok) == MASK, cfg.mask_id, np.clip(tok, 0, cfg.V - 1))
    uniq = np.unique(ids)
    rows = dict(zip(uniq.tolist(), synth_rows(seed, cfg, TENSOR_ID["embed"], uniq)))
    return np.stack([rows[int(i)] for i in ids])


def forward(seed: int, cfg: ModelCfg, L: int, br_tok: np.ndarray, layers=None,
            prefix=None, round_points: bool = True) -> ForwardOut:
    """All branches' blocks br_tok [nb][B] through the model.  ``layers`` /
    ``prefix`` may carry already drawn weights (synth_layer) and prefix
    caches (synth_prefix) to save time."""
    R = rnd if round_points else (lambda a: a)
    br_tok = np.asarray(br_tok)
    nb, B = br_tok.shape
    if layers is None:
        layers = [synth_layer(seed, cfg, l) for l in range(cfg.n_layers)]
    if prefix is None:
        prefix = [synth_prefix(seed, cfg, l, L) for l in range(cfg.n_layers)]
    final = synth_tensor(seed, 7, 0, 1, cfg.hidden, "norm")[0]
    Kb = np.zeros((cfg.n_layers, nb, B, cfg.Hkv, cfg.d))
    Vb = np.zeros_like(Kb)
    x = np.stack([embed_rows(seed, cfg, br_tok[b]) for b in range(nb)])
    for l in range(cfg.n_layers):
        x, Kb[l], Vb[l] = layer_forward(cfg, layers[l], x, prefix[l][0], prefix[l][1], L,
                                        round_points)
    return ForwardOut(R(rmsnorm(x, final, cfg.rms_eps)), Kb, Vb)


# ---------------------------------------------------------------------------
# Decoding blocks with the model
# ---------------------------------------------------------------------------

def lm_head_weight(seed: int, cfg: ModelCfg) -> np.ndarray:
    """The model's LM head [V][hidden] (bf16 values)."""
    return synth_rows(seed, cfg, TENSOR_ID["lm_head"], np.arange(cfg.V)).astype(np.float32)


def initial_pass(seed: int, cfg: ModelCfg, L: int, tok, layers, prefix, W):
    """The block as it stands through the model and the LM head on its masked
    positions.  Returns (conf [B] float32, arg [B] int32, margin [B]: the
    top-2 logit gap behind each masked position's token, inf elsewhere,
    the forward's output)."""
    from .lopa_oracle import lmhead_conf
    tok = np.asarray(tok, np.int32)
    B = len(tok)
    out = forward(seed, cfg, L, tok[None], layers, prefix)
    masked = np.flatnonzero(tok == MASK)
    head = lmhead_conf(out.H[0, masked, :], W)
    conf = np.zeros(B, np.float32)
    arg = np.full(B, -1, np.int32)
    conf[masked] = head.conf.astype(np.float32)
    arg[masked] = head.arg
    margin = np.full(B, np.inf)
    margin[masked] = head.margin
    return conf, arg, margin, out


def decode_step(seed: int, cfg: ModelCfg, L: int, tok, conf, arg, margin, k: int, tau: float,
                nb_max: int, layers, prefix, W):
    """One verification step with the model from the state (tok, conf, arg):
    explore (lopa_oracle.branch_build), every branch through the model, the
    LM head on the still-masked rows, select and reuse.  ``margin`` [B] is
    the top-2 logit gap behind each masked position's arg.  Returns
    (decode_oracle.DecodeStep, the next (tok, conf, arg, margin), the
    forward's output, the winner, the branches (lopa_oracle.Branches) and
    the top-2 logit gap of every LM-head row [nb_max * B], inf elsewhere)."""
    from .decode_oracle import DecodeStep, _explore_gaps
    from .lopa_oracle import branch_build, branch_select, lmhead_conf
    B = len(tok)
    rank_gap, tau_gap = _explore_gaps(tok, conf, np.float64(np.float32(tau)), k)
    br = branch_build(tok, conf, arg, k, np.float32(tau), nb_max)
    out = forward(seed, cfg, L, br.br_tok[:br.nb], layers, prefix)
    rows = np.asarray(br.rows)
    n = nb_max * B
    conf_pos, arg_pos, margin_pos = np.zeros(n), np.full(n, -1), np.full(n, np.inf)
    if rows.size:
        h = lmhead_conf(np.stack([out.H[r // B, r % B] for r in rows]), W)
        conf_pos[rows], arg_pos[rows], margin_pos[rows] = h.conf, h.arg, h.margin
    sel = branch_select(br.nb, br.br_mask, br.br_tok, conf_pos, arg_pos)
    bc = np.sort(np.asarray(sel.bconf[:br.nb], np.float64))[::-1]
    new_tok = np.asarray(sel.tok_next, np.int32)
    filled = (tok == MASK) & (new_tok != MASK)
    w = int(sel.winner)
    step = DecodeStep(br.nb, w, new_tok.copy(), int(filled.sum()),
                      float(margin[filled].min()) if filled.any() else np.inf,
                      rank_gap, tau_gap, float(bc[0] - bc[1]) if bc.size > 1 else np.inf)
    nxt = (new_tok, np.asarray(sel.conf_next, np.float32), np.asarray(sel.arg_next, np.int32),
           np.where(new_tok == MASK, margin_pos[w * B:(w + 1) * B], np.inf))
    return step, nxt, out, w, br, margin_pos


def decode_block(seed: int, cfg: ModelCfg, L: int, tok0, k: int, tau: float, nb_max: int,
                 layers=None, prefix=None, max_steps: int | None = None):
    """Decode tok0's masked positions with the model: the initial pass (the
    block alone through the model, the LM head on its masked positions),
    then verification steps (decode_step) until none is masked (news
    article, section "LoPA 的核心设计：前瞻并行与分支验证"; the LM head weight
    is the model's).  Returns the trace (decode_oracle.DecodeTrace) and the
    winner's block keys and values of every layer from the last pass
    ([n_layers][B][Hkv][d] each), the cache a commit appends."""
    from .decode_oracle import DecodeTrace
    if layers is None:
        layers = [synth_layer(seed, cfg, l) for l in range(cfg.n_layers)]
    if prefix is None:
        prefix = [synth_prefix(seed, cfg, l, L) for l in range(cfg.n_layers)]
    W = lm_head_weight(seed, cfg)
    tok = np.asarray(tok0, np.int32).copy()
    conf, arg, margin, out = initial_pass(seed, cfg, L, tok, layers, prefix, W)
    masked = np.isfinite(margin)
    tr = DecodeTrace(tok.copy(), conf.copy(), arg.copy(),
                     float(margin[masked].min()) if masked.any() else np.inf)
    Kw, Vw = out.Kb[:, 0], out.Vb[:, 0]
    limit = int(np.sum(tok == MASK)) if max_steps is None else max_steps
    for _ in range(limit):
        if not np.any(tok == MASK):
            break
        st, (tok, conf, arg, margin), out, w, _, _ = decode_step(
            seed, cfg, L, tok, conf, arg, margin, k, tau, nb_max, layers, prefix, W)
        tr.steps.append(st)
        Kw, Vw = out.Kb[:, w], out.Vb[:, w]
    return tr, Kw, Vw


def decode_sequence(seed: int, cfg: ModelCfg, L: int, blocks, k: int, tau: float, nb_max: int):
    """Decode ``blocks`` one after another, appending each decoded block's
    winner keys and values of every layer to that layer's prefix (the
    commit of the news article's section "系统级创新：LoPA-Dist 分布式推理",
    one GPU).  Returns the traces and the final per-layer prefixes."""
    layers = [synth_layer(seed, cfg, l) for l in range(cfg.n_layers)]
    prefix = [synth_prefix(seed, cfg, l, L) for l in range(cfg.n_layers)]
    traces = []
    for tok0 in blocks:
        tr, Kw, Vw = decode_block(seed, cfg, L, tok0, k, tau, nb_max, layers, prefix)
        traces.append(tr)
        prefix = [(np.concatenate([prefix[l][0], Kw[l]]), np.concatenate([prefix[l][1], Vw[l]]))
                  for l in range(cfg.n_layers)]
        L += len(tok0)
    return traces, prefix
