"""Seeded synthetic inputs for one LoPA branch-verification step.

This module is shared by the CPU oracle (``oracle/``), the tests and the
benchmark.  It holds none of the method's arithmetic: it only draws the
random inputs of a step (block tokens, prefix K/V, per-branch Q/K/V and the
LM-head weight) and stores them in the byte layouts that the C-ABI library
reads.  Nothing here decodes, attends or scores.

Workload shapes follow the 7B D2F-Dream setting that the LoPA articles
report on (Qwen2.5/Dream-7B geometry: 28 query heads, 4 KV heads, head dim
128, hidden 3584, vocabulary 152064); the GSM8K / MBPP / HumanEval+ runs the
articles quote are replaced by these seeded draws.

Draw recipe (each workload carries its own default seed):
  1. masked block positions: ``choice(B, m, replace=False)``
  2. committed block tokens: ``integers(0, V, size=B)`` (masked ones set to -1)
  3. prefix keys Kp [L][Hkv][d], 4. prefix values Vp,
  5. Qb [nb_max][B][Hq][d], 6. Kb [nb_max][B][Hkv][d], 7. Vb (same shape)
     -- all ``standard_normal`` float32, rounded to bf16 (RNE) for bf16 configs;
  8. the LM-head weight W [V][hidden] (vocab-major): ``standard_normal``
     float32 drawn in 64 fixed row chunks from child streams of
     ``SeedSequence([seed, 87])`` (so it can be drawn by several threads and
     still be identical), times ``4 / (sigma_h * sqrt(hidden))`` with
     ``sigma_h = sqrt(e / (L + B))``, then rounded to the activation dtype.

``sigma_h`` is the expected RMS of one attention-output element when scores
are N(0,1) over n = L + B keys and values are N(0,1): the sum of squared
softmax weights concentrates at e/n.  With that scale a row's logits over
the vocabulary have a standard deviation of about 4, as the workload asks.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, asdict

import numpy as np

MASK = -1
F32 = "f32"
BF16 = "bf16"
W_CHUNKS = 64


@dataclass(frozen=True)
class StepConfig:
    """Shape of one verification step.

    ``k`` is the lookahead count, so a step has at most ``1 + k`` branches;
    ``m`` is the number of masked block positions at step start; ``tau`` is
    the anchor's fill threshold.
    """
    name: str
    dtype: str
    L: int
    B: int
    m: int
    k: int
    Hq: int
    Hkv: int
    d: int
    V: int
    tau: float = 0.9
    seed: int = 1000

    @property
    def hidden(self) -> int:
        return self.Hq * self.d

    @property
    def nb_max(self) -> int:
        return 1 + self.k

    def describe(self) -> dict:
        out = asdict(self)
        out["hidden"] = self.hidden
        out["nb_max"] = self.nb_max
        return out


# The five workloads: a tiny fp32 case the oracle finishes instantly, and
# four 7B-shaped bf16 cases (prefix 512..4096, block 32/64, 5..16 branches).
# Threshold 0.9 for all; the 16-branch case has 24 of 32 positions masked.
_W = [
    StepConfig("tiny-f32-L64-B16-m8-k3", F32, L=64, B=16, m=8, k=3,
               Hq=4, Hkv=4, d=64, V=1024, seed=1001),
    StepConfig("7b-bf16-L512-B32-m24-k4", BF16, L=512, B=32, m=24, k=4,
               Hq=28, Hkv=4, d=128, V=152064, seed=1002),
    StepConfig("7b-bf16-L2048-B32-m28-k8", BF16, L=2048, B=32, m=28, k=8,
               Hq=28, Hkv=4, d=128, V=152064, seed=1003),
    StepConfig("7b-bf16-L1024-B32-m24-k15", BF16, L=1024, B=32, m=24, k=15,
               Hq=28, Hkv=4, d=128, V=152064, seed=1004),
    StepConfig("7b-bf16-L4096-B64-m48-k8", BF16, L=4096, B=64, m=48, k=8,
               Hq=28, Hkv=4, d=128, V=152064, seed=1005),
]
WORKLOADS = {c.name: c for c in _W}
TINY = _W[0].name
SEVEN_B = [c.name for c in _W[1:]]
HEADLINE = _W[1].name   # prefix 512, block 32, 5 branches


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); return the raw
    16-bit patterns as uint16.  Used only to store drawn inputs."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == F32:
        return np.ascontiguousarray(x, dtype=np.float32)
    return f32_to_bf16_bits(x)


def weight_scale(cfg: StepConfig) -> float:
    sigma_h = math.sqrt(math.e / (cfg.L + cfg.B))
    return 4.0 / (sigma_h * math.sqrt(cfg.hidden))


def draw_weight(cfg: StepConfig, seed: int, scale: float | None = None,
                threads: int | None = None) -> np.ndarray:
    """W [V][hidden] in the activation dtype (uint16 bits for bf16)."""
    scale = weight_scale(cfg) if scale is None else scale
    V, hid = cfg.V, cfg.hidden
    bounds = np.linspace(0, V, W_CHUNKS + 1).astype(np.int64)
    children = np.random.SeedSequence([seed, 87]).spawn(W_CHUNKS)
    out_dtype = np.float32 if cfg.dtype == F32 else np.uint16
    W = np.empty((V, hid), dtype=out_dtype)
    sc = np.float32(scale)

    def fill(i: int) -> None:
        lo, hi = int(bounds[i]), int(bounds[i + 1])
        if hi == lo:
            return
        g = np.random.Generator(np.random.PCG64(children[i]))
        w0 = g.standard_normal((hi - lo, hid), dtype=np.float32)
        w0 *= sc
        W[lo:hi] = _store(w0, cfg.dtype)

    n = threads or min(16, os.cpu_count() or 1)
    with ThreadPoolExecutor(max_workers=n) as ex:
        list(ex.map(fill, range(W_CHUNKS)))
    return W


@dataclass
class StepInputs:
    cfg: StepConfig
    seed: int
    tok: np.ndarray          # [B] int32, MASK at masked positions
    Kp: np.ndarray           # [L][Hkv][d]
    Vp: np.ndarray           # [L][Hkv][d]
    Qb: np.ndarray           # [nb_max][B][Hq][d]
    Kb: np.ndarray           # [nb_max][B][Hkv][d]
    Vb: np.ndarray           # [nb_max][B][Hkv][d]
    W: np.ndarray | None = field(default=None)   # [V][hidden]

    def arrays(self) -> dict:
        return {k: getattr(self, k) for k in ("tok", "Kp", "Vp", "Qb", "Kb", "Vb", "W")}


def make_inputs(cfg: StepConfig | str, seed: int | None = None,
                with_weight: bool = True, **overrides) -> StepInputs:
    """Draw every input of one step, in the fixed order stated above.

    ``cfg`` is a StepConfig or a workload name; ``overrides`` replaces
    fields of it (parity cases with ragged or edge-case shapes), e.g.
    ``make_inputs(TINY, L=0, B=5)``.
    """
    if isinstance(cfg, str):
        cfg = WORKLOADS[cfg]
    if overrides:
        cfg = StepConfig(**{**asdict(cfg), **overrides})
    if seed is None:
        seed = cfg.seed
    if not (0 <= cfg.m <= cfg.B):
        raise ValueError("m must lie in [0, B]")
    g = np.random.Generator(np.random.PCG64(seed))
    masked = g.choice(cfg.B, cfg.m, replace=False)
    tok = g.integers(0, cfg.V, size=cfg.B).astype(np.int32)
    tok[masked] = MASK
    nbm = cfg.nb_max
    Kp = _store(g.standard_normal((cfg.L, cfg.Hkv, cfg.d), dtype=np.float32), cfg.dtype)
    Vp = _store(g.standard_normal((cfg.L, cfg.Hkv, cfg.d), dtype=np.float32), cfg.dtype)
    Qb = _store(g.standard_normal((nbm, cfg.B, cfg.Hq, cfg.d), dtype=np.float32), cfg.dtype)
    Kb = _store(g.standard_normal((nbm, cfg.B, cfg.Hkv, cfg.d), dtype=np.float32), cfg.dtype)
    Vb = _store(g.standard_normal((nbm, cfg.B, cfg.Hkv, cfg.d), dtype=np.float32), cfg.dtype)
    W = draw_weight(cfg, seed) if with_weight else None
    return StepInputs(cfg, seed, tok, Kp, Vp, Qb, Kb, Vb, W)
