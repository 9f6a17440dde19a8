"""Temperature sampling in the LM head (test infrastructure; only tests/,
__graft_entry__.smoke() and the benchmark's CPU-baseline leg use it).

"解码效率革命：LoPA如何突破扩散语言模型的并行瓶颈", section 5, recommends a
temperature between 0.7 and 1.1 instead of greedy decoding.  Reading: a
masked position's token is drawn from softmax(l / T) and its confidence is
that token's probability under the same distribution (greedy decoding is the
limit T -> 0).  The draw is Gumbel-max -- the argmax over v of l_v / T + G_v
with G_v = -ln(-ln u_v) is distributed as softmax(l / T) -- with the
uniforms u from Philox4x32-10 (this package's own implementation): key (seed
low, seed high), counter (v / 4, block position p, SAMPLE_TAG, 0), word
v % 4, u = (2 (x >> 9) + 1) 2^-24.  The noise depends on the position, not on
the branch.  float64 throughout.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

from .decode_oracle import philox4x32_10

SAMPLE_TAG = 0x5AB1E


def uniforms(seed: int, pos: int, V: int) -> np.ndarray:
    """u_v for v < V at block position pos (exact values in (0, 1))."""
    quads = (V + 3) // 4
    key = np.array([seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF], np.uint32)
    ctr = np.stack([np.arange(quads, dtype=np.uint32), np.full(quads, pos, np.uint32),
                    np.full(quads, SAMPLE_TAG, np.uint32), np.zeros(quads, np.uint32)], axis=-1)
    x = philox4x32_10(ctr, key).reshape(quads * 4)[:V].astype(np.int64)
    return (2 * (x >> 9) + 1) / float(1 << 24)


def gumbel(seed: int, pos: int, V: int) -> np.ndarray:
    return -np.log(-np.log(uniforms(seed, pos, V)))


@dataclass
class SampleOut:
    conf: np.ndarray     # [M] probability of the drawn token under softmax(l / T)
    arg: np.ndarray      # [M] drawn token
    margin: np.ndarray   # [M] best minus second-best perturbed score
    top_tok: np.ndarray | None = None     # [M][T] tokens of the T best perturbed scores
    top_score: np.ndarray | None = None   # [M][T] those scores, descending


def lmhead_sample(Hrows64: np.ndarray, W, T: float, seed: int, positions,
                  top: int = 16) -> SampleOut:
    """Rows Hrows64 [M][hidden] (float64) at block positions ``positions``
    [M]; W [V][hidden] (float32 or bf16 bits).  ``top``: also each row's
    ``top`` best perturbed scores and their tokens."""
    from .lopa_oracle import to_f64, top_logits
    W64 = to_f64(W)
    logits = Hrows64 @ W64.T
    V = W64.shape[0]
    M = logits.shape[0]
    conf = np.zeros(M)
    arg = np.zeros(M, dtype=np.int64)
    margin = np.full(M, math.inf)
    scores = np.zeros((M, V))
    for r in range(M):
        z = logits[r] / T
        score = z + gumbel(seed, int(positions[r]), V)
        scores[r] = score
        a = int(np.argmax(score))          # lowest index on a tie
        e = np.exp(z - z.max())
        conf[r] = e[a] / e.sum()
        arg[r] = a
        if V > 1:
            top2 = np.partition(score, -2)[-2:]
            margin[r] = float(top2[1] - top2[0])
    top_tok, top_score = top_logits(scores, top)
    return SampleOut(conf, arg, margin, top_tok, top_score)
