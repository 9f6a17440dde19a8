"""Pins of the temperature-sampling oracle (oracle/sample_oracle.py), CPU.

* The noise is Gumbel: mean Euler-Mascheroni's constant, variance pi^2/6;
  every uniform is (2k + 1) / 2^24 in (0, 1).
* Gumbel-max draws from softmax(l / T): token frequencies over many seeds
  match scipy's softmax within four binomial standard deviations.
* T -> 0 gives the greedy argmax; the confidence is scipy's softmax(l / T)
  at the drawn token; equal logits at equal positions draw equal tokens.
"""
import math

import numpy as np
import pytest
from scipy.special import softmax

from oracle import sample_oracle as S


def test_gumbel_moments_and_uniform_grid():
    g = np.concatenate([S.gumbel(s, 7, 50000) for s in range(4)])
    se = math.pi / math.sqrt(6) / math.sqrt(g.size)
    assert abs(g.mean() - 0.5772156649015329) < 4 * se
    assert g.var() == pytest.approx(math.pi ** 2 / 6, rel=0.02)
    u = S.uniforms(3, 1, 4096)
    k = u * (1 << 24)
    assert np.all((u > 0) & (u < 1)) and np.array_equal(k, np.round(k)) and np.all(k % 2 == 1)


def test_draws_follow_softmax_at_temperature():
    l = np.array([[1.0, 0.2, -0.5, 2.0, 0.0, 1.1]])
    T = 0.8
    W = np.eye(6, dtype=np.float32)
    n = 6000
    counts = np.zeros(6)
    for s in range(n):
        counts[S.lmhead_sample(l, W, T, s, [0]).arg[0]] += 1
    p = softmax(l[0] / T)
    assert np.all(np.abs(counts / n - p) <= 4 * np.sqrt(p * (1 - p) / n))


def test_low_temperature_is_greedy_and_conf_is_the_softmax():
    rng = np.random.default_rng(0)
    H = rng.standard_normal((6, 16))
    W = rng.standard_normal((300, 16)).astype(np.float32)
    logits = H @ W.astype(np.float64).T
    srt = np.sort(logits, axis=1)
    assert np.all(srt[:, -1] - srt[:, -2] > 0.05)
    out = S.lmhead_sample(H, W, 1e-3, 9, np.arange(6))
    assert np.array_equal(out.arg, np.argmax(logits, axis=1))
    hot = S.lmhead_sample(H, W, 1.1, 9, np.arange(6))
    for r in range(6):
        assert hot.conf[r] == pytest.approx(softmax(logits[r] / 1.1)[hot.arg[r]], rel=1e-12)


def test_noise_depends_on_position_not_branch():
    rng = np.random.default_rng(1)
    h = rng.standard_normal((1, 8))
    W = rng.standard_normal((500, 8)).astype(np.float32)
    a = S.lmhead_sample(np.vstack([h, h]), W, 1.0, 4, [5, 5])   # two branches, one position
    assert a.arg[0] == a.arg[1]
    draws = {int(S.lmhead_sample(h, W, 1.0, 4, [p]).arg[0]) for p in range(12)}
    assert len(draws) > 1                                       # positions draw differently
