"""Pins of the explore stage with a confidence floor for lookahead
candidates (branch_build's ``gamma``: a branch count that follows the
state).  CPU only."""
import itertools

import numpy as np
import pytest

from oracle import lopa_oracle as O

M = O.MASK


def _state(rng, B, levels=None):
    tok = rng.integers(0, 500, B).astype(np.int32)
    tok[rng.random(B) < 0.7] = M
    conf = (rng.random(B) if levels is None else rng.choice(levels, B)).astype(np.float32)
    arg = rng.integers(0, 500, B).astype(np.int32)
    return tok, conf, arg


@pytest.mark.parametrize("seed", range(20))
def test_floor_at_or_below_zero_is_the_plain_build(seed):
    rng = np.random.default_rng(seed)
    tok, conf, arg = _state(rng, int(rng.integers(1, 40)))
    k = int(rng.integers(0, 8))
    a = O.branch_build(tok, conf, arg, k, np.float32(0.9), 8)
    for g in (0.0, -1.0):
        b = O.branch_build(tok, conf, arg, k, np.float32(0.9), 8, np.float32(g))
        assert a.nb == b.nb and np.array_equal(a.br_tok, b.br_tok)
        assert np.array_equal(a.rows, b.rows) and np.array_equal(a.row_ptr, b.row_ptr)


@pytest.mark.parametrize("seed", range(20))
def test_lookahead_set_by_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    levels = np.array([0.1, 0.2, 0.2, 0.5, 0.95], np.float32) if seed % 2 else None
    tok, conf, arg = _state(rng, int(rng.integers(1, 30)), levels)
    k = int(rng.integers(0, 8))
    gamma = np.float32([0.15, 0.2, 0.5, 2.0][seed % 4])
    br = O.branch_build(tok, conf, arg, k, np.float32(0.9), 9, gamma)
    masked = [p for p in range(len(tok)) if tok[p] == M]
    fill = O.anchor_fill_set(tok, conf, np.float32(0.9))
    cand = [p for p in masked if p not in fill and conf[p] >= gamma]
    # every subset of the candidates of the right size, ordered by (conf desc, pos asc):
    # the chosen one is the lexicographically best
    want = min(k, len(cand))
    best = sorted(cand, key=lambda p: (-float(conf[p]), p))[:want]
    for sub in itertools.combinations(cand, want):
        assert sorted((-float(conf[p]), p) for p in sub) >= sorted((-float(conf[p]), p) for p in best)
    assert br.lookahead == best and br.nb == 1 + want
    # the anchor is untouched by the floor
    assert br.anchor_fill == fill


def test_floor_above_every_confidence_leaves_the_anchor_alone():
    tok = np.array([M, M, 3, M], np.int32)
    conf = np.array([0.4, 0.3, 0.0, 0.2], np.float32)
    br = O.branch_build(tok, conf, np.array([7, 8, 0, 9], np.int32), 3, np.float32(0.9), 4,
                        np.float32(0.5))
    assert br.nb == 1 and br.anchor_fill == [0]
    assert list(br.br_tok[0]) == [7, M, 3, M]


def test_branch_count_never_grows_with_the_floor():
    rng = np.random.default_rng(7)
    for _ in range(30):
        tok, conf, arg = _state(rng, 24)
        nbs = [O.branch_build(tok, conf, arg, 6, np.float32(0.9), 7, np.float32(g)).nb
               for g in np.linspace(0, 1, 11)]
        assert all(a >= b for a, b in zip(nbs, nbs[1:]))
