"""Pins for the oracle's branch construction (explore stage).

What the articles fix: the anchor is the ordinary greedy confidence-driven
branch, and each lookahead branch additionally fills one of the currently
most confident positions.  The tests below pin the oracle with a worked
example done by hand, the k = 0 reduction to plain confidence-driven
sampling (written separately here), a rank-count recomputation of the
lookahead positions, and structural invariants on random inputs with ties.
"""
import itertools

import numpy as np
import pytest

import oracle as O

M = O.MASK


def test_oracle_build_hand_example():
    # B = 6, positions 0,2,3,5 masked.  conf: p2 = 0.95 passes tau = 0.9, so
    # the anchor fills p2 only.  Remaining {0, 3, 5} ranked by confidence:
    # p5 (0.6), p0 (0.4), p3 (0.4; ties go to the lower position -> p0 first).
    tok = np.array([M, 7, M, M, 9, M], np.int32)
    conf = np.array([0.4, 0, 0.95, 0.4, 0, 0.6], np.float32)
    arg = np.array([10, -1, 12, 13, -1, 15], np.int32)
    br = O.branch_build(tok, conf, arg, k=2, tau=np.float32(0.9), nb_max=4)
    assert br.nb == 3
    assert br.anchor_fill == [2]
    assert br.lookahead == [5, 0]
    assert br.br_tok[0].tolist() == [M, 7, 12, M, 9, M]
    assert br.br_tok[1].tolist() == [M, 7, 12, M, 9, 15]
    assert br.br_tok[2].tolist() == [10, 7, 12, M, 9, M]
    assert br.br_tok[3].tolist() == br.br_tok[0].tolist()      # unused slot
    assert br.br_mask[3].tolist() == [0] * 6
    # rows b*B+p, branch-major, p ascending
    assert br.rows.tolist() == [0, 3, 5, 6, 9, 15, 17]
    assert br.row_ptr.tolist() == [0, 3, 5, 7, 7]


def test_oracle_build_fallback_fills_top1():
    # nothing above tau: the anchor fills the single most confident masked
    # position, lowest position on a tie
    tok = np.array([M, M, M, 4], np.int32)
    conf = np.array([0.3, 0.5, 0.5, 0.99], np.float32)   # p3 is not masked
    arg = np.array([1, 2, 3, -1], np.int32)
    br = O.branch_build(tok, conf, arg, k=5, tau=np.float32(0.9), nb_max=6)
    assert br.anchor_fill == [1]
    assert br.lookahead == [2, 0]        # k clipped to the 2 remaining
    assert br.nb == 3


def test_oracle_build_threshold_is_strict():
    tok = np.array([M, M], np.int32)
    conf = np.array([0.9, 0.2], np.float32)
    br = O.branch_build(tok, conf, np.array([5, 6], np.int32), 1, np.float32(0.9), 2)
    assert br.anchor_fill == [0]         # via the top-1 fallback, not the threshold
    conf = np.array([0.9, 0.95], np.float32)
    br = O.branch_build(tok, conf, np.array([5, 6], np.int32), 1, np.float32(0.9), 2)
    assert br.anchor_fill == [1]


def test_oracle_build_nothing_masked():
    tok = np.array([1, 2, 3], np.int32)
    br = O.branch_build(tok, np.zeros(3, np.float32), np.zeros(3, np.int32), 3,
                        np.float32(0.9), 4)
    assert br.nb == 1 and br.anchor_fill == [] and len(br.rows) == 0
    assert br.row_ptr.tolist() == [0] * 5
    assert br.br_tok[0].tolist() == [1, 2, 3]


def _confidence_driven(tok, conf, arg, tau):
    """Plain confidence-driven sampling, written independently: fill every
    masked position above tau, else the single argmax of confidence."""
    tok = tok.copy()
    idx = np.flatnonzero(tok == M)
    if idx.size == 0:
        return tok
    above = idx[conf[idx] > tau]
    pick = above if above.size else idx[[int(np.argmax(conf[idx]))]]
    tok[pick] = arg[pick]
    return tok


def _random_state(rng, B, levels=None):
    tok = rng.integers(0, 50, B).astype(np.int32)
    nmask = rng.integers(0, B + 1)
    tok[rng.choice(B, nmask, replace=False)] = M
    if levels is None:
        conf = rng.random(B).astype(np.float32)
    else:   # few distinct values -> many exact ties
        conf = rng.choice(np.array(levels, np.float32), B)
    arg = rng.integers(100, 200, B).astype(np.int32)
    return tok, conf, arg


@pytest.mark.parametrize("seed", range(200))
def test_oracle_build_k0_is_confidence_driven(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 12))
    tok, conf, arg = _random_state(rng, B, [0.2, 0.5, 0.91, 0.95] if seed % 2 else None)
    br = O.branch_build(tok, conf, arg, 0, np.float32(0.9), 1)
    assert br.nb == 1
    assert np.array_equal(br.br_tok[0], _confidence_driven(tok, conf, arg, np.float32(0.9)))


@pytest.mark.parametrize("seed", range(300))
def test_oracle_build_invariants_and_rank_count(seed):
    rng = np.random.default_rng(10_000 + seed)
    B = int(rng.integers(1, 10))
    k = int(rng.integers(0, 6))
    tok, conf, arg = _random_state(rng, B, [0.1, 0.3, 0.3, 0.95] if seed % 3 == 0 else None)
    nb_max = 1 + k
    br = O.branch_build(tok, conf, arg, k, np.float32(0.9), nb_max)
    U = [p for p in range(B) if tok[p] == M]
    if U:
        assert len(br.anchor_fill) >= 1
    R = [p for p in U if p not in br.anchor_fill]
    # rank-count recomputation of the lookahead positions
    def key(p):
        return (float(conf[p]), -p)
    rank = {p: sum(1 for q in R if key(q) > key(p)) for p in R}
    k_eff = min(k, len(R))
    assert br.lookahead == [p for r in range(k_eff) for p in R if rank[p] == r]
    assert br.nb == 1 + k_eff
    # each lookahead branch differs from the anchor at exactly its q_j
    for j, q in enumerate(br.lookahead, start=1):
        diff = np.flatnonzero(br.br_tok[j] != br.br_tok[0])
        assert diff.tolist() == [q] and br.br_tok[j, q] == arg[q]
        assert br.br_tok[0, q] == M
    # masks and rows agree
    rows = [b * B + p for b in range(br.nb) for p in range(B) if br.br_tok[b, p] == M]
    assert br.rows.tolist() == rows
    for b in range(nb_max):
        lo, hi = br.row_ptr[b], br.row_ptr[b + 1]
        assert all(r // B == b for r in br.rows[lo:hi])
        if b >= br.nb:
            assert lo == hi == len(rows)
    assert br.br_mask[:br.nb].sum() == len(rows)


def test_oracle_build_exhaustive_tiny():
    # every masked pattern and every ordering of three confidence levels on B=4
    levels = np.array([0.2, 0.6, 0.95], np.float32)
    for pattern in itertools.product([0, 1], repeat=4):
        for lv in itertools.product(range(3), repeat=4):
            tok = np.where(np.array(pattern) == 1, M, 3).astype(np.int32)
            conf = levels[list(lv)]
            arg = np.array([20, 21, 22, 23], np.int32)
            for k in range(0, 4):
                br = O.branch_build(tok, conf, arg, k, np.float32(0.9), 4)
                U = [p for p in range(4) if tok[p] == M]
                above = [p for p in U if conf[p] > np.float32(0.9)]
                if U and not above:
                    best = max(U, key=lambda p: (conf[p], -p))
                    above = [best]
                assert br.anchor_fill == above
                R = [p for p in U if p not in above]
                # brute force: the chosen set is the lexicographically best
                # k_eff-subset ordered by (conf desc, p asc)
                k_eff = min(k, len(R))
                best_seq = max(itertools.permutations(R, k_eff),
                               key=lambda s: [(conf[p], -p) for p in s])
                assert br.lookahead == list(best_seq)
