"""Pins of the block-decoding oracle (oracle/decode_oracle.py).

* Philox4x32-10 against the known-answer vectors published with the
  generator (Random123 distribution, kat_vectors: philox4x32 with 10 rounds).
* The Irwin-Hall values: exact multiples of 2^-16 inside [-6, 6], and the
  moments of a sum of twelve uniforms (mean 0, variance 1, excess kurtosis
  -1/10) -- a sum of eight, or halves taken from one draw twice, fails them.
* Token keying: the same token at the same position gives the same vectors
  in every branch, anything else differs.
* The decoding loop against cases with closed-form outcomes and invariants.
* The explore-stage gaps against brute force: no perturbation of the
  confidences smaller than the gaps (every sign corner of the box, tiny
  blocks) changes what the explore stage builds, and one just past the rank
  gap -- or past the threshold gap where crossing the threshold must matter
  -- does.
"""
import numpy as np
import pytest

import synth
from oracle import decode_oracle as D
from oracle import lopa_oracle as O

KAT = [  # (counter, key, output) -- Random123 kat_vectors, philox4x32 R = 10
    ((0x00000000, 0x00000000, 0x00000000, 0x00000000), (0x00000000, 0x00000000),
     (0x6627e8d5, 0xe169c58d, 0xbc57ac4c, 0x9b00dbd8)),
    ((0xffffffff, 0xffffffff, 0xffffffff, 0xffffffff), (0xffffffff, 0xffffffff),
     (0x408f276d, 0x41c83b0e, 0xa20bc7c6, 0x6d5451fd)),
    ((0x243f6a88, 0x85a308d3, 0x13198a2e, 0x03707344), (0xa4093822, 0x299f31d0),
     (0xd16cfe09, 0x94fdcceb, 0x5001e420, 0x24126ea1)),
]


@pytest.mark.parametrize("ctr,key,out", KAT)
def test_philox_known_answers(ctr, key, out):
    got = D.philox4x32_10(np.array(ctr, np.uint32), np.array(key, np.uint32))
    assert tuple(int(x) for x in got) == out


def test_philox_vectorised_matches_scalar():
    rng = np.random.default_rng(5)
    ctr = rng.integers(0, 2**32, size=(50, 4), dtype=np.uint64).astype(np.uint32)
    key = np.array([0x12345678, 0x9abcdef0], np.uint32)
    batch = D.philox4x32_10(ctr, key)
    for i in range(50):
        assert np.array_equal(batch[i], D.philox4x32_10(ctr[i], key))


def _values(n=200_000, seed=3):
    tok = np.zeros((1, 1), np.int64)
    vals = []
    for kind in range(3):
        x = D.synth_values(seed, kind, 1, tok, n // 3, dtype=np.float32).astype(np.float64)
        vals.append(x.ravel())
    return np.concatenate(vals)


def test_irwin_hall_exact_grid_and_range():
    x = _values(30_000)
    assert np.all(x >= -6) and np.all(x < 6)
    assert np.all(x * 65536 == np.round(x * 65536))


def test_irwin_hall_moments():
    x = _values()
    n = x.size
    assert abs(x.mean()) < 5 / np.sqrt(n)
    assert abs(x.var() - 1.0) < 0.02
    kurt = np.mean((x - x.mean()) ** 4) / x.var() ** 2 - 3.0
    assert abs(kurt - (-0.1)) < 0.05


def test_bf16_values_round_the_exact_ones():
    tok = np.array([[3, -1, 7]])
    exact = D.synth_values(11, D.KIND_K, 2, tok, 16, dtype=np.float32).astype(np.float64)
    bits = D.synth_values(11, D.KIND_K, 2, tok, 16, dtype=np.uint16)
    assert np.array_equal(bits, O.f64_to_bf16(exact))


def test_token_keying():
    tok = np.array([[5, -1, 9, 9], [5, 4, 9, 2]])
    Q, K, V = D.token_qkv(7, tok, 4, 2, 32)
    assert Q.shape == (2, 4, 4, 32) and K.shape == (2, 4, 2, 32) and V.shape == K.shape
    for A in (Q, K, V):
        assert np.array_equal(A[0, 0], A[1, 0])          # same token, same position
        assert np.array_equal(A[0, 2], A[1, 2])
        assert not np.array_equal(A[0, 1], A[1, 1])      # masked vs token 4
        assert not np.array_equal(A[0, 3], A[1, 3])      # 9 vs 2
        assert not np.array_equal(A[0, 2], A[0, 3])      # same token, other position
    assert not np.array_equal(K, V)                       # the tensor enters the key
    Q2, _, _ = D.token_qkv(8, tok, 4, 2, 32)
    assert not np.array_equal(Q, Q2)                      # the seed enters the key


def _inp(**kw):
    base = dict(dtype="bf16", L=40, B=16, m=10, k=3, Hq=4, Hkv=2, d=32, V=600)
    base.update(kw)
    return synth.make_inputs(synth.TINY, **base)


def test_decode_fills_every_position_and_never_changes_filled_ones():
    inp = _inp()
    tr = D.decode_block(inp, seed=21, k=3, tau=0.9)
    tok = tr.tok0.copy()
    for st in tr.steps:
        assert st.filled >= 1
        kept = tok != O.MASK
        assert np.array_equal(st.tok[kept], tok[kept])
        tok = st.tok
    assert not np.any(tok == O.MASK)
    assert len(tr.steps) <= int(np.sum(tr.tok0 == O.MASK))
    assert 1 <= len(tr.steps)


def test_decode_threshold_below_every_confidence_fills_all_in_one_step():
    # tau < 0: the anchor fills every masked position with the initial pass's
    # argmax, in one step
    inp = _inp()
    tr = D.decode_block(inp, seed=4, k=2, tau=-1.0)
    assert len(tr.steps) == 1
    m = tr.tok0 == O.MASK
    assert np.array_equal(tr.steps[0].tok[m], tr.arg0[m])


def test_decode_unreachable_threshold_without_lookahead_fills_one_per_step():
    # tau > 1 and k = 0: only the fallback fill, one position per step, in the
    # order of the confidences each step reports
    inp = _inp(m=6)
    tr = D.decode_block(inp, seed=9, k=0, tau=2.0)
    assert len(tr.steps) == 6
    assert all(st.filled == 1 and st.nb == 1 and st.winner == 0 for st in tr.steps)
    assert tr.tpf == 1.0


def test_decode_lookahead_never_slower_than_one_per_step():
    inp = _inp(k=4)
    tr = D.decode_block(inp, seed=33, k=4, tau=2.0)
    # with tau unreachable each step fills 1 (anchor) or 2 (a lookahead branch wins)
    assert all(st.filled in (1, 2) for st in tr.steps)
    assert all((st.filled == 2) == (st.winner > 0) for st in tr.steps)
    assert tr.tpf >= 1.0


def _blocks(B, n, m, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        tok = rng.integers(0, 500, size=B).astype(np.int32)
        tok[rng.choice(B, m, replace=False)] = O.MASK
        out.append(tok)
    return out


def test_sequence_appends_final_tokens_kv_and_later_blocks_see_it():
    inp = _inp(L=24, B=16, m=8, k=3)
    blocks = _blocks(16, 3, 6, 1)
    sq = D.decode_sequence(inp, seed=5, k=3, tau=0.9, blocks=blocks)
    L0, B = inp.Kp.shape[0], 16
    assert sq.Kp.shape[0] == L0 + 3 * B and sq.Vp.shape == sq.Kp.shape
    assert np.array_equal(sq.Kp[:L0], inp.Kp) and np.array_equal(sq.Vp[:L0], inp.Vp)
    for j, tr in enumerate(sq.blocks):
        final = tr.steps[-1].tok
        assert not np.any(final == O.MASK)
        _, K, V = D.token_qkv(5, final[None, :], inp.cfg.Hq, inp.cfg.Hkv, inp.cfg.d)
        assert np.array_equal(sq.Kp[L0 + j * B:L0 + (j + 1) * B], K[0])
        assert np.array_equal(sq.Vp[L0 + j * B:L0 + (j + 1) * B], V[0])
    # block 1 decoded on the extended prefix, not on the original one
    from dataclasses import replace
    ext = replace(inp, tok=blocks[1], Kp=sq.Kp[:L0 + B], Vp=sq.Vp[:L0 + B],
                  cfg=replace(inp.cfg, L=L0 + B))
    again = D.decode_block(ext, 5, 3, 0.9)
    assert np.array_equal(again.conf0, sq.blocks[1].conf0)
    orig = D.decode_block(replace(inp, tok=blocks[1]), 5, 3, 0.9)
    assert not np.array_equal(orig.conf0, sq.blocks[1].conf0)


def _random_state(rng, gamma=False):
    B = int(rng.integers(3, 8))
    tok = rng.integers(0, 100, B).astype(np.int32)
    masked = rng.random(B) < 0.7
    masked[rng.integers(B)] = True
    tok[masked] = O.MASK
    # values on a coarse grid plus a small jitter: many near-ties, no exact ones
    grid = np.linspace(0.1, 0.9, 9)
    conf = rng.choice(grid, B) + rng.uniform(-2e-3, 2e-3, B)
    conf[~masked] = 0.0
    arg = rng.integers(0, 100, B).astype(np.int32)
    tau = float(rng.choice(grid) + rng.uniform(-2e-3, 2e-3))
    k = int(rng.integers(0, 5))
    g = float(rng.choice(grid) + rng.uniform(-2e-3, 2e-3)) if gamma else None
    return tok, conf, arg, tau, k, g


def _built(tok, conf, arg, k, tau, g):
    br = O.branch_build(tok, conf, arg, k, tau, k + 1, g)
    M = int(br.row_ptr[-1])
    return (br.nb, br.br_tok.tobytes(), br.br_mask.tobytes(), br.rows[:M].tobytes(),
            br.row_ptr.tobytes())


def _corners(n):
    for bits in range(1 << n):
        yield np.array([1.0 if bits >> i & 1 else -1.0 for i in range(n)])


@pytest.mark.parametrize("gamma", [False, True])
def test_explore_gaps_bound_every_perturbation_that_keeps_the_branches(gamma):
    rng = np.random.default_rng(11 + gamma)
    checked = 0
    for _ in range(300):
        tok, conf, arg, tau, k, g = _random_state(rng, gamma)
        rank_gap, tau_gap = D._explore_gaps(tok, conf, tau, k, g)
        r = 0.999 * min(rank_gap / 2, tau_gap)
        m = np.flatnonzero(tok == O.MASK)
        ref = _built(tok, conf, arg, k, tau, g)
        for sgn in _corners(m.size):
            c = conf.copy()
            c[m] += r * sgn
            assert _built(tok, c, arg, k, tau, g) == ref, (tok, conf, tau, k, g, sgn)
        for _ in range(8):
            c = conf.copy()
            c[m] += rng.uniform(-r, r, m.size)
            assert _built(tok, c, arg, k, tau, g) == ref
        checked += 1
    assert checked == 300


def test_explore_gaps_are_tight():
    """Just past the rank gap some sign corner changes the branches; just past
    the threshold gap moving the nearest position alone across the threshold
    does, whenever another position stays above it or the nearest was
    above it with company."""
    rng = np.random.default_rng(12)
    rank_cases = tau_cases = 0
    for _ in range(300):
        tok, conf, arg, tau, k, _ = _random_state(rng)
        rank_gap, tau_gap = D._explore_gaps(tok, conf, tau, k)
        m = np.flatnonzero(tok == O.MASK)
        ref = _built(tok, conf, arg, k, tau, None)
        if np.isfinite(rank_gap) and 1.01 * rank_gap / 2 < tau_gap:
            r = 1.01 * rank_gap / 2
            changed = False
            for sgn in _corners(m.size):
                c = conf.copy()
                c[m] += r * sgn
                changed |= _built(tok, c, arg, k, tau, None) != ref
            assert changed, (tok, conf, tau, k)
            rank_cases += 1
        near = m[np.argmin(np.abs(conf[m] - tau))]
        above = m[conf[m] > tau]
        if 1.01 * tau_gap < rank_gap / 2 and (above.size >= 2 or (above.size == 1 and
                                                                   near not in above)):
            c = conf.copy()
            c[near] = tau + (1.01 * tau_gap if conf[near] < tau else -1.01 * tau_gap)
            assert _built(tok, c, arg, k, tau, None) != ref
            tau_cases += 1
    assert rank_cases >= 50 and tau_cases >= 20, (rank_cases, tau_cases)
