"""Pins of the alternative branch score ([blog] section 3.2): the normalised
entropy the LM head reports and branch_select_alpha."""
import math

import numpy as np
import pytest
from scipy.stats import entropy as scipy_entropy

import synth
from oracle import decode_oracle as D
from oracle import lopa_oracle as O


def test_entropy_matches_library_routine():
    rng = np.random.default_rng(0)
    H = rng.standard_normal((7, 24))
    W = rng.standard_normal((300, 24)).astype(np.float32)
    out = O.lmhead_conf(H, W)
    logits = H @ W.astype(np.float64).T
    for r in range(7):
        p = np.exp(logits[r] - logits[r].max())
        assert out.ent[r] == pytest.approx(scipy_entropy(p / p.sum()) / math.log(300), rel=1e-12)


def test_entropy_extremes():
    H = np.ones((2, 8))
    assert np.allclose(O.lmhead_conf(H, np.zeros((50, 8), np.float32)).ent, 1.0)   # uniform
    W = np.zeros((50, 8), np.float32)
    W[3] = 100.0
    assert np.all(O.lmhead_conf(H, W).ent < 1e-100)                              # one-hot
    assert np.all(O.lmhead_conf(H, np.ones((1, 8), np.float32)).ent == 0.0)      # V = 1


def test_alpha_score_by_hand():
    # B = 4; state: positions 1, 2, 3 masked with confidences .9 .5 .3
    tok_state = np.array([7, -1, -1, -1])
    conf_state = np.array([0, .9, .5, .3], np.float32)
    # anchor fills 1; branch 1 fills 1 and 2; branch 2 fills 1 and 3
    br_mask = np.array([[0, 0, 1, 1], [0, 0, 0, 1], [0, 0, 1, 0]], bool)
    br_tok = np.array([[7, 4, -1, -1], [7, 4, 5, -1], [7, 4, -1, 6]])
    ent = np.zeros(12)
    ent[[2, 3]] = [.2, .4]          # anchor's remaining positions
    ent[4 + 3] = .1                 # branch 1's remaining
    ent[8 + 2] = .6                 # branch 2's remaining
    conf_pos = np.zeros(12)
    arg_pos = np.full(12, -1)
    conf_pos[[2, 3, 7, 10]] = [.55, .35, .32, .7]
    arg_pos[[2, 3, 7, 10]] = [11, 12, 13, 14]
    a = 0.7
    sel = O.branch_select_alpha(3, br_mask, br_tok, conf_pos, arg_pos, ent, tok_state,
                                conf_state, a)
    want = [a * .9 + (1 - a) * ((1 - .2) + (1 - .4)),
            a * (.9 + .5) + (1 - a) * (1 - .1),
            a * (.9 + .3) + (1 - a) * (1 - .6)]
    assert np.allclose(sel.bconf[:3], want)
    assert sel.winner == 1
    assert list(sel.tok_next) == [7, 4, 5, -1]
    assert sel.conf_next[3] == pytest.approx(.32) and sel.arg_next[3] == 13
    assert sel.arg_next[2] == -1
    # with all weight on the future term, branch 0's two remaining positions win
    assert O.branch_select_alpha(3, br_mask, br_tok, conf_pos, arg_pos, ent, tok_state,
                                 conf_state, 0.0).winner == 0


def test_alpha_one_prefers_the_most_confident_extra_fill():
    # alpha = 1: score = sum of the fill probabilities; every lookahead branch
    # adds one fill to the anchor's, so branch 1 (the most confident extra
    # position) wins whenever its confidence is positive
    inp = synth.make_inputs(synth.TINY, dtype="bf16", L=30, B=16, m=9, k=3, Hq=4, Hkv=2, d=32,
                            V=500)
    tr = D.decode_block(inp, seed=3, k=3, tau=2.0, alpha=1.0)
    assert all(st.winner == (1 if st.nb > 1 else 0) for st in tr.steps)
    assert all(st.filled == (2 if st.nb > 1 else 1) for st in tr.steps)
