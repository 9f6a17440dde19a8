"""Pins for the oracle's LM head (confidence, argmax) and branch selection.

LM head: confidence is the largest softmax probability and lies in
[1/V, 1]; checked against scipy's softmax, the all-zero weight (uniform
distribution: 1/V, token 0), a dominant logit, and exact ties.
Selection: branch confidence is the mean confidence over the branch's
still-masked positions (the articles' definition); checked by brute force,
tie-to-anchor, the empty-branch rule and the next-state copy.
"""
import numpy as np
import pytest
import scipy.special

import oracle as O


def test_oracle_head_matches_scipy_softmax():
    rng = np.random.default_rng(0)
    H = rng.standard_normal((9, 12))
    W = rng.standard_normal((50, 12)).astype(np.float32)
    out = O.lmhead_conf(H, W, keep_logits=True)
    logits = H @ W.astype(np.float64).T
    P = scipy.special.softmax(logits, axis=1)
    np.testing.assert_allclose(out.conf, P.max(axis=1), rtol=1e-13)
    assert out.arg.tolist() == P.argmax(axis=1).tolist()
    srt = np.sort(logits, axis=1)
    np.testing.assert_allclose(out.margin, srt[:, -1] - srt[:, -2], rtol=1e-13)
    # conf = 1 / sum exp(l - max)
    np.testing.assert_allclose(out.conf, 1 / np.exp(logits - logits.max(1, keepdims=True)).sum(1),
                               rtol=1e-13)


def test_oracle_head_top_logits_by_full_sort():
    """The T largest logits per row (tokens of equal logits lowest first)
    against a full lexicographic sort of every row, with planted ties and
    T reaching V."""
    rng = np.random.default_rng(7)
    H = rng.standard_normal((6, 5))
    W = rng.standard_normal((40, 5)).astype(np.float32)
    W[[3, 11, 29]] = W[17]          # four tokens share every row's logit
    for T in (1, 4, 16, 40, 60):
        out = O.lmhead_conf(H, W, keep_logits=True, top=T)
        for r in range(H.shape[0]):
            l = out.logits[r]
            order = np.lexsort((np.arange(40), -l))[:min(T, 40)]
            assert out.top_tok[r].tolist() == order.tolist()
            assert np.array_equal(out.top_logit[r], l[order])
        assert np.array_equal(out.top_tok[:, 0], out.arg)
        if T >= 2:
            np.testing.assert_array_equal(out.top_logit[:, 0] - out.top_logit[:, 1], out.margin)


def test_oracle_head_zero_weight_is_uniform():
    H = np.ones((3, 8))
    W = np.zeros((777, 8), np.float32)
    out = O.lmhead_conf(H, W)
    assert np.all(out.conf == 1 / 777) and np.all(out.arg == 0)
    assert np.all(out.margin == 0)


def test_oracle_head_dominant_logit():
    W = np.zeros((100, 4), np.float32)
    W[37, 0] = 1.0
    for x in (10.0, 60.0):
        out = O.lmhead_conf(np.array([[x, 0, 0, 0]]), W)
        assert out.arg[0] == 37
        np.testing.assert_allclose(out.conf[0], 1 / (1 + 99 * np.exp(-x)), rtol=1e-14)


def test_oracle_head_tie_lowest_index():
    W = np.zeros((10, 2), np.float32)
    W[[3, 6, 8], 0] = 2.0
    out = O.lmhead_conf(np.array([[1.0, 0.0]]), W)
    assert out.arg[0] == 3
    np.testing.assert_allclose(out.conf[0], 1 / (3 + 7 * np.exp(-2.0)), rtol=1e-14)


def test_oracle_head_conf_bounds_random():
    rng = np.random.default_rng(1)
    for V in (1, 2, 5, 300):
        H = rng.standard_normal((20, 6)) * 10
        W = rng.standard_normal((V, 6)).astype(np.float32)
        c = O.lmhead_conf(H, W).conf
        assert np.all(c >= 1 / V * (1 - 1e-12)) and np.all(c <= 1)


def test_oracle_head_reads_bf16_weights():
    rng = np.random.default_rng(2)
    Wf = rng.standard_normal((30, 8)).astype(np.float32)
    import torch
    bits = torch.from_numpy(Wf).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    vals = torch.from_numpy(Wf).to(torch.bfloat16).float().numpy()
    H = rng.standard_normal((4, 8))
    a, b = O.lmhead_conf(H, bits), O.lmhead_conf(H, vals)
    assert np.array_equal(a.conf, b.conf) and np.array_equal(a.arg, b.arg)


def _mask(rows, nb_max, B):
    m = np.zeros((nb_max, B), np.uint8)
    for b, ps in enumerate(rows):
        m[b, ps] = 1
    return m


def test_oracle_select_brute_force():
    rng = np.random.default_rng(3)
    for trial in range(200):
        B = int(rng.integers(1, 9))
        nb_max = int(rng.integers(1, 6))
        nb = int(rng.integers(1, nb_max + 1))
        br_mask = (rng.random((nb_max, B)) < 0.5).astype(np.uint8)
        br_mask[nb:] = 0
        br_tok = np.where(br_mask == 1, -1, rng.integers(0, 9, (nb_max, B))).astype(np.int32)
        conf = rng.random(nb_max * B)
        arg = rng.integers(0, 100, nb_max * B)
        s = O.branch_select(nb, br_mask, br_tok, conf, arg)
        means = []
        for b in range(nb):
            v = [conf[b * B + p] for p in range(B) if br_mask[b, p]]
            means.append(np.mean(v) if v else 1.0)
        w = int(np.argmax(means))        # first maximum
        assert s.winner == w
        np.testing.assert_allclose(s.bconf[:nb], means, rtol=1e-14)
        assert np.all(s.bconf[nb:] == -1)
        assert s.tok_next.tolist() == br_tok[w].tolist()
        for p in range(B):
            if br_mask[w, p]:
                assert s.conf_next[p] == conf[w * B + p] and s.arg_next[p] == arg[w * B + p]
            else:
                assert s.conf_next[p] == 0 and s.arg_next[p] == -1


def test_oracle_select_tie_goes_to_anchor_and_empty_is_one():
    B = 3
    br_mask = _mask([[0, 1], [1, 2], []], 3, B)
    br_tok = np.where(br_mask == 1, -1, 5).astype(np.int32)
    conf = np.array([0.5, 0.7, 0, 0, 0.7, 0.5, 0, 0, 0])
    s = O.branch_select(2, br_mask, br_tok, conf, np.zeros(9, int))
    assert s.winner == 0 and s.margin == 0
    s = O.branch_select(3, br_mask, br_tok, conf, np.zeros(9, int))
    assert s.bconf[2] == 1.0 and s.winner == 2
    assert s.tok_next.tolist() == [5, 5, 5]
    assert abs(s.margin - 0.4) < 1e-15
