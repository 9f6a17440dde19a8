"""Pins for the oracle's whole verification step on the tiny fp32 workload
and small bf16 variants.

* k = 0: the step reduces to plain confidence-driven sampling (one branch,
  which wins, and fills exactly what greedy sampling fills);
* each branch's verification outputs equal running that branch alone
  (attention over prefix + its own block, then the LM head);
* the winner maximises the mean confidence of its remaining positions,
  recomputed here from the per-branch runs;
* reuse: the next state's confidences/tokens are the winner's rows;
* the synthetic recipe gives H with RMS about sqrt(e/(L+B)) and logits with
  a standard deviation of about 4.
"""
import math

import numpy as np
import pytest

import oracle as O
import synth

M = O.MASK


@pytest.fixture(scope="module")
def tiny():
    inp = synth.make_inputs(synth.TINY)
    c, a, head = O.initial_state(inp)
    return inp, c, a, head


def test_oracle_step_initial_state_shape(tiny):
    inp, c, a, head = tiny
    masked = inp.tok == M
    assert masked.sum() == inp.cfg.m
    assert np.all(c[~masked] == 0) and np.all(a[~masked] == -1)
    assert np.all(c[masked] >= 1 / inp.cfg.V) and np.all(c[masked] <= 1)
    assert np.all((a[masked] >= 0) & (a[masked] < inp.cfg.V))


def test_oracle_step_k0_reduces_to_confidence_driven(tiny):
    inp, c, a, _ = tiny
    out = O.verification_step(inp, c, a, k=0)
    assert out.br.nb == 1 and out.sel.winner == 0
    greedy = inp.tok.copy()
    idx = np.flatnonzero(greedy == M)
    above = idx[c[idx] > np.float32(inp.cfg.tau)]
    pick = above if above.size else idx[[int(np.argmax(c[idx]))]]
    greedy[pick] = a[pick]
    assert out.sel.tok_next.tolist() == greedy.tolist()


def test_oracle_step_branches_equal_running_alone(tiny):
    inp, c, a, _ = tiny
    cfg = inp.cfg
    out = O.verification_step(inp, c, a)
    assert out.br.nb == 1 + cfg.k
    W = inp.W
    means = []
    for b in range(out.br.nb):
        Hb = O.attention_one_branch(*(O.to_f64(x) for x in (inp.Kp, inp.Vp)),
                                    O.to_f64(inp.Qb[b]), O.to_f64(inp.Kb[b]),
                                    O.to_f64(inp.Vb[b]), cfg.Hq, cfg.Hkv)
        Hb = O.round_like(Hb, inp.Qb.dtype)
        ps = [p for p in range(cfg.B) if out.br.br_tok[b, p] == M]
        head = O.lmhead_conf(Hb[ps], W)
        for i, p in enumerate(ps):
            assert out.conf_pos[b * cfg.B + p] == head.conf[i]
            assert out.arg_pos[b * cfg.B + p] == head.arg[i]
        means.append(np.mean(head.conf) if ps else 1.0)
    w = int(np.argmax(means))
    assert out.sel.winner == w
    assert means[w] == max(means)
    # reuse: next state is exactly the winner's rows, nothing recomputed
    for p in range(cfg.B):
        if out.br.br_tok[w, p] == M:
            assert out.sel.conf_next[p] == out.conf_pos[w * cfg.B + p]
            assert out.sel.arg_next[p] == out.arg_pos[w * cfg.B + p]
    assert out.sel.tok_next.tolist() == out.br.br_tok[w].tolist()


def test_oracle_step_bf16_small(tiny):
    # the same step on a small bf16 GQA variant: H is rounded to bf16 once
    inp = synth.make_inputs(synth.TINY, dtype=synth.BF16, Hq=4, Hkv=2, d=32, V=700, B=12, m=9, L=20)
    c, a, _ = O.initial_state(inp)
    out = O.verification_step(inp, c, a)
    Hb = O.round_like(O.branch_attn(inp.Kp, inp.Vp, inp.Qb, inp.Kb, inp.Vb, out.br.nb, 4, 2),
                      np.uint16)
    assert np.array_equal(out.H, Hb)
    # every rounded value is a bf16 value
    assert np.array_equal(O.bf16_to_f64(O.f64_to_bf16(out.H)), out.H)


def test_oracle_step_workload_statistics(tiny):
    inp, c, a, head = tiny
    cfg = inp.cfg
    H = O.branch_attn(inp.Kp, inp.Vp, inp.Qb, inp.Kb, inp.Vb, 1, cfg.Hq, cfg.Hkv)
    rms = math.sqrt(np.mean(H[0] ** 2))
    assert abs(rms / math.sqrt(math.e / (cfg.L + cfg.B)) - 1) < 0.2
    logits = H[0] @ O.to_f64(inp.W).T
    std = logits.std(axis=1).mean()
    assert 3.0 < std < 5.0
