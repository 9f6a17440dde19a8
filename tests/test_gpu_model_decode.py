"""GPU parity of block decoding with the model (model.model_decode_block /
model_decode_sequence) against oracle/model_oracle (initial_pass,
decode_step, forward).

Tolerances.  The GPU forward and the oracle's differ by bf16 rounding noise
(test_gpu_model.py).  tests/golden/forward_noise.json holds what that noise
does to the LM head under the rounding-noise model (every value entering a
bf16 rounding point perturbed by 2^-16 relative, run through the oracle),
over a block's first two passes: the largest change of a row's confidence
("conf"), of a branch confidence ("branch": the mean confidence of the rows
the branch leaves masked) and of a logit relative to the row's top logit
("lead").  Allowed, with a factor 2 of margin: CONF = 2 conf for a row
confidence (4.3e-2 on the wider geometry: this exceeds the 2e-2 that the
branch step meets from given hidden rows, because here the hidden rows
themselves carry the forward's rounding noise); LEAD = 2 lead for a token
(its top-2 logit gap must exceed LEAD for the GPU to be held to the same
token); two branches' order can flip only when their gap is below
GAP = 2 (2 branch), both moving.

A whole trajectory follows the oracle's only while every decision clears
those gaps, so each GPU step is checked from the GPU's own state: the oracle
takes one step from the state the GPU logged (the explore stage sees
identical inputs and builds identical branches), and
  * the GPU's next tokens are one of the step's branches, b;
  * the oracle's branch confidence of b is within GAP of the best one, and b
    is the oracle's winner whenever the winner leads by more than GAP
    ("clear-cut" steps: at least MIN_CLEAR of every block's steps);
  * the GPU's next confidences are within CONF of the oracle's for branch b,
    its next argmax tokens equal the oracle's where their lead exceeds LEAD
    and lie within LEAD of the top logit elsewhere.
The committed prefix of every layer is compared with the oracle's forward
of the GPU's decoded tokens to the forward's bound for that geometry.
"""
import json
import os

import numpy as np
import pytest
import torch

import lookahead_decoding_amd as lopa
from lookahead_decoding_amd.model import (Model, ModelDecodeBuffers, model_decode_block,
                                          model_decode_sequence, model_dims)
from oracle import lopa_oracle as O
from oracle import model_oracle as MO
from _model_cases import DECODE_CASES as CASES
from _model_cases import block as _block

pytestmark = pytest.mark.gpu
M = O.MASK
with open(os.path.join(os.path.dirname(__file__), "golden", "forward_noise.json")) as _f:
    _NOISE = json.load(_f)
MIN_CLEAR = 0.4   # share of a block's steps whose winner leads by more than GAP


def _tols(name):
    """(CONF, LEAD, GAP) of the geometry ``name`` belongs to."""
    g = _NOISE["decode"][name.split("-")[0]]
    return 2 * g["conf"], 2 * g["lead"], 2 * (2 * g["branch"])


def _setup(geo, seed, extra_rows=0):
    L, B, k, Hq, Hkv, d, inter, V, n = geo
    dims = lopa.Dims(L=L, B=B, Hq=Hq, Hkv=Hkv, d=d, V=V, k_max=k, dtype=lopa.BF16)
    md = model_dims(n, inter, V - 1)
    cfg = MO.ModelCfg(n_layers=n, Hq=Hq, Hkv=Hkv, d=d, inter=inter, V=V, mask_id=V - 1)
    return dims, md, cfg, Model(dims, md, seed, kv_rows=L + extra_rows)


def _logs(m, B):
    return (torch.zeros(m, B, dtype=torch.int32, device="cuda"),
            (torch.zeros(m + 1, B, dtype=torch.float32, device="cuda"),
             torch.zeros(m + 1, B, dtype=torch.int32, device="cuda")))


def _check_block(what, tols, seed, cfg, L, layers, prefix, W, tok0, k, tau, nb_max, log,
                 state_log):
    """Check the GPU's initial pass and every step from the GPU's own states.
    Returns (clear-cut steps, steps taken, the final tokens)."""
    CONF, LEAD, GAP = tols
    got_tok = log.cpu().numpy()
    got_conf, got_arg = state_log[0].cpu().numpy(), state_log[1].cpu().numpy()
    B = len(tok0)
    conf0, arg0, _, out0 = MO.initial_pass(seed, cfg, L, tok0, layers, prefix, W)
    masked = np.flatnonzero(tok0 == M)
    _check_rows(f"{what}: initial pass", got_conf[0][masked], got_arg[0][masked],
                out0.H[0, masked], W, CONF, LEAD)
    tok, conf, arg = tok0.copy(), got_conf[0], got_arg[0]
    margin = np.full(B, np.inf)        # decode_step's fill statistic only
    clear = steps = 0
    for s in range(len(got_tok)):
        if not np.any(tok == M):
            break
        steps += 1
        st, _, out, w, br, _ = MO.decode_step(seed, cfg, L, tok, conf, arg, margin, k, tau,
                                              nb_max, layers, prefix, W)
        took = [b for b in range(br.nb) if np.array_equal(br.br_tok[b], got_tok[s])]
        assert took, f"{what}: step {s}: the tokens are none of the {br.nb} branches"
        b = took[0]
        # the oracle's branch confidences (mean confidence of the rows a branch leaves masked)
        bconf = np.ones(br.nb)
        for c in range(br.nb):
            rows = np.flatnonzero(br.br_mask[c])
            if rows.size:
                bconf[c] = O.lmhead_conf(out.H[c, rows], W).conf.mean()
        assert bconf[b] >= bconf.max() - GAP, f"{what}: step {s}: branch {b} far from the best"
        if st.win_margin > GAP:
            assert b == w, f"{what}: step {s}: winner {b}, the oracle's {w}"
            clear += 1
        rem = np.flatnonzero(br.br_mask[b])
        _check_rows(f"{what}: step {s}", got_conf[s + 1][rem], got_arg[s + 1][rem],
                    out.H[b, rem], W, CONF, LEAD)
        tok, conf, arg = got_tok[s], got_conf[s + 1], got_arg[s + 1]
    assert not np.any(tok == M), f"{what}: block not finished after {steps} steps"
    return clear, steps, tok


def _check_rows(what, conf_gpu, arg_gpu, H, W, CONF, LEAD):
    """The GPU's confidences and argmax tokens of rows whose oracle hidden
    rows are H."""
    if not len(H):
        return
    head = O.lmhead_conf(H, W)
    d = np.abs(conf_gpu - head.conf).max()
    assert d <= CONF, f"{what}: confidences differ by {d:.3g}"
    sure = head.margin > LEAD
    assert np.array_equal(arg_gpu[sure], head.arg[sure]), f"{what}: argmax tokens"
    lg = H @ W.astype(np.float64).T
    for r in np.flatnonzero(~sure):
        lead = lg[r].max() - lg[r, int(arg_gpu[r])]
        assert lead <= LEAD, f"{what}: row {r}: token {int(arg_gpu[r])} {lead:.3g} below the top"


@pytest.mark.parametrize("name,geo,m,seed", CASES, ids=[c[0] for c in CASES])
def test_gpu_model_decode_block(name, geo, m, seed):
    dims, md, cfg, model = _setup(geo, seed)
    tok = _block(seed, dims.B, m, cfg.V)
    buf = ModelDecodeBuffers(dims, md)
    log, state_log = _logs(m, dims.B)
    model_decode_block(model, dims, dims.k_max, 0.9, tok, buf, m, log, state_log=state_log)
    torch.cuda.synchronize()
    layers = [MO.synth_layer(seed, cfg, l) for l in range(cfg.n_layers)]
    prefix = [MO.synth_prefix(seed, cfg, l, dims.L) for l in range(cfg.n_layers)]
    W = MO.lm_head_weight(seed, cfg)
    clear, steps, _ = _check_block(name, _tols(name), seed, cfg, dims.L, layers, prefix, W,
                                   tok, dims.k_max, 0.9, dims.nb_max, log, state_log)
    print(f"[model decode] {name}: {clear} of {steps} steps clear-cut", flush=True)
    assert clear >= MIN_CLEAR * steps, f"{name}: {clear} of {steps} steps clear-cut"
    # the log is complete: steps past the end repeat the final tokens
    got = log.cpu().numpy()
    assert np.all(got[steps - 1:] == got[steps - 1])


def test_gpu_model_decode_sequence_commits_every_layer():
    geo = (40, 16, 3, 4, 2, 64, 512, 1000, 2)
    seed = 1
    dims, md, cfg, model = _setup(geo, seed, extra_rows=2 * 16)
    blocks = [_block(1, 16, 10, cfg.V), _block(5, 16, 10, cfg.V)]
    buf = ModelDecodeBuffers(dims, md)
    logs = [_logs(10, 16) for _ in blocks]
    L = model_decode_sequence(model, dims.k_max, 0.9, blocks, buf, [lg[0] for lg in logs],
                              state_logs=[lg[1] for lg in logs])
    torch.cuda.synchronize()
    assert L == dims.L + 32
    layers = [MO.synth_layer(seed, cfg, l) for l in range(cfg.n_layers)]
    prefix = [MO.synth_prefix(seed, cfg, l, dims.L) for l in range(cfg.n_layers)]
    W = MO.lm_head_weight(seed, cfg)
    g = lambda t: O.bf16_to_f64(t.cpu().view(torch.int16).numpy().view(np.uint16))  # noqa: E731
    for l in range(cfg.n_layers):   # the original prefix is untouched
        assert np.array_equal(g(model.Kp[l, :dims.L]), prefix[l][0])
        assert np.array_equal(g(model.Vp[l, :dims.L]), prefix[l][1])
    Lj = dims.L
    for j, tok0 in enumerate(blocks):
        clear, steps, final = _check_block(f"block {j}", _tols("small"), seed, cfg, Lj, layers,
                                           prefix, W, tok0, dims.k_max, 0.9, dims.nb_max,
                                           *logs[j])
        print(f"[model decode] block {j}: {clear} of {steps} steps clear-cut", flush=True)
        assert clear >= MIN_CLEAR * steps, f"block {j}: {clear} of {steps} steps clear-cut"
        # the commit appended the keys and values of the decoded block: the
        # last pass's winner slot, whose input was the final tokens
        out = MO.forward(seed, cfg, Lj, final[None], layers, prefix)
        for l in range(cfg.n_layers):
            for got, want, key in ((g(model.Kp[l, Lj:Lj + 16]), out.Kb[l, 0], "K"),
                                   (g(model.Vp[l, Lj:Lj + 16]), out.Vb[l, 0], "V")):
                rms = float(np.sqrt(np.mean(want ** 2)))
                err = np.abs(got - want)
                mx, mn = _NOISE["forward"]["commit"][key]
                assert err.max() <= 2 * mx * rms, (j, l, key)
                assert err.mean() <= 1.5 * mn * rms, (j, l, key)
        prefix = [(np.concatenate([prefix[l][0], out.Kb[l, 0]]),
                   np.concatenate([prefix[l][1], out.Vb[l, 0]])) for l in range(cfg.n_layers)]
        Lj += 16
