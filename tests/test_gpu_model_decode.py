"""GPU parity of block decoding with the model (model.model_decode_block /
model_decode_sequence) against oracle/model_oracle (initial_pass,
decode_step, forward).

The GPU forward and the oracle's agree to bf16 rounding noise (see
test_gpu_model.py); from identical states the confidences of one step
differ by up to 1.5e-2 on these geometries (measured).  A whole decoding
trajectory therefore follows the oracle's only while every decision is clear
by more than that, which few blocks are for long.  So each GPU step is
checked from the GPU's own state: the oracle takes one step from the state
the GPU logged (the explore stage then sees identical inputs and decides
identically), and whenever that step's outcome is clear-cut -- the top-2
logit gap behind every token it fills > FILL and the winner's
branch-confidence margin > GAP -- the GPU's next tokens must equal the
oracle's, its next confidences agree to GAP and its next argmax tokens
agree where their logit gap is > FILL.  The committed prefix of every layer
is compared with the oracle's forward of the GPU's decoded tokens, to the
forward's tolerance.
"""
import numpy as np
import pytest
import torch

import lookahead_decoding_amd as lopa
from lookahead_decoding_amd.model import (Model, ModelDecodeBuffers, model_decode_block,
                                          model_decode_sequence, model_dims)
from oracle import lopa_oracle as O
from oracle import model_oracle as MO

pytestmark = pytest.mark.gpu
M = O.MASK
FILL = 0.1    # logit gap behind a filled token
GAP = 3e-2    # confidence gaps: twice the largest difference measured from identical states


def _block(seed, B, m, V):
    rng = np.random.default_rng(100 + seed)
    tok = rng.integers(0, V - 1, B).astype(np.int32)
    tok[rng.choice(B, m, replace=False)] = M
    return tok


CASES = [
    # name, geometry (L, B, k, Hq, Hkv, d, inter, V, layers), masked, seed
    ("small-1", (40, 16, 3, 4, 2, 64, 512, 1000, 2), 10, 1),
    ("small-4", (40, 16, 3, 4, 2, 64, 512, 1000, 2), 10, 4),
    ("small-5", (40, 16, 3, 4, 2, 64, 512, 1000, 2), 10, 5),
    ("mfma-1", (64, 32, 4, 8, 2, 128, 1024, 2000, 2), 16, 1),
    ("mfma-2", (64, 32, 4, 8, 2, 128, 1024, 2000, 2), 16, 2),
]


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


def _check_block(what, seed, cfg, L, layers, prefix, W, tok0, k, tau, nb_max, log, state_log):
    """Check the GPU's initial pass and every clear-cut step from the GPU's
    own states.  Returns (steps checked, steps taken, the final tokens)."""
    got_tok = log.cpu().numpy()
    got_conf, got_arg = state_log[0].cpu().numpy(), state_log[1].cpu().numpy()
    conf0, arg0, margin, _ = MO.initial_pass(seed, cfg, L, tok0, layers, prefix, W)
    masked = tok0 == M
    assert np.abs(got_conf[0][masked] - conf0[masked]).max(initial=0) <= GAP, f"{what}: conf0"
    sure = masked & (margin > FILL)
    assert np.array_equal(got_arg[0][sure], arg0[sure]), f"{what}: initial tokens"
    tok, conf, arg = tok0.copy(), got_conf[0], got_arg[0]
    checked = steps = 0
    for s in range(len(got_tok)):
        if not np.any(tok == M):
            break
        steps += 1
        st, (ntok, nconf, narg, nmargin), _, _, br, bmargin = MO.decode_step(
            seed, cfg, L, tok, conf, arg, margin, k, tau, nb_max, layers, prefix, W)
        # whatever the noise, the GPU's next tokens are one of the step's branches
        took = [b for b in range(br.nb) if np.array_equal(br.br_tok[b], got_tok[s])]
        assert took, f"{what}: step {s}: the tokens are none of the {br.nb} branches"
        if st.fill_margin > FILL and st.win_margin > GAP:
            assert np.array_equal(got_tok[s], ntok), f"{what}: step {s} tokens"
            rem = ntok == M
            d = np.abs(got_conf[s + 1][rem] - nconf[rem]).max(initial=0)
            assert d <= GAP, f"{what}: step {s} confidences differ by {d:.3g}"
            sure = rem & (nmargin > FILL)
            assert np.array_equal(got_arg[s + 1][sure], narg[sure]), f"{what}: step {s} argmax"
            checked += 1
        # the logit gaps behind the argmax tokens of the branch the GPU took
        B = len(tok)
        margin = np.where(got_tok[s] == M, bmargin[took[0] * B:(took[0] + 1) * B], np.inf)
        tok, conf, arg = got_tok[s], got_conf[s + 1], got_arg[s + 1]
    assert not np.any(tok == M), f"{what}: block not finished after {steps} steps"
    return checked, steps, tok


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
    checked, steps, _ = _check_block(name, seed, cfg, dims.L, layers, prefix, W, tok,
                                     dims.k_max, 0.9, dims.nb_max, log, state_log)
    print(f"[model decode] {name}: {checked} of {steps} steps clear-cut and checked", flush=True)
    assert checked >= 1, f"{name}: no step clear-cut"
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
        checked, steps, final = _check_block(f"block {j}", seed, cfg, Lj, layers, prefix, W,
                                             tok0, dims.k_max, 0.9, dims.nb_max, *logs[j])
        print(f"[model decode] block {j}: {checked} of {steps} steps checked", flush=True)
        # the commit appended the keys and values of the decoded block: the
        # last pass's winner slot, whose input was the final tokens
        out = MO.forward(seed, cfg, Lj, final[None], layers, prefix)
        for l in range(cfg.n_layers):
            for got, want in ((g(model.Kp[l, Lj:Lj + 16]), out.Kb[l, 0]),
                              (g(model.Vp[l, Lj:Lj + 16]), out.Vb[l, 0])):
                rms = float(np.sqrt(np.mean(want ** 2)))
                err = np.abs(got - want)
                assert err.max() <= 2.0 ** -4 * rms, (j, l)
                assert err.mean() <= 2.0 ** -8 * rms * np.sqrt(cfg.n_layers), (j, l)
        prefix = [(np.concatenate([prefix[l][0], out.Kb[l, 0]]),
                   np.concatenate([prefix[l][1], out.Vb[l, 0]])) for l in range(cfg.n_layers)]
        Lj += 16
