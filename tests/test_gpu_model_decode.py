"""GPU parity of block decoding with the model (model.model_decode_block /
model_decode_sequence) against oracle/model_oracle.decode_block /
decode_sequence.

The GPU forward and the oracle's agree to bf16 rounding noise (see
test_gpu_model.py), so logits agree to ~1e-2 and confidences to ~1e-3: the
tokens after each step are compared while every decision the oracle took
was clear-cut by more than that -- the top-2 logit gap behind every filled
token > 0.1, the confidence gaps of the explore stage and the threshold test
> 3e-3, the winner's branch-confidence margin > 3e-3.  The committed prefix
of every layer is compared with the forward's tolerance.
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


def _clear(st):
    return (st.fill_margin > 0.1 and st.rank_gap > 3e-3 and st.tau_gap > 3e-3
            and st.win_margin > 3e-3)


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


@pytest.mark.parametrize("name,geo,m,seed", CASES, ids=[c[0] for c in CASES])
def test_gpu_model_decode_block(name, geo, m, seed):
    dims, md, cfg, model = _setup(geo, seed)
    tok = _block(seed, dims.B, m, cfg.V)
    tr, _, _ = MO.decode_block(seed, cfg, dims.L, tok, dims.k_max, 0.9, dims.nb_max)
    buf = ModelDecodeBuffers(dims, md)
    log = torch.zeros(m, dims.B, dtype=torch.int32, device="cuda")
    model_decode_block(model, dims, dims.k_max, 0.9, tok, buf, m, log)
    torch.cuda.synchronize()
    got = log.cpu().numpy()
    n = 0
    for s, st in enumerate(tr.steps):
        if not _clear(st):
            break
        assert np.array_equal(got[s], st.tok), f"{name}: step {s}"
        n += 1
    assert n == len(tr.steps), f"{name}: {n} of {len(tr.steps)} steps clear-cut"
    assert not np.any(got[n - 1] == M) and np.all(got[n - 1:] == got[n - 1])


def test_gpu_model_decode_sequence_commits_every_layer():
    geo = (40, 16, 3, 4, 2, 64, 512, 1000, 2)
    seed = 1
    dims, md, cfg, model = _setup(geo, seed, extra_rows=2 * 16)
    blocks = [_block(1, 16, 10, cfg.V), _block(5, 16, 10, cfg.V)]
    traces, prefix = MO.decode_sequence(seed, cfg, dims.L, blocks, dims.k_max, 0.9, dims.nb_max)
    buf = ModelDecodeBuffers(dims, md)
    logs = [torch.zeros(10, 16, dtype=torch.int32, device="cuda") for _ in blocks]
    L = model_decode_sequence(model, dims.k_max, 0.9, blocks, buf, logs)
    torch.cuda.synchronize()
    assert L == dims.L + 32
    for j, tr in enumerate(traces):
        got = logs[j].cpu().numpy()
        for s, st in enumerate(tr.steps):
            if not _clear(st):
                break
            assert np.array_equal(got[s], st.tok), f"block {j} step {s}"
    g = lambda t: O.bf16_to_f64(t.cpu().view(torch.int16).numpy().view(np.uint16))  # noqa: E731
    for l in range(cfg.n_layers):
        for got, want in ((g(model.Kp[l, :L]), prefix[l][0]), (g(model.Vp[l, :L]), prefix[l][1])):
            assert np.array_equal(got[:dims.L], want[:dims.L])          # the original prefix
            rms = float(np.sqrt(np.mean(want[dims.L:] ** 2)))
            err = np.abs(got[dims.L:] - want[dims.L:])
            assert err.max() <= 2.0 ** -4 * rms and err.mean() <= 2.0 ** -8 * rms * np.sqrt(2)
