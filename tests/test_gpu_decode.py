"""GPU parity of block decoding over several steps (lookahead_decoding_amd.decode
against oracle/decode_oracle.py).

* lopa_synth_qkv: bit-exact against the oracle's independent implementation of
  the same published generator (Philox4x32-10 + Irwin-Hall), slots >= nb
  untouched.
* Whole blocks: the GPU and the oracle each decode the block on their own.
  Their inputs at every step are bit-identical as long as they took the same
  decisions before, so the tokens after each step must be identical while
  every decision the oracle took was clear-cut: the argmax behind every token
  a step filled (top-2 logit gap > 1e-2), the confidence gaps the explore
  stage's choices hinged on and the threshold test (> 1e-4), and the winner
  (branch-confidence gap > 1e-3).
  After the first step with a near-tie the two may part ways legitimately and
  the comparison stops there; each case below is checked to stay clear-cut for
  most of its steps.
"""
import numpy as np
import pytest
import torch

import lookahead_decoding_amd as lopa
import synth
from lookahead_decoding_amd.decode import DecodeBuffers, decode_block
from lookahead_decoding_amd.step import dims_of, to_device
from oracle import decode_oracle as D
from oracle import lopa_oracle as O

pytestmark = pytest.mark.gpu

TOK_MARGIN, GAP, WIN = 1e-2, 1e-4, 1e-3


@pytest.mark.parametrize("dtype,Hq,Hkv,d,nb_live", [
    ("bf16", 8, 2, 128, 3), ("bf16", 28, 4, 128, 5), ("f32", 4, 4, 64, 2), ("bf16", 3, 1, 96, 1),
])
def test_gpu_synth_qkv_bit_exact(dtype, Hq, Hkv, d, nb_live):
    B, k_max = 20, 4
    dims = lopa.Dims(L=8, B=B, Hq=Hq, Hkv=Hkv, d=d, V=64, k_max=k_max,
                     dtype=lopa.F32 if dtype == "f32" else lopa.BF16)
    rng = np.random.default_rng(Hq * 100 + d)
    tok = rng.integers(-1, 152064, size=(k_max + 1, B)).astype(np.int32)
    tok[rng.random(tok.shape) < 0.3] = O.MASK
    seed = 0x1234_5678_9ABC_DEF0 + Hq
    act = torch.float32 if dtype == "f32" else torch.bfloat16
    Q = torch.full((k_max + 1, B, Hq, d), 3.0, dtype=act, device="cuda")
    K = torch.full((k_max + 1, B, Hkv, d), 3.0, dtype=act, device="cuda")
    V = torch.full_like(K, 3.0)
    lopa.lopa_synth_qkv(dims, seed, to_device(tok.reshape(-1)),
                        to_device(np.array([nb_live], np.int32)), Q, K, V)
    torch.cuda.synchronize()
    like = np.float32 if dtype == "f32" else np.uint16
    ref = D.token_qkv(seed, tok[:nb_live], Hq, Hkv, d, like)
    for got, want in zip((Q, K, V), ref):
        g = got.cpu()
        g = g.numpy() if dtype == "f32" else g.view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(g[:nb_live], want)
        fill = np.float32(3.0) if dtype == "f32" else O.f64_to_bf16(np.array(3.0))
        assert np.all(g[nb_live:] == fill)


DECODE_CASES = [
    # name, workload overrides, k, tau, seed
    ("bf16-mfma-k3", dict(dtype="bf16", L=100, B=32, m=20, Hq=8, Hkv=2, d=128, V=4096, k=3), 3, 0.9, 7),
    ("bf16-mfma-k0", dict(dtype="bf16", L=100, B=32, m=12, Hq=8, Hkv=2, d=128, V=4096, k=3), 0, 0.9, 8),
    ("bf16-mfma-k7-lowtau", dict(dtype="bf16", L=64, B=32, m=24, Hq=8, Hkv=2, d=128, V=3000, k=7),
     7, 0.05, 9),
    ("bf16-plain-d64", dict(dtype="bf16", L=40, B=16, m=10, Hq=4, Hkv=2, d=64, V=700, k=2), 2, 0.9, 10),
    ("f32-k4", dict(dtype="f32", L=30, B=16, m=12, Hq=4, Hkv=4, d=64, V=500, k=4), 4, 0.9, 11),
]


@pytest.mark.parametrize("name,ov,k,tau,seed", DECODE_CASES, ids=[c[0] for c in DECODE_CASES])
def test_gpu_decode_block(name, ov, k, tau, seed):
    inp = synth.make_inputs(synth.TINY, **ov)
    cfg = inp.cfg
    dims = dims_of(cfg)
    tr = D.decode_block(inp, seed, k, tau)
    m = int(np.sum(inp.tok == O.MASK))
    buf = DecodeBuffers(dims)
    x = {n: to_device(getattr(inp, n)) for n in ("Kp", "Vp", "W")}
    log = torch.zeros(m, cfg.B, dtype=torch.int32, device="cuda")
    decode_block(dims, k, tau, seed, inp.tok, x["Kp"], x["Vp"], x["W"], buf, m, log)
    torch.cuda.synchronize()
    got = log.cpu().numpy()
    compared = 0
    for s, st in enumerate(tr.steps):
        if not (st.fill_margin > TOK_MARGIN and st.rank_gap > GAP and st.tau_gap > GAP
                and st.win_margin > WIN):
            break
        assert np.array_equal(got[s], st.tok), f"{name}: step {s} tokens differ"
        compared += 1
    assert compared >= min(3, len(tr.steps)), f"{name}: only {compared} clear-cut steps"
    if compared == len(tr.steps):
        n = len(tr.steps)
        assert not np.any(got[n - 1] == O.MASK)
        # steps after completion change nothing
        assert np.all(got[n - 1:] == got[n - 1])
        if n > 1:
            assert np.any(got[n - 2] == O.MASK)


def test_gpu_commit_block_copies_winner_slot():
    from lookahead_decoding_amd import lopa_commit_block
    dims = lopa.Dims(L=10, B=12, Hq=4, Hkv=2, d=64, V=64, k_max=3, dtype=lopa.BF16)
    Kb = torch.randn(4, 12, 2, 64, device="cuda").to(torch.bfloat16)
    Vb = torch.randn(4, 12, 2, 64, device="cuda").to(torch.bfloat16)
    Kp = torch.zeros(10 + 24, 2, 64, dtype=torch.bfloat16, device="cuda")
    Vp = torch.zeros_like(Kp)
    for w, at in ((2, 10), (0, 22)):
        lopa_commit_block(dims, to_device(np.array([w], np.int32)), Kb, Vb, Kp, Vp, at)
    torch.cuda.synchronize()
    assert torch.equal(Kp[10:22], Kb[2]) and torch.equal(Vp[10:22], Vb[2])
    assert torch.equal(Kp[22:34], Kb[0]) and torch.equal(Vp[22:34], Vb[0])
    assert torch.count_nonzero(Kp[:10]) == 0


def test_gpu_decode_sequence_three_blocks():
    from lookahead_decoding_amd.decode import decode_sequence
    ov = dict(dtype="bf16", L=64, B=32, m=10, Hq=8, Hkv=2, d=128, V=4096, k=3)
    inp = synth.make_inputs(synth.TINY, **ov)
    cfg = inp.cfg
    rng = np.random.default_rng(5)   # blocks whose decisions are clear-cut throughout
    blocks = []
    for m in (10, 14, 0):
        tok = rng.integers(0, cfg.V, size=cfg.B).astype(np.int32)
        tok[rng.choice(cfg.B, m, replace=False)] = O.MASK
        blocks.append(tok)
    seed, k, tau = 77, 3, 0.9
    sq = D.decode_sequence(inp, seed, k, tau, blocks)
    L0, B = cfg.L, cfg.B
    dims_max = dims_of(cfg)
    dims_max.L = L0 + 2 * B
    buf = DecodeBuffers(dims_max)
    Kp = torch.zeros(L0 + 3 * B, cfg.Hkv, cfg.d, dtype=torch.bfloat16, device="cuda")
    Vp = torch.zeros_like(Kp)
    Kp[:L0] = to_device(inp.Kp)
    Vp[:L0] = to_device(inp.Vp)
    W = to_device(inp.W)
    logs = [torch.zeros(max(int(np.sum(b == O.MASK)), 1), B, dtype=torch.int32, device="cuda")
            for b in blocks]
    dims = dims_of(cfg)
    L = decode_sequence(dims, k, tau, seed, blocks, Kp, Vp, W, buf, logs)
    torch.cuda.synchronize()
    assert L == L0 + 3 * B
    for j, tr in enumerate(sq.blocks):
        clear = all(st.fill_margin > TOK_MARGIN and st.rank_gap > GAP and st.tau_gap > GAP
                    and st.win_margin > WIN for st in tr.steps)
        assert clear, f"block {j} not clear-cut"
        got = logs[j].cpu().numpy()
        for s, st in enumerate(tr.steps):
            assert np.array_equal(got[s], st.tok), f"block {j} step {s}"
    # the committed prefix, bit for bit
    g = lambda t: t.cpu().view(torch.int16).numpy().view(np.uint16)  # noqa: E731
    assert np.array_equal(g(Kp), sq.Kp) and np.array_equal(g(Vp), sq.Vp)
