"""GPU parity of the alternative branch score (entropy in the LM head,
lopa_branch_select_alpha) against oracle/lopa_oracle.py and
oracle/decode_oracle.py.

* lopa_lmhead_conf_ent on the oracle's rounded H (identical inputs): the
  normalised entropy within 2e-4 (logits agree to ~1e-5 relative; the entropy
  moves by at most twice the largest logit error, divided by ln V), and conf /
  arg bit-identical to lopa_lmhead_conf's (the entropy term is carried beside
  the unchanged sums).  A zero weight gives the uniform distribution: entropy
  exactly 1.
* lopa_branch_select_alpha on random consistent states: scores within float32
  summation error, winner where the oracle's margin exceeds 1e-3 (and on exact
  ties: the anchor), next state bit-exact.
* Whole blocks decoded with the alternative score, compared step by step while
  every decision is clear-cut (as for the mean-confidence score, with the
  winner's score margin > 5e-3: a score sums up to B entropy terms).
"""
import numpy as np
import pytest
import torch

import lookahead_decoding_amd as lopa
import synth
from lookahead_decoding_amd.decode import DecodeBuffers, decode_block
from lookahead_decoding_amd.step import StepBuffers, dims_of, to_device
from oracle import decode_oracle as D
from oracle import lopa_oracle as O
from _parity import assert_winner_valid, device_inputs

pytestmark = pytest.mark.gpu
M = O.MASK

ENT_CASES = [
    ("f32-tiny", dict()),
    ("bf16-mfma-ragged-V", dict(dtype="bf16", Hq=4, Hkv=2, d=64, V=1000, B=16, m=12, k=3)),
    ("bf16-plain-hidden96", dict(dtype="bf16", Hq=3, Hkv=1, d=32, V=513, B=8, m=6, k=2)),
    ("bf16-mfma-V1", dict(dtype="bf16", Hq=1, Hkv=1, d=64, V=1, B=4, m=4, k=1)),
    ("bf16-stream-12tiles", dict(dtype="bf16", Hq=2, Hkv=1, d=64, V=1000, B=32, m=30, k=5)),
    ("bf16-three-groups", dict(dtype="bf16", Hq=2, Hkv=1, d=64, V=2500, B=32, m=30, k=9)),
    ("bf16-two-wide-groups", dict(dtype="bf16", Hq=2, Hkv=2, d=128, V=1900, B=64, m=50, k=8)),
    ("bf16-7b-shape", dict(dtype="bf16", L=64, Hq=28, Hkv=4, d=128, V=152064, B=32, m=24, k=2)),
]


@pytest.mark.parametrize("name,ov", ENT_CASES, ids=[c[0] for c in ENT_CASES])
def test_gpu_lmhead_entropy(name, ov):
    inp = synth.make_inputs(synth.TINY, **ov)
    cfg = inp.cfg
    dims = dims_of(cfg)
    nb = dims.nb_max
    Hx = O.round_like(O.branch_attn(inp.Kp, inp.Vp, inp.Qb, inp.Kb, inp.Vb, nb, cfg.Hq, cfg.Hkv),
                      inp.Qb.dtype)
    masked = np.flatnonzero(inp.tok == M)
    r = np.array([b * cfg.B + p for b in range(nb) for p in masked], np.int32)
    row_ptr = np.array([b * len(masked) for b in range(nb + 1)], np.int32)
    rows = np.zeros(dims.nb_max * dims.B, np.int32)
    rows[:len(r)] = r
    Hin = O.f64_to_bf16(Hx) if cfg.dtype == "bf16" else Hx.astype(np.float32)
    x = device_inputs(inp)
    buf = StepBuffers(dims)
    H, R, P, NB = (to_device(Hin), to_device(rows), to_device(row_ptr),
                   to_device(np.array([nb], np.int32)))
    buf.ent.fill_(-5.0)
    lopa.lopa_lmhead_conf_ent(dims, H, x["W"], R, P, NB, buf.conf, buf.arg, buf.ent, None, buf.ws)
    torch.cuda.synchronize()
    c1, a1, e1 = buf.conf.clone(), buf.arg.clone(), buf.ent.cpu().numpy()
    lopa.lopa_lmhead_conf(dims, H, x["W"], R, P, NB, buf.conf, buf.arg, None, buf.ws)
    torch.cuda.synchronize()
    assert torch.equal(c1[r.tolist()], buf.conf[r.tolist()])
    assert torch.equal(a1[r.tolist()], buf.arg[r.tolist()])
    ref = O.lmhead_conf(np.stack([Hx[q // cfg.B, q % cfg.B] for q in r]), inp.W)
    np.testing.assert_allclose(e1[r], ref.ent, rtol=0, atol=2e-4)
    assert np.all(e1[r] >= -1e-6) and np.all(e1[r] <= 1 + 1e-6)
    unlisted = np.setdiff1d(np.arange(dims.nb_max * dims.B), r)
    assert np.all(e1[unlisted] == -5.0)


def test_gpu_lmhead_entropy_uniform():
    """Zero weight: every logit is 0, the distribution is uniform, the
    normalised entropy is 1 and the confidence 1 / V."""
    cfg = synth.StepConfig("zero-w", "bf16", L=4, B=8, m=5, k=0, Hq=2, Hkv=1, d=64, V=152064)
    dims = dims_of(cfg)
    buf = StepBuffers(dims)
    H = torch.randn(1, 8, 128, device="cuda").to(torch.bfloat16)
    W = torch.zeros(cfg.V, 128, dtype=torch.bfloat16, device="cuda")
    rows = to_device(np.array([0, 2, 3, 5, 7, 0, 0, 0], np.int32))
    lopa.lopa_lmhead_conf_ent(dims, H, W, rows, to_device(np.array([0, 5], np.int32)),
                              to_device(np.array([1], np.int32)), buf.conf, buf.arg, buf.ent,
                              None, buf.ws)
    torch.cuda.synchronize()
    e = buf.ent.cpu().numpy()[[0, 2, 3, 5, 7]]
    np.testing.assert_allclose(e, 1.0, rtol=0, atol=1e-6)


def _alpha_state(rng, B, nbm, nb):
    """A consistent explore result: the state's masked set S; every branch
    leaves a subset of S masked; a filled position holds some token."""
    tok = rng.integers(0, 99, B).astype(np.int32)
    S = rng.random(B) < 0.7
    tok[S] = M
    conf_state = np.where(S, rng.random(B), 0).astype(np.float32)
    br_mask = ((rng.random((nbm, B)) < 0.6) & S[None, :]).astype(np.uint8)
    br_mask[nb:] = 0
    br_tok = np.where(br_mask == 1, M, np.where(S[None, :], rng.integers(0, 99, (nbm, B)),
                                                 tok[None, :])).astype(np.int32)
    return tok, conf_state, br_mask, br_tok


@pytest.mark.parametrize("seed", range(24))
def test_gpu_select_alpha(seed):
    rng = np.random.default_rng(500 + seed)
    B = int(rng.integers(1, 65))
    nbm = int(rng.integers(1, 17))
    nb = int(rng.integers(1, nbm + 1))
    alpha = [0.0, 1.0, 0.5, float(rng.random())][seed % 4]
    tok, conf_state, br_mask, br_tok = _alpha_state(rng, B, nbm, nb)
    tie = seed % 6 == 5
    if tie:
        # every branch fills and leaves the same positions: an exact tie
        br_mask[:nb] = br_mask[0]
        br_tok[:nb] = br_tok[0]
    conf = rng.random(nbm * B).astype(np.float32)
    ent = rng.random(nbm * B).astype(np.float32)
    if tie:
        ent[:] = np.tile(ent[:B], nbm)
    arg = rng.integers(0, 9999, nbm * B).astype(np.int32)
    ref = O.branch_select_alpha(nb, br_mask, br_tok, conf.astype(np.float64), arg,
                                ent.astype(np.float64), tok, conf_state, alpha)
    dims = lopa.Dims(L=0, B=B, Hq=1, Hkv=1, d=8, V=10000, k_max=nbm - 1, dtype=lopa.F32)
    buf = StepBuffers(dims)
    lopa.lopa_branch_select_alpha(
        dims, alpha, to_device(tok), to_device(conf_state), to_device(np.array([nb], np.int32)),
        to_device(br_mask.reshape(-1)), to_device(br_tok.reshape(-1)), to_device(conf),
        to_device(arg), to_device(ent), buf.bconf, buf.winner, buf.tok_next, buf.conf_next,
        buf.arg_next)
    torch.cuda.synchronize()
    sc = buf.bconf.cpu().numpy().astype(np.float64)
    np.testing.assert_allclose(sc[:nb], ref.bconf[:nb], rtol=1e-5, atol=1e-5)
    assert np.all(sc[nb:] == -1)
    w = int(buf.winner.item())
    if tie:
        assert w == 0
    assert_winner_valid(buf.bconf.cpu().numpy(), w, nb, ref.bconf, ref.winner, ref.margin)
    np.testing.assert_array_equal(buf.tok_next.cpu().numpy(), br_tok[w])
    m = br_mask[w] == 1
    cn, an = buf.conf_next.cpu().numpy(), buf.arg_next.cpu().numpy()
    np.testing.assert_array_equal(cn[m], conf[w * B:(w + 1) * B][m])
    np.testing.assert_array_equal(an[m], arg[w * B:(w + 1) * B][m])
    assert np.all(cn[~m] == 0) and np.all(an[~m] == -1)


TOK_MARGIN, GAP, WIN = 1e-2, 1e-4, 5e-3

ALPHA_DECODE = [
    # name, workload overrides, k, tau, seed, alpha (each stays clear-cut for
    # most of its steps)
    ("bf16-half", dict(dtype="bf16", L=100, B=32, m=20, Hq=8, Hkv=2, d=128, V=4096, k=3),
     3, 0.9, 24, 0.5),
    ("bf16-0.7", dict(dtype="bf16", L=100, B=32, m=20, Hq=8, Hkv=2, d=128, V=4096, k=3),
     3, 0.9, 22, 0.7),
    ("bf16-one", dict(dtype="bf16", L=64, B=32, m=16, Hq=8, Hkv=2, d=128, V=3000, k=4),
     4, 0.9, 13, 1.0),
    ("bf16-zero", dict(dtype="bf16", L=64, B=32, m=16, Hq=8, Hkv=2, d=128, V=3000, k=4),
     4, 0.9, 12, 0.0),
    ("f32-0.3", dict(dtype="f32", L=30, B=16, m=12, Hq=4, Hkv=4, d=64, V=500, k=4), 4, 0.9, 11, 0.3),
]


@pytest.mark.parametrize("name,ov,k,tau,seed,alpha", ALPHA_DECODE,
                         ids=[c[0] for c in ALPHA_DECODE])
def test_gpu_decode_block_alpha(name, ov, k, tau, seed, alpha):
    inp = synth.make_inputs(synth.TINY, **ov)
    cfg = inp.cfg
    dims = dims_of(cfg)
    tr = D.decode_block(inp, seed, k, tau, alpha=alpha)
    m = int(np.sum(inp.tok == M))
    buf = DecodeBuffers(dims)
    x = {n: to_device(getattr(inp, n)) for n in ("Kp", "Vp", "W")}
    log = torch.zeros(m, cfg.B, dtype=torch.int32, device="cuda")
    decode_block(dims, k, tau, seed, inp.tok, x["Kp"], x["Vp"], x["W"], buf, m, log, alpha=alpha)
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
