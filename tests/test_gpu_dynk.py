"""GPU parity of the explore stage with a confidence floor for lookahead
candidates (lopa_branch_build_floor) against the oracle's branch_build, and
of whole blocks decoded with it (decode.decode_block(gamma=...)).

Explore is integer and compare logic: bit-exact, ties at the floor
included (conf == gamma is a candidate on both sides, in float32).  Blocks:
compared step by step while every decision was clear-cut (as for the plain
explore, with the floor test's gaps |conf - gamma| > 1e-4 added)."""
import numpy as np
import pytest
import torch

import lookahead_decoding_amd as lopa
import synth
from _parity import assert_build_equal
from lookahead_decoding_amd.decode import DecodeBuffers, decode_block
from lookahead_decoding_amd.step import StepBuffers, dims_of, to_device
from oracle import decode_oracle as D
from oracle import lopa_oracle as O

pytestmark = pytest.mark.gpu
M = O.MASK


@pytest.mark.parametrize("seed", range(40))
def test_gpu_build_floor_bit_exact(seed):
    rng = np.random.default_rng(900 + seed)
    B = int(rng.integers(1, 65))
    k_max = int(rng.integers(0, 16))
    k = int(rng.integers(0, k_max + 1))
    tok = rng.integers(0, 5000, B).astype(np.int32)
    tok[rng.random(B) < rng.random()] = M
    levels = np.array([0.1, 0.3, 0.3, 0.5, 0.95], np.float32)
    conf = (rng.choice(levels, B) if seed % 2 else rng.random(B)).astype(np.float32)
    arg = rng.integers(0, 5000, B).astype(np.int32)
    gamma = np.float32([0.0, 0.3, 0.45, 0.3, 2.0, -1.0][seed % 6])
    tau = np.float32(0.9)
    dims = lopa.Dims(L=0, B=B, Hq=1, Hkv=1, d=8, V=5000, k_max=k_max, dtype=lopa.F32)
    buf = StepBuffers(dims)
    lopa.lopa_branch_build_floor(dims, k, tau, gamma, to_device(tok), to_device(conf),
                                 to_device(arg), buf.nb, buf.br_tok, buf.br_mask, buf.rows,
                                 buf.row_ptr)
    torch.cuda.synchronize()
    nbm = dims.nb_max
    g = dict(nb=int(buf.nb.item()), br_tok=buf.br_tok.cpu().numpy().reshape(nbm, B),
             br_mask=buf.br_mask.cpu().numpy().reshape(nbm, B), rows=buf.rows.cpu().numpy(),
             row_ptr=buf.row_ptr.cpu().numpy())
    assert_build_equal(g, O.branch_build(tok, conf, arg, k, tau, nbm, gamma))


def test_gpu_build_floor_edges():
    """One position; nothing masked; everything masked with the floor
    exactly at every confidence (ties at the floor are candidates)."""
    for tok, conf, k, gamma in (
            (np.array([M], np.int32), np.array([0.2], np.float32), 0, 0.5),
            (np.array([3, 4, 5], np.int32), np.zeros(3, np.float32), 2, 0.1),
            (np.full(8, M, np.int32), np.full(8, 0.25, np.float32), 3, 0.25)):
        B = len(tok)
        arg = np.arange(B, dtype=np.int32) + 10
        dims = lopa.Dims(L=0, B=B, Hq=1, Hkv=1, d=8, V=100, k_max=3, dtype=lopa.F32)
        buf = StepBuffers(dims)
        lopa.lopa_branch_build_floor(dims, k, np.float32(0.9), np.float32(gamma), to_device(tok),
                                     to_device(conf), to_device(arg), buf.nb, buf.br_tok,
                                     buf.br_mask, buf.rows, buf.row_ptr)
        torch.cuda.synchronize()
        nbm = dims.nb_max
        g = dict(nb=int(buf.nb.item()), br_tok=buf.br_tok.cpu().numpy().reshape(nbm, B),
                 br_mask=buf.br_mask.cpu().numpy().reshape(nbm, B), rows=buf.rows.cpu().numpy(),
                 row_ptr=buf.row_ptr.cpu().numpy())
        assert_build_equal(g, O.branch_build(tok, conf, arg, k, np.float32(0.9), nbm,
                                             np.float32(gamma)))


FLOOR_DECODE = [
    ("floor-0.25", 0.25, 7), ("floor-0.3", 0.3, 21), ("floor-0.4", 0.4, 24),
]


@pytest.mark.parametrize("name,gamma,seed", FLOOR_DECODE, ids=[c[0] for c in FLOOR_DECODE])
def test_gpu_decode_block_floor(name, gamma, seed):
    ov = dict(dtype="bf16", L=100, B=32, m=20, Hq=8, Hkv=2, d=128, V=4096, k=3)
    inp = synth.make_inputs(synth.TINY, **ov)
    cfg = inp.cfg
    dims = dims_of(cfg)
    k, tau = 3, 0.9
    tr = D.decode_block(inp, seed, k, tau, gamma=gamma)
    m = int(np.sum(inp.tok == M))
    buf = DecodeBuffers(dims)
    x = {n: to_device(getattr(inp, n)) for n in ("Kp", "Vp", "W")}
    log = torch.zeros(m, cfg.B, dtype=torch.int32, device="cuda")
    decode_block(dims, k, tau, seed, inp.tok, x["Kp"], x["Vp"], x["W"], buf, m, log, gamma=gamma)
    torch.cuda.synchronize()
    got = log.cpu().numpy()
    compared = 0
    for s, st in enumerate(tr.steps):
        if not (st.fill_margin > 1e-2 and st.rank_gap > 1e-4 and st.tau_gap > 1e-4
                and st.win_margin > 1e-3):
            break
        assert np.array_equal(got[s], st.tok), f"{name}: step {s}"
        compared += 1
    assert compared >= min(3, len(tr.steps))
    # the floor does shrink the branch count on the way
    assert min(st.nb for st in tr.steps) < max(st.nb for st in tr.steps)
