"""GPU parity: liblopa against the CPU oracle on identical seeded inputs.

Per call (build, attention, LM head, select) on small and ragged shapes that
exercise both kernel families (MFMA and plain) and their edges, then the
whole step on every workload shape, including the full 7B-shaped ones in the
launch configuration the benchmark times.
"""
import math

import numpy as np
import pytest
import torch

import lookahead_decoding_amd as lopa
from lookahead_decoding_amd.step import StepBuffers, dims_of, to_device
import oracle as O
import synth
from _parity import (assert_build_equal, assert_h_close, assert_head_close, assert_winner_valid,
                     check_step, conf_tol, gpu_build, gpu_initial, run_gpu_step, act_to_f64,
                     device_inputs)

pytestmark = pytest.mark.gpu
M = O.MASK


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lopa.lib()
    yield
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# build
# ---------------------------------------------------------------------------

def _rand_state(rng, B, V=5000, tie_levels=None):
    tok = rng.integers(0, V, B).astype(np.int32)
    nm = int(rng.integers(0, B + 1))
    tok[rng.choice(B, nm, replace=False)] = M
    if tie_levels is None:
        conf = rng.random(B).astype(np.float32)
    else:
        conf = rng.choice(np.array(tie_levels, np.float32), B)
    arg = rng.integers(0, V, B).astype(np.int32)
    return tok, conf, arg


@pytest.mark.parametrize("seed", range(60))
def test_gpu_build_bit_exact(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 65))
    k_max = int(rng.integers(0, 16))
    k = int(rng.integers(0, k_max + 1))
    levels = [0.3, 0.5, 0.5, 0.92, 0.95] if seed % 3 == 0 else None
    tok, conf, arg = _rand_state(rng, B, tie_levels=levels)
    tau = np.float32(0.9)
    dims = lopa.Dims(L=0, B=B, Hq=1, Hkv=1, d=8, V=5000, k_max=k_max, dtype=lopa.F32)
    g = gpu_build(dims, k, tau, tok, conf, arg)
    assert_build_equal(g, O.branch_build(tok, conf, arg, k, tau, k_max + 1))


@pytest.mark.parametrize("case", ["none_masked", "all_above", "single", "full64", "one_left"])
def test_gpu_build_edges(case):
    B, k_max, k = 64, 15, 15
    tok = np.full(B, M, np.int32)
    conf = np.linspace(0.1, 0.8, B).astype(np.float32)
    arg = np.arange(B, dtype=np.int32) + 100
    if case == "none_masked":
        tok = np.arange(B, dtype=np.int32)
    elif case == "all_above":
        conf[:] = 0.99
    elif case == "single":
        tok[:] = 7
        tok[40] = M
    elif case == "one_left":
        conf[:] = 0.95
        conf[10] = 0.5
    dims = lopa.Dims(L=0, B=B, Hq=1, Hkv=1, d=8, V=5000, k_max=k_max, dtype=lopa.F32)
    g = gpu_build(dims, k, np.float32(0.9), tok, conf, arg)
    assert_build_equal(g, O.branch_build(tok, conf, arg, k, np.float32(0.9), k_max + 1))


@pytest.mark.parametrize("B,k_max,case", [(1, 0, "rand"), (17, 4, "rand"), (32, 4, "rand"),
                                            (64, 15, "rand"), (64, 15, "none"), (64, 15, "all"),
                                            (33, 1, "last"), (64, 8, "first")])
def test_gpu_block_rows(B, k_max, case):
    """Initial-pass rows on the device: every masked position, ascending, in
    slot 0; the other slots empty; the LM head's outputs cleared."""
    rng = np.random.default_rng(B * 100 + k_max)
    tok = rng.integers(0, 5000, B).astype(np.int32)
    if case == "rand":
        tok[rng.random(B) < 0.5] = M
    elif case == "all":
        tok[:] = M
    elif case == "last":
        tok[-1] = M
    elif case == "first":
        tok[0] = M
    dims = lopa.Dims(L=0, B=B, Hq=1, Hkv=1, d=8, V=5000, k_max=k_max, dtype=lopa.F32)
    n = (k_max + 1) * B
    dev = "cuda"
    nb = torch.full((1,), 7, dtype=torch.int32, device=dev)
    rows = torch.full((n,), 12345, dtype=torch.int32, device=dev)
    row_ptr = torch.full((k_max + 2,), -9, dtype=torch.int32, device=dev)
    conf = torch.full((n,), 3.5, dtype=torch.float32, device=dev)
    arg = torch.full((n,), 77, dtype=torch.int32, device=dev)
    lopa.lopa_block_rows(dims, to_device(tok), nb, rows, row_ptr, conf, arg)
    torch.cuda.synchronize()
    masked = np.flatnonzero(tok == M)
    want_rows = np.zeros(n, np.int32)
    want_rows[:len(masked)] = masked
    want_ptr = np.full(k_max + 2, len(masked), np.int32)
    want_ptr[0] = 0
    assert int(nb.item()) == 1
    assert np.array_equal(rows.cpu().numpy(), want_rows)
    assert np.array_equal(row_ptr.cpu().numpy(), want_ptr)
    assert np.all(conf.cpu().numpy() == 0.0) and np.all(arg.cpu().numpy() == -1)
    # conf / arg may be left out
    rows.fill_(5)
    lopa.lopa_block_rows(dims, to_device(tok), nb, rows, row_ptr)
    torch.cuda.synchronize()
    assert np.array_equal(rows.cpu().numpy(), want_rows)


# ---------------------------------------------------------------------------
# select
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(30))
def test_gpu_select(seed):
    rng = np.random.default_rng(100 + seed)
    B = int(rng.integers(1, 65))
    nbm = int(rng.integers(1, 17))
    nb = int(rng.integers(1, nbm + 1))
    br_mask = (rng.random((nbm, B)) < 0.6).astype(np.uint8)
    br_mask[nb:] = 0
    if seed % 5 == 0:
        br_mask[nb - 1] = 0            # a branch with nothing left: confidence 1
    br_tok = np.where(br_mask == 1, M, rng.integers(0, 99, (nbm, B))).astype(np.int32)
    conf = rng.random(nbm * B).astype(np.float32)
    if seed % 4 == 0:
        conf[:] = 0.25                 # every branch ties: the anchor must win
    arg = rng.integers(0, 9999, nbm * B).astype(np.int32)
    ref = O.branch_select(nb, br_mask, br_tok, conf.astype(np.float64), arg)
    dims = lopa.Dims(L=0, B=B, Hq=1, Hkv=1, d=8, V=10000, k_max=nbm - 1, dtype=lopa.F32)
    buf = StepBuffers(dims)
    lopa.lopa_branch_select(dims, to_device(np.array([nb], np.int32)),
                            to_device(br_mask.reshape(-1)), to_device(br_tok.reshape(-1)),
                            to_device(conf), to_device(arg), buf.bconf, buf.winner,
                            buf.tok_next, buf.conf_next, buf.arg_next)
    torch.cuda.synchronize()
    bc = buf.bconf.cpu().numpy().astype(np.float64)
    np.testing.assert_allclose(bc[:nb], ref.bconf[:nb], rtol=1e-6, atol=1e-7)
    assert np.all(bc[nb:] == -1)
    w = int(buf.winner.item())
    # identical float32 inputs: a float32 mean of n <= 64 values in [0, 1]
    # is within n * 2^-24 of the exact mean, so two branches whose exact
    # means differ by more than twice that are ordered as the oracle orders
    # them; closer ones may go either way, to a near-best branch
    sel_margin = 2 * 64 * 2.0 ** -24
    assert_winner_valid(buf.bconf.cpu().numpy(), w, nb, ref.bconf, ref.winner, ref.margin,
                        sel_margin)
    if seed % 4 == 0:
        assert w == ref.winner
    np.testing.assert_array_equal(buf.tok_next.cpu().numpy(), br_tok[w])
    m = br_mask[w] == 1
    cn, an = buf.conf_next.cpu().numpy(), buf.arg_next.cpu().numpy()
    np.testing.assert_array_equal(cn[m], conf[w * B:(w + 1) * B][m])
    np.testing.assert_array_equal(an[m], arg[w * B:(w + 1) * B][m])
    assert np.all(cn[~m] == 0) and np.all(an[~m] == -1)


# ---------------------------------------------------------------------------
# attention (per call, identical inputs)
# ---------------------------------------------------------------------------

ATTN_CASES = [
    # name, overrides of the tiny workload, nb
    ("f32-mha", dict(), 4),
    ("bf16-mfma-ragged-L", dict(dtype="bf16", L=100, B=16, Hq=4, Hkv=1, d=128, k=2), 3),
    ("bf16-mfma-L0", dict(dtype="bf16", L=0, B=32, Hq=28, Hkv=4, d=128, k=1), 2),
    ("bf16-mfma-span", dict(dtype="bf16", L=70, B=32, Hq=14, Hkv=2, d=128, k=4), 4),
    ("bf16-mfma-G1", dict(dtype="bf16", L=129, B=16, Hq=2, Hkv=2, d=128, k=3), 4),
    ("bf16-plain-d64", dict(dtype="bf16", L=33, B=8, Hq=4, Hkv=2, d=64, k=2), 3),
    ("bf16-mfma-split3", dict(dtype="bf16", L=1500, B=16, m=8, Hq=4, Hkv=1, d=128, k=2), 3),
    ("bf16-mfma-split-nb1", dict(dtype="bf16", L=1100, B=16, m=8, Hq=8, Hkv=2, d=128, k=3), 1),
    ("f32-gqa-d96", dict(L=1030, B=5, m=3, Hq=6, Hkv=3, d=96, k=1), 2),
    # a full 64-key own block; 32-row tiles straddling branches (B*G = 140)
    ("bf16-mfma-B64", dict(dtype="bf16", L=200, B=64, m=8, Hq=28, Hkv=4, d=128, k=2), 3),
    ("bf16-mfma-B20-G7", dict(dtype="bf16", L=64, B=20, m=8, Hq=28, Hkv=4, d=128, k=3), 4),
    # prefixes of 4096 keys and more: the 128-row kernel.  192 rows over 2 row
    # groups (the second half empty), branches of 64 rows, 16 splits
    ("bf16-wide-16splits", dict(dtype="bf16", L=4133, B=16, m=8, Hq=4, Hkv=1, d=128, k=2), 3),
    # G = 7: 128-row workgroups straddle branches (B*G = 140); dead slots
    ("bf16-wide-B20-G7", dict(dtype="bf16", L=4100, B=20, m=8, Hq=28, Hkv=4, d=128, k=3), 3),
    # a full 64-key own block, 2 splits
    ("bf16-wide-B64", dict(dtype="bf16", L=4096, B=64, m=8, Hq=14, Hkv=2, d=128, k=4), 5),
    ("bf16-wide-nb1", dict(dtype="bf16", L=5000, B=16, m=8, Hq=8, Hkv=2, d=128, k=3), 1),
]


@pytest.mark.parametrize("name,ov,nb", ATTN_CASES, ids=[c[0] for c in ATTN_CASES])
def test_gpu_attn(name, ov, nb):
    inp = synth.make_inputs(synth.TINY, with_weight=False, **ov)
    cfg = inp.cfg
    dims = dims_of(cfg)
    x = device_inputs(inp)
    buf = StepBuffers(dims)
    buf.H.fill_(7.0)                        # slots b >= nb must stay untouched
    lopa.lopa_branch_attn(dims, x["Kp"], x["Vp"], x["Qb"], x["Kb"], x["Vb"],
                          to_device(np.array([nb], np.int32)), buf.H, buf.ws)
    torch.cuda.synchronize()
    Hg = act_to_f64(buf.H)
    Hx = O.branch_attn(inp.Kp, inp.Vp, inp.Qb, inp.Kb, inp.Vb, nb, cfg.Hq, cfg.Hkv)
    assert_h_close(Hg[:nb], Hx[:nb], cfg.dtype, name)
    assert np.all(Hg[nb:] == 7.0)


@pytest.mark.parametrize("kn", [1, 8, 15, 16, 23, 24, 27, 28, 31, 32, 33, 40, 47, 48, 55, 56, 63])
def test_gpu_attn_ragged_last_unit(kn):
    """Every way a prefix can end inside a 64-key unit: kn valid keys in the
    last one, so each 32-key half of it holds none, some or all of them (a
    toolchain hazard once corrupted exactly the kn = 24..31 and 56..63
    cases)."""
    ov = dict(dtype="bf16", L=64 + kn, B=16, m=8, Hq=4, Hkv=1, d=128, k=2)
    inp = synth.make_inputs(synth.TINY, with_weight=False, **ov)
    cfg = inp.cfg
    dims = dims_of(cfg)
    x = device_inputs(inp)
    buf = StepBuffers(dims)
    nb = dims.nb_max
    lopa.lopa_branch_attn(dims, x["Kp"], x["Vp"], x["Qb"], x["Kb"], x["Vb"],
                          to_device(np.array([nb], np.int32)), buf.H, buf.ws)
    torch.cuda.synchronize()
    Hx = O.branch_attn(inp.Kp, inp.Vp, inp.Qb, inp.Kb, inp.Vb, nb, cfg.Hq, cfg.Hkv)
    assert_h_close(act_to_f64(buf.H)[:nb], Hx[:nb], cfg.dtype, f"kn={kn}")


@pytest.mark.parametrize("kn", [1, 31, 32, 33, 63])
def test_gpu_attn_wide_ragged_last_unit(kn):
    """The 128-row kernel with the prefix ending inside a 64-key unit."""
    ov = dict(dtype="bf16", L=4096 + kn, B=16, m=8, Hq=4, Hkv=1, d=128, k=2)
    inp = synth.make_inputs(synth.TINY, with_weight=False, **ov)
    cfg = inp.cfg
    dims = dims_of(cfg)
    x = device_inputs(inp)
    buf = StepBuffers(dims)
    nb = dims.nb_max
    lopa.lopa_branch_attn(dims, x["Kp"], x["Vp"], x["Qb"], x["Kb"], x["Vb"],
                          to_device(np.array([nb], np.int32)), buf.H, buf.ws)
    torch.cuda.synchronize()
    Hx = O.branch_attn(inp.Kp, inp.Vp, inp.Qb, inp.Kb, inp.Vb, nb, cfg.Hq, cfg.Hkv)
    assert_h_close(act_to_f64(buf.H)[:nb], Hx[:nb], cfg.dtype, f"kn={kn}")


@pytest.mark.parametrize("L", [1500, 4100])
def test_gpu_attn_scores_outgrow_the_first_units(L):
    """Keys in the second half of the prefix score up to ~40 (log2 units)
    above the first ones, so a row's exponent reference moves many times and
    O and l are rescaled (both attention kernels)."""
    ov = dict(dtype="bf16", L=L, B=16, m=8, Hq=8, Hkv=2, d=128, k=3)
    inp = synth.make_inputs(synth.TINY, with_weight=False, **ov)
    K = O.bf16_to_f64(inp.Kp)
    K[L // 2:] *= 1.0 + 11.0 * np.linspace(0.0, 1.0, L - L // 2)[:, None, None]
    inp.Kp = synth.f32_to_bf16_bits(K.astype(np.float32)).reshape(inp.Kp.shape)
    cfg = inp.cfg
    dims = dims_of(cfg)
    x = device_inputs(inp)
    buf = StepBuffers(dims)
    nb = dims.nb_max
    lopa.lopa_branch_attn(dims, x["Kp"], x["Vp"], x["Qb"], x["Kb"], x["Vb"],
                          to_device(np.array([nb], np.int32)), buf.H, buf.ws)
    torch.cuda.synchronize()
    Hx = O.branch_attn(inp.Kp, inp.Vp, inp.Qb, inp.Kb, inp.Vb, nb, cfg.Hq, cfg.Hkv)
    assert_h_close(act_to_f64(buf.H)[:nb], Hx[:nb], cfg.dtype, f"L={L}")


# ---------------------------------------------------------------------------
# LM head (per call, identical inputs: the oracle's rounded H)
# ---------------------------------------------------------------------------

HEAD_CASES = [
    ("f32-tiny", dict(), None),
    # the float32 MFMA kernel: a hidden size that is not a multiple of its
    # 32-wide K chunk, a vocabulary that is not a multiple of its 256-entry
    # tile (and one smaller than a tile), three 32-row tiles, the last ragged
    ("f32-hidden30-V1001-90rows", dict(Hq=3, Hkv=3, d=10, V=1001, B=32, m=30, k=2), None),
    ("f32-V100-1row", dict(Hq=2, Hkv=1, d=40, V=100, B=4, m=1, k=0), None),
    ("bf16-mfma-ragged-V", dict(dtype="bf16", Hq=4, Hkv=2, d=64, V=1000, B=16, m=12, k=3), None),
    ("bf16-mfma-two-groups", dict(dtype="bf16", Hq=2, Hkv=1, d=64, V=700, B=64, m=64, k=15), None),
    ("bf16-plain-hidden96", dict(dtype="bf16", Hq=3, Hkv=1, d=32, V=513, B=8, m=6, k=2), None),
    ("bf16-mfma-V1", dict(dtype="bf16", Hq=1, Hkv=1, d=64, V=1, B=4, m=4, k=1), None),
    ("bf16-stream-12tiles", dict(dtype="bf16", Hq=2, Hkv=1, d=64, V=1000, B=32, m=30, k=5), None),
    ("bf16-stream-1row", dict(dtype="bf16", Hq=2, Hkv=2, d=128, V=3001, B=8, m=1, k=0), None),
    ("bf16-tiled-hidden192", dict(dtype="bf16", Hq=3, Hkv=1, d=64, V=777, B=16, m=15, k=2), None),
    # 300 rows: three row groups of <= 4 tiles; 450 rows: two groups of <= 8 tiles
    ("bf16-three-groups", dict(dtype="bf16", Hq=2, Hkv=1, d=64, V=2500, B=32, m=30, k=9), None),
    ("bf16-two-wide-groups", dict(dtype="bf16", Hq=2, Hkv=2, d=128, V=1900, B=64, m=50, k=8), None),
    # vocabulary parts of 316, 384 and 448 rows (256 parts): a last pass of 60
    # and of 128 rows runs as the half-width tail pipeline after a full pass;
    # one of 192 rows stays in the full-width pipeline with idle columns
    ("bf16-vocab-tail-60", dict(dtype="bf16", Hq=1, Hkv=1, d=64, V=80896, B=16, m=10, k=1), None),
    ("bf16-vocab-tail-128", dict(dtype="bf16", Hq=1, Hkv=1, d=64, V=98304, B=16, m=10, k=1), None),
    ("bf16-vocab-no-tail-192", dict(dtype="bf16", Hq=1, Hkv=1, d=64, V=114688, B=16, m=10, k=1),
     None),
]


@pytest.mark.parametrize("name,ov,_", HEAD_CASES, ids=[c[0] for c in HEAD_CASES])
def test_gpu_lmhead(name, ov, _):
    """Every originally masked position of every branch slot is listed (the
    LM-head call does not care how the row list was built), on the oracle's
    rounded H, so both sides see identical inputs."""
    inp = synth.make_inputs(synth.TINY, **ov)
    cfg = inp.cfg
    dims = dims_of(cfg)
    nb = dims.nb_max
    Hx = O.round_like(O.branch_attn(inp.Kp, inp.Vp, inp.Qb, inp.Kb, inp.Vb, nb, cfg.Hq, cfg.Hkv),
                      inp.Qb.dtype)
    masked = np.flatnonzero(inp.tok == M)
    r = np.array([b * cfg.B + p for b in range(nb) for p in masked], np.int32)
    row_ptr = np.array([b * len(masked) for b in range(nb + 1)], np.int32)
    x = device_inputs(inp)
    buf = StepBuffers(dims)
    Hin = O.f64_to_bf16(Hx) if cfg.dtype == "bf16" else Hx.astype(np.float32)
    rows = np.zeros(dims.nb_max * dims.B, np.int32)
    rows[:len(r)] = r
    lo = torch.full((dims.nb_max * dims.B, dims.V), np.nan, dtype=torch.float32, device="cuda")
    lopa.lopa_lmhead_conf(dims, to_device(Hin), x["W"], to_device(rows), to_device(row_ptr),
                          to_device(np.array([nb], np.int32)), buf.conf, buf.arg, lo, buf.ws)
    torch.cuda.synchronize()
    ref = O.lmhead_conf(np.stack([Hx[q // cfg.B, q % cfg.B] for q in r]), inp.W, keep_logits=True)
    cg, ag = buf.conf.cpu().numpy()[r], buf.arg.cpu().numpy()[r]
    assert_head_close(cg, ag, ref.conf, ref.arg, ref.margin, cfg.dtype, name,
                      top_tok=ref.top_tok, top_logit=ref.top_logit)
    # identical inputs: confidences agree far inside the stated tolerance
    np.testing.assert_allclose(cg, ref.conf, rtol=1e-4, atol=1e-6)
    assert np.all(cg >= 1.0 / cfg.V * (1 - 1e-5)) and np.all(cg <= 1 + 1e-6)
    lg = lo.cpu().numpy()[r]
    np.testing.assert_allclose(lg, ref.logits, rtol=1e-5, atol=1e-5 * np.abs(ref.logits).max())


# Without full logits, m_max of 6 row tiles or more and hidden a multiple of
# 128: the wide kernel (four waves, register tiles of q owned row tiles plus
# a share of the r remaining ones, activation fragments loaded into
# registers from the operand-ordered copy) where it serves the row-tile count
# (6, 9-20, 23-26), the narrow one elsewhere (and alone when m_max is
# at most 5 tiles or hidden is not a multiple of 128).  Row groups of
# th = 4q + r tiles, 8 weight tiles per pass up to 8 row tiles, 4 from 9;
# vocabulary parts with empty parts (V < 4096), a last pass of 1 .. all live
# weight tiles (with 2 and with 4 K chunks: the activation register sets
# alternate by chunk), a vocabulary size that is not a multiple of 16, and 2
# and 3 row groups.  Rows: every masked position of every branch slot.
WIDE_CASES = [
    # name, overrides (M = (k + 1) m)
    ("tiles5-narrow-alone", dict(dtype="bf16", Hq=2, Hkv=1, d=64, V=3000, B=32, m=30, k=4)),
    ("th6-empty-parts", dict(dtype="bf16", Hq=2, Hkv=1, d=64, V=3000, B=48, m=45, k=3)),
    ("th6-tw8", dict(dtype="bf16", Hq=2, Hkv=2, d=64, V=9000, B=60, m=60, k=2)),
    ("th6-tw8-last-5", dict(dtype="bf16", Hq=2, Hkv=2, d=64, V=37100, B=60, m=60, k=2)),
    ("tiles7-narrow", dict(dtype="bf16", Hq=1, Hkv=1, d=128, V=65636, B=56, m=56, k=3)),
    ("tiles8-narrow", dict(dtype="bf16", Hq=2, Hkv=1, d=128, V=20000, B=32, m=30, k=7)),
    ("th9-ragged-V", dict(dtype="bf16", Hq=2, Hkv=1, d=64, V=33333, B=32, m=32, k=8)),
    ("th10", dict(dtype="bf16", Hq=4, Hkv=1, d=64, V=12000, B=64, m=64, k=4)),
    ("th11", dict(dtype="bf16", Hq=2, Hkv=1, d=64, V=100000, B=64, m=50, k=6)),
    ("th11-hidden64-narrow", dict(dtype="bf16", Hq=1, Hkv=1, d=64, V=100000, B=64, m=50, k=6)),
    ("th12-tw4", dict(dtype="bf16", Hq=4, Hkv=1, d=64, V=70000, B=64, m=48, k=7)),
    ("th12-hidden192-narrow", dict(dtype="bf16", Hq=3, Hkv=1, d=64, V=70000, B=64, m=48, k=7)),
    ("th13-last-pass-1-tile", dict(dtype="bf16", Hq=2, Hkv=1, d=64, V=40000, B=32, m=26, k=15)),
    ("th13-4-chunks-last-pass-1-tile",
     dict(dtype="bf16", Hq=4, Hkv=1, d=64, V=40000, B=32, m=26, k=15)),
    ("tiles14-two-groups-th7", dict(dtype="bf16", Hq=2, Hkv=1, d=64, V=9000, B=64, m=56, k=7)),
    ("tiles14-th7-two-passes-last-7",
     dict(dtype="bf16", Hq=2, Hkv=1, d=64, V=59392, B=64, m=56, k=7)),
    ("tiles15-two-groups-th8-tw8", dict(dtype="bf16", Hq=2, Hkv=1, d=64, V=7000, B=50, m=50, k=8)),
    ("tiles16-th8-tw8-last-1",
     dict(dtype="bf16", Hq=4, Hkv=1, d=64, V=35840, B=64, m=32, k=15)),
    ("tiles17-two-groups-th9", dict(dtype="bf16", Hq=2, Hkv=1, d=64, V=21000, B=60, m=60, k=8)),
    ("tiles18-two-groups-th9", dict(dtype="bf16", Hq=2, Hkv=1, d=64, V=9100, B=64, m=57, k=9)),
    ("tiles24-two-groups-th12", dict(dtype="bf16", Hq=2, Hkv=1, d=64, V=9000, B=64, m=48, k=15)),
    ("tiles26-two-groups-th13-last-1",
     dict(dtype="bf16", Hq=4, Hkv=1, d=64, V=20000, B=64, m=52, k=15)),
    ("tiles32-narrow-three-groups", dict(dtype="bf16", Hq=1, Hkv=1, d=64, V=5000, B=64, m=64, k=15)),
]


@pytest.mark.parametrize("name,ov", WIDE_CASES, ids=[c[0] for c in WIDE_CASES])
def test_gpu_lmhead_wide(name, ov):
    inp = synth.make_inputs(synth.TINY, **ov)
    cfg = inp.cfg
    dims = dims_of(cfg)
    nb = dims.nb_max
    Hx = O.round_like(O.branch_attn(inp.Kp, inp.Vp, inp.Qb, inp.Kb, inp.Vb, nb, cfg.Hq, cfg.Hkv),
                      inp.Qb.dtype)
    masked = np.flatnonzero(inp.tok == M)
    r = np.array([b * cfg.B + p for b in range(nb) for p in masked], np.int32)
    assert len(r) > 128
    row_ptr = np.array([b * len(masked) for b in range(nb + 1)], np.int32)
    rows = np.zeros(dims.nb_max * dims.B, np.int32)
    rows[:len(r)] = r
    x = device_inputs(inp)
    buf = StepBuffers(dims)
    H, R, P, NB = (to_device(O.f64_to_bf16(Hx)), to_device(rows), to_device(row_ptr),
                   to_device(np.array([nb], np.int32)))
    buf.conf.fill_(-3.0)
    buf.arg.fill_(-3)
    lopa.lopa_lmhead_conf(dims, H, x["W"], R, P, NB, buf.conf, buf.arg, None, buf.ws)
    torch.cuda.synchronize()
    cg, ag = buf.conf.cpu().numpy(), buf.arg.cpu().numpy()
    ref = O.lmhead_conf(np.stack([Hx[q // cfg.B, q % cfg.B] for q in r]), inp.W)
    assert_head_close(cg[r], ag[r], ref.conf, ref.arg, ref.margin, cfg.dtype, name,
                      top_tok=ref.top_tok, top_logit=ref.top_logit)
    np.testing.assert_allclose(cg[r], ref.conf, rtol=1e-4, atol=1e-6)
    unlisted = np.setdiff1d(np.arange(dims.nb_max * dims.B), r)
    assert np.all(cg[unlisted] == -3.0) and np.all(ag[unlisted] == -3)
    # the entropy-carrying head: same confidences and tokens, bit for bit
    lopa.lopa_lmhead_conf_ent(dims, H, x["W"], R, P, NB, buf.conf, buf.arg, buf.ent, None, buf.ws)
    torch.cuda.synchronize()
    assert np.array_equal(buf.conf.cpu().numpy()[r], cg[r])
    assert np.array_equal(buf.arg.cpu().numpy()[r], ag[r])
    np.testing.assert_allclose(buf.ent.cpu().numpy()[r], ref.ent, rtol=0, atol=2e-4)


def test_gpu_lmhead_zero_weight_uniform():
    cfg = synth.StepConfig("zero-w", "bf16", L=4, B=8, m=5, k=0, Hq=2, Hkv=1, d=64, V=152064)
    dims = dims_of(cfg)
    buf = StepBuffers(dims)
    H = torch.randn(1, 8, 128, device="cuda").to(torch.bfloat16)
    W = torch.zeros(cfg.V, 128, dtype=torch.bfloat16, device="cuda")
    rows = to_device(np.array([0, 2, 3, 5, 7, 0, 0, 0], np.int32))
    lopa.lopa_lmhead_conf(dims, H, W, rows, to_device(np.array([0, 5], np.int32)),
                          to_device(np.array([1], np.int32)), buf.conf, buf.arg, None, buf.ws)
    torch.cuda.synchronize()
    c = buf.conf.cpu().numpy()[[0, 2, 3, 5, 7]]
    a = buf.arg.cpu().numpy()[[0, 2, 3, 5, 7]]
    assert np.all(a == 0)
    np.testing.assert_allclose(c, 1.0 / cfg.V, rtol=1e-6)


# ---------------------------------------------------------------------------
# whole step
# ---------------------------------------------------------------------------

SMALL_STEPS = [
    ("tiny", dict()),
    ("tiny-k0", dict(k=0)),
    ("tiny-nothing-masked", dict(m=0)),
    ("bf16-small-gqa", dict(dtype="bf16", L=200, B=32, m=20, k=5, Hq=8, Hkv=2, d=128, V=3000)),
    ("bf16-B64-k15", dict(dtype="bf16", L=64, B=64, m=60, k=15, Hq=2, Hkv=1, d=128, V=2000)),
    ("f32-B1", dict(B=1, m=1, k=2)),
]


@pytest.mark.parametrize("name,ov", SMALL_STEPS, ids=[c[0] for c in SMALL_STEPS])
def test_gpu_step_small(name, ov):
    inp = synth.make_inputs(synth.TINY, **ov)
    c, a, head = O.initial_state(inp)
    # the GPU's own initial pass agrees with the oracle's
    cg, ag = gpu_initial(inp)
    masked = np.flatnonzero(inp.tok == M)
    if len(masked):
        assert_head_close(cg[masked], ag[masked], head.conf, head.arg, head.margin, inp.cfg.dtype,
                          "initial pass", top_tok=head.top_tok, top_logit=head.top_logit)
    ref = O.verification_step(inp, c, a)
    g = run_gpu_step(inp, c, a)
    check_step(inp, c, a, ref, g)


def _report(name, info):
    print(f"[parity] {name}: " + ", ".join(f"{k}={v}" for k, v in info.items()), flush=True)


@pytest.mark.parametrize("name", synth.SEVEN_B)
def test_gpu_step_7b(name):
    """Full 7B-shaped workloads (the benchmark's launch configuration)."""
    print(f"[parity] start {name}", flush=True)
    inp = synth.make_inputs(name)
    c, a, head = O.initial_state(inp)
    cg, ag = gpu_initial(inp)
    masked = np.flatnonzero(inp.tok == M)
    assert_head_close(cg[masked], ag[masked], head.conf, head.arg, head.margin, "bf16",
                      "initial pass", top_tok=head.top_tok, top_logit=head.top_logit)
    ref = O.verification_step(inp, c, a)
    g = run_gpu_step(inp, c, a)
    info = check_step(inp, c, a, ref, g)
    _report(name, info)
