"""Helpers shared by the GPU parity tests: run the library on the same seeded
inputs the oracle sees and compare to the agreement rules:

* integer outputs (branch count, tokens, masks, row lists, winner) are
  bit-exact; a predicted token only where the oracle's top-2 logit margin
  exceeds 1e-2, the winner only where the oracle's best-minus-second branch
  confidence exceeds 1e-3;
* below those margins the GPU's choice must still be a near-best one: a
  token whose oracle logit lies within 1e-2 of the row's largest, a winner
  whose oracle branch confidence lies within 1e-3 of the best (and the
  GPU's winner is the first maximum of its own branch confidences);
* confidences within 1e-4 absolute (fp32 workloads) or 2e-2 (bf16);
* the attention output H within what one bf16 (or fp32) rounding of the
  exact value allows, plus float32 accumulation error.
"""
from __future__ import annotations

import numpy as np
import torch

import lookahead_decoding_amd as lopa
from lookahead_decoding_amd.step import StepBuffers, dims_of, initial_pass, run_step, to_device
import oracle as O

TOK_MARGIN = 1e-2
WIN_MARGIN = 1e-3


def conf_tol(dtype: str) -> float:
    return 1e-4 if dtype == "f32" else 2e-2


def device_inputs(inp, conf=None, arg=None) -> dict:
    x = {k: to_device(v) for k, v in inp.arrays().items() if v is not None}
    if conf is not None:
        x["conf"] = to_device(np.asarray(conf, np.float32))
        x["arg"] = to_device(np.asarray(arg, np.int32))
    return x


def act_to_f64(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return O.bf16_to_f64(t.cpu().view(torch.int16).numpy().view(np.uint16))
    return t.cpu().numpy().astype(np.float64)


def assert_h_close(H_gpu: np.ndarray, H_exact: np.ndarray, dtype: str, what: str = "H"):
    """H_gpu is the library's (rounded) output, H_exact the oracle's value
    before rounding."""
    if dtype == "f32":
        tol = 2e-6 * np.abs(H_exact) + 2e-6 * np.abs(H_exact).max()
    else:
        # one bf16 rounding: <= 2^-9 relative; float32 accumulation and the
        # bf16 hi+lo probabilities add ~1e-5 relative: allow 2^-8.
        tol = 2.0 ** -8 * np.abs(H_exact) + 2.0 ** -16
    err = np.abs(H_gpu - H_exact)
    bad = err > tol
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} outside tolerance, "
                           f"max err {err.max():.3g}")


def assert_near_best_tokens(arg_gpu, top_tok, top_logit, rows_mask, what="head"):
    """Rows in ``rows_mask`` (near-tied in the oracle): the GPU's token must be
    one whose oracle logit is within TOK_MARGIN of the row's largest.  The
    oracle lists each row's largest logits and their tokens; a token outside
    that list is further than the list's last logit."""
    for r in np.flatnonzero(rows_mask):
        t = int(arg_gpu[r])
        hit = np.flatnonzero(top_tok[r] == t)
        assert hit.size == 1, f"{what}: row {r} token {t} not among the oracle's largest logits"
        gap = top_logit[r][0] - top_logit[r][hit[0]]
        assert gap <= TOK_MARGIN, f"{what}: row {r} token {t} is {gap:.3g} below the best logit"


def assert_head_close(conf_gpu, arg_gpu, conf_ref, arg_ref, margin_ref, dtype, what="head",
                      top_tok=None, top_logit=None):
    conf_gpu = np.asarray(conf_gpu, np.float64)
    err = np.abs(conf_gpu - conf_ref)
    tol = conf_tol(dtype)
    assert (err <= tol).all(), f"{what}: conf max err {err.max():.3g} > {tol}"
    sure = margin_ref > TOK_MARGIN
    mism = (np.asarray(arg_gpu) != np.asarray(arg_ref)) & sure
    assert not mism.any(), f"{what}: {mism.sum()} token mismatches among {sure.sum()} sure rows"
    if top_tok is not None:
        assert_near_best_tokens(np.asarray(arg_gpu), top_tok, top_logit, ~sure, what)
    return float(err.max()) if err.size else 0.0, int((~sure).sum())


def assert_winner_valid(bconf_gpu, w: int, nb: int, bconf_ref, winner_ref: int, margin_ref: float,
                        margin: float = WIN_MARGIN):
    """The GPU's winner is the first maximum of its own branch confidences;
    it equals the oracle's where the oracle's margin exceeds ``margin``, and
    is otherwise a branch whose oracle confidence is within ``margin`` of the
    oracle's best."""
    bc = np.asarray(bconf_gpu)[:nb]
    assert 0 <= w < nb and bc[w] == bc.max() and np.flatnonzero(bc == bc.max())[0] == w
    if margin_ref > margin:
        assert w == winner_ref
    else:
        best = float(np.max(bconf_ref[:nb]))
        assert bconf_ref[w] >= best - margin, (w, bconf_ref[w], best)


def gpu_build(dims, k, tau, tok, conf, arg):
    dev = "cuda"
    buf = StepBuffers(dims, dev)
    lopa.lopa_branch_build(dims, k, tau, to_device(tok), to_device(conf), to_device(arg),
                           buf.nb, buf.br_tok, buf.br_mask, buf.rows, buf.row_ptr)
    torch.cuda.synchronize()
    nbm, B = dims.nb_max, dims.B
    return dict(nb=int(buf.nb.item()),
                br_tok=buf.br_tok.cpu().numpy().reshape(nbm, B),
                br_mask=buf.br_mask.cpu().numpy().reshape(nbm, B),
                rows=buf.rows.cpu().numpy(), row_ptr=buf.row_ptr.cpu().numpy())


def assert_build_equal(g: dict, br: O.Branches):
    assert g["nb"] == br.nb
    np.testing.assert_array_equal(g["br_tok"], br.br_tok)
    np.testing.assert_array_equal(g["br_mask"], br.br_mask)
    np.testing.assert_array_equal(g["row_ptr"], br.row_ptr)
    M = int(br.row_ptr[-1])
    np.testing.assert_array_equal(g["rows"][:M], br.rows)


def run_gpu_step(inp, conf, arg, k=None, tau=None, logits=False):
    cfg = inp.cfg
    dims = dims_of(cfg)
    k = cfg.k if k is None else k
    tau = cfg.tau if tau is None else tau
    x = device_inputs(inp, conf, arg)
    buf = StepBuffers(dims)
    lo = None
    if logits:
        lo = torch.zeros(dims.nb_max * dims.B, dims.V, dtype=torch.float32, device="cuda")
    run_step(dims, k, tau, x, buf, logits_out=lo)
    torch.cuda.synchronize()
    nbm, B = dims.nb_max, dims.B
    out = dict(nb=int(buf.nb.item()), br_tok=buf.br_tok.cpu().numpy().reshape(nbm, B),
               br_mask=buf.br_mask.cpu().numpy().reshape(nbm, B), rows=buf.rows.cpu().numpy(),
               row_ptr=buf.row_ptr.cpu().numpy(), H=act_to_f64(buf.H),
               conf=buf.conf.cpu().numpy(), arg=buf.arg.cpu().numpy(),
               bconf=buf.bconf.cpu().numpy(), winner=int(buf.winner.item()),
               tok_next=buf.tok_next.cpu().numpy(), conf_next=buf.conf_next.cpu().numpy(),
               arg_next=buf.arg_next.cpu().numpy())
    if logits:
        out["logits"] = lo.cpu().numpy()
    return out


def gpu_initial(inp):
    dims = dims_of(inp.cfg)
    x = device_inputs(inp)
    buf = StepBuffers(dims)
    c, a = initial_pass(dims, inp.tok, x, buf)
    torch.cuda.synchronize()
    return c.cpu().numpy(), a.cpu().numpy()


def check_step(inp, conf, arg, ref: O.StepOut, g: dict):
    """Compare a whole GPU step against the oracle's step on identical inputs."""
    cfg = inp.cfg
    br = ref.br
    assert_build_equal(g, br)
    nb = br.nb
    # attention: the oracle's H before rounding
    H_exact = O.branch_attn(inp.Kp, inp.Vp, inp.Qb, inp.Kb, inp.Vb, nb, cfg.Hq, cfg.Hkv)
    assert_h_close(g["H"][:nb], H_exact[:nb], cfg.dtype)
    rows = br.rows
    cerr, excl = assert_head_close(g["conf"][rows], g["arg"][rows], ref.conf_pos[rows],
                                   ref.arg_pos[rows], ref.margin_pos[rows], cfg.dtype,
                                   top_tok=ref.top_tok_pos[rows],
                                   top_logit=ref.top_logit_pos[rows])
    # select
    bc = np.asarray(g["bconf"], np.float64)
    assert np.all(np.abs(bc[:nb] - ref.sel.bconf[:nb]) <= conf_tol(cfg.dtype))
    assert np.all(bc[nb:] == -1)
    assert_winner_valid(g["bconf"], g["winner"], nb, ref.sel.bconf, ref.sel.winner,
                        ref.sel.margin)
    # reuse: the GPU's next state is exactly its own winner's rows
    w = g["winner"]
    np.testing.assert_array_equal(g["tok_next"], g["br_tok"][w])
    for p in range(cfg.B):
        if g["br_mask"][w, p]:
            assert g["conf_next"][p] == g["conf"][w * cfg.B + p]
            assert g["arg_next"][p] == g["arg"][w * cfg.B + p]
        else:
            assert g["conf_next"][p] == 0 and g["arg_next"][p] == -1
    if w == ref.sel.winner:
        np.testing.assert_array_equal(g["tok_next"], ref.sel.tok_next)
    return dict(conf_max_err=cerr, rows=int(len(rows)), rows_excluded_by_margin=excl,
                winner=w, winner_margin=float(ref.sel.margin), nb=nb)
