"""Derive the tolerances of the model tests from the arithmetic: writes
tests/golden/forward_noise.json.  Calls only oracle/ (and the seeded case
tables in tests/_model_cases.py).

Error model.  The library and the oracle round to bf16 at the same points
(after each norm, q/k/v, the attention output, the MLP activation, the final
norm); between them the library computes in float32 and the oracle in
float64.  So the library's value entering a rounding point is the oracle's
times (1 + e), e a float32-level discrepancy: accumulation over K terms
gives |e| ~ 2^-24 sqrt(K) (K <= 18944: ~8e-6), and the attention weights
carried as a bf16 high + low pair give ~1.5e-5.  The model takes e as
independent normal noise of standard deviation 2^-16 (1.53e-5, the largest
of these) at every rounding point and runs the oracle's own forward with it:
a value near a rounding boundary then rounds the other way, exactly as it
does in the library, and the one-ulp differences propagate through the rest
of the network as they do there.  Over SAMPLES noise draws the script keeps,
per case,

  * the largest |difference| / RMS and the mean |difference| / RMS of the
    final rows H and of every layer's block K and V;
  * for block decoding, over the initial pass and the first verification
    step's rows: the largest change of a row's confidence (the probability
    of its most likely token), of a branch confidence (the mean confidence
    of the rows a branch leaves masked) and of a logit relative to the row's
    top logit (its most likely token keeps first place whenever its lead
    exceeds that change).

The tests allow twice the largest deviation and 1.5 times the mean one.

Run: python tests/golden/make_forward_noise.py   (a few minutes on 8 cores)
"""
from __future__ import annotations

import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.dirname(HERE))

from oracle import lopa_oracle as O  # noqa: E402
from oracle import model_oracle as MO  # noqa: E402
import _model_cases as C  # noqa: E402

NOISE = 2.0 ** -16
SAMPLES = 4
_exact_rnd = MO.rnd


def _noisy(rng):
    def rnd(x):
        x = np.asarray(x, np.float64)
        return _exact_rnd(x * (1.0 + NOISE * rng.standard_normal(x.shape)))
    return rnd


def _forward_noisy(rng, *args, **kw):
    MO.rnd = _noisy(rng)
    try:
        return MO.forward(*args, **kw)
    finally:
        MO.rnd = _exact_rnd


def _stats(got, want):
    rms = float(np.sqrt(np.mean(want * want))) or 1.0
    err = np.abs(got - want)
    return float(err.max() / rms), float(err.mean() / rms)


def _worst(acc, key, st):
    mx, mn = acc.get(key, (0.0, 0.0))
    acc[key] = (max(mx, st[0]), max(mn, st[1]))


def forward_case(cfg, seed, L, tok, keys=("H", "K", "V")):
    layers = [MO.synth_layer(seed, cfg, l) for l in range(cfg.n_layers)]
    prefix = [MO.synth_prefix(seed, cfg, l, L) for l in range(cfg.n_layers)]
    ref = MO.forward(seed, cfg, L, tok, layers, prefix)
    acc = {}
    for s in range(SAMPLES):
        out = _forward_noisy(np.random.default_rng(1000 + s), seed, cfg, L, tok, layers, prefix)
        for key, a, b in (("H", out.H, ref.H), ("K", out.Kb, ref.Kb), ("V", out.Vb, ref.Vb)):
            if key in keys:
                _worst(acc, key, _stats(a, b))
    return {k: list(v) for k, v in acc.items()}


def _cfg(case, n_layers=None):
    return MO.ModelCfg(n_layers=case.get("n_layers", n_layers), Hq=case["Hq"], Hkv=case["Hkv"],
                       d=case["d"], inter=case["inter"], V=case["V"], mask_id=case["V"] - 1)


def _head(H, W):
    lg = H @ W.astype(np.float64).T
    p = np.exp(lg - lg.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    return lg, p.max(1)


def decode_case(geo, m, seed):
    """Confidence and logit changes over the initial pass and the first
    verification step of the block decoding case."""
    L, B, k, Hq, Hkv, d, inter, V, n = geo
    cfg = MO.ModelCfg(n_layers=n, Hq=Hq, Hkv=Hkv, d=d, inter=inter, V=V, mask_id=V - 1)
    layers = [MO.synth_layer(seed, cfg, l) for l in range(n)]
    prefix = [MO.synth_prefix(seed, cfg, l, L) for l in range(n)]
    W = MO.lm_head_weight(seed, cfg)
    tok0 = C.block(seed, B, m, V)
    conf, arg, margin, _ = MO.initial_pass(seed, cfg, L, tok0, layers, prefix, W)
    br = O.branch_build(tok0, conf, arg, k, np.float32(0.9), k + 1)
    passes = [(tok0[None], [int(p) for p in np.flatnonzero(tok0 == C.MASK)]),
              (br.br_tok[:br.nb], [int(r) for r in br.rows])]
    dconf = dlead = dbranch = 0.0
    for toks, rows in passes:
        ref = MO.forward(seed, cfg, L, toks, layers, prefix)
        pick = lambda H: np.stack([H[r // B, r % B] for r in rows])  # noqa: E731
        lg0, c0 = _head(pick(ref.H), W)
        top = np.argmax(lg0, axis=1)
        for s in range(SAMPLES):
            out = _forward_noisy(np.random.default_rng(2000 + s), seed, cfg, L, toks, layers,
                                 prefix)
            lg, c = _head(pick(out.H), W)
            dl = lg - lg0
            dconf = max(dconf, float(np.abs(c - c0).max()))
            dlead = max(dlead, float(np.abs(dl - dl[np.arange(len(top)), top][:, None]).max()))
            owner = np.array(rows) // B
            for b in np.unique(owner):
                dbranch = max(dbranch, abs(float(c[owner == b].mean() - c0[owner == b].mean())))
    return dconf, dlead, dbranch


def main():
    res = {"noise_rel": NOISE, "samples": SAMPLES, "forward": {}, "decode": {}}
    for name, case, nb in C.FWD_CASES:
        tok = C.fwd_tokens(name, case)[:nb]
        res["forward"][name] = forward_case(_cfg(case), C.fwd_seed(name), case["L"], tok)
        print(name, res["forward"][name], flush=True)
    tok, conf, arg, k, tau = C.step_state()
    br = O.branch_build(tok, conf, arg, k, np.float32(tau), 1 + C.STEP_CASE["k_max"])
    res["forward"]["step"] = forward_case(_cfg(C.STEP_CASE), C.STEP_SEED, C.STEP_CASE["L"],
                                          br.br_tok[:br.nb], ("H",))
    print("step", res["forward"]["step"], flush=True)
    res["forward"]["7b-2"] = forward_case(_cfg(C.SEVEN_B, 2), C.SEVEN_B_SEED, C.SEVEN_B["L"],
                                          C.seven_b_tokens(), ("H", "K"))
    print("7b-2", res["forward"]["7b-2"], flush=True)
    # the committed K/V of a decoded block (the sequence test's geometry, at
    # both prefix lengths it reaches), a stand-in block with every position set
    geo = C.DECODE_CASES[0][1]
    L, B, _, Hq, Hkv, d, inter, V, n = geo
    case = dict(Hq=Hq, Hkv=Hkv, d=d, inter=inter, V=V, n_layers=n)
    full = C.block(1, B, 0, V)[None]
    acc = {}
    for Lj in (L, L + B):
        for key, v in forward_case(_cfg(case), 1, Lj, full, ("K", "V")).items():
            _worst(acc, key, v)
    res["forward"]["commit"] = {k: list(v) for k, v in acc.items()}
    print("commit", res["forward"]["commit"], flush=True)
    for name, geo, m, seed in C.DECODE_CASES:
        new = dict(zip(("conf", "lead", "branch"), decode_case(geo, m, seed)))
        g = name.split("-")[0]
        cur = res["decode"].get(g, {})
        res["decode"][g] = {k: max(cur.get(k, 0.0), v) for k, v in new.items()}
        print(name, new, flush=True)
    with open(os.path.join(HERE, "forward_noise.json"), "w") as f:
        json.dump(res, f, indent=1, sort_keys=True)
        f.write("\n")


if __name__ == "__main__":
    main()
