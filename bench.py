#!/usr/bin/env python3
"""Throughput of one LoPA branch-verification step on one MI355X.

A step = lopa_branch_build -> lopa_branch_attn -> lopa_lmhead_conf ->
lopa_branch_select on one batch of seeded synthetic inputs already resident
in HBM, enqueued on one stream.  Default workload: 7B D2F-Dream-like shapes
(28 q-heads / 4 kv-heads / d 128, hidden 3584, vocabulary 152064, bf16),
committed prefix 512, block 32 with 24 masked positions, k = 4 (5 branches).

Prints ONE JSON line: verification steps/s (value), branch-tokens/s, the
LM-head call's roofline (algorithmic bytes per call / its HIP-event-timed
duration vs 8 TB/s) and the CPU oracle timed on a bounded sample on this
host.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s

# HBM bytes per lopa_lmhead_conf call (k_lmhead_mfma, + k_lmhead_wide where it
# serves, + k_lmhead_merge) and per lopa_branch_attn call (k_attn_dma or k_attn_wide +
# k_attn_combine) from two rocprofv3 --pmc runs of this script: FETCH_SIZE x
# 2.0 + WRITE_SIZE x 1.0 (KiB per dispatch; the factors are what the same
# counters read for a 1 GiB device copy).  Keyed by workload and by a hash of
# the kernel sources the counters were taken on: after any change to those
# sources the figure is not reported.
HEAD_SOURCES = ("lmhead.hip", "head_plan.hpp", "stream_tile.hpp", "lopa_common.hpp")
ATTN_SOURCES = ("attn.hip", "attn_plan.hpp", "lopa_common.hpp")
HEAD_TRAFFIC = {
    "7b-bf16-L512-B32-m24-k4": ("31b4d9616e416850", 1104627674),
    "7b-bf16-L2048-B32-m28-k8": ("31b4d9616e416850", 1111034330),
    "7b-bf16-L1024-B32-m24-k15": ("31b4d9616e416850", 1131087997),
    "7b-bf16-L4096-B64-m48-k8": ("31b4d9616e416850", 1136817484),
}
ATTN_TRAFFIC = {
    "7b-bf16-L512-B32-m24-k4": ("63b58100ea765173", 26504587),
    "7b-bf16-L2048-B32-m28-k8": ("63b58100ea765173", 57528880),
    "7b-bf16-L1024-B32-m24-k15": ("63b58100ea765173", 28514114),
    "7b-bf16-L4096-B64-m48-k8": ("63b58100ea765173", 56802098),
}


def source_hash(files) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "lookahead_decoding_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def head_source_hash() -> str:
    return source_hash(HEAD_SOURCES)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None, help="workload name (default: prefix 512, k=4)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the block-decoding measurement (steps per block, TPF)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="lower bound on the oracle's timed CPU work")
    ap.add_argument("--graph", action="store_true", help="replay the step as a captured HIP graph")
    ap.add_argument("--no-model", action="store_true",
                    help="skip the step with the 28-layer model forward")
    ap.add_argument("--model-no-decode", action="store_true",
                    help="time the model step only, not the block decoded with the model")
    ap.add_argument("--model-steps", type=int, default=30)
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run 3 device copies of 1 GiB (a reference for byte counters)")
    return ap.parse_args()


def algorithmic(cfg, nb: int, M: int) -> dict:
    """Bytes and flops one step must move / do (each input read once, each
    output written once), with nb live branches and M LM-head rows."""
    e = 4 if cfg.dtype == "f32" else 2
    hid = cfg.hidden
    w = cfg.V * hid * e
    head_bytes = w + M * hid * e + M * 8                     # W, H rows, conf+arg
    attn_bytes = (2 * cfg.L * cfg.Hkv * cfg.d + nb * cfg.B * (cfg.Hq + 2 * cfg.Hkv) * cfg.d) * e \
        + nb * cfg.B * hid * e                               # prefix K/V, Q/K/V, H write
    small = cfg.B * 12 + nb * cfg.B * 9 + cfg.B * 12         # build/select state
    head_flops = 2.0 * M * hid * cfg.V
    attn_flops = 4.0 * nb * cfg.B * cfg.Hq * (cfg.L + cfg.B) * cfg.d
    return dict(step_bytes=head_bytes + attn_bytes + small, head_bytes=head_bytes,
                attn_bytes=attn_bytes, head_flops=head_flops, attn_flops=attn_flops,
                w_bytes=w)


def decode_measure(dims, cfg, inp, x, k: int, seed: int, reps: int = 10, alpha=None,
                   gamma=None, temperature=None) -> dict:
    """Decode the workload's block (its masked positions) from the initial
    pass until none is masked, with token-keyed projections: steps, tokens per
    step (TPF), and the time of the whole block (initial pass + its steps).
    ``alpha``: select with the entropy-weighted branch score instead;
    ``gamma``: lookahead candidates need confidence >= gamma ("median": the
    median confidence of the block's masked positions after the initial
    pass)."""
    import torch
    from lookahead_decoding_amd import MASK
    from lookahead_decoding_amd.decode import DecodeBuffers, decode_block

    m = int(np.sum(inp.tok == MASK))
    buf = DecodeBuffers(dims)
    log = torch.zeros(max(m, 1), cfg.B, dtype=torch.int32, device="cuda")
    if gamma == "median":
        from lookahead_decoding_amd.decode import start_block
        start_block(dims, seed, inp.tok, x["Kp"], x["Vp"], x["W"], buf)
        c = buf.conf_s.cpu().numpy()[np.asarray(inp.tok) == MASK]
        gamma = float(np.median(c)) if c.size else 0.0
    opts = dict(alpha=alpha, gamma=gamma, temperature=temperature, sample_seed=seed)
    decode_block(dims, k, cfg.tau, seed, inp.tok, x["Kp"], x["Vp"], x["W"], buf, m, log, **opts)
    torch.cuda.synchronize()
    got = log.cpu().numpy()
    done = [s for s in range(m) if not np.any(got[s] == MASK)]
    steps = done[0] + 1 if done else m
    decode_block(dims, k, cfg.tau, seed, inp.tok, x["Kp"], x["Vp"], x["W"], buf, steps, **opts)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        decode_block(dims, k, cfg.tau, seed, inp.tok, x["Kp"], x["Vp"], x["W"], buf, steps, **opts)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / reps * 1e3
    return {"k": k, "alpha": alpha, "gamma": gamma, "temperature": temperature, "masked": m,
            "steps": steps, "tpf": round(m / steps, 3),
            "ms_per_block": round(ms, 3), "decoded_tokens_per_s": round(m / (ms * 1e-3), 1)}


def model_bytes(dims, md) -> dict:
    """Algorithmic bytes of one lopa_branch_forward: every weight once, the
    embedding rows, each layer's prefix K/V, the block K/V and H written."""
    hid, e = dims.hidden, 2
    qkv = (dims.Hq + 2 * dims.Hkv) * dims.d
    M = dims.nb_max * dims.B
    layer_w = (qkv * hid + qkv + hid * hid + 2 * hid + 2 * md.inter * hid + hid * md.inter) * e
    kv = 2 * dims.Hkv * dims.d * e
    fwd = md.n_layers * (layer_w + dims.L * kv + M * kv) + hid * e + 2 * M * hid * e
    return dict(forward_bytes=fwd, weight_bytes=md.n_layers * layer_w + hid * e,
                flops=2.0 * M * (md.n_layers * layer_w / e))


def model_measure(cfg, inp, steps: int, warmup: int, decode: bool = True) -> dict:
    """A verification step with the 28-layer Qwen2.5/Dream-7B-shaped forward
    (synthetic weights): build -> lopa_branch_forward -> lopa_lmhead_conf
    (the model's LM head) -> select; and the same with one branch (k_max 0)
    for the cost of the extra branches."""
    import torch
    import lookahead_decoding_amd as lopa
    from lookahead_decoding_amd.model import QWEN7B, ForwardBuffers, Model, forward, model_dims
    from lookahead_decoding_amd.step import StepBuffers, dims_of, to_device

    md = model_dims(**QWEN7B)
    out = {"model": "Qwen2.5/Dream-7B geometry, 28 layers, synthetic bf16 weights (Philox)",
           "weights_gb": None}

    def run(k_max: int, k: int) -> dict:
        progress(f"28-layer model step, k_max {k_max}")
        dims = dims_of(cfg)
        dims.k_max = k_max
        model = Model(dims, md, seed=0x7B00 + inp.seed)
        out["weights_gb"] = round(model.layout.total / 1e9, 2)
        buf, fb = StepBuffers(dims), ForwardBuffers(dims, md)
        stream = torch.cuda.current_stream()
        B, nbm = dims.B, dims.nb_max
        # the state a step starts from: slot 0 alone through the model, LM head on the masked rows
        tok = np.asarray(inp.tok, np.int32)
        masked = np.flatnonzero(tok == lopa.MASK).astype(np.int32)
        rows = np.zeros(nbm * B, np.int32)
        rows[:len(masked)] = masked
        row_ptr = np.full(nbm + 1, len(masked), np.int32)
        row_ptr[0] = 0
        one = to_device(np.array([1], np.int32))
        forward(model, to_device(np.tile(tok, nbm)), one, fb, dims=dims)
        lopa.lopa_lmhead_conf(dims, fb.H, model.lm_head, to_device(rows), to_device(row_ptr), one,
                              buf.conf, buf.arg, None, buf.ws)
        conf = buf.conf[:B].clone()
        arg = buf.arg[:B].clone()
        tk = to_device(tok)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]

        def step(e=None):
            lopa.lopa_branch_build(dims, k, cfg.tau, tk, conf, arg, buf.nb, buf.br_tok,
                                   buf.br_mask, buf.rows, buf.row_ptr)
            if e is not None:
                e[0].record(stream)
            forward(model, buf.br_tok, buf.nb, fb, dims=dims)
            if e is not None:
                e[1].record(stream)
            lopa.lopa_lmhead_conf(dims, fb.H, model.lm_head, buf.rows, buf.row_ptr, buf.nb,
                                  buf.conf, buf.arg, None, buf.ws)
            if e is not None:
                e[2].record(stream)
            lopa.lopa_branch_select(dims, buf.nb, buf.br_mask, buf.br_tok, buf.conf, buf.arg,
                                    buf.bconf, buf.winner, buf.tok_next, buf.conf_next,
                                    buf.arg_next)

        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            step(ev[i])
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) / steps * 1e3
        fwd_ms = float(np.mean([a.elapsed_time(b) for a, b, _ in ev]))
        head_ms = float(np.mean([b.elapsed_time(c) for _, b, c in ev]))
        alg = model_bytes(dims, md)
        ach = alg["forward_bytes"] / (fwd_ms * 1e-3) / 1e9
        res = {"k": k, "branches": int(buf.nb.item()), "rows": nbm * B,
               "steps_per_s": round(1e3 / ms, 2), "ms_per_step": round(ms, 3),
               "forward_ms": round(fwd_ms, 3), "lmhead_ms": round(head_ms, 3),
               "forward_roofline": {"bound": "hbm", "achieved": round(ach, 1),
                                    "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                    "frac": round(ach / HBM_PEAK_GBS, 4),
                                    "algorithmic_bytes": alg["forward_bytes"],
                                    "mfma_tflops": round(alg["flops"] / (fwd_ms * 1e-3) / 1e12, 1)}}
        if not decode:
            del model, buf, fb
            torch.cuda.empty_cache()
            return res
        # the block decoded with the model until nothing is masked
        progress(f"28-layer model decode, k_max {k_max}")
        from lookahead_decoding_amd.model import ModelDecodeBuffers, model_decode_block
        m = len(masked)
        dbuf = ModelDecodeBuffers(dims, md)
        log = torch.zeros(max(m, 1), B, dtype=torch.int32, device="cuda")
        model_decode_block(model, dims, k, cfg.tau, tok, dbuf, m, log)
        torch.cuda.synchronize()
        got = log.cpu().numpy()
        done = [s for s in range(m) if not np.any(got[s] == lopa.MASK)]
        dsteps = done[0] + 1 if done else m
        t0 = time.perf_counter()
        for _ in range(2):
            model_decode_block(model, dims, k, cfg.tau, tok, dbuf, dsteps)
        torch.cuda.synchronize()
        dms = (time.perf_counter() - t0) / 2 * 1e3
        res["decode"] = {"masked": m, "steps": dsteps, "tpf": round(m / dsteps, 3),
                         "ms_per_block": round(dms, 2),
                         "decoded_tokens_per_s": round(m / (dms * 1e-3), 1)}
        del model, buf, fb, dbuf
        torch.cuda.empty_cache()
        return res

    out["lookahead"] = run(cfg.k, cfg.k)
    out["one_branch"] = run(0, 0)
    out["extra_branch_cost"] = round(out["lookahead"]["ms_per_step"] /
                                     out["one_branch"]["ms_per_step"] - 1.0, 4)
    return out


def cpu_baseline(inp, conf, arg, seconds: float) -> dict:
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = 1
    n = 0
    t0 = time.perf_counter()
    while True:
        O.verification_step(inp, conf, arg)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds or n >= 50:
            break
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            cpu = next((l.split(":", 1)[1].strip() for l in fh if l.startswith("model name")), cpu)
    except OSError:
        pass
    return {"value": n / el, "unit": "steps/s", "cores": threads, "kind": "oracle",
            "cpu": cpu, "affinity_cpus": len(os.sched_getaffinity(0)),
            "sample": f"{n} full oracle step(s) of the same workload (build, per-branch fp64 "
                      f"attention, fp64 LM head over all {inp.cfg.V} entries of every listed row, "
                      f"select) in {el:.1f} s; cores = BLAS threads of the fp64 matmul"}


PAGES_CONTEXT = {
    "note": "the pages' own figures, on trained D2F weights and real benchmarks (other "
            "hardware); not comparable to a single synthetic verification step",
    "tpf_d2f_dream_gsm8k": [3.1, 10.1],
    "tpf_d2f_diffucoder_humanevalplus": [2.8, 8.3],
    "tokens_per_s_lopa_dist_ascend910c_mbpp": 1073.9,
    "tokens_per_s_lopa_dist_ascend910c_gsm8k": 856.5,
    "extra_branch_compute_overhead": "10-15%",
}


def progress(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def measure_workload(name: str, args, headline: bool) -> tuple[dict, dict]:
    """Time the four-call step on one workload.  Returns the per-workload
    record and the context the headline extras need."""
    import torch

    import lookahead_decoding_amd as lopa
    import synth
    from lookahead_decoding_amd.step import StepBuffers, dims_of, initial_pass, run_step, to_device

    progress(f"workload {name}: drawing inputs")
    inp = synth.make_inputs(name)
    cfg = inp.cfg
    dims = dims_of(cfg)
    stream = torch.cuda.current_stream()
    x = {k: to_device(v) for k, v in inp.arrays().items()}
    buf = StepBuffers(dims)
    conf0, arg0 = initial_pass(dims, inp.tok, x, buf)
    x["conf"], x["arg"] = conf0, arg0
    torch.cuda.synchronize()

    def learn(k):
        # one step to learn nb and M (the state is fixed, so every step is identical)
        run_step(dims, k, cfg.tau, x, buf)
        torch.cuda.synchronize()
        nb = int(buf.nb.item())
        return nb, int(buf.row_ptr[nb].item())

    nb0, M0 = learn(0) if cfg.k > 0 else (None, None)
    nb, M = learn(cfg.k)
    alg = algorithmic(cfg, nb, M)

    graph = None
    if args.graph:
        graph = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(stream)
        with torch.cuda.stream(s):
            run_step(dims, cfg.k, cfg.tau, x, buf)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=s):
            run_step(dims, cfg.k, cfg.tau, x, buf)
        torch.cuda.synchronize()

    # Eager: every SAMPLE-th step of the timed loop carries HIP events around
    # its LM-head call (the roofline's duration, taken inside the timed
    # region); the other steps carry none.  Event records between kernels
    # hold the stream up: three per step cost 6 us a step (4340 against 4460
    # steps/s at prefix 512, batch 32, k 4).  The k = 0 leg (the anchor
    # alone, for the cost of the extra branches) runs the same loop.
    SAMPLE = 10

    def timed_loop(k):
        head_ev = {i: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for i in range(0, args.steps, SAMPLE)}

        def timed_step(i):
            ev_i = head_ev.get(i)
            lopa.lopa_branch_build(dims, k, cfg.tau, x["tok"], x["conf"], x["arg"], buf.nb,
                                   buf.br_tok, buf.br_mask, buf.rows, buf.row_ptr)
            lopa.lopa_branch_attn(dims, x["Kp"], x["Vp"], x["Qb"], x["Kb"], x["Vb"], buf.nb,
                                  buf.H, buf.ws)
            if ev_i:
                ev_i[0].record(stream)
            lopa.lopa_lmhead_conf(dims, buf.H, x["W"], buf.rows, buf.row_ptr, buf.nb, buf.conf,
                                  buf.arg, None, buf.ws)
            if ev_i:
                ev_i[1].record(stream)
            lopa.lopa_branch_select(dims, buf.nb, buf.br_mask, buf.br_tok, buf.conf, buf.arg,
                                    buf.bconf, buf.winner, buf.tok_next, buf.conf_next,
                                    buf.arg_next)

        use_graph = graph is not None and k == cfg.k
        for i in range(args.warmup):
            graph.replay() if use_graph else timed_step(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            graph.replay() if use_graph else timed_step(i)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) / args.steps * 1e3
        head_us = None if use_graph else \
            float(np.mean([a.elapsed_time(b) for a, b in head_ev.values()])) * 1e3
        return ms, head_us

    progress(f"workload {name}: timing {args.steps} steps")
    ms, head_timed_us = timed_loop(cfg.k)
    ms0, head0_us = timed_loop(0) if cfg.k > 0 else (None, None)

    # the distribution of step times, from a second pass of the same steps
    # with an event at every step boundary (outside the timed region)
    step_ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    step_ev[0].record(stream)
    for i in range(args.steps):
        graph.replay() if graph else run_step(dims, cfg.k, cfg.tau, x, buf)
        step_ev[i + 1].record(stream)
    torch.cuda.synchronize()
    step_us = np.array([step_ev[i].elapsed_time(step_ev[i + 1]) for i in range(args.steps)]) * 1e3

    # Per-call durations with HIP events on the stream the calls run on.
    K = max(20, min(args.steps, 100))
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(K)]
    for i in range(K):
        e = ev[i]
        e[0].record(stream)
        lopa.lopa_branch_build(dims, cfg.k, cfg.tau, x["tok"], x["conf"], x["arg"], buf.nb,
                               buf.br_tok, buf.br_mask, buf.rows, buf.row_ptr)
        e[1].record(stream)
        lopa.lopa_branch_attn(dims, x["Kp"], x["Vp"], x["Qb"], x["Kb"], x["Vb"], buf.nb, buf.H,
                              buf.ws)
        e[2].record(stream)
        lopa.lopa_lmhead_conf(dims, buf.H, x["W"], buf.rows, buf.row_ptr, buf.nb, buf.conf,
                              buf.arg, None, buf.ws)
        e[3].record(stream)
        lopa.lopa_branch_select(dims, buf.nb, buf.br_mask, buf.br_tok, buf.conf, buf.arg,
                                buf.bconf, buf.winner, buf.tok_next, buf.conf_next, buf.arg_next)
        e[4].record(stream)
    torch.cuda.synchronize()
    per = np.array([[ev[i][j].elapsed_time(ev[i][j + 1]) for j in range(4)] for i in range(K)])
    call_us = per.mean(axis=0) * 1e3
    calls = {"branch_build": round(float(call_us[0]), 2),
             "branch_attn": round(float(call_us[1]), 2),
             "lmhead_conf": round(float(call_us[2]), 2),
             "branch_select": round(float(call_us[3]), 2)}
    if headline:
        # the entropy-carrying LM head and the alternative select on the same rows
        ev2 = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
        for i in range(K):
            e = ev2[i]
            e[0].record(stream)
            lopa.lopa_lmhead_conf_ent(dims, buf.H, x["W"], buf.rows, buf.row_ptr, buf.nb,
                                      buf.conf, buf.arg, buf.ent, None, buf.ws)
            e[1].record(stream)
            lopa.lopa_branch_select_alpha(dims, 0.5, x["tok"], x["conf"], buf.nb, buf.br_mask,
                                          buf.br_tok, buf.conf, buf.arg, buf.ent, buf.bconf,
                                          buf.winner, buf.tok_next, buf.conf_next, buf.arg_next)
            e[2].record(stream)
            lopa.lopa_lmhead_sample(dims, 0.9, 1000 + i, buf.H, x["W"], buf.rows, buf.row_ptr,
                                    buf.nb, buf.conf, buf.arg, None, buf.ws)
            e[3].record(stream)
        torch.cuda.synchronize()
        alt_us = np.array([[ev2[i][j].elapsed_time(ev2[i][j + 1]) for j in range(3)]
                           for i in range(K)]).mean(axis=0) * 1e3
        calls.update({"lmhead_conf_ent": round(float(alt_us[0]), 2),
                      "branch_select_alpha": round(float(alt_us[1]), 2),
                      "lmhead_sample": round(float(alt_us[2]), 2)})
    # the roofline uses the LM-head call timed inside the timed loop (eager), else the
    # separate per-call loop (graph replay has no per-call events)
    head_us = head_timed_us if head_timed_us is not None else float(call_us[2])
    steps_s = 1e3 / ms
    rec = {
        "steps_per_s": round(steps_s, 2),
        "ms_per_step": round(ms, 4),
        "config": {"workload": cfg.name, "L": cfg.L, "B": cfg.B, "masked": cfg.m, "k": cfg.k,
                   "branches": nb, "lmhead_rows": M, "Hq": cfg.Hq, "Hkv": cfg.Hkv, "d": cfg.d,
                   "hidden": cfg.hidden, "V": cfg.V, "tau": cfg.tau,
                   "graph": bool(args.graph)},
        "branch_tokens_per_s": round(steps_s * nb * cfg.B, 1),
        "lmhead_rows_per_s": round(steps_s * M, 1),
        "step_hbm_frac": round(alg["step_bytes"] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "step_mfma_frac": round((alg["head_flops"] + alg["attn_flops"]) / (ms * 1e-3) / 1e12
                                / BF16_PEAK_TFLOPS, 4),
        # max(time at the HBM roof, time at the MFMA roof) / measured step time
        "step_roofline_frac": round(max(alg["step_bytes"] / (HBM_PEAK_GBS * 1e9),
                                        (alg["head_flops"] + alg["attn_flops"]) /
                                        (BF16_PEAK_TFLOPS * 1e12)) / (ms * 1e-3), 4),
        "step_us_p10_p50_p90": [round(float(np.percentile(step_us, q)), 2) for q in (10, 50, 90)],
        "k0": None if ms0 is None else {"branches": nb0, "lmhead_rows": M0,
                                        "ms_per_step": round(ms0, 4),
                                        "lmhead_us": None if head0_us is None
                                        else round(head0_us, 2)},
        "t_k_over_t_k0": None if ms0 is None else round(ms / ms0, 4),
        "call_us": calls,
        "roofline": head_roofline(cfg, alg, head_us),
        "attn_roofline": attn_roofline(cfg, alg, float(call_us[1])),
    }
    ctx = dict(inp=inp, cfg=cfg, dims=dims, x=x, buf=buf)
    return rec, ctx


def head_roofline(cfg, alg, head_us: float) -> dict:
    """LM-head call: algorithmic bytes (or flops, past the bf16 ridge) per
    call / its event-timed duration, against the MI355X peak of that roof."""
    tr = HEAD_TRAFFIC.get(cfg.name)
    traffic = tr[1] if tr is not None and tr[0] == head_source_hash() else None
    achieved = alg["head_bytes"] / (head_us * 1e-6) / 1e9
    tflops = alg["head_flops"] / (head_us * 1e-6) / 1e12
    # the roof whose time at peak is the longer (rows above ~315 per call
    # pass the bf16 ridge and make it MFMA-bound)
    mfma_bound = (alg["head_flops"] / (BF16_PEAK_TFLOPS * 1e12) >
                  alg["head_bytes"] / (HBM_PEAK_GBS * 1e9))
    kern = "lopa_lmhead_conf (k_lmhead_mfma, + k_lmhead_wide where it serves, + k_lmhead_merge)"
    if mfma_bound:
        return {"kernel": kern, "bound": "mfma", "achieved": round(tflops, 1),
                "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tflops / BF16_PEAK_TFLOPS, 4), "traffic": traffic,
                "algorithmic_flops_per_call": alg["head_flops"],
                "algorithmic_bytes_per_call": alg["head_bytes"], "call_us": round(head_us, 2),
                "hbm_gbs": round(achieved, 1), "hbm_frac": round(achieved / HBM_PEAK_GBS, 4)}
    return {"kernel": kern, "bound": "hbm", "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic, "algorithmic_bytes_per_call": alg["head_bytes"],
            "call_us": round(head_us, 2), "mfma_tflops": round(tflops, 1),
            "mfma_frac": round(tflops / BF16_PEAK_TFLOPS, 4)}


def attn_roofline(cfg, alg, attn_us: float) -> dict:
    """Attention call (event-timed, so it includes one event gap of a few
    microseconds): its flops against the bf16 MFMA peak and its algorithmic
    bytes against HBM; traffic as for the LM head."""
    tr = ATTN_TRAFFIC.get(cfg.name)
    traffic = tr[1] if tr is not None and tr[0] == source_hash(ATTN_SOURCES) else None
    tflops = alg["attn_flops"] / (attn_us * 1e-6) / 1e12
    gbs = alg["attn_bytes"] / (attn_us * 1e-6) / 1e9
    return {"call_us": round(attn_us, 2), "tflops": round(tflops, 1), "traffic": traffic,
            "mfma_frac": round(tflops / BF16_PEAK_TFLOPS, 4), "gbs": round(gbs, 1),
            "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
            "algorithmic_flops_per_call": alg["attn_flops"],
            "algorithmic_bytes_per_call": alg["attn_bytes"]}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): the verification step "
              "runs on a single GPU and is not sharded across GPUs.", file=sys.stderr)
        sys.exit(2)
    import torch

    import lookahead_decoding_amd as lopa
    import synth

    torch.cuda.set_device(0)
    lopa.lib()
    head_name = args.workload or synth.HEADLINE
    rec, ctx = measure_workload(head_name, args, headline=True)
    inp, cfg, dims, x = ctx["inp"], ctx["cfg"], ctx["dims"], ctx["x"]
    out = {
        "metric": "LoPA verification steps/s (7B shapes, 1 GPU)",
        "value": rec["steps_per_s"],
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": rec["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic (seeded; random Q/K/V and LM-head weight of 7B shape)",
        "config": rec["config"],
    }
    for key in ("branch_tokens_per_s", "lmhead_rows_per_s", "step_hbm_frac", "step_mfma_frac",
                "step_roofline_frac", "step_us_p10_p50_p90", "k0", "t_k_over_t_k0", "call_us",
                "roofline", "attn_roofline"):
        out[key] = rec[key]
    if args.copy_probe:
        a = torch.empty(1 << 29, dtype=torch.int16, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        out["copy_probe_bytes"] = a.numel() * a.element_size()
    if not args.no_decode:
        progress("block decoding")
        seed = 0x10FA + inp.seed
        out["decode"] = {
            "data": "token-keyed synthetic Q/K/V (Philox4x32-10, Irwin-Hall N(0,1)) and "
                    "random weights: TPF shows the mechanism, not a trained model's rate",
            "lookahead": decode_measure(dims, cfg, inp, x, cfg.k, seed),
            "anchor_only": decode_measure(dims, cfg, inp, x, 0, seed),
            "lookahead_alpha_0.5": decode_measure(dims, cfg, inp, x, cfg.k, seed, alpha=0.5),
            "lookahead_floor_median": decode_measure(dims, cfg, inp, x, cfg.k, seed,
                                                     gamma="median"),
            "lookahead_sampled_T0.9": decode_measure(dims, cfg, inp, x, cfg.k, seed,
                                                     temperature=0.9),
        }
    if not args.no_model and cfg.dtype == "bf16":
        progress("28-layer model step")
        out["model_step"] = model_measure(cfg, inp, args.model_steps, 5,
                                          decode=not args.model_no_decode)
    del ctx, x
    torch.cuda.empty_cache()
    # every 7B workload, each timed like the headline (its own inputs)
    names = [] if args.workload else list(synth.SEVEN_B)
    others = {}
    cpu_inputs = {head_name: inp}
    for name in names:
        if name == head_name:
            others[name] = {k: v for k, v in rec.items()}
            continue
        r, c = measure_workload(name, args, headline=False)
        others[name] = r
        cpu_inputs[name] = c["inp"]
        del c
        torch.cuda.empty_cache()
    if others:
        out["workloads"] = others
    out["pages_context"] = PAGES_CONTEXT
    if not args.no_cpu_baseline:
        progress("CPU oracle baseline")
        import oracle as O  # noqa: F401  (CPU baseline leg only)
        c, a, _ = O.initial_state(inp)
        out["cpu_baseline"] = cpu_baseline(inp, c, a, args.cpu_seconds)
        # one bounded oracle step of every other workload
        for name, winp in cpu_inputs.items():
            if name == head_name or name not in others:
                continue
            c, a, _ = O.initial_state(winp)
            others[name]["cpu_baseline"] = cpu_baseline(winp, c, a, 0.0)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
