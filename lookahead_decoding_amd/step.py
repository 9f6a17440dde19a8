"""Device buffers for one verification step and the four-call sequence.

Plumbing only: torch allocates device memory; the step itself is the four
library calls enqueued back to back on one stream with no host sync.
"""
from __future__ import annotations

import numpy as np

from . import (BF16, F32, Dims, lopa_block_rows, lopa_branch_attn,
               lopa_branch_build, lopa_branch_select, lopa_lmhead_conf, workspace_bytes)


def dims_of(cfg) -> Dims:
    """Dims from any object with L, B, Hq, Hkv, d, V, k and dtype ('f32'/'bf16')."""
    return Dims(L=cfg.L, B=cfg.B, Hq=cfg.Hq, Hkv=cfg.Hkv, d=cfg.d, V=cfg.V, k_max=cfg.k,
                dtype=F32 if cfg.dtype == "f32" else BF16)


def to_device(a: np.ndarray, device="cuda"):
    """numpy array -> torch device tensor; uint16 arrays are bf16 bit patterns."""
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


class StepBuffers:
    """Every device array one step reads or writes, sized for nb_max branches."""

    def __init__(self, dims: Dims, device="cuda"):
        import torch
        B, nbm = dims.B, dims.nb_max
        act = torch.float32 if dims.dtype == F32 else torch.bfloat16
        i32 = torch.int32
        z = lambda *s, dt=i32: torch.zeros(*s, dtype=dt, device=device)  # noqa: E731
        self.dims = dims
        self.nb = z(1)
        self.br_tok = z(nbm * B)
        self.br_mask = z(nbm * B, dt=torch.uint8)
        self.rows = z(nbm * B)
        self.row_ptr = z(nbm + 1)
        self.H = z(nbm, B, dims.hidden, dt=act)
        self.conf = z(nbm * B, dt=torch.float32)
        self.arg = z(nbm * B)
        self.ent = z(nbm * B, dt=torch.float32)
        self.ws = z(max(workspace_bytes(dims), 16), dt=torch.uint8)
        self.bconf = z(nbm, dt=torch.float32)
        self.winner = z(1)
        self.tok_next = z(B)
        self.conf_next = z(B, dt=torch.float32)
        self.arg_next = z(B)


def run_step(dims: Dims, k: int, tau: float, x: dict, buf: StepBuffers, stream=None,
             logits_out=None) -> None:
    """Enqueue build -> attention -> LM head -> select.  ``x`` holds device
    tensors tok, conf, arg (step-start state) and Kp, Vp, Qb, Kb, Vb, W."""
    lopa_branch_build(dims, k, tau, x["tok"], x["conf"], x["arg"], buf.nb, buf.br_tok,
                      buf.br_mask, buf.rows, buf.row_ptr, stream)
    lopa_branch_attn(dims, x["Kp"], x["Vp"], x["Qb"], x["Kb"], x["Vb"], buf.nb, buf.H, buf.ws, stream)
    lopa_lmhead_conf(dims, buf.H, x["W"], buf.rows, buf.row_ptr, buf.nb, buf.conf, buf.arg,
                     logits_out, buf.ws, stream)
    lopa_branch_select(dims, buf.nb, buf.br_mask, buf.br_tok, buf.conf, buf.arg, buf.bconf,
                       buf.winner, buf.tok_next, buf.conf_next, buf.arg_next, stream)


def initial_pass(dims: Dims, tok: np.ndarray, x: dict, buf: StepBuffers, stream=None):
    """State a step starts from, computed on the GPU: branch slot 0 alone,
    LM head on the block's masked positions.  Returns device tensors
    (conf [B] float32, 0 where filled; arg [B] int32, -1 where filled)."""
    import torch
    dev = buf.H.device
    B = dims.B
    tok_d = to_device(np.asarray(tok, np.int32), dev)
    nb1 = torch.empty(1, dtype=torch.int32, device=dev)
    rows = torch.empty(dims.nb_max * B, dtype=torch.int32, device=dev)
    row_ptr = torch.empty(dims.nb_max + 1, dtype=torch.int32, device=dev)
    conf = torch.empty(dims.nb_max * B, dtype=torch.float32, device=dev)
    arg = torch.empty(dims.nb_max * B, dtype=torch.int32, device=dev)
    lopa_block_rows(dims, tok_d, nb1, rows, row_ptr, conf, arg, stream)
    lopa_branch_attn(dims, x["Kp"], x["Vp"], x["Qb"], x["Kb"], x["Vb"], nb1, buf.H, buf.ws, stream)
    lopa_lmhead_conf(dims, buf.H, x["W"], rows, row_ptr, nb1, conf, arg, None, buf.ws, stream)
    return conf[:B].clone(), arg[:B].clone()
