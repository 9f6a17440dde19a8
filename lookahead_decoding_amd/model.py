"""Device buffers of the model forward and the verification step that runs
it (plumbing only: torch allocates, the library computes).

A step with the model is build -> lopa_branch_forward -> lopa_lmhead_conf
(the model's LM head weight) -> lopa_branch_select, enqueued on one stream
with no host synchronisation.  The forward writes every layer's block K/V of
every branch slot; lopa_model_commit appends the winner's slot to the prefix
once a block is decoded.
"""
from __future__ import annotations

from . import (ModelDims, lopa_block_rows, lopa_branch_build, lopa_branch_forward,
               lopa_branch_select, lopa_lmhead_conf, lopa_model_synth, model_layout,
               model_workspace_bytes)

# A block decoded with the model repeats the step above from the initial
# pass's state until no position is masked (model_decode_block), and
# model_decode_sequence commits each decoded block's winner K/V of every
# layer so the next block attends to it.

# Qwen2.5-7B / Dream-7B geometry (hidden 3584 = 28 x 128)
QWEN7B = dict(n_layers=28, inter=18944, mask_id=151666, rope_theta=1e6, rms_eps=1e-6)


def model_dims(n_layers: int, inter: int, mask_id: int, rope_theta: float = 1e6,
               rms_eps: float = 1e-6) -> ModelDims:
    return ModelDims(n_layers=n_layers, inter=inter, mask_id=mask_id, rope_theta=rope_theta,
                     rms_eps=rms_eps)


class Model:
    """Synthetic weights (lopa_model_synth) and the per-layer prefix cache
    [n_layers][kv_rows][Hkv][d], on the device."""

    def __init__(self, dims, md: ModelDims, seed: int, kv_rows: int | None = None,
                 device="cuda"):
        import torch
        self.dims, self.md, self.seed = dims, md, seed
        self.kv_rows = dims.L if kv_rows is None else kv_rows
        self.layout = model_layout(dims, md)
        self.weights = torch.empty(self.layout.total, dtype=torch.uint8, device=device)
        shape = (md.n_layers, max(self.kv_rows, 1), dims.Hkv, dims.d)
        self.Kp = torch.zeros(shape, dtype=torch.bfloat16, device=device)
        self.Vp = torch.zeros_like(self.Kp)
        lopa_model_synth(dims, md, seed, self.weights, self.Kp, self.Vp, self.kv_rows)

    def tensor(self, offset: int, *shape):
        """bf16 view of the weight buffer at a byte offset."""
        import math
        import torch
        n = math.prod(shape) * 2
        return self.weights[offset:offset + n].view(torch.bfloat16).view(*shape)

    @property
    def lm_head(self):
        return self.tensor(self.layout.lm_head, self.dims.V, self.dims.hidden)


class ForwardBuffers:
    """Outputs and workspace of lopa_branch_forward."""

    def __init__(self, dims, md: ModelDims, device="cuda"):
        import torch
        bf = torch.bfloat16
        nbm, B = dims.nb_max, dims.B
        self.Kb = torch.zeros(md.n_layers, nbm, B, dims.Hkv, dims.d, dtype=bf, device=device)
        self.Vb = torch.zeros_like(self.Kb)
        self.H = torch.zeros(nbm, B, dims.hidden, dtype=bf, device=device)
        self.ws = torch.zeros(model_workspace_bytes(dims, md), dtype=torch.uint8, device=device)


def forward(model: Model, br_tok, nb, fb: ForwardBuffers, stream=None, dims=None) -> None:
    """``dims`` may differ from the model's in k_max (the weight layout does
    not depend on it); ``fb`` must be sized for the dims used."""
    lopa_branch_forward(model.dims if dims is None else dims, model.md, model.weights, model.Kp,
                        model.Vp, model.kv_rows, br_tok, nb, fb.Kb, fb.Vb, fb.H, fb.ws, stream)


def model_step(model: Model, k: int, tau: float, tok, conf, arg, buf, fb: ForwardBuffers,
               stream=None) -> None:
    """One verification step with the model: explore from the state (tok,
    conf, arg device tensors), run every branch through the model, score the
    still-masked rows with the model's LM head, select."""
    dims = model.dims
    lopa_branch_build(dims, k, tau, tok, conf, arg, buf.nb, buf.br_tok, buf.br_mask, buf.rows,
                      buf.row_ptr, stream)
    forward(model, buf.br_tok, buf.nb, fb, stream)
    lopa_lmhead_conf(dims, fb.H, model.lm_head, buf.rows, buf.row_ptr, buf.nb, buf.conf, buf.arg,
                     None, buf.ws, stream)
    lopa_branch_select(dims, buf.nb, buf.br_mask, buf.br_tok, buf.conf, buf.arg, buf.bconf,
                       buf.winner, buf.tok_next, buf.conf_next, buf.arg_next, stream)


class ModelDecodeBuffers:
    """State and per-step buffers of block decoding with the model."""

    def __init__(self, dims, md: ModelDims, device="cuda"):
        import torch
        from .step import StepBuffers
        self.step = StepBuffers(dims, device)
        self.fwd = ForwardBuffers(dims, md, device)
        B, nbm = dims.B, dims.nb_max
        i32 = torch.int32
        self.one = torch.ones(1, dtype=i32, device=device)
        self.tok = torch.zeros(B, dtype=i32, device=device)
        self.conf = torch.zeros(B, dtype=torch.float32, device=device)
        self.arg = torch.zeros(B, dtype=i32, device=device)
        self.tok0 = torch.zeros(nbm * B, dtype=i32, device=device)
        self.rows0 = torch.zeros(nbm * B, dtype=i32, device=device)
        self.row_ptr0 = torch.zeros(nbm + 1, dtype=i32, device=device)

    def swap_state(self):
        s = self.step
        self.tok, s.tok_next = s.tok_next, self.tok
        self.conf, s.conf_next = s.conf_next, self.conf
        self.arg, s.arg_next = s.arg_next, self.arg


def model_decode_block(model: Model, dims, k: int, tau: float, tok0, buf: ModelDecodeBuffers,
                       steps: int, log=None, stream=None, state_log=None) -> None:
    """Decode one block with the model: the initial pass (the block as it
    stands in slot 0, the LM head on its masked positions), then ``steps``
    verification steps, each build -> forward -> LM head -> select with the
    winner's state swapped in.  ``dims`` carries the current prefix length
    (dims.L rows of the model's cache are the committed prefix).  ``log``
    (device int32 [steps][B]) receives the tokens after each step;
    ``state_log`` (device float32 and int32 tensors [steps + 1][B]) the
    confidences and tokens of the state: row 0 after the initial pass, row
    s + 1 after step s."""
    import numpy as np
    import torch
    tok0 = np.asarray(tok0, np.int32)
    dev = buf.tok.device
    B, nbm = dims.B, dims.nb_max
    s = buf.step
    buf.tok.copy_(torch.from_numpy(tok0).to(dev))
    buf.tok0.view(nbm, B).copy_(buf.tok.expand(nbm, B))
    # rows of the masked positions, the LM head's outputs cleared (on the device)
    lopa_block_rows(dims, buf.tok, buf.one, buf.rows0, buf.row_ptr0, s.conf, s.arg, stream)
    forward(model, buf.tok0, buf.one, buf.fwd, stream, dims=dims)
    lopa_lmhead_conf(dims, buf.fwd.H, model.lm_head, buf.rows0, buf.row_ptr0, buf.one, s.conf,
                     s.arg, None, s.ws, stream)
    buf.conf.copy_(s.conf[:B])
    buf.arg.copy_(s.arg[:B])
    if state_log is not None:
        state_log[0][0].copy_(buf.conf)
        state_log[1][0].copy_(buf.arg)
    for i in range(steps):
        lopa_branch_build(dims, k, tau, buf.tok, buf.conf, buf.arg, s.nb, s.br_tok, s.br_mask,
                          s.rows, s.row_ptr, stream)
        forward(model, s.br_tok, s.nb, buf.fwd, stream, dims=dims)
        lopa_lmhead_conf(dims, buf.fwd.H, model.lm_head, s.rows, s.row_ptr, s.nb, s.conf, s.arg,
                         None, s.ws, stream)
        lopa_branch_select(dims, s.nb, s.br_mask, s.br_tok, s.conf, s.arg, s.bconf, s.winner,
                           s.tok_next, s.conf_next, s.arg_next, stream)
        buf.swap_state()
        if log is not None:
            log[i].copy_(buf.tok)
        if state_log is not None:
            state_log[0][i + 1].copy_(buf.conf)
            state_log[1][i + 1].copy_(buf.arg)


def model_decode_sequence(model: Model, k: int, tau: float, blocks, buf: ModelDecodeBuffers,
                          logs=None, stream=None, state_logs=None) -> int:
    """Decode ``blocks`` one after another with the model, committing each
    decoded block's winner K/V of every layer (lopa_model_commit) at the end
    of the prefix, so the next block attends to it.  The model's cache must
    have room for the prefix plus len(blocks) * B rows.  ``logs`` /
    ``state_logs`` hold one model_decode_block log / state_log per block.
    Returns the final prefix length."""
    import numpy as np
    from . import MASK, Dims, lopa_model_commit
    import torch
    d0 = model.dims
    L = d0.L
    zero = torch.zeros(1, dtype=torch.int32, device=buf.tok.device)
    for j, tok0 in enumerate(blocks):
        dj = Dims(L=L, B=d0.B, Hq=d0.Hq, Hkv=d0.Hkv, d=d0.d, V=d0.V, k_max=d0.k_max,
                  dtype=d0.dtype)
        m = int(np.sum(np.asarray(tok0) == MASK))
        model_decode_block(model, dj, k, tau, tok0, buf, m, None if logs is None else logs[j],
                           stream, None if state_logs is None else state_logs[j])
        # with no step taken, slot 0 holds the block (written by the initial pass)
        lopa_model_commit(dj, model.md, buf.step.winner if m else zero, buf.fwd.Kb, buf.fwd.Vb,
                          model.Kp, model.Vp, model.kv_rows, L, stream)
        L += d0.B
    return L
