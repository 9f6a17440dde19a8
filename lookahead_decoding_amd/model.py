"""Device buffers of the model forward and the verification step that runs
it (plumbing only: torch allocates, the library computes).

A step with the model is build -> lopa_branch_forward -> lopa_lmhead_conf
(the model's LM head weight) -> lopa_branch_select, enqueued on one stream
with no host synchronisation.  The forward writes every layer's block K/V of
every branch slot; lopa_model_commit appends the winner's slot to the prefix
once a block is decoded.
"""
from __future__ import annotations

from . import (ModelDims, lopa_branch_build, lopa_branch_forward, lopa_branch_select,
               lopa_lmhead_conf, lopa_model_synth, model_layout, model_workspace_bytes)

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
        n = math.prod(shape) * 2
        return self.weights[offset:offset + n].view(__import__("torch").bfloat16).view(*shape)

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
