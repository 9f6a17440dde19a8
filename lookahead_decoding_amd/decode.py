"""Decoding one block over several LoPA steps on the device (plumbing only).

The news article "上交大 × 华为小艺推出LoPA：7B扩散语言模型单样例1000+ tokens/s！"
(section "LoPA 的核心设计：前瞻并行与分支验证") repeats explore, verify and
select, reusing the winner's verification outputs, until the block is
decoded.  This module only sequences library calls on one stream: an initial
pass of the block as it stands, then per step lopa_branch_build ->
lopa_synth_qkv (the token-keyed stand-in for the model's projections of every
branch) -> lopa_branch_attn -> lopa_lmhead_conf -> lopa_branch_select, with the
state (tokens, confidence, argmax) ping-ponged between two device buffers and
never read back by the host.  A step taken after the block is complete
changes nothing (no position is masked, so nothing is filled).

With ``alpha`` given, the LM head also returns each row's normalised entropy
(lopa_lmhead_conf_ent) and the winner is chosen by the alternative branch
score of "解码效率革命：LoPA如何突破扩散语言模型的并行瓶颈", section 3.2
(lopa_branch_select_alpha).
"""
from __future__ import annotations

import numpy as np

from . import (MASK, lopa_block_rows, lopa_branch_attn, lopa_branch_build,
               lopa_branch_build_floor, lopa_branch_select, lopa_branch_select_alpha,
               lopa_lmhead_conf, lopa_lmhead_conf_ent, lopa_lmhead_sample, lopa_synth_qkv)
from .step import StepBuffers


class DecodeBuffers(StepBuffers):
    """StepBuffers plus the per-branch projections and a second state."""

    def __init__(self, dims, device="cuda"):
        import torch
        super().__init__(dims, device)
        act = torch.float32 if dims.dtype == 0 else torch.bfloat16
        nbm, B = dims.nb_max, dims.B
        self.Qb = torch.zeros(nbm, B, dims.Hq, dims.d, dtype=act, device=device)
        self.Kb = torch.zeros(nbm, B, dims.Hkv, dims.d, dtype=act, device=device)
        self.Vb = torch.zeros_like(self.Kb)
        self.one = torch.ones(1, dtype=torch.int32, device=device)
        # state a step reads: tokens [B], confidence [B], argmax [B]
        self.tok = torch.zeros(B, dtype=torch.int32, device=device)
        self.conf_s = torch.zeros(B, dtype=torch.float32, device=device)
        self.arg_s = torch.zeros(B, dtype=torch.int32, device=device)
        self.rows0 = torch.zeros(nbm * B, dtype=torch.int32, device=device)
        self.row_ptr0 = torch.zeros(nbm + 1, dtype=torch.int32, device=device)

    def swap_state(self):
        self.tok, self.tok_next = self.tok_next, self.tok
        self.conf_s, self.conf_next = self.conf_next, self.conf_s
        self.arg_s, self.arg_next = self.arg_next, self.arg_s


def start_block(dims, seed, tok0, Kp, Vp, W, buf: DecodeBuffers, stream=None,
                temperature=None, sample_seed=0) -> None:
    """Load the block ``tok0`` (host int32 [B], MASK where masked) and run the
    initial pass: slot 0's projections, attention, and the LM head on every
    masked position, which gives the state the first step starts from."""
    import torch
    tok0 = np.asarray(tok0, np.int32)
    dev = buf.tok.device
    B = dims.B
    buf.tok.copy_(torch.from_numpy(tok0).to(dev))
    # rows of the masked positions, the LM head's outputs cleared (on the device)
    lopa_block_rows(dims, buf.tok, buf.one, buf.rows0, buf.row_ptr0, buf.conf, buf.arg, stream)
    lopa_synth_qkv(dims, seed, buf.tok, buf.one, buf.Qb, buf.Kb, buf.Vb, stream)
    lopa_branch_attn(dims, Kp, Vp, buf.Qb, buf.Kb, buf.Vb, buf.one, buf.H, buf.ws, stream)
    if temperature is None:
        lopa_lmhead_conf(dims, buf.H, W, buf.rows0, buf.row_ptr0, buf.one, buf.conf, buf.arg,
                         None, buf.ws, stream)
    else:
        lopa_lmhead_sample(dims, temperature, sample_seed, buf.H, W, buf.rows0, buf.row_ptr0,
                           buf.one, buf.conf, buf.arg, None, buf.ws, stream)
    buf.conf_s.copy_(buf.conf[:B])
    buf.arg_s.copy_(buf.arg[:B])


def decode_step(dims, k, tau, seed, Kp, Vp, W, buf: DecodeBuffers, stream=None,
                alpha=None, gamma=None, temperature=None, sample_seed=0) -> None:
    """One explore / verify / select step on the current state, then swap in
    the winner's state.  ``gamma``: lookahead candidates need confidence >=
    gamma (lopa_branch_build_floor)."""
    if gamma is None:
        lopa_branch_build(dims, k, tau, buf.tok, buf.conf_s, buf.arg_s, buf.nb, buf.br_tok,
                          buf.br_mask, buf.rows, buf.row_ptr, stream)
    else:
        lopa_branch_build_floor(dims, k, tau, gamma, buf.tok, buf.conf_s, buf.arg_s, buf.nb,
                                buf.br_tok, buf.br_mask, buf.rows, buf.row_ptr, stream)
    lopa_synth_qkv(dims, seed, buf.br_tok, buf.nb, buf.Qb, buf.Kb, buf.Vb, stream)
    lopa_branch_attn(dims, Kp, Vp, buf.Qb, buf.Kb, buf.Vb, buf.nb, buf.H, buf.ws, stream)
    if temperature is not None:
        lopa_lmhead_sample(dims, temperature, sample_seed, buf.H, W, buf.rows, buf.row_ptr,
                           buf.nb, buf.conf, buf.arg, None, buf.ws, stream)
        lopa_branch_select(dims, buf.nb, buf.br_mask, buf.br_tok, buf.conf, buf.arg, buf.bconf,
                           buf.winner, buf.tok_next, buf.conf_next, buf.arg_next, stream)
    elif alpha is None:
        lopa_lmhead_conf(dims, buf.H, W, buf.rows, buf.row_ptr, buf.nb, buf.conf, buf.arg, None,
                         buf.ws, stream)
        lopa_branch_select(dims, buf.nb, buf.br_mask, buf.br_tok, buf.conf, buf.arg, buf.bconf,
                           buf.winner, buf.tok_next, buf.conf_next, buf.arg_next, stream)
    else:
        lopa_lmhead_conf_ent(dims, buf.H, W, buf.rows, buf.row_ptr, buf.nb, buf.conf, buf.arg,
                             buf.ent, None, buf.ws, stream)
        lopa_branch_select_alpha(dims, alpha, buf.tok, buf.conf_s, buf.nb, buf.br_mask,
                                 buf.br_tok, buf.conf, buf.arg, buf.ent, buf.bconf, buf.winner,
                                 buf.tok_next, buf.conf_next, buf.arg_next, stream)
    buf.swap_state()


def decode_block(dims, k, tau, seed, tok0, Kp, Vp, W, buf: DecodeBuffers, steps: int,
                 log=None, stream=None, alpha=None, gamma=None, temperature=None,
                 sample_seed=0) -> None:
    """The initial pass and ``steps`` steps; ``log`` (device int32
    [steps][B]) receives the tokens after each step.  With ``temperature``
    pass s draws its tokens with seed sample_seed + s (0: the initial pass)."""
    start_block(dims, seed, tok0, Kp, Vp, W, buf, stream, temperature, sample_seed)
    for s in range(steps):
        decode_step(dims, k, tau, seed, Kp, Vp, W, buf, stream, alpha, gamma, temperature,
                    sample_seed + s + 1)
        if log is not None:
            log[s].copy_(buf.tok)


def decode_sequence(dims, k, tau, seed, blocks, Kp, Vp, W, buf: DecodeBuffers,
                    logs=None, stream=None) -> int:
    """Decode ``blocks`` (host int32 [B] arrays) one after another.  Kp and Vp
    hold the committed prefix in their first dims.L rows and have room for
    len(blocks) * B more; after block j is decoded (as many steps as it has
    masked positions -- later steps change nothing) the winner's K and V slot
    is appended at row L + j*B by lopa_commit_block, and block j+1 attends to
    it.  ``buf`` must be sized for the longest prefix.  ``logs[j]`` (device
    int32 [m_j][B]) receives block j's tokens after each step.  Returns the
    final prefix length."""
    from . import Dims, lopa_commit_block
    import torch
    L = dims.L
    zero = torch.zeros(1, dtype=torch.int32, device=buf.tok.device)
    for j, tok0 in enumerate(blocks):
        dj = Dims(L=L, B=dims.B, Hq=dims.Hq, Hkv=dims.Hkv, d=dims.d, V=dims.V, k_max=dims.k_max,
                  dtype=dims.dtype)
        m = int(np.sum(np.asarray(tok0) == MASK))
        decode_block(dj, k, tau, seed, tok0, Kp, Vp, W, buf, m,
                     None if logs is None else logs[j], stream)
        # with no step taken, slot 0 holds the block (written by the initial pass)
        lopa_commit_block(dj, buf.winner if m else zero, buf.Kb, buf.Vb, Kp, Vp, L, stream)
        L += dims.B
    return L
