"""Pins of the layer-forward oracle (oracle/model_oracle.py), CPU only.

* The whole forward (mask-token embedding row, two layers over per-layer
  prefix caches, final RMSNorm), rounding points off, equals transformers'
  Qwen2Model in float64.
* The decoder layer, with the rounding points switched off, equals the
  transformers library's own Qwen2 decoder layer in float64 (an independent
  implementation) on the same weights, with the prefix keys/values in its
  cache and a mask that shows every key (full-sequence attention), to
  float32 precision (transformers keeps the norm statistics and the softmax
  in float32).
* The rotary angles equal transformers' Qwen2 rotary embedding (which works
  in float32, hence the tolerance); rotation keeps norms and makes q.k depend
  on the position difference only.
* RMSNorm equals transformers' Qwen2RMSNorm.
* The weight generator: every value exact in bf16, the C fast path equal to
  the numpy definition, the stated ranges and spreads, and rows drawn alone
  equal to rows drawn with the rest.
* Branch isolation through the whole model: changing one branch's tokens
  leaves every other branch's outputs bit for bit unchanged.
"""
import math

import numpy as np
import pytest
import torch

from oracle import lopa_oracle as O
from oracle import model_oracle as MO

transformers = pytest.importorskip("transformers")
from transformers.cache_utils import DynamicCache  # noqa: E402
from transformers.models.qwen2.modeling_qwen2 import (  # noqa: E402
    Qwen2Config, Qwen2DecoderLayer, Qwen2RMSNorm, Qwen2RotaryEmbedding)

CFG = MO.ModelCfg(n_layers=2, Hq=4, Hkv=2, d=64, inter=512, V=1000, mask_id=999)


def _hf_config(cfg, layers=1):
    c = Qwen2Config(hidden_size=cfg.hidden, intermediate_size=cfg.inter,
                    num_attention_heads=cfg.Hq, num_key_value_heads=cfg.Hkv,
                    rms_norm_eps=cfg.rms_eps, rope_theta=cfg.rope_theta,
                    num_hidden_layers=layers, vocab_size=cfg.V)
    c._attn_implementation = "eager"
    return c


@pytest.mark.parametrize("L", [0, 17])
def test_layer_equals_transformers_qwen2_layer(L):
    seed, B = 31, 12
    cfg = CFG
    w = MO.synth_layer(seed, cfg, 0)
    Kp, Vp = MO.synth_prefix(seed, cfg, 0, L)
    rng = np.random.default_rng(0)
    x = rng.standard_normal((1, B, cfg.hidden))
    got, k, v = MO.layer_forward(cfg, w, x, Kp, Vp, L, round_points=False)

    layer = Qwen2DecoderLayer(_hf_config(cfg), 0).double()
    qd, kd = cfg.Hq * cfg.d, cfg.Hkv * cfg.d
    wqkv, wgu = w.wqkv.full(), w.wgu.full()
    t = lambda a: torch.tensor(np.ascontiguousarray(a), dtype=torch.float64)  # noqa: E731
    with torch.no_grad():
        at = layer.self_attn
        at.q_proj.weight.copy_(t(wqkv[:qd]))
        at.q_proj.bias.copy_(t(w.bqkv[:qd]))
        at.k_proj.weight.copy_(t(wqkv[qd:qd + kd]))
        at.k_proj.bias.copy_(t(w.bqkv[qd:qd + kd]))
        at.v_proj.weight.copy_(t(wqkv[qd + kd:]))
        at.v_proj.bias.copy_(t(w.bqkv[qd + kd:]))
        at.o_proj.weight.copy_(t(w.wo.full()))
        layer.input_layernorm.weight.copy_(t(w.attn_norm))
        layer.post_attention_layernorm.weight.copy_(t(w.mlp_norm))
        layer.mlp.gate_proj.weight.copy_(t(wgu[:cfg.inter]))
        layer.mlp.up_proj.weight.copy_(t(wgu[cfg.inter:]))
        layer.mlp.down_proj.weight.copy_(t(w.wd.full()))
        cache = DynamicCache(config=_hf_config(cfg))
        if L:
            cache.update(t(Kp.transpose(1, 0, 2))[None], t(Vp.transpose(1, 0, 2))[None], 0)
        cos, sin = MO.rope_cos_sin(L + np.arange(B), cfg.d, cfg.rope_theta)
        pe = (t(np.concatenate([cos, cos], -1))[None], t(np.concatenate([sin, sin], -1))[None])
        mask = torch.zeros(1, 1, B, L + B, dtype=torch.float64)
        ref = layer(t(x), attention_mask=mask, position_embeddings=pe, past_key_values=cache,
                    use_cache=True)
    # transformers takes the norm's statistics and the softmax in float32 even
    # for a float64 model: agreement to float32 precision
    np.testing.assert_allclose(got[0], ref.numpy()[0], rtol=1e-5, atol=1e-5)
    keys = cache.layers[0].keys[0, :, L:, :].numpy().transpose(1, 0, 2)
    vals = cache.layers[0].values[0, :, L:, :].numpy().transpose(1, 0, 2)
    np.testing.assert_allclose(k[0], keys, rtol=1e-5, atol=1e-5)
    np.testing.assert_allclose(v[0], vals, rtol=1e-5, atol=1e-5)


class _FixedRope(torch.nn.Module):
    """Stands in for Qwen2Model's rotary module with the oracle's cos/sin (the
    angles are pinned separately: transformers evaluates them in float32)."""

    def __init__(self, cos, sin):
        super().__init__()
        self.cos, self.sin = cos, sin

    def forward(self, x, position_ids):
        return self.cos, self.sin


@pytest.mark.parametrize("L", [0, 23])
def test_forward_equals_transformers_qwen2_model(L):
    """The whole stack -- the mask token's own embedding row, two decoder
    layers over per-layer prefix caches, the final RMSNorm -- against
    transformers' Qwen2Model in float64 with the rounding points off."""
    seed, B = 41, 10
    cfg = CFG
    rng = np.random.default_rng(5)
    tok = rng.integers(0, cfg.V - 1, B)
    tok[[1, 4, 5, 8]] = O.MASK
    layers = [MO.synth_layer(seed, cfg, l) for l in range(cfg.n_layers)]
    prefix = [MO.synth_prefix(seed, cfg, l, L) for l in range(cfg.n_layers)]
    got = MO.forward(seed, cfg, L, tok[None], layers, prefix, round_points=False).H[0]

    from transformers.models.qwen2.modeling_qwen2 import Qwen2Model
    hc = _hf_config(cfg, cfg.n_layers)
    model = Qwen2Model(hc).double()
    qd, kd = cfg.Hq * cfg.d, cfg.Hkv * cfg.d
    t = lambda a: torch.tensor(np.ascontiguousarray(a), dtype=torch.float64)  # noqa: E731
    with torch.no_grad():
        model.embed_tokens.weight.copy_(t(MO.synth_rows(seed, cfg, MO.TENSOR_ID["embed"],
                                                        np.arange(cfg.V))))
        model.norm.weight.copy_(t(MO.synth_tensor(seed, 7, 0, 1, cfg.hidden, "norm")[0]))
        for l, w in enumerate(layers):
            layer = model.layers[l]
            at = layer.self_attn
            wqkv, wgu = w.wqkv.full(), w.wgu.full()
            at.q_proj.weight.copy_(t(wqkv[:qd]))
            at.q_proj.bias.copy_(t(w.bqkv[:qd]))
            at.k_proj.weight.copy_(t(wqkv[qd:qd + kd]))
            at.k_proj.bias.copy_(t(w.bqkv[qd:qd + kd]))
            at.v_proj.weight.copy_(t(wqkv[qd + kd:]))
            at.v_proj.bias.copy_(t(w.bqkv[qd + kd:]))
            at.o_proj.weight.copy_(t(w.wo.full()))
            layer.input_layernorm.weight.copy_(t(w.attn_norm))
            layer.post_attention_layernorm.weight.copy_(t(w.mlp_norm))
            layer.mlp.gate_proj.weight.copy_(t(wgu[:cfg.inter]))
            layer.mlp.up_proj.weight.copy_(t(wgu[cfg.inter:]))
            layer.mlp.down_proj.weight.copy_(t(w.wd.full()))
        cos, sin = MO.rope_cos_sin(L + np.arange(B), cfg.d, cfg.rope_theta)
        model.rotary_emb = _FixedRope(t(np.concatenate([cos, cos], -1))[None],
                                      t(np.concatenate([sin, sin], -1))[None])
        cache = DynamicCache(config=hc)
        for l in range(cfg.n_layers):
            if L:
                cache.update(t(prefix[l][0].transpose(1, 0, 2))[None],
                             t(prefix[l][1].transpose(1, 0, 2))[None], l)
        ids = torch.tensor(np.where(tok == O.MASK, cfg.mask_id, tok))[None]
        mask = torch.zeros(1, 1, B, L + B, dtype=torch.float64)   # every key visible
        ref = model(input_ids=ids, attention_mask={"full_attention": mask},
                    position_ids=torch.tensor(L + np.arange(B))[None], past_key_values=cache,
                    use_cache=True).last_hidden_state[0].numpy()
    # transformers keeps the norms' statistics and the softmax in float32
    np.testing.assert_allclose(got, ref, rtol=1e-5, atol=1e-5)
    # the masked positions took the mask token's row: with no prefix they only
    # differ through their position
    assert not np.allclose(got[1], got[4])


def test_rope_angles_match_transformers():
    cfg = MO.ModelCfg(n_layers=1, Hq=28, Hkv=4, d=128, inter=64, V=10, mask_id=9)
    pos = np.arange(500, 540)
    cos, sin = MO.rope_cos_sin(pos, cfg.d, cfg.rope_theta)
    rot = Qwen2RotaryEmbedding(_hf_config(cfg))
    c, s = rot(torch.zeros(1, len(pos), 8, dtype=torch.float32), torch.tensor(pos)[None])
    # transformers evaluates the angles in float32: agreement to its precision
    np.testing.assert_allclose(cos, c[0, :, :64].double().numpy(), atol=2e-4)
    np.testing.assert_allclose(sin, s[0, :, :64].double().numpy(), atol=2e-4)


def test_rope_rotation_properties():
    rng = np.random.default_rng(1)
    d = 64
    q = rng.standard_normal((1, 1, d))
    k = rng.standard_normal((1, 1, d))
    dots = []
    for p in (3, 10, 40):
        cq, sq = MO.rope_cos_sin(np.array([p + 5]), d, 1e4)
        ck, sk = MO.rope_cos_sin(np.array([p]), d, 1e4)
        qr, kr = MO.rope(q, cq, sq), MO.rope(k, ck, sk)
        assert np.linalg.norm(qr) == pytest.approx(np.linalg.norm(q), rel=1e-6)
        dots.append(float(np.sum(qr * kr)))
    # the score depends on the offset (5) only
    assert dots[0] == pytest.approx(dots[1], rel=1e-5) and dots[1] == pytest.approx(dots[2], rel=1e-5)
    c0, s0 = MO.rope_cos_sin(np.array([0]), d, 1e6)
    assert np.array_equal(MO.rope(q, c0, s0), q)      # position 0: identity


def test_rmsnorm_matches_transformers():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((5, 96)) * 3
    g = 1 + rng.standard_normal(96) * 0.1
    n = Qwen2RMSNorm(96, eps=1e-6).double()
    with torch.no_grad():
        n.weight.copy_(torch.tensor(g))
        ref = n(torch.tensor(x)).numpy()
    # transformers' statistics are float32
    np.testing.assert_allclose(MO.rmsnorm(x, g, 1e-6), ref, rtol=1e-6)


@pytest.mark.parametrize("rule,shift", [("uniform", 4), ("uniform", -1), ("uniform", 2),
                                        ("norm", 0)])
def test_generator_values(rule, shift):
    a = MO.synth_tensor(77, 5, 3, 130, 258, rule, shift, use_c=False)
    b = MO.synth_tensor(77, 5, 3, 130, 258, rule, shift, use_c=True)
    assert np.array_equal(a, b)                                  # C fast path == definition
    assert np.array_equal(MO.rnd(a), a)                          # exact in bf16
    if rule == "norm":
        assert a.min() >= 0.875 and a.max() <= 1 + 15 / 128
        assert len(np.unique(a)) == 32
    else:
        half = 2.0 ** (-1 - shift)
        assert np.abs(a).max() <= half
        assert a.std() == pytest.approx(2.0 * half / math.sqrt(12), rel=0.03)
    # a block of rows drawn alone equals the same rows drawn with the rest
    part = MO._synth_rows_np(77, 5, 3, 40, 57, 258, rule, shift)
    assert np.array_equal(part, a[40:57])


def test_generator_rows_and_projection():
    cfg = CFG
    E = MO.synth_tensor(9, 8, 0, 50, cfg.hidden, "uniform", 1)
    assert np.array_equal(MO.synth_rows(9, cfg, 8, [0, 7, 49]), E[[0, 7, 49]])
    p = MO.Proj(9, 5, 1, 2100, cfg.hidden, 2)
    W = MO.synth_tensor(9, 5, 1, 2100, cfg.hidden, "uniform", 2)
    assert np.array_equal(p.full(), W)
    x = np.random.default_rng(3).standard_normal((3, cfg.hidden))
    np.testing.assert_allclose(p(x), x @ W.T, rtol=1e-12)
    assert MO.fan_in_shift(3584) == 4 and MO.fan_in_shift(18944) == 5 and MO.fan_in_shift(256) == 2


def test_branch_isolation_through_the_model():
    seed, L = 5, 30
    rng = np.random.default_rng(4)
    tok = rng.integers(0, CFG.V, (3, 10))
    tok[:, 2:6] = O.MASK
    a = MO.forward(seed, CFG, L, tok)
    tok2 = tok.copy()
    tok2[1] = rng.integers(0, CFG.V, 10)
    b = MO.forward(seed, CFG, L, tok2)
    for i in (0, 2):
        assert np.array_equal(a.H[i], b.H[i]) and np.array_equal(a.Kb[:, i], b.Kb[:, i])
    assert not np.array_equal(a.H[1], b.H[1])
    # each branch alone gives the same rows
    alone = MO.forward(seed, CFG, L, tok[2:3])
    assert np.array_equal(alone.H[0], a.H[2])


def test_rounding_points_are_bf16():
    out = MO.forward(5, CFG, 20, np.full((2, 8), O.MASK))
    for arr in (out.H, out.Kb, out.Vb):
        assert np.array_equal(MO.rnd(arr), arr)
    # the mask token's embedding feeds every masked position: identical rows
    assert np.array_equal(out.H[0], out.H[1])
