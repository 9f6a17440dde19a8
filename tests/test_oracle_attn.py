"""Pins for the oracle's branch attention (verify stage, attention part).

The articles fix that a branch attends to the original input and to its own
tokens but never to another branch's, and that all branches are verified in
one pass.  The oracle computes each branch alone; these tests check that
this equals one packed pass over all branches with an explicitly
materialised isolation mask (torch's scaled_dot_product_attention in
float64), plus closed forms (zero queries), the textbook single-block case
(scipy softmax) and GQA = MHA with repeated KV heads.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle as O


def _rand(rng, shape):
    return rng.standard_normal(shape).astype(np.float32)


def _inputs(rng, L, B, nb, Hq, Hkv, d):
    return (_rand(rng, (L, Hkv, d)), _rand(rng, (L, Hkv, d)),
            _rand(rng, (nb, B, Hq, d)), _rand(rng, (nb, B, Hkv, d)),
            _rand(rng, (nb, B, Hkv, d)))


def _packed_sdpa(Kp, Vp, Qb, Kb, Vb, Hq, Hkv):
    """All branches in ONE attention call over keys [prefix | block of branch
    0 | block of branch 1 | ...] with an explicit boolean mask: row (b, i)
    may see every prefix key and the keys of block b only."""
    L, _, d = Kp.shape
    nb, B = Qb.shape[:2]
    G = Hq // Hkv
    nk = L + nb * B
    mask = np.zeros((nb * B, nk), dtype=bool)
    mask[:, :L] = True
    for b in range(nb):
        mask[b * B:(b + 1) * B, L + b * B:L + (b + 1) * B] = True
    out = np.zeros((nb, B, Hq * d))
    for h in range(Hq):
        g = h // G
        q = torch.from_numpy(Qb[:, :, h, :].reshape(nb * B, d).astype(np.float64))
        k = torch.from_numpy(np.concatenate([Kp[:, g], Kb[:, :, g].reshape(nb * B, d)]).astype(np.float64))
        v = torch.from_numpy(np.concatenate([Vp[:, g], Vb[:, :, g].reshape(nb * B, d)]).astype(np.float64))
        o = torch.nn.functional.scaled_dot_product_attention(
            q[None], k[None], v[None], attn_mask=torch.from_numpy(mask)[None])
        out[:, :, h * d:(h + 1) * d] = o[0].numpy().reshape(nb, B, d)
    return out


@pytest.mark.parametrize("L,B,nb,Hq,Hkv,d", [
    (7, 5, 3, 4, 2, 8), (0, 4, 2, 2, 2, 4), (13, 1, 4, 6, 3, 16), (1, 3, 1, 1, 1, 2),
])
def test_oracle_attn_equals_packed_masked_pass(L, B, nb, Hq, Hkv, d):
    rng = np.random.default_rng(L * 100 + B)
    Kp, Vp, Qb, Kb, Vb = _inputs(rng, L, B, nb, Hq, Hkv, d)
    got = O.branch_attn(Kp, Vp, Qb, Kb, Vb, nb, Hq, Hkv)
    ref = _packed_sdpa(Kp, Vp, Qb, Kb, Vb, Hq, Hkv)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_oracle_attn_only_live_branches_written():
    rng = np.random.default_rng(3)
    Kp, Vp, Qb, Kb, Vb = _inputs(rng, 4, 3, 4, 2, 1, 4)
    H = O.branch_attn(Kp, Vp, Qb, Kb, Vb, 2, 2, 1)
    assert np.all(H[2:] == 0) and np.all(np.abs(H[:2]).sum(axis=-1) > 0)


def test_oracle_attn_isolation_by_perturbation():
    rng = np.random.default_rng(4)
    Kp, Vp, Qb, Kb, Vb = _inputs(rng, 6, 4, 3, 4, 2, 8)
    H = O.branch_attn(Kp, Vp, Qb, Kb, Vb, 3, 4, 2)
    Kb2, Vb2, Qb2 = Kb.copy(), Vb.copy(), Qb.copy()
    Kb2[1] += 3.0
    Vb2[1] -= 2.0
    Qb2[1] *= -1
    H2 = O.branch_attn(Kp, Vp, Qb2, Kb2, Vb2, 3, 4, 2)
    assert np.array_equal(H[0], H2[0]) and np.array_equal(H[2], H2[2])
    assert not np.allclose(H[1], H2[1])


def test_oracle_attn_zero_query_is_mean_of_visible_values():
    rng = np.random.default_rng(5)
    L, B, nb, Hq, Hkv, d = 5, 3, 2, 4, 2, 6
    Kp, Vp, Qb, Kb, Vb = _inputs(rng, L, B, nb, Hq, Hkv, d)
    Qb[:] = 0
    H = O.branch_attn(Kp, Vp, Qb, Kb, Vb, nb, Hq, Hkv)
    for b in range(nb):
        for h in range(Hq):
            g = h // 2
            mean = (Vp[:, g].astype(np.float64).sum(0) + Vb[b, :, g].astype(np.float64).sum(0)) / (L + B)
            for i in range(B):
                np.testing.assert_allclose(H[b, i, h * d:(h + 1) * d], mean, rtol=1e-13, atol=1e-14)


def test_oracle_attn_single_block_textbook():
    rng = np.random.default_rng(6)
    B, d = 7, 16
    Kp, Vp, Qb, Kb, Vb = _inputs(rng, 0, B, 1, 1, 1, d)
    H = O.branch_attn(Kp, Vp, Qb, Kb, Vb, 1, 1, 1)
    q, k, v = (x[0, :, 0].astype(np.float64) for x in (Qb, Kb, Vb))
    ref = scipy.special.softmax(q @ k.T / math.sqrt(d), axis=1) @ v
    np.testing.assert_allclose(H[0], ref, rtol=1e-12, atol=1e-13)


def test_oracle_attn_gqa_equals_mha_with_repeated_kv():
    rng = np.random.default_rng(7)
    L, B, nb, Hq, Hkv, d = 9, 4, 2, 6, 2, 8
    Kp, Vp, Qb, Kb, Vb = _inputs(rng, L, B, nb, Hq, Hkv, d)
    G = Hq // Hkv
    rep = lambda x: np.repeat(x, G, axis=-2)   # kv head g -> q heads g*G..g*G+G-1
    H_gqa = O.branch_attn(Kp, Vp, Qb, Kb, Vb, nb, Hq, Hkv)
    H_mha = O.branch_attn(rep(Kp), rep(Vp), Qb, rep(Kb), rep(Vb), nb, Hq, Hq)
    np.testing.assert_allclose(H_gqa, H_mha, rtol=1e-13, atol=1e-14)


def test_oracle_attn_reads_bf16_bits():
    rng = np.random.default_rng(8)
    Kp, Vp, Qb, Kb, Vb = _inputs(rng, 3, 2, 1, 2, 1, 4)
    bits = [torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
            for x in (Kp, Vp, Qb, Kb, Vb)]
    vals = [torch.from_numpy(x).to(torch.bfloat16).float().numpy() for x in (Kp, Vp, Qb, Kb, Vb)]
    np.testing.assert_array_equal(O.branch_attn(*bits, 1, 2, 1), O.branch_attn(*vals, 1, 2, 1))
