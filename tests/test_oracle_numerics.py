"""Pins for the oracle's number-format helpers (bf16 decode and rounding).

The oracle rounds the attention output H to bf16 once, straight from
float64.  These tests pin that rounding to torch's float32->bf16 conversion
on values where the two must agree (every float32 value), and to closed-form
cases where rounding through float32 first would give a different answer.
"""
import numpy as np
import pytest
import torch

import oracle as O


def _torch_bits(x32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(x32).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_oracle_bf16_decode_matches_torch():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 16, size=20000, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    got = O.bf16_to_f64(bits)
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.isnan(got), np.isnan(ref))


def test_oracle_bf16_round_matches_torch_on_float32_values():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(20000),
        rng.standard_normal(2000) * 1e-39,          # subnormal range
        rng.standard_normal(2000) * 1e37,
        np.ldexp(rng.integers(1, 1 << 9, 4000) * 2 + 1, rng.integers(-20, 20, 4000)),
    ]).astype(np.float32)
    # exact halfway points between adjacent bf16 values
    base = rng.integers(0, 0x7F00, size=4000, dtype=np.uint32)
    half = ((base << 16) | 0x8000).view(np.float32)
    x = np.concatenate([x, half, -half])
    got = O.f64_to_bf16(x.astype(np.float64))
    assert np.array_equal(got, _torch_bits(x))


@pytest.mark.parametrize("x,bits", [
    (1 + 2.0**-8 + 2.0**-30, 0x3F81),  # just above a tie: up (via fp32: tie -> 0x3F80)
    (1 + 2.0**-8, 0x3F80),             # tie -> even
    (1 + 3 * 2.0**-8, 0x3F82),         # tie -> even (up)
    (-(1 + 2.0**-8 + 2.0**-40), 0xBF81),
    (3.4e38, 0x7F80),                  # past the halfway point above the largest finite
    (3.3e38, 0x7F78),
    (2.0**-133, 0x0001),               # smallest subnormal
    (2.0**-134, 0x0000),               # tie -> even (zero)
    (3 * 2.0**-135, 0x0001),
    (0.0, 0x0000),
])
def test_oracle_bf16_round_single_step(x, bits):
    assert int(O.f64_to_bf16(np.array([x]))[0]) == bits


def test_oracle_round_like_f32_is_rne():
    x = np.array([1 + 2.0**-24, 1 + 3 * 2.0**-24, 1 + 2.0**-24 + 2.0**-50])
    got = O.round_like(x, np.float32)
    assert list(got) == [1.0, 1 + 2.0**-22, 1 + 2.0**-23]
