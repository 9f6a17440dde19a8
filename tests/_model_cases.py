"""Model geometries and seeded tokens shared by the GPU model tests and the
script that derives their tolerances (tests/golden/make_forward_noise.py).
numpy only: no torch, no library import."""
from __future__ import annotations

import numpy as np

MASK = -1

# name, geometry, live branches
FWD_CASES = [
    ("small-d64-M64", dict(L=40, B=16, k_max=3, Hq=4, Hkv=2, d=64, inter=512, V=1000,
                           n_layers=2), 4),
    ("mfma-attn-M160", dict(L=100, B=32, k_max=4, Hq=8, Hkv=2, d=128, inter=2048, V=3000,
                            n_layers=2), 5),
    ("dead-slots-M128", dict(L=70, B=32, k_max=3, Hq=8, Hkv=2, d=128, inter=1536, V=2000,
                             n_layers=3), 2),
    ("two-row-groups-M288", dict(L=64, B=32, k_max=8, Hq=4, Hkv=1, d=128, inter=1024, V=1500,
                                 n_layers=2), 9),
    ("no-prefix", dict(L=0, B=16, k_max=1, Hq=4, Hkv=4, d=64, inter=256, V=500, n_layers=2), 2),
    # 144 rows: the 160-row projection tile with 16 padding rows
    ("tile160-M144", dict(L=50, B=48, k_max=2, Hq=4, Hkv=2, d=64, inter=512, V=800,
                          n_layers=2), 3),
    # gate/up with its SwiGLU in one kernel: the 7B model's 18944-wide MLP
    # gives four and five weight tiles per workgroup, 10240 two and three
    ("glu-tiles4-5-M160", dict(L=32, B=32, k_max=4, Hq=4, Hkv=2, d=64, inter=18944, V=600,
                               n_layers=1), 5),
    ("glu-tiles2-3-M72", dict(L=20, B=24, k_max=2, Hq=2, Hkv=1, d=64, inter=10240, V=300,
                              n_layers=1), 3),
    # the 2-D wave blocks with padding rows (150 of 160 staged), and four
    # activation tiles against four or five weight tiles (one wave per tile)
    ("glu-blocks-M150", dict(L=24, B=30, k_max=4, Hq=4, Hkv=2, d=64, inter=18944, V=400,
                             n_layers=1), 4),
    ("glu-tiles4-5-M128", dict(L=16, B=32, k_max=3, Hq=8, Hkv=2, d=64, inter=18944, V=350,
                               n_layers=1), 4),
    # the 7B model's depth at a small width: errors compounding over 28 layers
    ("deep-28-layers", dict(L=40, B=16, k_max=3, Hq=4, Hkv=2, d=64, inter=512, V=1000,
                            n_layers=28), 4),
]

STEP_CASE = dict(L=64, B=32, k_max=4, Hq=8, Hkv=2, d=128, inter=2048, V=3000, n_layers=2)
STEP_SEED = 4242

SEVEN_B = dict(L=512, B=32, k_max=4, Hq=28, Hkv=4, d=128, inter=18944, V=152064)
SEVEN_B_SEED = 2026

# block decoding: name, geometry (L, B, k, Hq, Hkv, d, inter, V, layers), masked, seed
DECODE_CASES = [
    ("small-1", (40, 16, 3, 4, 2, 64, 512, 1000, 2), 10, 1),
    ("small-4", (40, 16, 3, 4, 2, 64, 512, 1000, 2), 10, 4),
    ("small-5", (40, 16, 3, 4, 2, 64, 512, 1000, 2), 10, 5),
    ("mfma-1", (64, 32, 4, 8, 2, 128, 1024, 2000, 2), 16, 1),
    ("mfma-2", (64, 32, 4, 8, 2, 128, 1024, 2000, 2), 16, 2),
]


def fwd_seed(name: str) -> int:
    return 99 + len(name)


def tokens(rng, nbm: int, B: int, V: int, frac: float = 0.5) -> np.ndarray:
    """[nbm][B] tokens, a share ``frac`` of them masked."""
    tok = rng.integers(0, V, (nbm, B)).astype(np.int32)
    tok[rng.random((nbm, B)) < frac] = MASK
    return tok


def fwd_tokens(name: str, case: dict) -> np.ndarray:
    rng = np.random.default_rng(fwd_seed(name))
    return tokens(rng, 1 + case["k_max"], case["B"], case["V"])


def seven_b_tokens() -> np.ndarray:
    return tokens(np.random.default_rng(11), 1 + SEVEN_B["k_max"], SEVEN_B["B"],
                  SEVEN_B["V"], 0.6)


def block(seed: int, B: int, m: int, V: int) -> np.ndarray:
    """A block of B tokens with m of them masked."""
    rng = np.random.default_rng(100 + seed)
    tok = rng.integers(0, V - 1, B).astype(np.int32)
    tok[rng.choice(B, m, replace=False)] = MASK
    return tok


def step_state():
    """(tok, conf, arg, k, tau) of the whole-step test: 20 of 32 positions
    masked, random confidences and tokens."""
    B, V = STEP_CASE["B"], STEP_CASE["V"]
    rng = np.random.default_rng(7)
    tok = rng.integers(0, V, B).astype(np.int32)
    tok[rng.choice(B, 20, replace=False)] = MASK
    conf = np.where(tok == MASK, rng.random(B), 0).astype(np.float32)
    arg = np.where(tok == MASK, rng.integers(0, V, B), -1).astype(np.int32)
    return tok, conf, arg, 4, 0.9
