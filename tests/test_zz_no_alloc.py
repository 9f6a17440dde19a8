"""The allocation-free LM head (lopa_lmhead_conf_noalloc) against the
workspace entry point (lopa_lmhead_conf) on identical inputs: bit-identical
confidences and tokens, on two calls in a row whose second has fewer rows
(stale partials of the first call must not leak into the second), on the
bfloat16 MFMA kernels (narrow and wide row counts) and the float32 path."""
import numpy as np
import pytest
import torch

import lookahead_decoding_amd as lopa
from lookahead_decoding_amd.step import StepBuffers, dims_of, to_device
import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lopa.lib()
    yield
    torch.cuda.synchronize()


def _case(dims, M, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    m_max = dims.nb_max * dims.B
    act = torch.float32 if dims.dtype == lopa.F32 else torch.bfloat16
    H = torch.randn(m_max, dims.hidden, generator=g).to(act).cuda()
    W = (torch.randn(dims.V, dims.hidden, generator=g) * 0.3).to(act).cuda()
    rows = torch.randperm(m_max, generator=g)[:m_max].to(torch.int32).cuda()
    row_ptr = torch.full((dims.nb_max + 1,), M, dtype=torch.int32)
    row_ptr[0] = 0
    nb = torch.ones(1, dtype=torch.int32)
    return H, W, rows, row_ptr.cuda(), nb.cuda()


SHAPES = [
    # name, dims, rows of the first call, rows of the second call
    ("bf16-wide-then-narrow", dict(L=0, B=64, Hq=2, Hkv=1, d=128, V=9000, k_max=15, dtype=lopa.BF16),
     415, 100),
    ("bf16-wide-twice", dict(L=0, B=64, Hq=2, Hkv=1, d=128, V=9000, k_max=15, dtype=lopa.BF16),
     540, 300),
    ("bf16-narrow-three-groups", dict(L=0, B=64, Hq=2, Hkv=1, d=64, V=30000, k_max=15,
                                      dtype=lopa.BF16), 700, 37),
    ("f32-plain", dict(L=0, B=32, Hq=2, Hkv=2, d=32, V=5000, k_max=3, dtype=lopa.F32), 120, 9),
]


@pytest.mark.parametrize("name,dd,m1,m2", SHAPES, ids=[s[0] for s in SHAPES])
def test_noalloc_head_matches_workspace_head(name, dd, m1, m2):
    dims = lopa.Dims(**dd)
    m_max = dims.nb_max * dims.B
    for M, seed in ((m1, 1), (m2, 2)):
        print(f"[noalloc] {name}: {M} rows", flush=True)
        H, W, rows, row_ptr, nb = _case(dims, M, seed)
        ws = torch.zeros(lopa.workspace_bytes(dims), dtype=torch.uint8, device="cuda")
        c1 = torch.full((m_max,), -7.0, device="cuda")
        a1 = torch.full((m_max,), -7, dtype=torch.int32, device="cuda")
        c2, a2 = c1.clone(), a1.clone()
        lopa.lopa_lmhead_conf(dims, H, W, rows, row_ptr, nb, c1, a1, None, ws)
        lopa.lopa_lmhead_conf_noalloc(dims, H, W, rows, row_ptr, nb, c2, a2)
        torch.cuda.synchronize()
        listed = rows[:M].long()
        assert torch.equal(c1, c2) and torch.equal(a1, a2)
        assert bool((c2[listed] > 0).all()) and bool((a2[listed] >= 0).all())
        unlisted = torch.ones(m_max, dtype=torch.bool, device="cuda")
        unlisted[listed] = False
        assert bool((c2[unlisted] == -7.0).all()) and bool((a2[unlisted] == -7).all())
        del ws
