"""C-ABI checks that need no GPU: the library loads, exports every function
include/lopa.h declares, and rejects bad arguments on the host before any
launch (each call below returns before touching the HIP runtime)."""
import ctypes
import os
import re
import subprocess

import pytest

import lookahead_decoding_amd as lopa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lopa.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lopa_\w+)\s*\(", text)))


def test_header_declares_the_step_calls():
    names = _declared()
    for fn in ("lopa_branch_build", "lopa_branch_attn", "lopa_lmhead_conf", "lopa_branch_select",
               "lopa_abi_version", "lopa_status_string", "lopa_workspace_bytes"):
        assert fn in names


def test_library_exports_every_declared_symbol():
    L = lopa.lib()
    out = subprocess.run(["nm", "-D", "--defined-only", lopa.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (lopa_\w+)", out))
    for fn in _declared():
        assert fn in exported, fn
        assert hasattr(L, fn)
    assert set(lopa.EXPORTS) == set(_declared())


def test_version_and_status_strings():
    assert lopa.abi_version() == 1
    for s in (0, -1, -2, -3, -4, 7):
        assert isinstance(lopa.status_string(s), str) and lopa.status_string(s)


def _dims(**kw):
    base = dict(L=512, B=32, Hq=28, Hkv=4, d=128, V=152064, k_max=4, dtype=lopa.BF16)
    base.update(kw)
    return lopa.Dims(**base)


@pytest.mark.parametrize("bad", [
    dict(B=0), dict(B=65), dict(Hq=28, Hkv=5), dict(Hkv=0), dict(d=0), dict(d=257),
    dict(V=0), dict(k_max=-1), dict(k_max=16), dict(dtype=7), dict(L=-1),
])
def test_invalid_dims_rejected(bad):
    d = _dims(**bad)
    n = ctypes.c_size_t(0)
    assert lopa.lib().lopa_workspace_bytes(ctypes.byref(d), ctypes.byref(n)) == -1
    fake = ctypes.c_void_p(16)
    st = lopa.lib().lopa_branch_build(ctypes.byref(d), 0, 0.9, *([fake] * 8), None)
    assert st == -1


def test_null_pointers_and_k_rejected():
    d = _dims()
    fake = ctypes.c_void_p(16)
    L = lopa.lib()
    assert L.lopa_branch_build(ctypes.byref(d), 0, 0.9, None, *([fake] * 7), None) == -1
    assert L.lopa_branch_build(ctypes.byref(d), 5, 0.9, *([fake] * 8), None) == -1   # k > k_max
    assert L.lopa_branch_build(ctypes.byref(d), -1, 0.9, *([fake] * 8), None) == -1
    assert L.lopa_branch_attn(ctypes.byref(d), fake, fake, fake, fake, fake, None, fake, fake,
                              1 << 30, None) == -1
    assert L.lopa_branch_attn(ctypes.byref(d), None, fake, fake, fake, fake, fake, fake, fake,
                              1 << 30, None) == -1
    assert L.lopa_branch_select(ctypes.byref(d), *([fake] * 9), None, None) == -1
    assert L.lopa_lmhead_conf(None, *([fake] * 8), fake, 1 << 30, None) == -1
    assert L.lopa_synth_qkv(ctypes.byref(d), 1, None, fake, fake, fake, fake, None) == -1
    # confidence-floor explore: NaN floor, k out of range, null arrays
    assert L.lopa_branch_build_floor(ctypes.byref(d), 0, 0.9, float("nan"), *([fake] * 8),
                                     None) == -1
    assert L.lopa_branch_build_floor(ctypes.byref(d), 5, 0.9, 0.1, *([fake] * 8), None) == -1
    assert L.lopa_branch_build_floor(ctypes.byref(d), 0, 0.9, 0.1, None, *([fake] * 7),
                                     None) == -1
    # sampling: temperature > 0 and finite
    for T in (0.0, -1.0, float("inf"), float("nan")):
        assert L.lopa_lmhead_sample(ctypes.byref(d), T, 1, *([fake] * 9), 1 << 30, None) == -1
    assert L.lopa_lmhead_sample(ctypes.byref(d), 0.8, 1, None, *([fake] * 8), 1 << 30, None) == -1
    # entropy variant: ent is required
    assert L.lopa_lmhead_conf_ent(ctypes.byref(d), *([fake] * 7), None, None, fake, 1 << 30,
                                  None) == -1
    # alpha variant: alpha in [0, 1], every array required
    for alpha in (-0.1, 1.5, float("nan")):
        assert L.lopa_branch_select_alpha(ctypes.byref(d), alpha, *([fake] * 13), None) == -1
    for i in range(13):
        args = [fake] * 13
        args[i] = None
        assert L.lopa_branch_select_alpha(ctypes.byref(d), 0.5, *args, None) == -1
    assert L.lopa_synth_qkv(ctypes.byref(d), 1, fake, fake, fake, None, fake, None) == -1


def test_workspace_size_and_shortfall():
    d = _dims()
    need = lopa.workspace_bytes(d)
    # prefix 512 = 8 key blocks + 1 own block, 9 row groups x 4 KV heads = 36
    # workgroups: min(256 // 36, 9 // 2) = 4 splits of attention partials
    # (O, max, sum = 130 floats per row) dominate the LM head's partials
    assert need == 4 * 4 * (5 * 32 * 7) * 130 * 4
    assert lopa.workspace_bytes(_dims(k_max=8)) == 4 * 4 * (9 * 32 * 7) * 130 * 4
    # a long prefix: 16 row groups x 4 heads = 128 workgroups -> 2 splits
    split = _dims(L=4096, B=64, k_max=8)
    assert lopa.workspace_bytes(split) == 2 * 4 * (9 * 64 * 7) * 130 * 4
    # the LM head alone needs rows x 256 vocabulary parts x (max, sum, argmax,
    # entropy term or perturbed score, sampled logit)
    head_need = 5 * 32 * 256 * 20
    fake = ctypes.c_void_p(16)
    L = lopa.lib()
    args = [fake] * 8
    assert L.lopa_lmhead_conf(ctypes.byref(d), *args, fake, head_need - 1, None) == -3
    assert L.lopa_lmhead_conf(ctypes.byref(d), *args, None, need, None) == -3
    assert L.lopa_branch_attn(ctypes.byref(d), fake, fake, fake, fake, fake, fake, fake, fake,
                              need - 1, None) == -3
    f32 = _dims(dtype=lopa.F32, V=1000)
    assert lopa.workspace_bytes(f32) == 5 * 32 * 4 * 20
