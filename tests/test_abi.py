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
    assert lopa.abi_version() == 2
    for s in (0, -1, -2, -3, -4, -5, 7):
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
    # initial-pass rows: tok, nb, rows and row_ptr are required (conf / arg optional)
    for i in range(4):
        args = [fake] * 4
        args[i] = None
        assert L.lopa_block_rows(ctypes.byref(d), *args, None, None, None) == -1
    assert L.lopa_block_rows(None, *([fake] * 6), None) == -1
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
    # the LM head needs rows x 256 vocabulary parts x (max, sum, argmax,
    # entropy term or perturbed score, sampled logit)
    head_need = 5 * 32 * 256 * 20
    # prefix 512 = 8 key blocks + 1 own block over 18 row groups x 4 KV heads
    # = 72 workgroups: 3 splits (3 units + the merge's 5 < 9) of attention
    # partials (O, max, sum = 130 floats per row), which dominate
    assert need == 3 * 4 * (5 * 32 * 7) * 130 * 4
    # 9 branches: 128 workgroups leave room for 2 splits, which would not pay;
    # the LM head's 288 rows (9 tiles) may reach the wide kernel, which also
    # takes the operand-ordered copy of the rows (288 x hidden bf16) after
    # the partials
    assert lopa.workspace_bytes(_dims(k_max=8)) == 9 * 32 * 256 * 20 + 9 * 32 * 3584 * 2
    # prefix 4096 takes the 128-row kernel: 32 row groups x 4 heads = 128
    # workgroups -> 2 splits (33 units + the merge's 8 < 65)
    assert lopa.workspace_bytes(_dims(L=4096, B=64, k_max=8)) == 2 * 4 * (9 * 64 * 7) * 130 * 4
    # prefix 2048: 33 units over 32 row groups x 4 heads = 128 workgroups ->
    # 2 splits (17 + 5 < 33)
    split = _dims(L=2048, k_max=8)
    assert lopa.workspace_bytes(split) == 2 * 4 * (9 * 32 * 7) * 130 * 4
    fake = ctypes.c_void_p(16)
    L = lopa.lib()
    args = [fake] * 8
    assert L.lopa_lmhead_conf(ctypes.byref(d), *args, fake, head_need - 1, None) == -3
    assert L.lopa_lmhead_conf(ctypes.byref(d), *args, None, need, None) == -3
    assert L.lopa_branch_attn(ctypes.byref(split), fake, fake, fake, fake, fake, fake, fake,
                              fake, lopa.workspace_bytes(split) - 1, None) == -3
    f32 = _dims(dtype=lopa.F32, V=1000)
    assert lopa.workspace_bytes(f32) == 5 * 32 * 4 * 20


def _model_dims(**kw):
    base = dict(n_layers=2, inter=512, mask_id=999, rope_theta=1e6, rms_eps=1e-6)
    base.update(kw)
    return lopa.ModelDims(**base)


def test_model_layout_and_workspace():
    d = _dims(L=40, B=16, Hq=4, Hkv=2, d=64, V=1000, k_max=3)
    md = _model_dims()
    lay = lopa.model_layout(d, md)
    h, qkv = 256, (4 + 4) * 64
    # every tensor 256-byte aligned, in the documented order, sized as declared
    assert lay.attn_norm == 0 and lay.wqkv == 512
    assert lay.bqkv == lay.wqkv + qkv * h * 2
    assert lay.wo == lay.bqkv + 1024 and lay.mlp_norm == lay.wo + h * h * 2
    assert lay.wgu == lay.mlp_norm + 512 and lay.wd == lay.wgu + 2 * 512 * h * 2
    assert lay.layer_stride == lay.wd + h * 512 * 2
    assert lay.final_norm == 2 * lay.layer_stride
    assert lay.embed == lay.final_norm + 512 and lay.lm_head == lay.embed + 1000 * h * 2
    assert lay.total == lay.lm_head + 1000 * h * 2
    assert lopa.model_workspace_bytes(d, md) > 0
    # the 7B geometry: 15.2 GB of weights
    d7 = _dims(L=512, B=32, Hq=28, Hkv=4, d=128, V=152064, k_max=4)
    lay7 = lopa.model_layout(d7, _model_dims(n_layers=28, inter=18944, mask_id=151666))
    assert lay7.total == 15231233024


@pytest.mark.parametrize("bad,status", [
    (dict(md=dict(n_layers=0)), -1), (dict(md=dict(inter=0)), -1), (dict(md=dict(mask_id=1000)), -1),
    (dict(md=dict(rope_theta=1.0)), -1), (dict(md=dict(rms_eps=-1.0)), -1),
    (dict(d=dict(dtype=lopa.F32)), -2), (dict(md=dict(inter=100)), -2), (dict(d=dict(d=60)), -2),
])
def test_model_dims_rejected(bad, status):
    dd = dict(L=40, B=16, Hq=4, Hkv=2, d=64, V=1000, k_max=3)
    dd.update(bad.get("d", {}))
    d = _dims(**dd)
    md = _model_dims(**bad.get("md", {}))
    out = lopa.ModelLayout()
    assert lopa.lib().lopa_model_layout_of(ctypes.byref(d), ctypes.byref(md), ctypes.byref(out)) == status


def test_model_calls_reject_null_and_small_workspace():
    d = _dims(L=40, B=16, Hq=4, Hkv=2, d=64, V=1000, k_max=3)
    md = _model_dims()
    L = lopa.lib()
    fake = ctypes.c_void_p(256)
    need = lopa.model_workspace_bytes(d, md)
    args = [fake, fake, fake, 40, fake, fake, fake, fake, fake]
    assert L.lopa_branch_forward(ctypes.byref(d), ctypes.byref(md), *args, fake, need - 1,
                                 None) == -3
    a2 = list(args)
    a2[4] = None                                   # br_tok
    assert L.lopa_branch_forward(ctypes.byref(d), ctypes.byref(md), *a2, fake, need, None) == -1
    a3 = list(args)
    a3[3] = 39                                     # fewer cache rows than the prefix
    assert L.lopa_branch_forward(ctypes.byref(d), ctypes.byref(md), *a3, fake, need, None) == -1
    assert L.lopa_model_synth(ctypes.byref(d), ctypes.byref(md), 1, None, fake, fake, 40,
                              None) == -1
    # the commit must fit the cache
    assert L.lopa_model_commit(ctypes.byref(d), ctypes.byref(md), fake, fake, fake, fake, fake,
                               40, 30, None) == -1


@pytest.mark.parametrize("shape", [dict(Hq=8, Hkv=2, B=16, k_max=2, d=128),
                                   dict(Hq=28, Hkv=4, B=32, k_max=4, d=128),
                                   dict(Hq=28, Hkv=4, B=32, k_max=8, d=128),
                                   dict(Hq=4, Hkv=1, B=16, k_max=2, d=128)])
def test_workspace_never_shrinks_as_the_prefix_grows(shape):
    """A decoded sequence grows its prefix block by block and keeps one
    workspace: the size for a prefix must cover every shorter one, although
    the split count of the attention partials is not monotone in the prefix
    (8 q-heads over 2 KV heads, block 16, 3 branches: 4 splits at prefix 448
    but 3 at 512)."""
    prev = 0
    for L in range(0, 4097, 32):
        n = lopa.workspace_bytes(_dims(L=L, V=4096, **shape))
        assert n >= prev, (L, n, prev)
        prev = n


def test_offsets_past_32_bits_rejected():
    """The MFMA kernels address K/V and the weight range of a vocabulary part
    with 32-bit byte offsets: shapes past that are refused, not computed
    wrongly."""
    L = lopa.lib()
    fake = ctypes.c_void_p(256)
    # prefix K/V of 2^20 keys x 8 KV heads x 128 x 2 bytes = 2^31 bytes
    d = _dims(L=1 << 20, Hq=8, Hkv=8, B=16, k_max=0)
    assert L.lopa_branch_attn(ctypes.byref(d), fake, fake, fake, fake, fake, fake, fake, fake,
                              1 << 40, None) == -2
    # 2^22 vocabulary rows of 65536 bf16 values over 256 parts: 16384 rows
    # (+ one pass of overrun) of 128 KiB each per part
    d = _dims(Hq=512, Hkv=8, d=128, V=1 << 22, B=16, k_max=0)
    assert L.lopa_lmhead_conf(ctypes.byref(d), *([fake] * 7), None, fake, 1 << 40, None) == -2


def test_model_slot_table_overflow_rejected():
    """A projection whose single unit spans all 256 workgroups (hidden 256,
    inter 16384: the down projection's K range is 256 chunks) would need 256
    slots, more than the consumers' one-byte slot table counts."""
    d = _dims(L=40, B=16, Hq=4, Hkv=2, d=64, V=1000, k_max=0)
    out = lopa.ModelLayout()
    md = _model_dims(inter=16384)
    assert lopa.lib().lopa_model_layout_of(ctypes.byref(d), ctypes.byref(md),
                                           ctypes.byref(out)) == -2
    md = _model_dims(inter=8192)
    assert lopa.lib().lopa_model_layout_of(ctypes.byref(d), ctypes.byref(md),
                                           ctypes.byref(out)) == 0


def test_noalloc_head_rejects_before_any_launch():
    """The allocation-free LM head checks its arguments, and that its partials
    fit the library's fixed 16 MiB array, before touching the HIP runtime."""
    L = lopa.lib()
    fake = ctypes.c_void_p(256)
    d = _dims()
    assert L.lopa_lmhead_conf_noalloc(ctypes.byref(d), None, *([fake] * 7), None) == -1
    assert L.lopa_lmhead_conf_noalloc(None, *([fake] * 8), None) == -1
    # float32 path over a 400000-entry vocabulary with 16 x 64 rows: 1024 x 1563
    # partials of 20 bytes (32 MB) do not fit
    d = _dims(dtype=lopa.F32, V=400000, B=64, k_max=15)
    assert L.lopa_lmhead_conf_noalloc(ctypes.byref(d), *([fake] * 8), None) == -5
    # bfloat16 at hidden 28 x 256 with 1024 rows: 5 MiB of partials plus the
    # wide kernel's 14 MiB copy of the rows do not fit
    d = _dims(d=256, B=64, k_max=15)
    assert lopa.workspace_bytes(d) == 1024 * 256 * 20 + 1024 * 7168 * 2
    assert L.lopa_lmhead_conf_noalloc(ctypes.byref(d), *([fake] * 8), None) == -5
    assert "scratch" in lopa.status_string(-5)

def test_forward_cases_are_supported_shapes():
    """Every geometry the GPU forward tests run is one the library accepts
    (checked here on the host, before any of them reaches a GPU)."""
    from _model_cases import FWD_CASES
    for name, case, _ in FWD_CASES:
        d = _dims(L=case["L"], B=case["B"], Hq=case["Hq"], Hkv=case["Hkv"], d=case["d"],
                  V=case["V"], k_max=case["k_max"])
        md = _model_dims(n_layers=case["n_layers"], inter=case["inter"], mask_id=case["V"] - 1)
        out = lopa.ModelLayout()
        assert lopa.lib().lopa_model_layout_of(ctypes.byref(d), ctypes.byref(md),
                                               ctypes.byref(out)) == 0, name
