"""Python binding of liblopa: one LoPA branch-verification step on MI355X.

Argument marshalling only.  Every function below forwards torch device
tensors (as raw pointers) and sizes to the C ABI declared in
``include/lopa.h``; all of the step's arithmetic runs in the library's HIP
kernels.  There is no CPU fallback: if ``liblopa.so`` is missing the import of
the library raises.

    import lookahead_decoding_amd as lopa
    dims = lopa.Dims(L=512, B=32, Hq=28, Hkv=4, d=128, V=152064, k_max=4,
                     dtype=lopa.BF16)
    lopa.lopa_branch_build(dims, k, tau, tok, conf, arg, nb, br_tok, br_mask,
                           rows, row_ptr)
    ...
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "liblopa.so")

F32 = 0
BF16 = 1
MASK = -1
MAX_BLOCK = 64
MAX_BRANCHES = 16

STATUS = {0: "LOPA_OK", -1: "LOPA_ERR_INVALID", -2: "LOPA_ERR_UNSUPPORTED",
          -3: "LOPA_ERR_WORKSPACE", -4: "LOPA_ERR_HIP", -5: "LOPA_ERR_TOO_LARGE"}


class Dims(ctypes.Structure):
    """Mirror of ``lopa_dims``."""
    _fields_ = [(n, ctypes.c_int32) for n in ("L", "B", "Hq", "Hkv", "d", "V", "k_max", "dtype")]

    @property
    def hidden(self) -> int:
        return self.Hq * self.d

    @property
    def nb_max(self) -> int:
        return self.k_max + 1

    def __repr__(self) -> str:
        return "Dims(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_) + ")"


class ModelDims(ctypes.Structure):
    """Mirror of ``lopa_model_dims``."""
    _fields_ = [("n_layers", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("mask_id", ctypes.c_int32), ("rope_theta", ctypes.c_float),
                ("rms_eps", ctypes.c_float)]

    def __repr__(self) -> str:
        return "ModelDims(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_) + ")"


class ModelLayout(ctypes.Structure):
    """Mirror of ``lopa_model_layout`` (byte offsets into the weight buffer)."""
    _fields_ = [(n, ctypes.c_size_t) for n in (
        "attn_norm", "wqkv", "bqkv", "wo", "mlp_norm", "wgu", "wd", "layer0", "layer_stride",
        "final_norm", "embed", "lm_head", "total")]


class LopaError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} returned {STATUS.get(status, status)}: {text}")
        self.status = status


_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int32

_SIGS = {
    "lopa_abi_version": ([], ctypes.c_int),
    "lopa_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "lopa_workspace_bytes": ([ctypes.POINTER(Dims), ctypes.POINTER(ctypes.c_size_t)], ctypes.c_int),
    "lopa_block_rows": ([ctypes.POINTER(Dims), _P, _P, _P, _P, _P, _P, _P], ctypes.c_int),
    "lopa_branch_build": ([ctypes.POINTER(Dims), _I, ctypes.c_float, _P, _P, _P, _P, _P, _P, _P, _P, _P],
                          ctypes.c_int),
    "lopa_branch_build_floor": ([ctypes.POINTER(Dims), _I, ctypes.c_float, ctypes.c_float] +
                                [_P] * 9, ctypes.c_int),
    "lopa_branch_attn": ([ctypes.POINTER(Dims), _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P],
                         ctypes.c_int),
    "lopa_lmhead_conf": ([ctypes.POINTER(Dims), _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P],
                         ctypes.c_int),
    "lopa_lmhead_conf_noalloc": ([ctypes.POINTER(Dims), _P, _P, _P, _P, _P, _P, _P, _P, _P],
                                 ctypes.c_int),
    "lopa_branch_select": ([ctypes.POINTER(Dims), _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P],
                           ctypes.c_int),
    "lopa_lmhead_conf_ent": ([ctypes.POINTER(Dims), _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                              ctypes.c_size_t, _P], ctypes.c_int),
    "lopa_branch_select_alpha": ([ctypes.POINTER(Dims), ctypes.c_float] + [_P] * 14,
                                 ctypes.c_int),
    "lopa_lmhead_sample": ([ctypes.POINTER(Dims), ctypes.c_float, ctypes.c_uint64] + [_P] * 9 +
                           [ctypes.c_size_t, _P], ctypes.c_int),
    "lopa_synth_qkv": ([ctypes.POINTER(Dims), ctypes.c_uint64, _P, _P, _P, _P, _P, _P],
                       ctypes.c_int),
    "lopa_commit_block": ([ctypes.POINTER(Dims), _P, _P, _P, _P, _P, _I, _P], ctypes.c_int),
    "lopa_model_layout_of": ([ctypes.POINTER(Dims), ctypes.POINTER(ModelDims),
                              ctypes.POINTER(ModelLayout)], ctypes.c_int),
    "lopa_model_workspace_bytes": ([ctypes.POINTER(Dims), ctypes.POINTER(ModelDims),
                                    ctypes.POINTER(ctypes.c_size_t)], ctypes.c_int),
    "lopa_model_synth": ([ctypes.POINTER(Dims), ctypes.POINTER(ModelDims), ctypes.c_uint64, _P,
                          _P, _P, ctypes.c_size_t, _P], ctypes.c_int),
    "lopa_branch_forward": ([ctypes.POINTER(Dims), ctypes.POINTER(ModelDims), _P, _P, _P,
                             ctypes.c_size_t, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P],
                            ctypes.c_int),
    "lopa_model_commit": ([ctypes.POINTER(Dims), ctypes.POINTER(ModelDims), _P, _P, _P, _P, _P,
                           ctypes.c_size_t, _I, _P], ctypes.c_int),
}
EXPORTS = tuple(_SIGS)


def lib():
    """The loaded liblopa (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -c 'import __graft_entry__ as g; g.build()'`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise LopaError(fn, status, lib().lopa_status_string(status).decode())


def _ptr(t, dtype=None, name="tensor"):
    """Raw device pointer of a contiguous CUDA tensor (None -> NULL)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _act_dtype(dims):
    import torch
    return torch.float32 if dims.dtype == F32 else torch.bfloat16


def abi_version() -> int:
    return lib().lopa_abi_version()


def status_string(status: int) -> str:
    return lib().lopa_status_string(status).decode()


def workspace_bytes(dims: Dims) -> int:
    n = ctypes.c_size_t(0)
    _check("lopa_workspace_bytes", lib().lopa_workspace_bytes(ctypes.byref(dims), ctypes.byref(n)))
    return n.value


def lopa_block_rows(dims, tok, nb, rows, row_ptr, conf=None, arg=None, stream=None) -> None:
    import torch
    i32, f32 = torch.int32, torch.float32
    _check("lopa_block_rows", lib().lopa_block_rows(
        ctypes.byref(dims), _ptr(tok, i32, "tok"), _ptr(nb, i32, "nb"), _ptr(rows, i32, "rows"),
        _ptr(row_ptr, i32, "row_ptr"), _ptr(conf, f32, "conf"), _ptr(arg, i32, "arg"),
        _stream(stream)))


def lopa_branch_build(dims, k, tau, tok, conf, arg, nb, br_tok, br_mask, rows, row_ptr,
                      stream=None) -> None:
    import torch
    i32, f32, u8 = torch.int32, torch.float32, torch.uint8
    _check("lopa_branch_build", lib().lopa_branch_build(
        ctypes.byref(dims), int(k), float(tau),
        _ptr(tok, i32, "tok"), _ptr(conf, f32, "conf"), _ptr(arg, i32, "arg"),
        _ptr(nb, i32, "nb"), _ptr(br_tok, i32, "br_tok"), _ptr(br_mask, u8, "br_mask"),
        _ptr(rows, i32, "rows"), _ptr(row_ptr, i32, "row_ptr"), _stream(stream)))


def lopa_branch_build_floor(dims, k, tau, gamma, tok, conf, arg, nb, br_tok, br_mask, rows,
                            row_ptr, stream=None) -> None:
    import torch
    i32, f32, u8 = torch.int32, torch.float32, torch.uint8
    _check("lopa_branch_build_floor", lib().lopa_branch_build_floor(
        ctypes.byref(dims), int(k), float(tau), float(gamma),
        _ptr(tok, i32, "tok"), _ptr(conf, f32, "conf"), _ptr(arg, i32, "arg"),
        _ptr(nb, i32, "nb"), _ptr(br_tok, i32, "br_tok"), _ptr(br_mask, u8, "br_mask"),
        _ptr(rows, i32, "rows"), _ptr(row_ptr, i32, "row_ptr"), _stream(stream)))


def lopa_branch_attn(dims, Kp, Vp, Qb, Kb, Vb, nb, H, ws=None, stream=None) -> None:
    import torch
    a = _act_dtype(dims)
    _check("lopa_branch_attn", lib().lopa_branch_attn(
        ctypes.byref(dims), _ptr(Kp, a, "Kp"), _ptr(Vp, a, "Vp"), _ptr(Qb, a, "Qb"),
        _ptr(Kb, a, "Kb"), _ptr(Vb, a, "Vb"), _ptr(nb, torch.int32, "nb"), _ptr(H, a, "H"),
        _ptr(ws, None, "ws"), 0 if ws is None else ws.numel() * ws.element_size(),
        _stream(stream)))


def lopa_lmhead_conf(dims, H, W, rows, row_ptr, nb, conf, arg, logits_out, ws,
                     stream=None) -> None:
    import torch
    a = _act_dtype(dims)
    i32 = torch.int32
    _check("lopa_lmhead_conf", lib().lopa_lmhead_conf(
        ctypes.byref(dims), _ptr(H, a, "H"), _ptr(W, a, "W"), _ptr(rows, i32, "rows"),
        _ptr(row_ptr, i32, "row_ptr"), _ptr(nb, i32, "nb"), _ptr(conf, torch.float32, "conf"),
        _ptr(arg, i32, "arg"), _ptr(logits_out, torch.float32, "logits_out"),
        _ptr(ws, None, "ws"), 0 if ws is None else ws.numel() * ws.element_size(),
        _stream(stream)))


def lopa_lmhead_conf_noalloc(dims, H, W, rows, row_ptr, nb, conf, arg, logits_out=None,
                             stream=None) -> None:
    """lopa_lmhead_conf with its partials in the library's fixed device array
    (no workspace argument; allocates nothing)."""
    import torch
    a = _act_dtype(dims)
    i32 = torch.int32
    _check("lopa_lmhead_conf_noalloc", lib().lopa_lmhead_conf_noalloc(
        ctypes.byref(dims), _ptr(H, a, "H"), _ptr(W, a, "W"), _ptr(rows, i32, "rows"),
        _ptr(row_ptr, i32, "row_ptr"), _ptr(nb, i32, "nb"), _ptr(conf, torch.float32, "conf"),
        _ptr(arg, i32, "arg"), _ptr(logits_out, torch.float32, "logits_out"), _stream(stream)))


def lopa_branch_select(dims, nb, br_mask, br_tok, conf, arg, bconf, winner, tok_next,
                       conf_next, arg_next, stream=None) -> None:
    import torch
    i32, f32 = torch.int32, torch.float32
    _check("lopa_branch_select", lib().lopa_branch_select(
        ctypes.byref(dims), _ptr(nb, i32, "nb"), _ptr(br_mask, torch.uint8, "br_mask"),
        _ptr(br_tok, i32, "br_tok"), _ptr(conf, f32, "conf"), _ptr(arg, i32, "arg"),
        _ptr(bconf, f32, "bconf"), _ptr(winner, i32, "winner"), _ptr(tok_next, i32, "tok_next"),
        _ptr(conf_next, f32, "conf_next"), _ptr(arg_next, i32, "arg_next"), _stream(stream)))


def lopa_lmhead_conf_ent(dims, H, W, rows, row_ptr, nb, conf, arg, ent, logits_out, ws,
                         stream=None) -> None:
    import torch
    a = _act_dtype(dims)
    i32, f32 = torch.int32, torch.float32
    if ent is None:
        raise ValueError("ent is required")
    _check("lopa_lmhead_conf_ent", lib().lopa_lmhead_conf_ent(
        ctypes.byref(dims), _ptr(H, a, "H"), _ptr(W, a, "W"), _ptr(rows, i32, "rows"),
        _ptr(row_ptr, i32, "row_ptr"), _ptr(nb, i32, "nb"), _ptr(conf, f32, "conf"),
        _ptr(arg, i32, "arg"), _ptr(ent, f32, "ent"), _ptr(logits_out, f32, "logits_out"),
        _ptr(ws, None, "ws"), 0 if ws is None else ws.numel() * ws.element_size(),
        _stream(stream)))


def lopa_lmhead_sample(dims, temperature, seed, H, W, rows, row_ptr, nb, conf, arg, logits_out,
                       ws, stream=None) -> None:
    import torch
    a = _act_dtype(dims)
    i32, f32 = torch.int32, torch.float32
    _check("lopa_lmhead_sample", lib().lopa_lmhead_sample(
        ctypes.byref(dims), float(temperature), int(seed) & 0xFFFFFFFFFFFFFFFF, _ptr(H, a, "H"),
        _ptr(W, a, "W"), _ptr(rows, i32, "rows"), _ptr(row_ptr, i32, "row_ptr"),
        _ptr(nb, i32, "nb"), _ptr(conf, f32, "conf"), _ptr(arg, i32, "arg"),
        _ptr(logits_out, f32, "logits_out"), _ptr(ws, None, "ws"),
        0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def lopa_branch_select_alpha(dims, alpha, tok, conf_state, nb, br_mask, br_tok, conf, arg, ent,
                             score, winner, tok_next, conf_next, arg_next, stream=None) -> None:
    import torch
    i32, f32 = torch.int32, torch.float32
    _check("lopa_branch_select_alpha", lib().lopa_branch_select_alpha(
        ctypes.byref(dims), float(alpha), _ptr(tok, i32, "tok"),
        _ptr(conf_state, f32, "conf_state"), _ptr(nb, i32, "nb"),
        _ptr(br_mask, torch.uint8, "br_mask"), _ptr(br_tok, i32, "br_tok"),
        _ptr(conf, f32, "conf"), _ptr(arg, i32, "arg"), _ptr(ent, f32, "ent"),
        _ptr(score, f32, "score"), _ptr(winner, i32, "winner"), _ptr(tok_next, i32, "tok_next"),
        _ptr(conf_next, f32, "conf_next"), _ptr(arg_next, i32, "arg_next"), _stream(stream)))


def lopa_synth_qkv(dims, seed, br_tok, nb, Qb, Kb, Vb, stream=None) -> None:
    import torch
    a = _act_dtype(dims)
    i32 = torch.int32
    _check("lopa_synth_qkv", lib().lopa_synth_qkv(
        ctypes.byref(dims), int(seed) & 0xFFFFFFFFFFFFFFFF, _ptr(br_tok, i32, "br_tok"),
        _ptr(nb, i32, "nb"), _ptr(Qb, a, "Qb"), _ptr(Kb, a, "Kb"), _ptr(Vb, a, "Vb"),
        _stream(stream)))


def lopa_commit_block(dims, winner, Kb, Vb, Kp, Vp, at, stream=None) -> None:
    import torch
    a = _act_dtype(dims)
    _check("lopa_commit_block", lib().lopa_commit_block(
        ctypes.byref(dims), _ptr(winner, torch.int32, "winner"), _ptr(Kb, a, "Kb"),
        _ptr(Vb, a, "Vb"), _ptr(Kp, a, "Kp"), _ptr(Vp, a, "Vp"), int(at), _stream(stream)))


def model_layout(dims, md) -> ModelLayout:
    out = ModelLayout()
    _check("lopa_model_layout_of", lib().lopa_model_layout_of(ctypes.byref(dims), ctypes.byref(md),
                                                              ctypes.byref(out)))
    return out


def model_workspace_bytes(dims, md) -> int:
    n = ctypes.c_size_t(0)
    _check("lopa_model_workspace_bytes", lib().lopa_model_workspace_bytes(
        ctypes.byref(dims), ctypes.byref(md), ctypes.byref(n)))
    return n.value


def lopa_model_synth(dims, md, seed, weights, Kp, Vp, kv_layer_rows, stream=None) -> None:
    import torch
    bf = torch.bfloat16
    _check("lopa_model_synth", lib().lopa_model_synth(
        ctypes.byref(dims), ctypes.byref(md), int(seed) & 0xFFFFFFFFFFFFFFFF,
        _ptr(weights, torch.uint8, "weights"), _ptr(Kp, bf, "Kp"), _ptr(Vp, bf, "Vp"),
        int(kv_layer_rows), _stream(stream)))


def lopa_branch_forward(dims, md, weights, Kp, Vp, kv_layer_rows, br_tok, nb, Kb, Vb, H, ws,
                        stream=None) -> None:
    import torch
    bf, i32 = torch.bfloat16, torch.int32
    _check("lopa_branch_forward", lib().lopa_branch_forward(
        ctypes.byref(dims), ctypes.byref(md), _ptr(weights, torch.uint8, "weights"),
        _ptr(Kp, bf, "Kp"), _ptr(Vp, bf, "Vp"), int(kv_layer_rows), _ptr(br_tok, i32, "br_tok"),
        _ptr(nb, i32, "nb"), _ptr(Kb, bf, "Kb"), _ptr(Vb, bf, "Vb"), _ptr(H, bf, "H"),
        _ptr(ws, None, "ws"), 0 if ws is None else ws.numel() * ws.element_size(),
        _stream(stream)))


def lopa_model_commit(dims, md, winner, Kb, Vb, Kp, Vp, kv_layer_rows, at, stream=None) -> None:
    import torch
    bf = torch.bfloat16
    _check("lopa_model_commit", lib().lopa_model_commit(
        ctypes.byref(dims), ctypes.byref(md), _ptr(winner, torch.int32, "winner"),
        _ptr(Kb, bf, "Kb"), _ptr(Vb, bf, "Vb"), _ptr(Kp, bf, "Kp"), _ptr(Vp, bf, "Vp"),
        int(kv_layer_rows), int(at), _stream(stream)))


from .step import StepBuffers, run_step, initial_pass  # noqa: E402,F401
