"""ctypes binding of ``liblora_mlp.so`` (declared in ``include/lora_mlp.h``).

Argument marshalling only: every function here converts its arguments
(torch tensors -> device pointers, ``None`` -> NULL, the current torch HIP
stream when no stream is given) and calls the C entry point of the same name.
Nothing is computed in Python, and there is no fallback: if the library is
not built, or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "liblora_mlp.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "lora_mlp.h")

LMLP_OK, LMLP_ERR_INVALID_ARG, LMLP_ERR_UNSUPPORTED, LMLP_ERR_WORKSPACE, LMLP_ERR_HIP = range(5)
LMLP_F32, LMLP_BF16 = 0, 1
LMLP_W_DENSE, LMLP_W_INT4_B64 = 0, 1
LMLP_CONSUME_SAVED = 0x1
LMLP_INT4_INKERNEL = 0x2
LMLP_RECOMPUTE_GU = 0x4
LMLP_RMSNORM = 0x8
LMLP_INT4_BF16_COPIES = 0x10


class lmlp_dims(ctypes.Structure):
    _fields_ = [("tokens", ctypes.c_int64), ("hidden", ctypes.c_int64), ("inter", ctypes.c_int64),
                ("rank", ctypes.c_int64), ("scale", ctypes.c_float), ("dtype", ctypes.c_int32),
                ("wfmt", ctypes.c_int32), ("flags", ctypes.c_uint32)]


def make_dims(tokens, hidden, inter, rank, scale, dtype="bf16", wfmt="dense", flags=0) -> lmlp_dims:
    dt = {"f32": LMLP_F32, "bf16": LMLP_BF16}[dtype] if isinstance(dtype, str) else int(dtype)
    wf = {"dense": LMLP_W_DENSE, "int4_b64": LMLP_W_INT4_B64}[wfmt] if isinstance(wfmt, str) else int(wfmt)
    return lmlp_dims(int(tokens), int(hidden), int(inter), int(rank), float(scale), dt, wf, int(flags))


class lmlp_kernel_time(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 40), ("ms", ctypes.c_float)]


class LoraMLPError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: {status_name(status)} ({detail})")


_lib = None
_P = ctypes.c_void_p
_SZ = ctypes.c_size_t

_SIGS = {
    "lora_mlp_saved_bytes": (_SZ, [ctypes.POINTER(lmlp_dims)]),
    "lora_mlp_workspace_bytes": (_SZ, [ctypes.POINTER(lmlp_dims), ctypes.c_int]),
    "lora_mlp_forward": (ctypes.c_int, [ctypes.POINTER(lmlp_dims)] + [_P] * 14 + [_P, _SZ, _P, _SZ, _P]),
    "lora_mlp_backward": (ctypes.c_int, [ctypes.POINTER(lmlp_dims)] + [_P] * 15 + [_SZ] + [_P] * 8
                          + [_SZ, _P]),
    "lora_mlp_norm_forward": (ctypes.c_int, [ctypes.POINTER(lmlp_dims), ctypes.c_float] + [_P] * 15
                              + [_P, _SZ, _P, _SZ, _P]),
    "lora_mlp_norm_backward": (ctypes.c_int, [ctypes.POINTER(lmlp_dims)] + [_P] * 16 + [_SZ] + [_P] * 8
                               + [_SZ, _P]),
    "lora_moe_saved_bytes": (_SZ, [ctypes.POINTER(lmlp_dims), ctypes.c_int64, _P]),
    "lora_moe_workspace_bytes": (_SZ, [ctypes.POINTER(lmlp_dims), ctypes.c_int64, _P, ctypes.c_int]),
    "lora_moe_forward": (ctypes.c_int, [ctypes.POINTER(lmlp_dims), ctypes.c_int64, _P] + [_P] * 14
                         + [_P, _SZ, _P, _SZ, _P]),
    "lora_moe_backward": (ctypes.c_int, [ctypes.POINTER(lmlp_dims), ctypes.c_int64, _P] + [_P] * 15 + [_SZ]
                          + [_P] * 8 + [_SZ, _P]),
    "lora_linear_saved_bytes": (_SZ, [ctypes.POINTER(lmlp_dims)]),
    "lora_linear_workspace_bytes": (_SZ, [ctypes.POINTER(lmlp_dims), ctypes.c_int]),
    "lora_linear_forward": (ctypes.c_int, [ctypes.POINTER(lmlp_dims)] + [_P] * 7 + [_SZ, _P, _SZ, _P]),
    "lora_linear_forward_noalloc": (ctypes.c_int, [ctypes.POINTER(lmlp_dims)] + [_P] * 7 + [_SZ, _P]),
    "lora_linear_backward": (ctypes.c_int, [ctypes.POINTER(lmlp_dims)] + [_P] * 7 + [_SZ] + [_P] * 4
                             + [_SZ, _P]),
    "lora_mlp_dequant_int4": (ctypes.c_int, [_P, _P, ctypes.c_int64, ctypes.c_int64, _P, _P]),
    "lora_mlp_profile_begin": (ctypes.c_int, []),
    "lora_mlp_profile_end": (ctypes.c_int, [ctypes.POINTER(lmlp_kernel_time), ctypes.c_int,
                                            ctypes.POINTER(ctypes.c_int)]),
    "lora_mlp_mfma_probe": (ctypes.c_int, [_P, _SZ, _P, ctypes.c_int, ctypes.c_int, _P]),
    "lora_mlp_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "lora_mlp_last_error": (ctypes.c_char_p, []),
}


def header_functions() -> list:
    """Names of the functions ``include/lora_mlp.h`` declares."""
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lora_(?:mlp|linear|moe)_\w+)\s*\(", text)))


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m lora_swiglu_mlp_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def status_name(code: int) -> str:
    return lib().lora_mlp_status_string(int(code)).decode()


def lora_mlp_status_string(code: int) -> str:
    return status_name(code)


def lora_mlp_last_error() -> str:
    return lib().lora_mlp_last_error().decode()


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _nbytes(t) -> int:
    if t is None:
        return 0
    if isinstance(t, int):
        raise TypeError("pass a tensor (or an explicit size) for sized buffers")
    return t.numel() * t.element_size()


def _check(rc: int, where: str):
    if rc != LMLP_OK:
        raise LoraMLPError(rc, where, lora_mlp_last_error())


def lora_mlp_saved_bytes(dims: lmlp_dims) -> int:
    return int(lib().lora_mlp_saved_bytes(ctypes.byref(dims)))


def lora_mlp_workspace_bytes(dims: lmlp_dims, is_backward: bool) -> int:
    return int(lib().lora_mlp_workspace_bytes(ctypes.byref(dims), int(bool(is_backward))))


def lora_mlp_forward(dims, x, w_gate, w_gate_scales, w_up, w_up_scales, w_down, w_down_scales,
                     a_gate, b_gate, a_up, b_up, a_down, b_down, y, saved, workspace,
                     stream=None, saved_bytes=None, workspace_bytes=None):
    rc = lib().lora_mlp_forward(
        ctypes.byref(dims), _ptr(x), _ptr(w_gate), _ptr(w_gate_scales), _ptr(w_up), _ptr(w_up_scales),
        _ptr(w_down), _ptr(w_down_scales), _ptr(a_gate), _ptr(b_gate), _ptr(a_up), _ptr(b_up),
        _ptr(a_down), _ptr(b_down), _ptr(y), _ptr(saved),
        _nbytes(saved) if saved_bytes is None else saved_bytes,
        _ptr(workspace), _nbytes(workspace) if workspace_bytes is None else workspace_bytes,
        _stream(stream))
    _check(rc, "lora_mlp_forward")


def lora_mlp_backward(dims, dy, x, w_gate, w_gate_scales, w_up, w_up_scales, w_down, w_down_scales,
                      a_gate, b_gate, a_up, b_up, a_down, b_down, saved, dx, da_gate, db_gate,
                      da_up, db_up, da_down, db_down, workspace, stream=None, saved_bytes=None,
                      workspace_bytes=None):
    rc = lib().lora_mlp_backward(
        ctypes.byref(dims), _ptr(dy), _ptr(x), _ptr(w_gate), _ptr(w_gate_scales), _ptr(w_up),
        _ptr(w_up_scales), _ptr(w_down), _ptr(w_down_scales), _ptr(a_gate), _ptr(b_gate), _ptr(a_up),
        _ptr(b_up), _ptr(a_down), _ptr(b_down), _ptr(saved),
        _nbytes(saved) if saved_bytes is None else saved_bytes,
        _ptr(dx), _ptr(da_gate), _ptr(db_gate), _ptr(da_up), _ptr(db_up), _ptr(da_down),
        _ptr(db_down), _ptr(workspace),
        _nbytes(workspace) if workspace_bytes is None else workspace_bytes, _stream(stream))
    _check(rc, "lora_mlp_backward")


def lora_mlp_norm_forward(dims, eps, x, gamma, w_gate, w_gate_scales, w_up, w_up_scales, w_down, w_down_scales,
                          a_gate, b_gate, a_up, b_up, a_down, b_down, y, saved, workspace, stream=None,
                          saved_bytes=None, workspace_bytes=None):
    rc = lib().lora_mlp_norm_forward(
        ctypes.byref(dims), float(eps), _ptr(x), _ptr(gamma), _ptr(w_gate), _ptr(w_gate_scales), _ptr(w_up),
        _ptr(w_up_scales), _ptr(w_down), _ptr(w_down_scales), _ptr(a_gate), _ptr(b_gate), _ptr(a_up),
        _ptr(b_up), _ptr(a_down), _ptr(b_down), _ptr(y), _ptr(saved),
        _nbytes(saved) if saved_bytes is None else saved_bytes,
        _ptr(workspace), _nbytes(workspace) if workspace_bytes is None else workspace_bytes,
        _stream(stream))
    _check(rc, "lora_mlp_norm_forward")


def lora_mlp_norm_backward(dims, dy, x, gamma, w_gate, w_gate_scales, w_up, w_up_scales, w_down, w_down_scales,
                           a_gate, b_gate, a_up, b_up, a_down, b_down, saved, dx, da_gate, db_gate, da_up, db_up,
                           da_down, db_down, workspace, stream=None, saved_bytes=None, workspace_bytes=None):
    rc = lib().lora_mlp_norm_backward(
        ctypes.byref(dims), _ptr(dy), _ptr(x), _ptr(gamma), _ptr(w_gate), _ptr(w_gate_scales), _ptr(w_up),
        _ptr(w_up_scales), _ptr(w_down), _ptr(w_down_scales), _ptr(a_gate), _ptr(b_gate), _ptr(a_up),
        _ptr(b_up), _ptr(a_down), _ptr(b_down), _ptr(saved),
        _nbytes(saved) if saved_bytes is None else saved_bytes,
        _ptr(dx), _ptr(da_gate), _ptr(db_gate), _ptr(da_up), _ptr(db_up), _ptr(da_down),
        _ptr(db_down), _ptr(workspace),
        _nbytes(workspace) if workspace_bytes is None else workspace_bytes, _stream(stream))
    _check(rc, "lora_mlp_norm_backward")


def offsets_array(offsets) -> "ctypes.Array":
    """Host int64 array of the expert row offsets (n_experts + 1 values)."""
    vals = [int(v) for v in offsets]
    return (ctypes.c_int64 * len(vals))(*vals)


def lora_moe_saved_bytes(dims: lmlp_dims, offsets) -> int:
    off = offsets_array(offsets)
    return int(lib().lora_moe_saved_bytes(ctypes.byref(dims), len(off) - 1, off))


def lora_moe_workspace_bytes(dims: lmlp_dims, offsets, is_backward: bool) -> int:
    off = offsets_array(offsets)
    return int(lib().lora_moe_workspace_bytes(ctypes.byref(dims), len(off) - 1, off, int(bool(is_backward))))


def lora_moe_forward(dims, offsets, x, w_gate, w_gate_scales, w_up, w_up_scales, w_down, w_down_scales,
                     a_gate, b_gate, a_up, b_up, a_down, b_down, y, saved, workspace, stream=None,
                     saved_bytes=None, workspace_bytes=None):
    """offsets: n_experts + 1 host ints (rows of expert e: offsets[e] .. offsets[e+1]-1)."""
    off = offsets_array(offsets)
    rc = lib().lora_moe_forward(
        ctypes.byref(dims), len(off) - 1, off, _ptr(x), _ptr(w_gate), _ptr(w_gate_scales), _ptr(w_up),
        _ptr(w_up_scales), _ptr(w_down), _ptr(w_down_scales), _ptr(a_gate), _ptr(b_gate), _ptr(a_up),
        _ptr(b_up), _ptr(a_down), _ptr(b_down), _ptr(y), _ptr(saved),
        _nbytes(saved) if saved_bytes is None else saved_bytes,
        _ptr(workspace), _nbytes(workspace) if workspace_bytes is None else workspace_bytes, _stream(stream))
    _check(rc, "lora_moe_forward")


def lora_moe_backward(dims, offsets, dy, x, w_gate, w_gate_scales, w_up, w_up_scales, w_down, w_down_scales,
                      a_gate, b_gate, a_up, b_up, a_down, b_down, saved, dx, da_gate, db_gate, da_up, db_up,
                      da_down, db_down, workspace, stream=None, saved_bytes=None, workspace_bytes=None):
    off = offsets_array(offsets)
    rc = lib().lora_moe_backward(
        ctypes.byref(dims), len(off) - 1, off, _ptr(dy), _ptr(x), _ptr(w_gate), _ptr(w_gate_scales),
        _ptr(w_up), _ptr(w_up_scales), _ptr(w_down), _ptr(w_down_scales), _ptr(a_gate), _ptr(b_gate),
        _ptr(a_up), _ptr(b_up), _ptr(a_down), _ptr(b_down), _ptr(saved),
        _nbytes(saved) if saved_bytes is None else saved_bytes,
        _ptr(dx), _ptr(da_gate), _ptr(db_gate), _ptr(da_up), _ptr(db_up), _ptr(da_down), _ptr(db_down),
        _ptr(workspace), _nbytes(workspace) if workspace_bytes is None else workspace_bytes, _stream(stream))
    _check(rc, "lora_moe_backward")


def lora_linear_saved_bytes(dims: lmlp_dims) -> int:
    return int(lib().lora_linear_saved_bytes(ctypes.byref(dims)))


def lora_linear_workspace_bytes(dims: lmlp_dims, is_backward: bool) -> int:
    return int(lib().lora_linear_workspace_bytes(ctypes.byref(dims), int(bool(is_backward))))


def lora_linear_forward(dims, x, w, w_scales, a, b, y, saved, workspace, stream=None, saved_bytes=None,
                        workspace_bytes=None):
    """dims: make_dims(tokens, in, out, rank, scale, ...) (hidden = in, inter = out)."""
    rc = lib().lora_linear_forward(
        ctypes.byref(dims), _ptr(x), _ptr(w), _ptr(w_scales), _ptr(a), _ptr(b), _ptr(y), _ptr(saved),
        _nbytes(saved) if saved_bytes is None else saved_bytes,
        _ptr(workspace), _nbytes(workspace) if workspace_bytes is None else workspace_bytes, _stream(stream))
    _check(rc, "lora_linear_forward")


def lora_linear_forward_noalloc(dims, x, w, w_scales, a, b, y, saved, stream=None, saved_bytes=None):
    """lora_linear_forward with the library's own scratch as the workspace."""
    rc = lib().lora_linear_forward_noalloc(
        ctypes.byref(dims), _ptr(x), _ptr(w), _ptr(w_scales), _ptr(a), _ptr(b), _ptr(y), _ptr(saved),
        _nbytes(saved) if saved_bytes is None else saved_bytes, _stream(stream))
    _check(rc, "lora_linear_forward_noalloc")


LMLP_NOALLOC_SCRATCH_BYTES = 96 << 20


def lora_linear_backward(dims, dy, x, w, w_scales, a, b, saved, dx, da, db, workspace, stream=None,
                         saved_bytes=None, workspace_bytes=None):
    rc = lib().lora_linear_backward(
        ctypes.byref(dims), _ptr(dy), _ptr(x), _ptr(w), _ptr(w_scales), _ptr(a), _ptr(b), _ptr(saved),
        _nbytes(saved) if saved_bytes is None else saved_bytes,
        _ptr(dx), _ptr(da), _ptr(db), _ptr(workspace),
        _nbytes(workspace) if workspace_bytes is None else workspace_bytes, _stream(stream))
    _check(rc, "lora_linear_backward")


def lora_mlp_dequant_int4(packed, scales, out: int, inn: int, w_bf16, stream=None):
    rc = lib().lora_mlp_dequant_int4(_ptr(packed), _ptr(scales), int(out), int(inn), _ptr(w_bf16),
                                     _stream(stream))
    _check(rc, "lora_mlp_dequant_int4")


def lora_mlp_profile_begin():
    _check(lib().lora_mlp_profile_begin(), "lora_mlp_profile_begin")


def lora_mlp_profile_end(capacity: int = 65536):
    """Stop recording; returns [(kernel name, ms), ...] in launch order."""
    buf = (lmlp_kernel_time * capacity)()
    n = ctypes.c_int(0)
    _check(lib().lora_mlp_profile_end(buf, capacity, ctypes.byref(n)), "lora_mlp_profile_end")
    return [(buf[i].name.decode(), float(buf[i].ms)) for i in range(n.value)]


def lora_mlp_mfma_probe(operands, sink, blocks: int, iters: int, stream=None):
    """One launch of the matrix-core ceiling probe (see the header)."""
    rc = lib().lora_mlp_mfma_probe(_ptr(operands), _nbytes(operands), _ptr(sink), int(blocks), int(iters),
                                   _stream(stream))
    _check(rc, "lora_mlp_mfma_probe")
