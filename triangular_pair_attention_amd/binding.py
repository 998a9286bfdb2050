"""ctypes binding of libtri_attn.so: the C ABI of include/tri_attn.h, same names.

Argument marshalling only: every step of the forward runs in the library's
HIP kernels. Pointer arguments accept an int address or any object with a
``data_ptr()`` method (torch tensors); streams accept an int handle, a torch
stream, or None (default stream). Failures raise TriAttnError; a missing
library raises at load time (there is no fallback).
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "lib", "libtri_attn.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "tri_attn.h")

TRI_ATTN_F32 = 0
TRI_ATTN_BF16 = 1
TRI_ATTN_OK = 0
TRI_ATTN_ERR_INVALID_ARG = -1
TRI_ATTN_ERR_UNSUPPORTED = -2
TRI_ATTN_ERR_WORKSPACE = -3
TRI_ATTN_ERR_HIP = -4
TRI_ATTN_ERR_OOM = -5

WEIGHT_FIELDS = ("ln_weight", "ln_bias", "w_query", "w_key", "w_value", "w_gate", "b_gate",
                 "w_bias_proj", "w_out", "b_out")


class tri_attn_config(ctypes.Structure):
    _fields_ = [
        ("pair_dim", ctypes.c_int),
        ("num_heads", ctypes.c_int),
        ("dtype", ctypes.c_int),
        ("ln_eps", ctypes.c_float),
        ("mask_fill", ctypes.c_float),
        ("ending_node", ctypes.c_int),
    ]


class tri_attn_weights(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in WEIGHT_FIELDS]


GRAD_FIELDS = ("d_pair_repr", "d_ln_weight", "d_ln_bias", "d_w_query", "d_w_key", "d_w_value", "d_w_gate",
               "d_b_gate", "d_w_bias_proj", "d_w_out", "d_b_out")


class tri_attn_grads(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in GRAD_FIELDS]


class tri_attn_workspace_layout(ctypes.Structure):
    _fields_ = [(name, ctypes.c_size_t)
                for name in ("q", "k", "vt", "g", "zm", "zmax", "kmax", "vsum", "recover_flags", "total")] + [
        ("padded_n", ctypes.c_int), ("attention_items", ctypes.c_int)
    ]


class TriAttnError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {tri_attn_strerror(code)} ({code})")


_lib = None


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load (once) and return the shared library; raise if it was not built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m triangular_pair_attention_amd.build`")
    lib = ctypes.CDLL(p)
    vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.tri_attn_create.argtypes = [ctypes.POINTER(tri_attn_config), ctypes.POINTER(tri_attn_weights), vp,
                                    ctypes.POINTER(vp)]
    lib.tri_attn_workspace_size.argtypes = [vp, i, i, ctypes.POINTER(sz)]
    lib.tri_attn_forward.argtypes = [vp, vp, vp, vp, i, i, vp, sz, vp]
    lib.tri_attn_destroy.argtypes = [vp]
    lib.tri_attn_strerror.argtypes = [i]
    lib.tri_attn_strerror.restype = ctypes.c_char_p
    lib.tri_attn_get_workspace_layout.argtypes = [vp, i, i, ctypes.POINTER(tri_attn_workspace_layout)]
    lib.tri_attn_project.argtypes = [vp, vp, vp, i, i, vp, sz, vp]
    lib.tri_attn_attend.argtypes = [vp, i, i, vp, sz, vp]
    lib.tri_attn_output.argtypes = [vp, vp, i, i, vp, sz, vp]
    lib.tri_attn_set_shift_slack.argtypes = [vp, ctypes.c_float]
    lib.tri_attn_set_alloc_fault.argtypes = [i]
    lib.tri_attn_set_backward_dz_ranges.argtypes = [vp, i]
    lib.tri_attn_onepass_workspace_size.argtypes = [vp, i, i, ctypes.POINTER(sz)]
    lib.tri_attn_forward_onepass.argtypes = [vp, vp, vp, vp, i, i, vp, sz, vp]
    lib.tri_attn_backward_workspace_size.argtypes = [vp, i, i, ctypes.POINTER(sz)]
    lib.tri_attn_backward_train.argtypes = [vp, vp, vp, vp, i, i, ctypes.c_double, ctypes.c_uint64, ctypes.c_uint32,
                                            ctypes.POINTER(tri_attn_grads), vp, sz, vp]
    lib.tri_attn_forward_noalloc.argtypes = [vp, vp, vp, vp, i, i, vp]
    lib.tri_attn_forward_train.argtypes = [vp, vp, vp, vp, vp, i, i, ctypes.c_double, ctypes.c_uint64,
                                           ctypes.c_uint32, vp, sz, vp]
    for name in ("tri_attn_create", "tri_attn_workspace_size", "tri_attn_forward", "tri_attn_destroy",
                 "tri_attn_get_workspace_layout", "tri_attn_project", "tri_attn_attend",
                 "tri_attn_output", "tri_attn_forward_train", "tri_attn_set_shift_slack",
                 "tri_attn_forward_noalloc", "tri_attn_backward_workspace_size", "tri_attn_backward_train",
                 "tri_attn_onepass_workspace_size", "tri_attn_forward_onepass", "tri_attn_set_alloc_fault",
                 "tri_attn_set_backward_dz_ranges"):
        getattr(lib, name).restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def declared_functions(header: str = HEADER_PATH) -> list:
    """Names of the functions include/tri_attn.h declares."""
    with open(header) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(tri_attn_\w+)\s*\(", text, re.M)))


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return int(x.data_ptr())
    raise TypeError(f"cannot take a device pointer from {type(x).__name__}")


def _stream(s) -> Optional[int]:
    if s is None:
        return None
    if isinstance(s, int):
        return s
    if hasattr(s, "cuda_stream"):
        return int(s.cuda_stream)
    raise TypeError(f"cannot take a stream handle from {type(s).__name__}")


def _check(code: int, where: str) -> None:
    if code != TRI_ATTN_OK:
        raise TriAttnError(code, where)


# ------------------------------------------------------------------ the C ABI, same names
def tri_attn_strerror(code: int) -> str:
    return load_library().tri_attn_strerror(int(code)).decode()


def tri_attn_create(cfg: tri_attn_config, weights: dict, stream=None) -> int:
    """weights: dict name -> pointer (see WEIGHT_FIELDS). Returns the handle."""
    w = tri_attn_weights(**{k: _ptr(weights[k]) for k in WEIGHT_FIELDS})
    h = ctypes.c_void_p()
    _check(load_library().tri_attn_create(ctypes.byref(cfg), ctypes.byref(w), _stream(stream), ctypes.byref(h)),
           "tri_attn_create")
    return h.value


def tri_attn_workspace_size(handle: int, B: int, N: int) -> int:
    n = ctypes.c_size_t()
    _check(load_library().tri_attn_workspace_size(handle, B, N, ctypes.byref(n)), "tri_attn_workspace_size")
    return n.value


def tri_attn_forward(handle: int, pair_repr, pair_mask, out, B: int, N: int, workspace, ws_bytes: int,
                     stream=None) -> None:
    _check(load_library().tri_attn_forward(handle, _ptr(pair_repr), _ptr(pair_mask), _ptr(out), B, N,
                                           _ptr(workspace), ws_bytes, _stream(stream)), "tri_attn_forward")


def tri_attn_forward_noalloc(handle: int, pair_repr, pair_mask, out, B: int, N: int, stream=None) -> None:
    _check(load_library().tri_attn_forward_noalloc(handle, _ptr(pair_repr), _ptr(pair_mask), _ptr(out), B, N,
                                                   _stream(stream)), "tri_attn_forward_noalloc")


def tri_attn_forward_train(handle: int, pair_repr, pair_mask, out, lse, B: int, N: int, dropout_rate: float,
                           seed: int, offset: int, workspace, ws_bytes: int, stream=None) -> None:
    _check(load_library().tri_attn_forward_train(handle, _ptr(pair_repr), _ptr(pair_mask), _ptr(out), _ptr(lse), B,
                                                 N, float(dropout_rate), int(seed), int(offset), _ptr(workspace),
                                                 ws_bytes, _stream(stream)), "tri_attn_forward_train")


def tri_attn_destroy(handle: Optional[int]) -> None:
    _check(load_library().tri_attn_destroy(handle), "tri_attn_destroy")


def tri_attn_get_workspace_layout(handle: int, B: int, N: int) -> tri_attn_workspace_layout:
    lay = tri_attn_workspace_layout()
    _check(load_library().tri_attn_get_workspace_layout(handle, B, N, ctypes.byref(lay)),
           "tri_attn_get_workspace_layout")
    return lay


def tri_attn_project(handle: int, pair_repr, pair_mask, B: int, N: int, workspace, ws_bytes: int,
                     stream=None) -> None:
    _check(load_library().tri_attn_project(handle, _ptr(pair_repr), _ptr(pair_mask), B, N, _ptr(workspace),
                                           ws_bytes, _stream(stream)), "tri_attn_project")


def tri_attn_attend(handle: int, B: int, N: int, workspace, ws_bytes: int, stream=None) -> None:
    _check(load_library().tri_attn_attend(handle, B, N, _ptr(workspace), ws_bytes, _stream(stream)),
           "tri_attn_attend")


def tri_attn_output(handle: int, out, B: int, N: int, workspace, ws_bytes: int, stream=None) -> None:
    _check(load_library().tri_attn_output(handle, _ptr(out), B, N, _ptr(workspace), ws_bytes, _stream(stream)),
           "tri_attn_output")


def tri_attn_set_shift_slack(handle: int, slack: float) -> None:
    _check(load_library().tri_attn_set_shift_slack(handle, float(slack)), "tri_attn_set_shift_slack")


def tri_attn_set_backward_dz_ranges(handle: int, ranges: int) -> None:
    _check(load_library().tri_attn_set_backward_dz_ranges(handle, int(ranges)), "tri_attn_set_backward_dz_ranges")


def tri_attn_set_alloc_fault(nth: int) -> None:
    """Testing hook: the next tri_attn_create fails its nth device allocation."""
    _check(load_library().tri_attn_set_alloc_fault(nth), "tri_attn_set_alloc_fault")


def tri_attn_onepass_workspace_size(handle: int, B: int, N: int) -> int:
    n = ctypes.c_size_t()
    _check(load_library().tri_attn_onepass_workspace_size(handle, B, N, ctypes.byref(n)),
           "tri_attn_onepass_workspace_size")
    return n.value


def tri_attn_forward_onepass(handle: int, pair_repr, pair_mask, out, B: int, N: int, workspace, ws_bytes: int,
                             stream=None) -> None:
    _check(load_library().tri_attn_forward_onepass(handle, _ptr(pair_repr), _ptr(pair_mask), _ptr(out), B, N,
                                                   _ptr(workspace), ws_bytes, _stream(stream)),
           "tri_attn_forward_onepass")


def tri_attn_backward_workspace_size(handle: int, B: int, N: int) -> int:
    n = ctypes.c_size_t()
    _check(load_library().tri_attn_backward_workspace_size(handle, B, N, ctypes.byref(n)),
           "tri_attn_backward_workspace_size")
    return n.value


def tri_attn_backward_train(handle: int, pair_repr, pair_mask, dy, B: int, N: int, dropout_rate: float, seed: int,
                            offset: int, grads: dict, workspace, ws_bytes: int, stream=None) -> None:
    """grads: dict name -> float32 device pointer (see GRAD_FIELDS)."""
    g = tri_attn_grads(**{k: _ptr(grads[k]) for k in GRAD_FIELDS})
    _check(load_library().tri_attn_backward_train(handle, _ptr(pair_repr), _ptr(pair_mask), _ptr(dy), B, N,
                                                  float(dropout_rate), int(seed), int(offset), ctypes.byref(g),
                                                  _ptr(workspace), ws_bytes, _stream(stream)),
           "tri_attn_backward_train")


def raw_call(name: str, *args) -> int:
    """Call an ABI function with raw ctypes arguments and return its status
    code (used by tests of the error paths)."""
    return getattr(load_library(), name)(*args)
