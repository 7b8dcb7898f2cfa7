"""Python binding of the per-channel W8A8 matmul (include/w8a8.h), same names
as the C ABI; the functions live in the same libi2s.so.

Argument marshalling only: every step runs in the library's HIP kernels.  No
fallback: a missing library or a failed call raises.
"""

from __future__ import annotations

import ctypes
import os
import re

import torch

from . import i2s
from .i2s import I2SError, _check, _dev, _stream

HEADER_PATH = os.path.join(os.path.dirname(i2s._PKG), "include", "w8a8.h")

_ready = False


def declared_symbols() -> list[str]:
    """Names of the functions include/w8a8.h declares."""
    with open(HEADER_PATH) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^[A-Za-z_][\w \*]*?\b(w8a8_\w+)\s*\(", text, flags=re.M)


def lib() -> ctypes.CDLL:
    global _ready
    L = i2s.lib()
    if not _ready:
        i64, p, sz, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
        L.w8a8_act_workspace_bytes.restype = sz
        L.w8a8_act_workspace_bytes.argtypes = [i64, i64]
        L.w8a8_quantize_weight.restype = ci
        L.w8a8_quantize_weight.argtypes = [p, i64, i64, p, p, p]
        L.w8a8_quantize_act.restype = ci
        L.w8a8_quantize_act.argtypes = [p, i64, i64, p, p, p]
        L.w8a8_matmul.restype = ci
        L.w8a8_matmul.argtypes = [p, p, i64, i64, p, p, i64, p, p, ci, p]
        L.w8a8_mul_mat.restype = ci
        L.w8a8_mul_mat.argtypes = [p, p, i64, i64, p, i64, p, sz, p, p]
        L.w8a8_mul_mat_ex.restype = ci
        L.w8a8_mul_mat_ex.argtypes = [p, p, i64, i64, p, i64, p, sz, p, p, ci, p]
        L.w8a8_mul_mat_variant.restype = ci
        L.w8a8_mul_mat_variant.argtypes = [i64, i64, i64]
        L.w8a8_variants.restype = ci
        L.w8a8_variants.argtypes = []
        _ready = True
    return L


def w8a8_act_workspace_bytes(M: int, K: int) -> int:
    return int(lib().w8a8_act_workspace_bytes(M, K))


def w8a8_variants() -> int:
    return int(lib().w8a8_variants())


def w8a8_mul_mat_variant(OC: int, K: int, M: int) -> int:
    return int(lib().w8a8_mul_mat_variant(OC, K, M))


def new_workspace(M: int, K: int, device) -> torch.Tensor:
    return torch.empty(max(w8a8_act_workspace_bytes(M, K), 1), dtype=torch.uint8, device=device)


def _rows(fn: str, t: torch.Tensor, q=None, scale=None, stream=None):
    rows, K = t.shape
    q = torch.empty((rows, K), dtype=torch.int8, device=t.device) if q is None else q
    scale = torch.empty(rows, dtype=torch.float32, device=t.device) if scale is None else scale
    if q.numel() < rows * K or scale.numel() < rows:
        raise ValueError("output buffers too small")
    _check(fn, getattr(lib(), fn)(_dev(t, torch.float32, "x"), rows, K, _dev(q, torch.int8, "q"),
                                  _dev(scale, torch.float32, "scale"), _stream(stream)))
    return q, scale


def w8a8_quantize_weight(w: torch.Tensor, wq=None, wscale=None, stream=None):
    """(int8 wq[OC][K], F32 wscale[OC]) of F32 w[OC][K], per output channel."""
    return _rows("w8a8_quantize_weight", w, wq, wscale, stream)


def w8a8_quantize_act(x: torch.Tensor, q=None, ascale=None, stream=None):
    """(int8 q[M][K], F32 ascale[M]) of F32 x[M][K], per row."""
    return _rows("w8a8_quantize_act", x, q, ascale, stream)


def w8a8_matmul(wq: torch.Tensor, wscale: torch.Tensor, aq: torch.Tensor, ascale: torch.Tensor, y=None,
                dot_out=None, variant: int = 0, stream=None):
    """F32 y[M][OC] (and the int32 product if dot_out is a tensor or True)."""
    OC, K = wq.shape
    M = aq.shape[0]
    if aq.shape[1] != K:
        raise ValueError("K mismatch")
    dev = wq.device
    y = torch.empty((M, OC), dtype=torch.float32, device=dev) if y is None else y
    if dot_out is True:
        dot_out = torch.empty((M, OC), dtype=torch.int32, device=dev)
    _check("w8a8_matmul", lib().w8a8_matmul(
        _dev(wq, torch.int8, "wq"), _dev(wscale, torch.float32, "wscale"), OC, K, _dev(aq, torch.int8, "aq"),
        _dev(ascale, torch.float32, "ascale"), M, _dev(y, torch.float32, "y"),
        None if dot_out is None else _dev(dot_out, torch.int32, "dot_out"), int(variant), _stream(stream)))
    return y if dot_out is None else (y, dot_out)


def w8a8_mul_mat_ex(wq: torch.Tensor, wscale: torch.Tensor, x: torch.Tensor, workspace=None, y=None, dot_out=None,
                    variant: int = 0, stream=None):
    """The whole op on F32 x[M][K]: quantize the rows, contract, dequantize
    (one launch for 1 <= M <= 4: variant 11)."""
    OC, K = wq.shape
    M = x.shape[0]
    if x.dim() != 2 or x.shape[1] != K:
        raise ValueError(f"x must be [M][{K}]")
    dev = x.device
    workspace = new_workspace(M, K, dev) if workspace is None else workspace
    y = torch.empty((M, OC), dtype=torch.float32, device=dev) if y is None else y
    if dot_out is True:
        dot_out = torch.empty((M, OC), dtype=torch.int32, device=dev)
    _check("w8a8_mul_mat_ex", lib().w8a8_mul_mat_ex(
        _dev(wq, torch.int8, "wq"), _dev(wscale, torch.float32, "wscale"), OC, K, _dev(x, torch.float32, "x"), M,
        _dev(workspace, torch.uint8, "workspace"), workspace.numel(), _dev(y, torch.float32, "y"),
        None if dot_out is None else _dev(dot_out, torch.int32, "dot_out"), int(variant), _stream(stream)))
    return y if dot_out is None else (y, dot_out)


def w8a8_mul_mat(wq: torch.Tensor, wscale: torch.Tensor, x: torch.Tensor, workspace=None, y=None, stream=None):
    OC, K = wq.shape
    M = x.shape[0]
    if x.dim() != 2 or x.shape[1] != K:
        raise ValueError(f"x must be [M][{K}]")
    dev = x.device
    workspace = new_workspace(M, K, dev) if workspace is None else workspace
    y = torch.empty((M, OC), dtype=torch.float32, device=dev) if y is None else y
    _check("w8a8_mul_mat", lib().w8a8_mul_mat(
        _dev(wq, torch.int8, "wq"), _dev(wscale, torch.float32, "wscale"), OC, K, _dev(x, torch.float32, "x"), M,
        _dev(workspace, torch.uint8, "workspace"), workspace.numel(), _dev(y, torch.float32, "y"), _stream(stream)))
    return y


__all__ = ["w8a8_variants", "I2SError", "w8a8_act_workspace_bytes", "w8a8_mul_mat_variant", "w8a8_quantize_weight",
           "w8a8_quantize_act", "w8a8_matmul", "w8a8_mul_mat", "w8a8_mul_mat_ex"]
