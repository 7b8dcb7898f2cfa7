"""Python binding of the I8_S type and mul_mat_add(_relu) (include/i8s.h), same
names as the C ABI; the functions live in the same libi2s.so as the I2_S op.

Argument marshalling only: every step runs in the library's HIP kernels.  An
I8_S tensor is a flat uint8 tensor of i8s_bytes(n) bytes (payload, then the
32-byte in-band scale slot).  No fallback: a missing library or a failed
call raises.
"""

from __future__ import annotations

import ctypes
import os
import re

import torch

from . import i2s
from .i2s import I2SError, _check, _dev, _stream

HEADER_PATH = os.path.join(os.path.dirname(i2s._PKG), "include", "i8s.h")
I8S_SCALE_SLOT = 32
I8S_MAX_IC = 133143
VARIANT_AUTO, VARIANT_PLAIN = 0, 1

_ready = False


def declared_symbols() -> list[str]:
    """Names of the functions include/i8s.h declares."""
    with open(HEADER_PATH) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^[A-Za-z_][\w \*]*?\b(i8s_\w+)\s*\(", text, flags=re.M)


def lib() -> ctypes.CDLL:
    global _ready
    L = i2s.lib()
    if not _ready:
        i64, p, sz, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
        L.i8s_bytes.restype = sz
        L.i8s_bytes.argtypes = [i64]
        L.i8s_workspace_bytes.restype = sz
        L.i8s_workspace_bytes.argtypes = []
        L.i8s_quantize.restype = ci
        L.i8s_quantize.argtypes = [p, i64, p, p, sz, p]
        L.i8s_dequantize.restype = ci
        L.i8s_dequantize.argtypes = [p, i64, p, p]
        L.i8s_mul_mat_add.restype = ci
        L.i8s_mul_mat_add.argtypes = [p, i64, i64, p, i64, p, p, p, sz, p]
        L.i8s_mul_mat_add_relu.restype = ci
        L.i8s_mul_mat_add_relu.argtypes = [p, i64, i64, p, i64, p, p, p, sz, p]
        L.i8s_mul_mat_add_ex.restype = ci
        L.i8s_mul_mat_add_ex.argtypes = [p, i64, i64, p, i64, p, ci, p, p, ci, p, sz, p]
        L.i8s_mul_mat_add_variant.restype = ci
        L.i8s_mul_mat_add_variant.argtypes = [i64, i64, i64]
        L.i8s_variants.restype = ci
        L.i8s_variants.argtypes = []
        _ready = True
    return L


def i8s_bytes(n: int) -> int:
    return int(lib().i8s_bytes(n))


def i8s_workspace_bytes() -> int:
    return int(lib().i8s_workspace_bytes())


def i8s_variants() -> int:
    return int(lib().i8s_variants())


def i8s_mul_mat_add_variant(OC: int, IC: int, N: int) -> int:
    return int(lib().i8s_mul_mat_add_variant(OC, IC, N))


def new_workspace(device) -> torch.Tensor:
    return torch.empty(i8s_workspace_bytes(), dtype=torch.uint8, device=device)


def i8s_tensor(q, scale: float, device) -> torch.Tensor:
    """An I8_S tensor on `device` holding the given int8 values (any shape,
    C order) and scale: the payload bytes, the F32 scale, 28 zero bytes (the
    layout of an I8_S tensor read from a checkpoint)."""
    import numpy as np
    q = np.ascontiguousarray(q, dtype=np.int8).reshape(-1)
    buf = np.zeros(q.size + I8S_SCALE_SLOT, dtype=np.uint8)
    buf[: q.size] = q.view(np.uint8)
    buf[q.size: q.size + 4] = np.array([scale], dtype="<f4").view(np.uint8)
    return torch.from_numpy(buf).to(device)


def _i8s_tensor(t: torch.Tensor, n: int, name: str) -> int:
    ptr = _dev(t, torch.uint8, name)
    if t.numel() < i8s_bytes(n):
        raise ValueError(f"{name} holds {t.numel()} bytes, an I8_S tensor of {n} values needs {i8s_bytes(n)}")
    return ptr


def i8s_quantize(x: torch.Tensor, out=None, workspace=None, stream=None) -> torch.Tensor:
    """I8_S bytes of the F32 tensor x (all of it, C order): one scale."""
    n = x.numel()
    out = torch.empty(i8s_bytes(n), dtype=torch.uint8, device=x.device) if out is None else out
    workspace = new_workspace(x.device) if workspace is None else workspace
    _check("i8s_quantize", lib().i8s_quantize(_dev(x, torch.float32, "x"), n, _i8s_tensor(out, n, "out"),
                                              _dev(workspace, torch.uint8, "workspace"), workspace.numel(),
                                              _stream(stream)))
    return out


def i8s_dequantize(t: torch.Tensor, n: int, y=None, stream=None) -> torch.Tensor:
    """F32 y[n] = q * s of the I8_S tensor t."""
    y = torch.empty(n, dtype=torch.float32, device=t.device) if y is None else y
    if y.numel() < n:
        raise ValueError("y too small")
    _check("i8s_dequantize", lib().i8s_dequantize(_i8s_tensor(t, n, "t"), n, _dev(y, torch.float32, "y"),
                                                  _stream(stream)))
    return y


def i8s_mul_mat_add_ex(w: torch.Tensor, OC: int, IC: int, x: torch.Tensor, N: int, bias=None, relu: bool = False,
                       out=None, dot_out=None, variant: int = VARIANT_AUTO, workspace=None, stream=None):
    """I8_S out[N][OC] of mul_mat_add (relu=False) or mul_mat_add_relu
    (relu=True); with dot_out (a tensor, or True) also the int32 acc[N][OC]."""
    dev = w.device
    out = torch.empty(i8s_bytes(N * OC), dtype=torch.uint8, device=dev) if out is None else out
    if dot_out is True:
        dot_out = torch.empty((N, OC), dtype=torch.int32, device=dev)
    if dot_out is not None and dot_out.numel() < N * OC:
        raise ValueError("dot_out too small")
    if bias is not None and bias.numel() < OC:
        raise ValueError("bias shorter than OC")
    workspace = new_workspace(dev) if workspace is None else workspace
    _check("i8s_mul_mat_add_ex", lib().i8s_mul_mat_add_ex(
        _i8s_tensor(w, OC * IC, "w"), OC, IC, _i8s_tensor(x, N * IC, "x"), N,
        None if bias is None else _dev(bias, torch.float32, "bias"), int(bool(relu)),
        _i8s_tensor(out, N * OC, "out"), None if dot_out is None else _dev(dot_out, torch.int32, "dot_out"),
        int(variant), _dev(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream)))
    return out if dot_out is None else (out, dot_out)


def i8s_mul_mat_add(w, OC: int, IC: int, x, N: int, bias=None, out=None, workspace=None, stream=None):
    """I8_S out[N][OC]: bias added, output requantized."""
    dev = w.device
    out = torch.empty(i8s_bytes(N * OC), dtype=torch.uint8, device=dev) if out is None else out
    workspace = new_workspace(dev) if workspace is None else workspace
    if bias is not None and bias.numel() < OC:
        raise ValueError("bias shorter than OC")
    _check("i8s_mul_mat_add", lib().i8s_mul_mat_add(
        _i8s_tensor(w, OC * IC, "w"), OC, IC, _i8s_tensor(x, N * IC, "x"), N,
        None if bias is None else _dev(bias, torch.float32, "bias"), _i8s_tensor(out, N * OC, "out"),
        _dev(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream)))
    return out


def i8s_mul_mat_add_relu(w, OC: int, IC: int, x, N: int, bias=None, out=None, workspace=None, stream=None):
    """I8_S out[N][OC]: bias added, ReLU, output requantized."""
    dev = w.device
    out = torch.empty(i8s_bytes(N * OC), dtype=torch.uint8, device=dev) if out is None else out
    workspace = new_workspace(dev) if workspace is None else workspace
    if bias is not None and bias.numel() < OC:
        raise ValueError("bias shorter than OC")
    _check("i8s_mul_mat_add_relu", lib().i8s_mul_mat_add_relu(
        _i8s_tensor(w, OC * IC, "w"), OC, IC, _i8s_tensor(x, N * IC, "x"), N,
        None if bias is None else _dev(bias, torch.float32, "bias"), _i8s_tensor(out, N * OC, "out"),
        _dev(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream)))
    return out


__all__ = ["I2SError", "i8s_bytes", "i8s_workspace_bytes", "i8s_variants", "i8s_mul_mat_add_variant",
           "i8s_quantize", "i8s_dequantize", "i8s_mul_mat_add", "i8s_mul_mat_add_relu", "i8s_mul_mat_add_ex"]
