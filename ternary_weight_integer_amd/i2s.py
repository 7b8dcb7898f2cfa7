"""Python binding of the gfx950 I2_S library (libi2s.so), same names as the C ABI.

Argument marshalling only: every step of the op runs in the library's HIP
kernels.  PyTorch supplies device memory and the current stream.  There is no
fallback: if libi2s.so is missing or a call fails, an exception is raised.
"""

from __future__ import annotations

import ctypes
import os
import re

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libi2s.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "i2s.h")

I2S_OK = 0
I2S_EINVAL = 1
I2S_EALIGN = 2
I2S_EWORKSPACE = 3
I2S_EHIP = 4
I2S_ERANGE = 5
I2S_EKERNEL = 6
I2S_ESCRATCH = 7

KERNEL_AUTO, KERNEL_GEMV, KERNEL_GEMM = 0, 1, 2

_lib = None


class I2SError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {i2s_strerror(status)} (status {status})")


class I2SProj(ctypes.Structure):
    """One projection of a grouped call (struct i2s_proj of include/i2s.h)."""
    _fields_ = [("packed", ctypes.c_void_p), ("rows", ctypes.c_int64), ("bias", ctypes.c_void_p),
                ("y", ctypes.c_void_p), ("dot_out", ctypes.c_void_p)]


I2S_GROUP_MAX = 8


def declared_symbols() -> list[str]:
    """Names of the functions include/i2s.h declares."""
    with open(HEADER_PATH) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^[A-Za-z_][\w \*]*?\b(i2s_\w+)\s*\(", text, flags=re.M)


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it first (python -m ternary_weight_integer_amd.build); "
                "there is no fallback path")
        L = ctypes.CDLL(LIB_PATH)
        i64, p, sz, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
        L.i2s_packed_bytes.restype = sz
        L.i2s_packed_bytes.argtypes = [i64, i64]
        L.i2s_act_workspace_bytes.restype = sz
        L.i2s_act_workspace_bytes.argtypes = [i64, i64]
        L.i2s_pack.restype = ci
        L.i2s_pack.argtypes = [p, ctypes.c_float, i64, i64, p, p]
        L.i2s_quantize_act.restype = ci
        L.i2s_quantize_act.argtypes = [p, i64, i64, p, p, p, p]
        L.i2s_mul_mat.restype = ci
        L.i2s_mul_mat.argtypes = [p, i64, i64, p, i64, p, sz, p, p, p]
        L.i2s_mul_mat_ex.restype = ci
        L.i2s_mul_mat_ex.argtypes = [p, i64, i64, p, i64, p, sz, p, p, ci, ci, p]
        L.i2s_quantize_act_ws.restype = ci
        L.i2s_quantize_act_ws.argtypes = [p, i64, i64, p, sz, p]
        L.i2s_mul_mat_ws.restype = ci
        L.i2s_mul_mat_ws.argtypes = [p, i64, i64, i64, p, sz, p, p, ci, ci, p]
        L.i2s_mul_mat_kernel.restype = ci
        L.i2s_mul_mat_kernel.argtypes = [i64, i64, i64]
        L.i2s_mul_mat_variant.restype = ci
        L.i2s_mul_mat_variant.argtypes = [i64, i64, i64]
        L.i2s_mul_mat_group.restype = ci
        L.i2s_mul_mat_group.argtypes = [ctypes.POINTER(I2SProj), ci, i64, p, i64, p, sz, p]
        L.i2s_mul_mat_group_ex.restype = ci
        L.i2s_mul_mat_group_ex.argtypes = [ctypes.POINTER(I2SProj), ci, i64, p, i64, p, sz, ci, ci, p]
        L.i2s_mul_mat_batched.restype = ci
        L.i2s_mul_mat_batched.argtypes = [p, i64, i64, p, i64, i64, i64, i64, p, sz, p, i64, i64, p, p]
        L.i2s_kernel_variants.restype = ci
        L.i2s_kernel_variants.argtypes = [ci]
        L.i2s_strerror.restype = ctypes.c_char_p
        L.i2s_strerror.argtypes = [ci]
        L.i2s_mul_mat_noalloc.restype = ci
        L.i2s_mul_mat_noalloc.argtypes = [p, i64, i64, p, i64, p, p, p]
        L.i2s_noalloc_scratch_bytes.restype = sz
        L.i2s_noalloc_scratch_bytes.argtypes = []
        _lib = L
    return _lib


def i2s_strerror(status: int) -> str:
    return lib().i2s_strerror(status).decode()


def i2s_packed_bytes(rows: int, K: int) -> int:
    return int(lib().i2s_packed_bytes(rows, K))


def i2s_act_workspace_bytes(N: int, K: int) -> int:
    return int(lib().i2s_act_workspace_bytes(N, K))


KERNEL_FUSED = 3
KERNEL_SKINNY = 4


def i2s_mul_mat_kernel(rows: int, K: int, N: int) -> int:
    """Kernel id i2s_mul_mat launches for this shape (1 GEMV, 2 GEMM, 3 fused, 4 skinny MFMA)."""
    k = int(lib().i2s_mul_mat_kernel(rows, K, N))
    if k < 0:
        raise I2SError("i2s_mul_mat_kernel", -k)
    return k


def i2s_mul_mat_variant(rows: int, K: int, N: int) -> int:
    """Tile configuration (1-based) of that kernel the automatic choice uses."""
    v = int(lib().i2s_mul_mat_variant(rows, K, N))
    if v < 0:
        raise I2SError("i2s_mul_mat_variant", -v)
    return v


def i2s_kernel_variants(kernel: int) -> int:
    return int(lib().i2s_kernel_variants(kernel))


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dev(t: torch.Tensor, dtype, name: str) -> int:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _check(fn: str, status: int):
    if status != I2S_OK:
        raise I2SError(fn, status)


def i2s_pack(w: torch.Tensor, weight_scale: float, packed: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Pack ternary int8 w[rows][K] with its F32 scale into I2_S bytes."""
    rows, K = w.shape
    nbytes = i2s_packed_bytes(rows, K)
    if nbytes == 0:
        raise I2SError("i2s_pack", I2S_EALIGN)
    if packed is None:
        packed = torch.empty(nbytes, dtype=torch.uint8, device=w.device)
    elif packed.numel() < nbytes:
        raise ValueError(f"packed holds {packed.numel()} bytes, needs {nbytes}")
    _check("i2s_pack", lib().i2s_pack(_dev(w, torch.int8, "w"), float(weight_scale), rows, K,
                                      _dev(packed, torch.uint8, "packed"), _stream(stream)))
    return packed


def i2s_quantize_act(x: torch.Tensor, q=None, act_scale=None, row_sum=None, stream=None):
    """(q int8[N][K], act_scale f32[N], row_sum i32[N]) of F32 x[N][K]."""
    N, K = x.shape
    dev = x.device
    q = torch.empty((N, K), dtype=torch.int8, device=dev) if q is None else q
    act_scale = torch.empty(N, dtype=torch.float32, device=dev) if act_scale is None else act_scale
    row_sum = torch.empty(N, dtype=torch.int32, device=dev) if row_sum is None else row_sum
    if q.numel() < N * K or act_scale.numel() < N or row_sum.numel() < N:
        raise ValueError("output buffers too small")
    _check("i2s_quantize_act", lib().i2s_quantize_act(
        _dev(x, torch.float32, "x"), N, K, _dev(q, torch.int8, "q"), _dev(act_scale, torch.float32, "act_scale"),
        _dev(row_sum, torch.int32, "row_sum"), _stream(stream)))
    return q, act_scale, row_sum


def new_workspace(N: int, K: int, device) -> torch.Tensor:
    return torch.empty(max(i2s_act_workspace_bytes(N, K), 1), dtype=torch.uint8, device=device)


def i2s_mul_mat_ex(packed: torch.Tensor, rows: int, K: int, x: torch.Tensor, workspace=None, y=None,
                   dot_out=None, kernel: int = KERNEL_AUTO, variant: int = 0, stream=None):
    """y[N][rows] F32 (and the int32 dot if dot_out is a tensor or True)."""
    N = x.shape[0]
    if x.dim() != 2 or x.shape[1] != K:
        raise ValueError(f"x must be [N][{K}], got {tuple(x.shape)}")
    if packed.numel() < i2s_packed_bytes(rows, K):
        raise ValueError("packed tensor smaller than i2s_packed_bytes(rows, K)")
    dev = x.device
    workspace = new_workspace(N, K, dev) if workspace is None else workspace
    y = torch.empty((N, rows), dtype=torch.float32, device=dev) if y is None else y
    if y.numel() < N * rows:
        raise ValueError("y too small")
    want_dot = dot_out is not None and dot_out is not False
    if dot_out is True:
        dot_out = torch.empty((N, rows), dtype=torch.int32, device=dev)
    dptr = _dev(dot_out, torch.int32, "dot_out") if want_dot else None
    if want_dot and dot_out.numel() < N * rows:
        raise ValueError("dot_out too small")
    _check("i2s_mul_mat_ex", lib().i2s_mul_mat_ex(
        _dev(packed, torch.uint8, "packed"), rows, K, _dev(x, torch.float32, "x"), N,
        _dev(workspace, torch.uint8, "workspace"), workspace.numel(), _dev(y, torch.float32, "y"), dptr,
        int(kernel), int(variant), _stream(stream)))
    return (y, dot_out) if want_dot else y


def i2s_mul_mat(packed: torch.Tensor, rows: int, K: int, x: torch.Tensor, workspace=None, y=None, dot_out=None,
                stream=None):
    """The I2_S matmul with the library's automatic kernel choice
    (i2s_mul_mat_kernel / i2s_mul_mat_variant report it): for N <= 3 at
    K <= 9216 one fused quantize + v_dot4 GEMV launch; otherwise a quantize
    launch, then the v_dot4 GEMV (N = 1, or N = 2 at K <= 2048), the skinny
    int8-MFMA kernel (N <= 32, or N <= 64 with at most 4096 weight rows),
    else the int8-MFMA GEMM."""
    N = x.shape[0]
    if x.dim() != 2 or x.shape[1] != K:
        raise ValueError(f"x must be [N][{K}], got {tuple(x.shape)}")
    if packed.numel() < i2s_packed_bytes(rows, K):
        raise ValueError("packed tensor smaller than i2s_packed_bytes(rows, K)")
    dev = x.device
    workspace = new_workspace(N, K, dev) if workspace is None else workspace
    y = torch.empty((N, rows), dtype=torch.float32, device=dev) if y is None else y
    if y.numel() < N * rows:
        raise ValueError("y too small")
    want_dot = dot_out is not None and dot_out is not False
    if dot_out is True:
        dot_out = torch.empty((N, rows), dtype=torch.int32, device=dev)
    dptr = _dev(dot_out, torch.int32, "dot_out") if want_dot else None
    _check("i2s_mul_mat", lib().i2s_mul_mat(
        _dev(packed, torch.uint8, "packed"), rows, K, _dev(x, torch.float32, "x"), N,
        _dev(workspace, torch.uint8, "workspace"), workspace.numel(), _dev(y, torch.float32, "y"), dptr,
        _stream(stream)))
    return (y, dot_out) if want_dot else y


def i2s_noalloc_scratch_bytes() -> int:
    return int(lib().i2s_noalloc_scratch_bytes())


def i2s_mul_mat_noalloc(packed: torch.Tensor, rows: int, K: int, x: torch.Tensor, y: torch.Tensor,
                        dot_out=None, stream=None):
    """i2s_mul_mat with the library's fixed device array as its workspace:
    the caller passes every buffer (y and, if wanted, dot_out), so nothing is
    allocated on the way in or inside."""
    N = x.shape[0]
    if x.dim() != 2 or x.shape[1] != K:
        raise ValueError(f"x must be [N][{K}], got {tuple(x.shape)}")
    if packed.numel() < i2s_packed_bytes(rows, K):
        raise ValueError("packed tensor smaller than i2s_packed_bytes(rows, K)")
    if y.numel() < N * rows or (dot_out is not None and dot_out.numel() < N * rows):
        raise ValueError("y or dot_out too small")
    dptr = _dev(dot_out, torch.int32, "dot_out") if dot_out is not None else None
    _check("i2s_mul_mat_noalloc", lib().i2s_mul_mat_noalloc(
        _dev(packed, torch.uint8, "packed"), rows, K, _dev(x, torch.float32, "x"), N, _dev(y, torch.float32, "y"),
        dptr, _stream(stream)))
    return y


def i2s_quantize_act_ws(x: torch.Tensor, workspace: torch.Tensor, stream=None) -> torch.Tensor:
    """Quantize F32 x[N][K] into the matmul workspace (private layout)."""
    N, K = x.shape
    _check("i2s_quantize_act_ws", lib().i2s_quantize_act_ws(
        _dev(x, torch.float32, "x"), N, K, _dev(workspace, torch.uint8, "workspace"), workspace.numel(),
        _stream(stream)))
    return workspace


def i2s_mul_mat_ws(packed: torch.Tensor, rows: int, K: int, N: int, workspace: torch.Tensor, y=None, dot_out=None,
                   kernel: int = KERNEL_AUTO, variant: int = 0, stream=None):
    """Contraction + epilogue against activations already in `workspace`."""
    if packed.numel() < i2s_packed_bytes(rows, K):
        raise ValueError("packed tensor smaller than i2s_packed_bytes(rows, K)")
    dev = packed.device
    y = torch.empty((N, rows), dtype=torch.float32, device=dev) if y is None else y
    if y.numel() < N * rows:
        raise ValueError("y too small")
    want_dot = dot_out is not None and dot_out is not False
    if dot_out is True:
        dot_out = torch.empty((N, rows), dtype=torch.int32, device=dev)
    dptr = _dev(dot_out, torch.int32, "dot_out") if want_dot else None
    _check("i2s_mul_mat_ws", lib().i2s_mul_mat_ws(
        _dev(packed, torch.uint8, "packed"), rows, K, N, _dev(workspace, torch.uint8, "workspace"),
        workspace.numel(), _dev(y, torch.float32, "y"), dptr, int(kernel), int(variant), _stream(stream)))
    return (y, dot_out) if want_dot else y


def i2s_mul_mat_group(weights, K: int, x: torch.Tensor, biases=None, workspace=None, dot_out: bool = False,
                      kernel: int = KERNEL_AUTO, variant: int = 0, stream=None, ys=None):
    """Several projections of one activation x[N][K]: weights is a list of
    (packed tensor, rows); biases a matching list of F32 [rows] tensors or
    None; ys optional preallocated outputs.  Returns the list of y[N][rows]
    (and of the int32 dots if dot_out)."""
    N = x.shape[0]
    if x.dim() != 2 or x.shape[1] != K:
        raise ValueError(f"x must be [N][{K}], got {tuple(x.shape)}")
    count = len(weights)
    if biases is None:
        biases = [None] * count
    if len(biases) != count:
        raise ValueError("one bias entry (or None) per projection")
    dev = x.device
    workspace = new_workspace(N, K, dev) if workspace is None else workspace
    projs = (I2SProj * max(count, 1))()
    outs, dots = [], []
    for i, ((packed, rows), b) in enumerate(zip(weights, biases)):
        if packed.numel() < i2s_packed_bytes(rows, K):
            raise ValueError(f"projection {i}: packed tensor smaller than i2s_packed_bytes(rows, K)")
        y = torch.empty((N, rows), dtype=torch.float32, device=dev) if ys is None else ys[i]
        if y.numel() < N * rows:
            raise ValueError(f"projection {i}: y too small")
        d = torch.empty((N, rows), dtype=torch.int32, device=dev) if dot_out else None
        if b is not None and b.numel() < rows:
            raise ValueError(f"projection {i}: bias shorter than rows")
        projs[i] = I2SProj(_dev(packed, torch.uint8, "packed"), rows,
                           _dev(b, torch.float32, "bias") if b is not None else None,
                           _dev(y, torch.float32, "y"), _dev(d, torch.int32, "dot_out") if dot_out else None)
        outs.append(y)
        dots.append(d)
    _check("i2s_mul_mat_group_ex", lib().i2s_mul_mat_group_ex(
        projs, count, K, _dev(x, torch.float32, "x"), N, _dev(workspace, torch.uint8, "workspace"),
        workspace.numel(), int(kernel), int(variant), _stream(stream)))
    return (outs, dots) if dot_out else outs


def i2s_mul_mat_batched(packed: torch.Tensor, rows: int, K: int, x: torch.Tensor, workspace=None, y=None,
                        dot_out=None, stream=None):
    """The op on a 3-D activation x[B][N][K] (any strides whose innermost is 1):
    y[B][N][rows] (allocated, or a given view with innermost stride 1), and
    the int32 dots (same strides as y) if dot_out is a tensor or True."""
    if x.dim() != 3 or x.shape[2] != K or x.stride(2) != 1:
        raise ValueError(f"x must be [B][N][{K}] with unit innermost stride, got {tuple(x.shape)}")
    if x.dtype != torch.float32 or not x.is_cuda:
        raise TypeError("x must be a float32 CUDA (HIP) tensor")
    B, N = x.shape[0], x.shape[1]
    if packed.numel() < i2s_packed_bytes(rows, K):
        raise ValueError("packed tensor smaller than i2s_packed_bytes(rows, K)")
    dev = x.device
    workspace = new_workspace(N * B, K, dev) if workspace is None else workspace
    y = torch.empty((B, N, rows), dtype=torch.float32, device=dev) if y is None else y
    if y.dim() != 3 or tuple(y.shape) != (B, N, rows) or y.stride(2) != 1 or y.dtype != torch.float32:
        raise ValueError(f"y must be float32 [B][N][{rows}] with unit innermost stride")
    want_dot = dot_out is not None and dot_out is not False
    if dot_out is True:
        dot_out = torch.empty_strided(y.shape, y.stride(), dtype=torch.int32, device=dev)
    if want_dot and (dot_out.stride() != y.stride() or dot_out.dtype != torch.int32):
        raise ValueError("dot_out must be int32 with y's strides")
    _check("i2s_mul_mat_batched", lib().i2s_mul_mat_batched(
        _dev(packed, torch.uint8, "packed"), rows, K, x.data_ptr(), N, B, x.stride(1), x.stride(0),
        _dev(workspace, torch.uint8, "workspace"), workspace.numel(), y.data_ptr(), y.stride(1), y.stride(0),
        dot_out.data_ptr() if want_dot else None, _stream(stream)))
    return (y, dot_out) if want_dot else y
