"""Python access to the CPU oracle (oracle.c) for the I2_S W2A8 matmul.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg load this; the product path never does.  It shares no code
with the GPU library and imports nothing from it.

``build()`` compiles oracle.c with gcc (no fast-math, no FP contraction, so
every float operation in it is one IEEE binary32 operation).  The wrappers
take and return numpy arrays.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_DIR = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_DIR, "oracle.c")
_LIB = os.path.join(_DIR, "liboracle.so")
_CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math", "-ffp-contract=off",
           "-fno-strict-aliasing", "-Wall", "-Wextra"]

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so next to it; returns the path."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", *_CFLAGS, _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build(force=False)
        lib = ctypes.CDLL(_LIB)
        i64, p = ctypes.c_int64, ctypes.c_void_p
        lib.oracle_packed_bytes.restype = ctypes.c_size_t
        lib.oracle_packed_bytes.argtypes = [i64, i64]
        lib.oracle_pack.restype = ctypes.c_int
        lib.oracle_pack.argtypes = [p, ctypes.c_float, i64, i64, p]
        lib.oracle_weight_scale.restype = ctypes.c_float
        lib.oracle_weight_scale.argtypes = [p, i64, i64]
        lib.oracle_quantize_act.restype = None
        lib.oracle_quantize_act.argtypes = [p, i64, i64, p, p, p]
        lib.oracle_dot.restype = None
        lib.oracle_dot.argtypes = [p, i64, i64, p, i64, p]
        lib.oracle_epilogue.restype = None
        lib.oracle_epilogue.argtypes = [p, p, p, ctypes.c_float, i64, i64, p]
        lib.oracle_mul_mat.restype = ctypes.c_int
        lib.oracle_mul_mat.argtypes = [p, i64, i64, p, i64, p, p]
        lib.oracle_add_bias.restype = None
        lib.oracle_add_bias.argtypes = [p, p, i64, i64]
        lib.oracle_i8s_bytes.restype = ctypes.c_size_t
        lib.oracle_i8s_bytes.argtypes = [i64]
        lib.oracle_i8s_scale.restype = ctypes.c_float
        lib.oracle_i8s_scale.argtypes = [p, i64]
        lib.oracle_i8s_quantize.restype = None
        lib.oracle_i8s_quantize.argtypes = [p, i64, p]
        lib.oracle_i8s_dequantize.restype = None
        lib.oracle_i8s_dequantize.argtypes = [p, i64, p]
        lib.oracle_i8s_mul_mat_add.restype = ctypes.c_int
        lib.oracle_i8s_mul_mat_add.argtypes = [p, i64, i64, p, i64, p, ctypes.c_int, p, p, p]
        lib.oracle_w8a8_quantize_weight.restype = None
        lib.oracle_w8a8_quantize_weight.argtypes = [p, i64, i64, p, p]
        lib.oracle_w8a8_quantize_act.restype = None
        lib.oracle_w8a8_quantize_act.argtypes = [p, i64, i64, p, p]
        lib.oracle_w8a8_matmul.restype = None
        lib.oracle_w8a8_matmul.argtypes = [p, p, i64, p, p, i64, i64, p, p]
        lib.oracle_w8a8_mul_mat.restype = ctypes.c_int
        lib.oracle_w8a8_mul_mat.argtypes = [p, p, i64, i64, p, i64, p, p]
        _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def packed_bytes(rows: int, K: int) -> int:
    return int(_load().oracle_packed_bytes(rows, K))


def pack(w: np.ndarray, ws: float) -> np.ndarray:
    """I2_S bytes (payload then the 32-byte scale slot) of ternary w[rows][K]."""
    w = np.ascontiguousarray(w, dtype=np.int8)
    rows, K = w.shape
    out = np.empty(packed_bytes(rows, K), dtype=np.uint8)
    rc = _load().oracle_pack(_ptr(w), float(np.float32(ws)), rows, K, _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle_pack: bad shape {w.shape}")
    return out


def weight_scale(packed: np.ndarray, rows: int, K: int) -> np.float32:
    return np.float32(_load().oracle_weight_scale(_ptr(np.ascontiguousarray(packed)), rows, K))


def quantize_act(x: np.ndarray):
    """(q int8[N][K], act_scale f32[N], row_sum i32[N]) of F32 x[N][K]."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    N, K = x.shape
    q = np.empty((N, K), dtype=np.int8)
    s = np.empty(N, dtype=np.float32)
    rs = np.empty(N, dtype=np.int32)
    _load().oracle_quantize_act(_ptr(x), N, K, _ptr(q), _ptr(s), _ptr(rs))
    return q, s, rs


def dot(packed: np.ndarray, rows: int, K: int, q: np.ndarray) -> np.ndarray:
    """int32 dot[N][rows] = sum_k code*q, codes decoded from packed bytes."""
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    q = np.ascontiguousarray(q, dtype=np.int8)
    N = q.shape[0]
    assert q.shape[1] == K and packed.size >= rows * K // 4
    out = np.empty((N, rows), dtype=np.int32)
    _load().oracle_dot(_ptr(packed), rows, K, _ptr(q), N, _ptr(out))
    return out


def epilogue(dot_: np.ndarray, row_sum: np.ndarray, act_scale: np.ndarray, ws: float) -> np.ndarray:
    dot_ = np.ascontiguousarray(dot_, dtype=np.int32)
    row_sum = np.ascontiguousarray(row_sum, dtype=np.int32)
    act_scale = np.ascontiguousarray(act_scale, dtype=np.float32)
    N, rows = dot_.shape
    y = np.empty((N, rows), dtype=np.float32)
    _load().oracle_epilogue(_ptr(dot_), _ptr(row_sum), _ptr(act_scale), float(np.float32(ws)), N, rows, _ptr(y))
    return y


def mul_mat(packed: np.ndarray, rows: int, K: int, x: np.ndarray, with_dot: bool = False):
    """F32 y[N][rows] (and optionally int32 dot[N][rows]) of the whole op."""
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    x = np.ascontiguousarray(x, dtype=np.float32)
    N = x.shape[0]
    assert x.shape[1] == K
    y = np.empty((N, rows), dtype=np.float32)
    d = np.empty((N, rows), dtype=np.int32) if with_dot else None
    rc = _load().oracle_mul_mat(_ptr(packed), rows, K, _ptr(x), N, _ptr(y), _ptr(d) if with_dot else None)
    if rc != 0:
        raise ValueError(f"oracle_mul_mat failed ({rc}) for rows={rows} K={K} N={N}")
    return (y, d) if with_dot else y


def host_threads() -> int:
    """Threads for the row-sliced oracle calls: the host cores this process
    may use, at most 16."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def mul_mat_sliced(packed: np.ndarray, rows: int, K: int, x: np.ndarray, with_dot: bool = False,
                   threads: int = 0):
    """mul_mat over slices of the output features, one slice per thread.
    A row slice of the payload followed by the scale slot is itself an I2_S
    tensor (groups never straddle rows), and every output feature depends on
    its own weight row only, so the concatenated slices are mul_mat's result
    exactly; this is the same oracle call, run in parallel (ctypes releases
    the GIL) so that whole outputs of the large shapes are checked in
    seconds."""
    import concurrent.futures

    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    x = np.ascontiguousarray(x, dtype=np.float32)
    rb = K // 4
    slot = packed[rows * rb: rows * rb + 32]
    n = max(1, min(threads or host_threads(), rows))
    bounds = [rows * i // n for i in range(n + 1)]
    parts = [(a, b) for a, b in zip(bounds, bounds[1:]) if b > a]
    if len(parts) <= 1:
        return mul_mat(packed, rows, K, x, with_dot=with_dot)

    def run(ab):
        a, b = ab
        return mul_mat(np.concatenate([packed[a * rb:b * rb], slot]), b - a, K, x, with_dot=True)

    with concurrent.futures.ThreadPoolExecutor(max_workers=len(parts)) as pool:
        outs = list(pool.map(run, parts))
    y = np.concatenate([o[0] for o in outs], axis=1)
    d = np.concatenate([o[1] for o in outs], axis=1)
    return (y, d) if with_dot else y


def add_bias(y: np.ndarray, bias: np.ndarray) -> np.ndarray:
    """y[N][rows] + bias[rows], one F32 add per element (oracle_add_bias)."""
    out = np.array(y, dtype=np.float32, order="C", copy=True)
    bias = np.ascontiguousarray(bias, dtype=np.float32)
    N, rows = out.shape
    assert bias.shape[0] >= rows
    _load().oracle_add_bias(_ptr(out), _ptr(bias), N, rows)
    return out


def mul_mat_group(projs, K: int, x: np.ndarray, with_dot: bool = False):
    """Several projections of one activation: projs is a list of
    (packed, rows, bias or None); each is the whole op on the same x followed
    by its bias add.  Returns the list of y (and of dots)."""
    ys, ds = [], []
    for packed, rows, bias in projs:
        y, d = mul_mat(packed, rows, K, x, with_dot=True)
        if bias is not None:
            y = add_bias(y, bias)
        ys.append(y)
        ds.append(d)
    return (ys, ds) if with_dot else ys


def mul_mat_batched(packed: np.ndarray, rows: int, K: int, x: np.ndarray, with_dot: bool = False):
    """The op on x[B][N][K]: every batch against the same 2-D weight
    (y[B][N][rows]); each activation row is quantized on its own."""
    x = np.asarray(x, dtype=np.float32)
    outs = [mul_mat(packed, rows, K, x[b], with_dot=True) for b in range(x.shape[0])]
    y = np.stack([o[0] for o in outs]) if outs else np.zeros((0, x.shape[1], rows), np.float32)
    d = np.stack([o[1] for o in outs]) if outs else np.zeros((0, x.shape[1], rows), np.int32)
    return (y, d) if with_dot else y


# ---------------------------------------------------------------------------
# I8_S: per-tensor int8 payload, then the 32-byte in-band F32 scale slot.


def i8s_bytes(n: int) -> int:
    return int(_load().oracle_i8s_bytes(n))


def i8s_make(q: np.ndarray, scale: float) -> np.ndarray:
    """An I8_S tensor from int8 values (any shape, flattened) and a scale:
    the payload bytes, the F32 scale, 28 zero bytes."""
    q = np.ascontiguousarray(q, dtype=np.int8).reshape(-1)
    out = np.zeros(i8s_bytes(q.size), dtype=np.uint8)
    out[: q.size] = q.view(np.uint8)
    out[q.size: q.size + 4] = np.array([scale], dtype="<f4").view(np.uint8)
    return out


def i8s_payload(t: np.ndarray, n: int) -> np.ndarray:
    return np.ascontiguousarray(t[:n]).view(np.int8)


def i8s_scale(t: np.ndarray, n: int) -> np.float32:
    return np.float32(_load().oracle_i8s_scale(_ptr(np.ascontiguousarray(t, dtype=np.uint8)), n))


def i8s_quantize(x: np.ndarray) -> np.ndarray:
    """I8_S bytes of the F32 tensor x (flattened in C order)."""
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
    out = np.empty(i8s_bytes(x.size), dtype=np.uint8)
    _load().oracle_i8s_quantize(_ptr(x), x.size, _ptr(out))
    return out


def i8s_dequantize(t: np.ndarray, n: int) -> np.ndarray:
    t = np.ascontiguousarray(t, dtype=np.uint8)
    assert t.size >= n + 4
    y = np.empty(n, dtype=np.float32)
    _load().oracle_i8s_dequantize(_ptr(t), n, _ptr(y))
    return y


def i8s_mul_mat_add(w: np.ndarray, OC: int, IC: int, x: np.ndarray, N: int, bias=None, relu: bool = False,
                    with_dot: bool = False, with_f: bool = False):
    """I8_S out[N][OC] (bytes, payload then scale slot) of mul_mat_add, or of
    mul_mat_add_relu when relu is set; optionally also int32 acc[N][OC] and
    the F32 values before requantization."""
    w = np.ascontiguousarray(w, dtype=np.uint8)
    x = np.ascontiguousarray(x, dtype=np.uint8)
    assert w.size >= OC * IC + 4 and x.size >= N * IC + 4
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    if b is not None:
        assert b.size >= OC
    out = np.empty(i8s_bytes(N * OC), dtype=np.uint8)
    d = np.empty((N, OC), dtype=np.int32)
    f = np.empty((N, OC), dtype=np.float32)
    rc = _load().oracle_i8s_mul_mat_add(_ptr(w), OC, IC, _ptr(x), N, None if b is None else _ptr(b), int(bool(relu)),
                                        _ptr(out), _ptr(d), _ptr(f))
    if rc != 0:
        raise MemoryError("oracle_i8s_mul_mat_add: allocation failed")
    res = [out]
    if with_dot:
        res.append(d)
    if with_f:
        res.append(f)
    return res[0] if len(res) == 1 else tuple(res)


# ---------------------------------------------------------------------------
# Per-channel W8A8 (the NPU page's scheme): int8 weights with per-channel
# scales, per-row int8 activations, d = aScale * bScale * C.


def w8a8_quantize_weight(w: np.ndarray):
    """(q int8[OC][K], scale f32[OC]) of F32 w[OC][K]."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    OC, K = w.shape
    q = np.empty((OC, K), dtype=np.int8)
    s = np.empty(OC, dtype=np.float32)
    _load().oracle_w8a8_quantize_weight(_ptr(w), OC, K, _ptr(q), _ptr(s))
    return q, s


def w8a8_quantize_act(x: np.ndarray):
    """(q int8[M][K], scale f32[M]) of F32 x[M][K]."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    M, K = x.shape
    q = np.empty((M, K), dtype=np.int8)
    s = np.empty(M, dtype=np.float32)
    _load().oracle_w8a8_quantize_act(_ptr(x), M, K, _ptr(q), _ptr(s))
    return q, s


def w8a8_matmul(a: np.ndarray, ascale: np.ndarray, w: np.ndarray, wscale: np.ndarray, with_c: bool = False):
    a = np.ascontiguousarray(a, dtype=np.int8)
    w = np.ascontiguousarray(w, dtype=np.int8)
    ascale = np.ascontiguousarray(ascale, dtype=np.float32)
    wscale = np.ascontiguousarray(wscale, dtype=np.float32)
    M, K = a.shape
    OC = w.shape[0]
    assert w.shape[1] == K
    d = np.empty((M, OC), dtype=np.float32)
    c = np.empty((M, OC), dtype=np.int32)
    _load().oracle_w8a8_matmul(_ptr(a), _ptr(ascale), M, _ptr(w), _ptr(wscale), OC, K, _ptr(d), _ptr(c))
    return (d, c) if with_c else d


def w8a8_mul_mat(wq: np.ndarray, wscale: np.ndarray, x: np.ndarray, with_c: bool = False):
    """F32 d[M][OC] of the whole op on F32 x[M][K] (activations quantized here)."""
    wq = np.ascontiguousarray(wq, dtype=np.int8)
    wscale = np.ascontiguousarray(wscale, dtype=np.float32)
    x = np.ascontiguousarray(x, dtype=np.float32)
    M, K = x.shape
    OC = wq.shape[0]
    d = np.empty((M, OC), dtype=np.float32)
    c = np.empty((M, OC), dtype=np.int32)
    rc = _load().oracle_w8a8_mul_mat(_ptr(wq), _ptr(wscale), OC, K, _ptr(x), M, _ptr(d), _ptr(c))
    if rc != 0:
        raise MemoryError("oracle_w8a8_mul_mat: allocation failed")
    return (d, c) if with_c else d


def _split_rows(M: int, threads: int):
    n = max(1, min(threads or host_threads(), M))
    bounds = [M * i // n for i in range(n + 1)]
    return [(a, b) for a, b in zip(bounds, bounds[1:]) if b > a]


def w8a8_matmul_sliced(a: np.ndarray, ascale: np.ndarray, w: np.ndarray, wscale: np.ndarray,
                       with_c: bool = False, threads: int = 0):
    """w8a8_matmul over slices of the activation rows, one slice per thread:
    each output row depends on its own activation row only, so the stacked
    slices are the whole result exactly (the same oracle call, in parallel)."""
    import concurrent.futures

    parts = _split_rows(a.shape[0], threads)
    if len(parts) <= 1:
        return w8a8_matmul(a, ascale, w, wscale, with_c=with_c)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(parts)) as pool:
        outs = list(pool.map(lambda ab: w8a8_matmul(a[ab[0]:ab[1]], ascale[ab[0]:ab[1]], w, wscale, with_c=True),
                             parts))
    d = np.concatenate([o[0] for o in outs], axis=0)
    c = np.concatenate([o[1] for o in outs], axis=0)
    return (d, c) if with_c else d


def w8a8_mul_mat_sliced(wq: np.ndarray, wscale: np.ndarray, x: np.ndarray, with_c: bool = False, threads: int = 0):
    """w8a8_mul_mat over slices of the activation rows (each row is quantized
    on its own), one slice per thread."""
    import concurrent.futures

    parts = _split_rows(x.shape[0], threads)
    if len(parts) <= 1:
        return w8a8_mul_mat(wq, wscale, x, with_c=with_c)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(parts)) as pool:
        outs = list(pool.map(lambda ab: w8a8_mul_mat(wq, wscale, x[ab[0]:ab[1]], with_c=True), parts))
    d = np.concatenate([o[0] for o in outs], axis=0)
    c = np.concatenate([o[1] for o in outs], axis=0)
    return (d, c) if with_c else d
