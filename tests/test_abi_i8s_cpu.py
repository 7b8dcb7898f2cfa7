"""CPU-side checks of the I8_S part of the C ABI (include/i8s.h): every
declared symbol is exported, the size queries, the automatic variant choice,
and the host-side argument checks (these calls return before any launch)."""

from __future__ import annotations

import ctypes

import pytest

from ternary_weight_integer_amd import i2s, i8s

FAKE = 1 << 20      # 16- and 256-byte aligned, never dereferenced here
FAKE_ODD = FAKE + 4  # 4- but not 16-byte aligned


def test_every_declared_symbol_is_exported():
    names = i8s.declared_symbols()
    assert set(names) >= {"i8s_bytes", "i8s_workspace_bytes", "i8s_quantize", "i8s_dequantize", "i8s_mul_mat_add",
                          "i8s_mul_mat_add_relu", "i8s_mul_mat_add_ex", "i8s_mul_mat_add_variant", "i8s_variants"}
    raw = ctypes.CDLL(i2s.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n


def test_sizes_and_variants():
    assert i8s.i8s_bytes(0) == 32
    assert i8s.i8s_bytes(1000) == 1032
    assert i8s.i8s_bytes(-5) == 0
    assert i8s.i8s_workspace_bytes() == 4096
    assert i8s.i8s_variants() >= 2
    # IC not a multiple of 16 takes the plain kernel; MFMA tiles otherwise.
    assert i8s.i8s_mul_mat_add_variant(128, 7, 1000) == 1
    assert i8s.i8s_mul_mat_add_variant(128, 24, 1000) == 1
    for shape in [(128, 32, 96000), (1024, 256, 6000), (2048, 8192, 30), (1536, 1536, 30)]:
        assert 2 <= i8s.i8s_mul_mat_add_variant(*shape) <= i8s.i8s_variants()


def _mm(w=FAKE, OC=64, IC=64, x=FAKE, N=64, bias=None, relu=0, out=FAKE, dot=None, variant=0, ws=FAKE,
        ws_bytes=4096):
    return i8s.lib().i8s_mul_mat_add_ex(w, OC, IC, x, N, bias, relu, out, dot, variant, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(w=None), i2s.I2S_EINVAL),
    (dict(x=None), i2s.I2S_EINVAL),
    (dict(out=None), i2s.I2S_EINVAL),
    (dict(OC=-1), i2s.I2S_EINVAL),
    (dict(IC=-1), i2s.I2S_EINVAL),
    (dict(N=-1), i2s.I2S_EINVAL),
    (dict(w=FAKE_ODD), i2s.I2S_EINVAL),
    (dict(out=FAKE + 8), i2s.I2S_EINVAL),
    (dict(bias=FAKE + 2), i2s.I2S_EINVAL),
    (dict(dot=FAKE + 1), i2s.I2S_EINVAL),
    (dict(IC=133144), i2s.I2S_ERANGE),
    (dict(OC=1 << 20, IC=4096), i2s.I2S_ERANGE),
    (dict(N=1 << 16, OC=1 << 15), i2s.I2S_ERANGE),
    (dict(ws=None), i2s.I2S_EWORKSPACE),
    (dict(ws=FAKE + 16), i2s.I2S_EWORKSPACE),
    (dict(ws_bytes=4095), i2s.I2S_EWORKSPACE),
    (dict(variant=-1), i2s.I2S_EKERNEL),
    (dict(variant=99), i2s.I2S_EKERNEL),
    (dict(IC=40, variant=2), i2s.I2S_EKERNEL),
])
def test_mul_mat_add_rejects_on_host(kw, expect):
    assert _mm(**kw) == expect


def test_quantize_and_dequantize_reject_on_host():
    L = i8s.lib()
    assert L.i8s_quantize(None, 16, FAKE, FAKE, 4096, None) == i2s.I2S_EINVAL
    assert L.i8s_quantize(FAKE, -1, FAKE, FAKE, 4096, None) == i2s.I2S_EINVAL
    assert L.i8s_quantize(FAKE_ODD, 16, FAKE, FAKE, 4096, None) == i2s.I2S_EINVAL
    assert L.i8s_quantize(FAKE, 16, FAKE, FAKE, 100, None) == i2s.I2S_EWORKSPACE
    assert L.i8s_quantize(FAKE, 1 << 31, FAKE, FAKE, 4096, None) == i2s.I2S_ERANGE
    assert L.i8s_dequantize(None, 16, FAKE, None) == i2s.I2S_EINVAL
    assert L.i8s_dequantize(FAKE, 16, FAKE_ODD, None) == i2s.I2S_EINVAL
    assert L.i8s_dequantize(FAKE, 1 << 30, FAKE, None) == i2s.I2S_ERANGE
