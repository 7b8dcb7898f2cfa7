"""CPU-side checks of the W8A8 part of the C ABI (include/w8a8.h): every
declared symbol is exported, the workspace size, the automatic variant and
the host-side argument checks (these calls return before any launch)."""

from __future__ import annotations

import ctypes

import pytest

from ternary_weight_integer_amd import i2s, i8s, w8a8

FAKE = 1 << 20


def test_every_declared_symbol_is_exported():
    names = w8a8.declared_symbols()
    assert set(names) >= {"w8a8_act_workspace_bytes", "w8a8_quantize_weight", "w8a8_quantize_act", "w8a8_matmul",
                          "w8a8_mul_mat", "w8a8_mul_mat_ex", "w8a8_mul_mat_variant"}
    raw = ctypes.CDLL(i2s.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n


def test_workspace_and_variant():
    assert w8a8.w8a8_act_workspace_bytes(512, 1536) == 512 * 1536 + 2048
    assert w8a8.w8a8_act_workspace_bytes(1, 1536) == 1536 + 256
    assert w8a8.w8a8_act_workspace_bytes(-1, 16) == 0
    for shape in [(8960, 1536, 512), (1536, 8960, 1), (256, 1536, 64), (32, 64, 1000)]:
        assert 2 <= w8a8.w8a8_mul_mat_variant(*shape) <= w8a8.w8a8_variants()
    assert w8a8.w8a8_variants() == i8s.i8s_variants() + 2  # variants 10 and 11: W8A8 only
    assert w8a8.w8a8_mul_mat_variant(8960, 1536, 512) == 10   # activation-resident
    assert w8a8.w8a8_mul_mat_variant(1536, 8960, 512) == 7    # K beyond its LDS tile
    assert w8a8.w8a8_mul_mat_variant(8960, 1536, 1) == 11     # fused decode kernel
    assert w8a8.w8a8_mul_mat_variant(1536, 8960, 4) == 11
    assert w8a8.w8a8_mul_mat_variant(8960, 1536, 5) == 9      # skinny, after the quantizer's launch
    assert w8a8.w8a8_mul_mat_variant(64, 9232, 1) == 9        # K beyond the fused kernel's registers


def _mm(wq=FAKE, ws=FAKE, OC=64, K=64, aq=FAKE, as_=FAKE, M=8, y=FAKE, dot=None, variant=0):
    return w8a8.lib().w8a8_matmul(wq, ws, OC, K, aq, as_, M, y, dot, variant, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(wq=None), i2s.I2S_EINVAL),
    (dict(y=None), i2s.I2S_EINVAL),
    (dict(OC=-1), i2s.I2S_EINVAL),
    (dict(wq=FAKE + 4), i2s.I2S_EINVAL),
    (dict(ws=FAKE + 2), i2s.I2S_EINVAL),
    (dict(dot=FAKE + 4), i2s.I2S_EINVAL),
    (dict(K=0), i2s.I2S_EALIGN),
    (dict(K=40), i2s.I2S_EALIGN),
    (dict(OC=1 << 20, K=4096), i2s.I2S_ERANGE),
    (dict(variant=1), i2s.I2S_EKERNEL),
    (dict(variant=99), i2s.I2S_EKERNEL),
    (dict(variant=11), i2s.I2S_EKERNEL),
    (dict(K=48, variant=10), i2s.I2S_EKERNEL),      # K % 64 != 0
    (dict(K=2560, variant=10), i2s.I2S_EKERNEL),    # activation tile beyond the LDS
])
def test_matmul_rejects_on_host(kw, expect):
    assert _mm(**kw) == expect


def test_mul_mat_and_quantizers_reject_on_host():
    L = w8a8.lib()
    assert L.w8a8_mul_mat(FAKE, FAKE, 64, 64, FAKE, 8, None, 1 << 20, FAKE, None) == i2s.I2S_EWORKSPACE
    assert L.w8a8_mul_mat(FAKE, FAKE, 64, 64, FAKE, 8, FAKE, 10, FAKE, None) == i2s.I2S_EWORKSPACE
    assert L.w8a8_mul_mat(FAKE, FAKE, 64, 64, FAKE + 8, 8, FAKE, 1 << 20, FAKE, None) == i2s.I2S_EINVAL
    assert L.w8a8_mul_mat(FAKE, FAKE, 64, 40, FAKE, 8, FAKE, 1 << 20, FAKE, None) == i2s.I2S_EALIGN
    assert L.w8a8_quantize_weight(None, 4, 16, FAKE, FAKE, None) == i2s.I2S_EINVAL
    assert L.w8a8_quantize_act(FAKE, -1, 16, FAKE, FAKE, None) == i2s.I2S_EINVAL
    assert L.w8a8_quantize_act(FAKE, 1 << 20, 4096, FAKE, FAKE, None) == i2s.I2S_ERANGE


def test_fused_variant_refused_on_host():
    """Variant 11 (the fused decode kernel) takes 1 <= M <= 4 and K <= 9216,
    and only on the F32-input entry point; the refusals come before any
    launch."""
    L = w8a8.lib()
    ex = lambda M, K, v: L.w8a8_mul_mat_ex(FAKE, FAKE, 64, K, FAKE, M, FAKE, 1 << 24, FAKE, None, v, None)
    assert ex(5, 64, 11) == i2s.I2S_EKERNEL
    assert ex(0, 64, 11) == i2s.I2S_EKERNEL
    assert ex(1, 9232, 11) == i2s.I2S_EKERNEL
    assert ex(1, 40, 11) == i2s.I2S_EALIGN
    assert _mm(variant=11) == i2s.I2S_EKERNEL
