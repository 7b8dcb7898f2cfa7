"""CPU-side checks of the C ABI: the built library loads, exports every symbol
include/i2s.h declares, answers the size queries, and rejects bad arguments on
the host before any launch (these calls return before touching the GPU)."""

from __future__ import annotations

import ctypes

import pytest

from ternary_weight_integer_amd import i2s


def test_every_declared_symbol_is_exported():
    names = i2s.declared_symbols()
    assert set(names) >= {"i2s_pack", "i2s_quantize_act", "i2s_mul_mat", "i2s_packed_bytes",
                          "i2s_act_workspace_bytes", "i2s_strerror"}
    raw = ctypes.CDLL(i2s.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n


def test_size_queries():
    # rows*K/4 payload + 32-byte scale slot
    assert i2s.i2s_packed_bytes(8960, 1536) == 8960 * 1536 // 4 + 32
    assert i2s.i2s_packed_bytes(0, 128) == 32
    assert i2s.i2s_packed_bytes(4, 100) == 0
    assert i2s.i2s_packed_bytes(-1, 128) == 0
    # q (N*K, 256-aligned) + scales + row sums (each 256-aligned) + the
    # MFMA-tiled copy (ceil(N/16) blocks x ceil(K/256) steps x 4 KiB)
    assert i2s.i2s_act_workspace_bytes(1, 1536) == 1536 + 256 + 256 + 1 * 6 * 4096
    assert i2s.i2s_act_workspace_bytes(512, 1536) == 512 * 1536 + 2048 + 2048 + 32 * 6 * 4096
    assert i2s.i2s_act_workspace_bytes(17, 1152) == 19712 + 256 + 256 + 2 * 5 * 4096  # 17*1152 rounded up to 256
    assert i2s.i2s_act_workspace_bytes(0, 1536) == 0
    assert i2s.i2s_act_workspace_bytes(3, 200) == 0


def test_kernel_variant_counts():
    assert i2s.i2s_kernel_variants(1) >= 2
    assert i2s.i2s_kernel_variants(2) >= 2
    assert i2s.i2s_kernel_variants(3) >= 1
    assert i2s.i2s_kernel_variants(4) >= 1
    assert i2s.i2s_kernel_variants(0) == 0
    assert i2s.i2s_kernel_variants(5) == 0


def test_strerror_covers_every_status():
    seen = set()
    for st in range(0, 8):
        msg = i2s.i2s_strerror(st)
        assert msg and msg != "unknown status"
        seen.add(msg)
    assert len(seen) == 8
    assert i2s.i2s_strerror(99) == "unknown status"


FAKE = 1 << 20  # a 16- and 256-byte aligned non-null address; never dereferenced here


@pytest.mark.parametrize("args,expect", [
    # (packed, rows, K, x, N, ws, ws_bytes, y, dot, kernel, variant) -> status
    ((FAKE, 4, 100, FAKE, 1, FAKE, 1 << 20, FAKE, None, 0, 0), i2s.I2S_EALIGN),
    ((FAKE, 4, 0, FAKE, 1, FAKE, 1 << 20, FAKE, None, 0, 0), i2s.I2S_EALIGN),
    ((FAKE, -1, 128, FAKE, 1, FAKE, 1 << 20, FAKE, None, 0, 0), i2s.I2S_EINVAL),
    ((FAKE, 4, 128, FAKE, -1, FAKE, 1 << 20, FAKE, None, 0, 0), i2s.I2S_EINVAL),
    ((None, 4, 128, FAKE, 1, FAKE, 1 << 20, FAKE, None, 0, 0), i2s.I2S_EINVAL),
    ((FAKE, 4, 128, None, 1, FAKE, 1 << 20, FAKE, None, 0, 0), i2s.I2S_EINVAL),
    ((FAKE, 4, 128, FAKE, 1, FAKE, 1 << 20, None, None, 0, 0), i2s.I2S_EINVAL),
    ((FAKE + 4, 4, 128, FAKE, 1, FAKE, 1 << 20, FAKE, None, 0, 0), i2s.I2S_EINVAL),
    ((FAKE, 4, 128, FAKE, 1, None, 1 << 20, FAKE, None, 0, 0), i2s.I2S_EWORKSPACE),
    ((FAKE, 4, 128, FAKE, 2, FAKE, 128, FAKE, None, 0, 0), i2s.I2S_EWORKSPACE),
    ((FAKE, 4, 128, FAKE, 1, FAKE + 16, 1 << 20, FAKE, None, 0, 0), i2s.I2S_EWORKSPACE),
    ((FAKE, 4, 128, FAKE, 9, FAKE, 1 << 20, FAKE, None, 1, 0), i2s.I2S_EKERNEL),
    ((FAKE, 4, 128, FAKE, 1, FAKE, 1 << 20, FAKE, None, 5, 0), i2s.I2S_EKERNEL),
    ((FAKE, 4, 128, FAKE, 65, FAKE, 1 << 20, FAKE, None, 4, 0), i2s.I2S_EKERNEL),
    ((FAKE, 4, 128, FAKE, 1, FAKE, 1 << 20, FAKE, None, 4, 9), i2s.I2S_EKERNEL),
    ((FAKE, 4, 128, FAKE, 5, FAKE, 1 << 20, FAKE, None, 3, 0), i2s.I2S_EKERNEL),
    ((FAKE, 4, 9344, FAKE, 1, FAKE, 1 << 20, FAKE, None, 3, 0), i2s.I2S_EKERNEL),
    ((FAKE, 4, 128, FAKE, 1, FAKE, 1 << 20, FAKE, None, 2, 99), i2s.I2S_EKERNEL),
    ((FAKE, 4, 128, FAKE, 1, FAKE, 1 << 20, FAKE, None, 0, 1), i2s.I2S_EKERNEL),
    ((FAKE, 4, 8454656, FAKE, 1, FAKE, 1 << 40, FAKE, None, 0, 0), i2s.I2S_ERANGE),
    # N == 0 or rows == 0: success, nothing launched
    ((None, 4, 128, None, 0, None, 0, None, None, 0, 0), i2s.I2S_OK),
    ((None, 0, 128, None, 3, None, 0, None, None, 0, 0), i2s.I2S_OK),
])
def test_mul_mat_ex_host_validation(args, expect):
    assert i2s.lib().i2s_mul_mat_ex(*args, None) == expect


def _batched(rows=4, K=128, N=2, B=2, ldx=128, bsx=256, ldy=4, bsy=8, ws_bytes=1 << 20, x=FAKE, y=FAKE):
    return i2s.lib().i2s_mul_mat_batched(FAKE, rows, K, x, N, B, ldx, bsx, FAKE, ws_bytes, y, ldy, bsy, None, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(N=-1), i2s.I2S_EINVAL),
    (dict(B=-1), i2s.I2S_EINVAL),
    (dict(N=1 << 16, B=1 << 16), i2s.I2S_ERANGE),     # N * B beyond 2^31 - 1
    (dict(x=None), i2s.I2S_EINVAL),
    (dict(x=FAKE + 4), i2s.I2S_EINVAL),
    (dict(ldx=64), i2s.I2S_EINVAL),                  # ldx < K
    (dict(ldx=130, bsx=260), i2s.I2S_EINVAL),        # activation rows not 16-byte aligned
    (dict(bsx=258), i2s.I2S_EINVAL),
    (dict(ldy=3), i2s.I2S_EINVAL),                   # ldy < rows
    (dict(bsy=7), i2s.I2S_EINVAL),                   # batch outputs would overlap
    (dict(B=1, bsy=0, ldx=1 << 31, bsx=0), i2s.I2S_ERANGE),   # strides the kernels cannot address
    (dict(B=1, bsy=0, ldy=1 << 31), i2s.I2S_ERANGE),
    (dict(ws_bytes=64), i2s.I2S_EWORKSPACE),
    (dict(K=96, ldx=96, bsx=192), i2s.I2S_EALIGN),
    (dict(N=0), i2s.I2S_OK),                         # nothing to do, nothing launched
    (dict(B=0), i2s.I2S_OK),
])
def test_batched_host_validation(kw, expect):
    """The batched entry point's refusals come before any launch."""
    assert _batched(**kw) == expect


def test_mul_mat_host_validation():
    L = i2s.lib()
    assert L.i2s_mul_mat(FAKE, 4, 96, FAKE, 1, FAKE, 1 << 20, FAKE, None, None) == i2s.I2S_EALIGN
    assert L.i2s_mul_mat(FAKE, 4, 128, FAKE, 1, FAKE, 16, FAKE, None, None) == i2s.I2S_EWORKSPACE


def test_pack_and_quantize_host_validation():
    L = i2s.lib()
    assert L.i2s_pack(FAKE, 1.0, 4, 192, FAKE, None) == i2s.I2S_EALIGN
    assert L.i2s_pack(None, 1.0, 4, 128, FAKE, None) == i2s.I2S_EINVAL
    assert L.i2s_pack(FAKE, 1.0, 4, 128, None, None) == i2s.I2S_EINVAL
    assert L.i2s_pack(FAKE + 8, 1.0, 4, 128, FAKE, None) == i2s.I2S_EINVAL
    assert L.i2s_quantize_act(FAKE, 2, 130, FAKE, FAKE, FAKE, None) == i2s.I2S_EALIGN
    assert L.i2s_quantize_act(FAKE, -2, 128, FAKE, FAKE, FAKE, None) == i2s.I2S_EINVAL
    assert L.i2s_quantize_act(FAKE, 2, 128, None, FAKE, FAKE, None) == i2s.I2S_EINVAL
    assert L.i2s_quantize_act(None, 0, 128, None, None, None, None) == i2s.I2S_OK


def test_mul_mat_kernel_choice():
    assert i2s.i2s_mul_mat_kernel(8960, 1536, 1) == i2s.KERNEL_FUSED   # decode: one launch
    assert i2s.i2s_mul_mat_kernel(1536, 8960, 1) == i2s.KERNEL_FUSED   # long K too
    assert i2s.i2s_mul_mat_kernel(1536, 8960, 3) == i2s.KERNEL_FUSED
    assert i2s.i2s_kernel_variants(3) == 8
    for rows, K, v in ((8960, 1536, 7), (8960, 2048, 8), (12288, 1664, 8), (8192, 2048, 2), (12289, 2048, 2),
                       (4096, 1536, 6), (2048, 2048, 3), (1536, 8960, 5)):
        assert i2s.i2s_mul_mat_variant(rows, K, 1) == v, (rows, K)
    assert i2s.i2s_mul_mat_kernel(1536, 9344, 1) == i2s.KERNEL_GEMV    # beyond the fused K limit
    assert i2s.i2s_mul_mat_kernel(1536, 9344, 2) == i2s.KERNEL_SKINNY
    assert i2s.i2s_mul_mat_kernel(1536, 8960, 4) == i2s.KERNEL_SKINNY
    assert i2s.i2s_mul_mat_kernel(1536, 8960, 8) == i2s.KERNEL_SKINNY
    assert i2s.i2s_mul_mat_kernel(8960, 1536, 16) == i2s.KERNEL_SKINNY
    assert i2s.i2s_mul_mat_kernel(8960, 1536, 32) == i2s.KERNEL_SKINNY   # N <= 32
    assert i2s.i2s_mul_mat_kernel(8960, 1536, 33) == i2s.KERNEL_GEMM     # N > 32, 560 subtiles
    assert i2s.i2s_mul_mat_kernel(4096, 1536, 64) == i2s.KERNEL_SKINNY   # 256 subtiles
    assert i2s.i2s_mul_mat_kernel(4112, 1536, 64) == i2s.KERNEL_GEMM     # 257 subtiles
    assert i2s.i2s_mul_mat_kernel(1536, 8960, 64) == i2s.KERNEL_SKINNY
    assert i2s.i2s_mul_mat_kernel(256, 1536, 64) == i2s.KERNEL_SKINNY
    assert i2s.i2s_mul_mat_kernel(256, 1536, 65) == i2s.KERNEL_GEMM
    assert i2s.i2s_mul_mat_kernel(8960, 1536, 512) == i2s.KERNEL_GEMM
    # fused configurations: chunk batches sized to the row where they can be
    assert i2s.i2s_mul_mat_variant(8960, 1536, 1) == 7
    assert i2s.i2s_mul_mat_variant(17920, 1536, 1) == 6
    assert i2s.i2s_mul_mat_variant(6144, 1536, 1) == 6
    assert i2s.i2s_mul_mat_variant(8960, 2048, 1) == 8   # 48-row workgroups
    assert i2s.i2s_mul_mat_variant(1536, 1536, 1) == 3
    assert i2s.i2s_mul_mat_variant(1536, 8960, 1) == 5
    with pytest.raises(i2s.I2SError):
        i2s.i2s_mul_mat_kernel(4, 100, 1)


def test_mul_mat_variant_choice():
    # every automatic variant is a valid index of its kernel
    for rows, K, N in [(8960, 1536, 1), (1536, 8960, 8), (8960, 1536, 512), (1536, 1536, 64), (256, 1536, 2048),
                       (1536, 9344, 1), (64, 128, 40)]:
        k = i2s.i2s_mul_mat_kernel(rows, K, N)
        v = i2s.i2s_mul_mat_variant(rows, K, N)
        assert 1 <= v <= i2s.i2s_kernel_variants(k), (rows, K, N, k, v)
    # the weight-resident GEMM up to 16 subtiles per block where K <= 1536;
    # beyond, the resident GEMM with row-contiguous weight loads, its group
    # size by the 16-row subtiles each wave holds
    assert i2s.i2s_mul_mat_variant(8960, 1536, 128) == 15   # 5 subtiles per block
    assert i2s.i2s_mul_mat_variant(1536, 1536, 128) == 15   # 1
    assert i2s.i2s_mul_mat_variant(1536, 1536, 512) == 15   # 3
    assert i2s.i2s_mul_mat_variant(256, 1536, 1024) == 15
    assert i2s.i2s_mul_mat_variant(8960, 1536, 256) == 15   # 9
    assert i2s.i2s_mul_mat_variant(4096, 1536, 512) == 15   # 16
    assert i2s.i2s_mul_mat_variant(8960, 1536, 512) == 16   # 18: 3 per wave, groups of 3, first two paired
    assert i2s.i2s_mul_mat_variant(8960, 1536, 1024) == 13  # 35: 5 per wave, groups of 4
    assert i2s.i2s_mul_mat_variant(8960, 1536, 2048) == 16  # 70: 9 per wave, groups of 3, first two paired
    assert i2s.i2s_mul_mat_variant(8960, 2304, 512) == 11   # past the 2-step chunks' LDS limit: 3-step chunks
    assert i2s.i2s_mul_mat_variant(1536, 2048, 512) == 12   # K past the weight-resident kernel
    assert i2s.i2s_mul_mat_variant(2048, 1792, 512) == 12   # 4 subtiles, K = 1792: 1 per wave, groups of 2
    with pytest.raises(i2s.I2SError):
        i2s.i2s_mul_mat_variant(4, 100, 1)


def test_noalloc_limit_is_checked_on_the_host():
    """i2s_mul_mat_noalloc refuses a shape whose workspace exceeds its fixed
    array before touching the GPU (fake pointers, no device needed)."""
    assert i2s.i2s_noalloc_scratch_bytes() == 32 << 20
    assert i2s.i2s_act_workspace_bytes(1024, 8960) <= i2s.i2s_noalloc_scratch_bytes()
    assert i2s.i2s_act_workspace_bytes(2048, 8960) > i2s.i2s_noalloc_scratch_bytes()
    st = i2s.lib().i2s_mul_mat_noalloc(FAKE, 4, 8960, FAKE, 2048, FAKE, None, None)
    assert st == i2s.I2S_ESCRATCH
    assert i2s.lib().i2s_mul_mat_noalloc(FAKE, 4, 100, FAKE, 1, FAKE, None, None) == i2s.I2S_EALIGN
