"""GPU parity of the batched (3-D, strided) op against the CPU oracle, bit for
bit: dense and strided activations and outputs, batch counts 1 and 3, N
covering every contraction path (fused, GEMV, skinny MFMA, MFMA GEMM), rows
not a multiple of 4, sentinel checks that nothing outside the output rows is
written, and the stride checks."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from ternary_weight_integer_amd import i2s, workloads

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU visible", allow_module_level=True)

DEV = torch.device("cuda:0")
SENTINEL = np.float32(-7.25)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def bits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def run_case(rows, K, B, N, pad_x=(0, 0), pad_y=(0, 0), seed=0):
    """pad_x / pad_y: (extra rows per batch, extra elements per row) around the
    dense views, so the strides are non-trivial."""
    print(f"[batched] rows={rows} K={K} B={B} N={N} pad_x={pad_x} pad_y={pad_y}", flush=True)
    rng = np.random.default_rng(seed)
    w = workloads.ternary(rng, rows, K)
    x = workloads.normal(rng, B * N, K).reshape(B, N, K)
    pnp = oracle.pack(w, 0.015)
    pg = i2s.i2s_pack(torch.from_numpy(w).to(DEV), 0.015)
    xbig = np.zeros((B, N + pad_x[0], K + pad_x[1]), np.float32)
    xbig[:, :N, :K] = x
    xg = torch.from_numpy(xbig).to(DEV)[:, :N, :K]
    ybig = torch.full((B, N + pad_y[0], rows + pad_y[1]), float(SENTINEL), dtype=torch.float32, device=DEV)
    yv = ybig[:, :N, :rows]
    dbig = torch.full((B, N + pad_y[0], rows + pad_y[1]), -5, dtype=torch.int32, device=DEV)
    dv = dbig[:, :N, :rows]
    i2s.i2s_mul_mat_batched(pg, rows, K, xg, y=yv, dot_out=dv)
    ye, de = oracle.mul_mat_batched(pnp, rows, K, x, with_dot=True)
    yh, dh = host(ybig), host(dbig)
    assert np.array_equal(dh[:, :N, :rows], de)
    assert np.array_equal(bits(yh[:, :N, :rows]), bits(ye))
    mask = np.ones(yh.shape, bool)
    mask[:, :N, :rows] = False
    assert (yh[mask] == SENTINEL).all() and (dh[mask] == -5).all(), "wrote outside the output rows"


@pytest.mark.parametrize("N", [1, 2, 3, 5, 8, 16, 40])
def test_dense_batches(N):
    run_case(70, 1152, 3, N)


@pytest.mark.parametrize("N", [1, 3, 5, 8, 24, 40])
def test_strided_batches(N):
    run_case(70, 1152, 3, N, pad_x=(2, 128), pad_y=(1, 8))


def test_strided_batches_past_64_rows_in_all():
    """Five batches of 17 rows (85 in all, batches starting inside a 16-row
    block of the workspace's tiled activation copy) through the skinny MFMA
    kernel."""
    assert i2s.i2s_mul_mat_kernel(70, 1152, 17) == i2s.KERNEL_SKINNY
    run_case(70, 1152, 5, 17, pad_x=(1, 0), pad_y=(1, 0), seed=7)


@pytest.mark.parametrize("seed", range(4))
def test_random_batched_shapes(seed):
    """Seeded random batch counts, row counts, K and padded strides (every
    contraction path: fused, GEMV, skinny MFMA with batches starting inside
    a 16-row block, GEMM)."""
    rng = np.random.default_rng(2000 + seed)
    for _ in range(4):
        rows = int(rng.integers(1, 300))
        K = 128 * int(rng.integers(1, 13))
        B = int(rng.integers(1, 5))
        N = int(rng.integers(1, 70))
        pad_x = (int(rng.integers(0, 3)), 4 * int(rng.integers(0, 40)))
        pad_y = (int(rng.integers(0, 3)), int(rng.integers(0, 20)))
        run_case(rows, K, B, N, pad_x=pad_x, pad_y=pad_y, seed=int(rng.integers(1 << 30)))


def test_strided_single_batch_and_long_k():
    run_case(64, 8960, 1, 4, pad_x=(0, 64), pad_y=(0, 4))
    run_case(36, 9344, 2, 2, pad_x=(1, 4), pad_y=(2, 0))    # beyond the fused K limit


def test_decoder_shapes_strided():
    run_case(1536, 1536, 2, 8, pad_x=(1, 0), pad_y=(0, 16), seed=3)


def test_stride_checks():
    K, rows = 128, 8
    pg = i2s.i2s_pack(torch.zeros((rows, K), dtype=torch.int8, device=DEV), 1.0)
    L = i2s.lib()
    x = torch.zeros((2, 3, 256), dtype=torch.float32, device=DEV)
    y = torch.zeros(256, dtype=torch.float32, device=DEV)  # room for every accepted stride below
    ws = i2s.new_workspace(6, K, DEV)
    args = lambda ldx, bsx, ldy, bsy: (pg.data_ptr(), rows, K, x.data_ptr(), 3, 2, ldx, bsx, ws.data_ptr(),
                                       ws.numel(), y.data_ptr(), ldy, bsy, None, None)
    assert L.i2s_mul_mat_batched(*args(256, 768, 16, 48)) == i2s.I2S_OK
    torch.cuda.synchronize()
    assert L.i2s_mul_mat_batched(*args(64, 768, 16, 48)) == i2s.I2S_EINVAL    # ldx < K
    assert L.i2s_mul_mat_batched(*args(130, 768, 16, 48)) == i2s.I2S_EINVAL   # ldx not a multiple of 4
    assert L.i2s_mul_mat_batched(*args(256, 768, 6, 48)) == i2s.I2S_EINVAL    # ldy < rows
    assert L.i2s_mul_mat_batched(*args(256, 768, 18, 54)) == i2s.I2S_OK      # ldy not a multiple of 4: fine
    assert L.i2s_mul_mat_batched(*args(256, 768, 16, 20)) == i2s.I2S_EINVAL   # batches overlap
    assert L.i2s_mul_mat_batched(*args(256, 766, 16, 48)) == i2s.I2S_EINVAL   # bsx not a multiple of 4
