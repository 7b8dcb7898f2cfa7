"""The allocation-free entry point i2s_mul_mat_noalloc against i2s_mul_mat:
two calls in a row on the library's fixed device array (the second with a
smaller input, so it runs on what the first left there), each compared bit
for bit with the workspace entry point and with the oracle; a third call
through the fused path; the size limit is refused before any launch."""

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


def bits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def run_pair(case):
    rows, K, N = case.rows, case.K, case.N
    print(f"[noalloc] rows={rows} K={K} N={N}", flush=True)
    pg = i2s.i2s_pack(torch.from_numpy(case.w).to(DEV), case.ws)
    x = torch.from_numpy(case.x).to(DEV)
    y = torch.full((N, rows), float("nan"), dtype=torch.float32, device=DEV)
    d = torch.full((N, rows), -1, dtype=torch.int32, device=DEV)
    i2s.i2s_mul_mat_noalloc(pg, rows, K, x, y, dot_out=d)
    y_ref, d_ref = i2s.i2s_mul_mat(pg, rows, K, x, dot_out=True)
    torch.cuda.synchronize()
    yh, dh = y.cpu().numpy(), d.cpu().numpy()
    assert np.array_equal(dh, d_ref.cpu().numpy())
    assert np.array_equal(bits(yh), bits(y_ref.cpu().numpy()))
    ye, de = oracle.mul_mat_sliced(oracle.pack(case.w, case.ws), rows, K, case.x, with_dot=True)
    assert np.array_equal(dh, de)
    assert np.array_equal(bits(yh), bits(ye))


def test_two_calls_in_a_row_then_smaller():
    run_pair(workloads.prefill_gate_case())                       # the MFMA GEMM path, N = 512
    run_pair(workloads.random_case(91, 1501, 1152, 40))           # smaller: the skinny path's tiled copy
    run_pair(workloads.random_case(92, 700, 384, 2))              # smaller still: the fused launch


def test_too_large_is_refused_before_launch():
    K, N = 8192, 4096
    assert i2s.i2s_act_workspace_bytes(N, K) > i2s.i2s_noalloc_scratch_bytes()
    pg = i2s.i2s_pack(torch.zeros((4, K), dtype=torch.int8, device=DEV), 1.0)
    x = torch.zeros((N, K), dtype=torch.float32, device=DEV)
    y = torch.full((N, 4), 3.0, dtype=torch.float32, device=DEV)
    with pytest.raises(i2s.I2SError) as e:
        i2s.i2s_mul_mat_noalloc(pg, 4, K, x, y)
    assert e.value.status == i2s.I2S_ESCRATCH
    torch.cuda.synchronize()
    assert (y.cpu().numpy() == 3.0).all()
