"""GPU parity of grouped projections (one activation, several I2_S weights,
optional F32 biases) against the CPU oracle, bit for bit: the decoder
layer's q/k/v (with biases) and gate/up groups at decode and prefill sizes,
every kernel and variant on small ragged shapes, and the argument checks."""

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


def say(msg):
    print(msg, flush=True)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def bits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def make_group(seed, shapes, K, N, with_bias):
    """shapes: list of rows; with_bias: list of bools."""
    rng = np.random.default_rng(seed)
    ws = [workloads.ternary(rng, r, K) for r in shapes]
    biases = [rng.standard_normal(r).astype(np.float32) if b else None for r, b in zip(shapes, with_bias)]
    x = workloads.normal(rng, N, K)
    return ws, biases, x


def oracle_group(ws, biases, K, x, scale):
    """Oracle y and dot of each projection on every output: the whole op on
    its own (over slices of its output features, in parallel), then its bias
    add, as oracle.mul_mat_group defines a group."""
    out = []
    for w, b in zip(ws, biases):
        rows = w.shape[0]
        if rows == 0:
            out.append((np.zeros((x.shape[0], 0), np.float32), np.zeros((x.shape[0], 0), np.int32)))
            continue
        y, d = oracle.mul_mat_sliced(oracle.pack(w, scale), rows, K, x, with_dot=True)
        if b is not None:
            y = oracle.add_bias(y, b)
        out.append((y, d))
    return out


def check_group(ws, biases, x, K, kernel=0, variant=0, scale=0.015):
    N = x.shape[0]
    say(f"[group] rows={[w.shape[0] for w in ws]} K={K} N={N} bias={[b is not None for b in biases]} "
        f"kernel={kernel} variant={variant}")
    packed = [(i2s.i2s_pack(dev(w), scale), w.shape[0]) for w in ws]
    bt = [dev(b) if b is not None else None for b in biases]
    ys, ds = i2s.i2s_mul_mat_group(packed, K, dev(x), biases=bt, dot_out=True, kernel=kernel, variant=variant)
    ys2 = i2s.i2s_mul_mat_group(packed, K, dev(x), biases=bt, kernel=kernel, variant=variant)
    for (ye, de), y, d, y2 in zip(oracle_group(ws, biases, K, x, scale), ys, ds, ys2):
        y, d, y2 = host(y), host(d), host(y2)
        assert np.array_equal(bits(y), bits(y2)), "y differs with and without dot_out"
        assert np.array_equal(d, de)
        assert np.array_equal(bits(y), bits(ye)), np.argwhere(bits(y) != bits(ye))[:5]


QKV = [1536, 256, 256]


@pytest.mark.parametrize("N", [1, 2, 3, 8, 64])
def test_decoder_qkv_group_with_biases(N):
    ws, b, x = make_group(41 + N, QKV, 1536, N, [True, True, True])
    check_group(ws, b, x, 1536)


@pytest.mark.parametrize("N", [1, 4])
def test_decoder_gate_up_group(N):
    ws, b, x = make_group(43 + N, [8960, 8960], 1536, N, [False, False])
    check_group(ws, b, x, 1536)


def test_down_projection_with_bias_long_k():
    ws, b, x = make_group(47, [1536], 8960, 3, [True])
    check_group(ws, b, x, 8960)


@pytest.mark.parametrize("K", [128, 1536])
def test_group_of_one_every_fused_variant(K):
    """A group of one projection runs the single-weight fused kernel: with
    and without a bias, ragged rows, N = 1..4, every fused variant."""
    for N in (1, 2, 4):
        for rows, with_bias in ((70, True), (1, False), (200, True)):
            ws, b, x = make_group(K + N + rows, [rows], K, N, [with_bias])
            for var in range(0, i2s.i2s_kernel_variants(3) + 1):
                check_group(ws, b, x, K, kernel=3, variant=var)
            check_group(ws, b, x, K)


@pytest.mark.parametrize("K", [128, 1152])
def test_group_every_kernel_and_variant(K):
    shapes = [70, 5, 64, 1]          # rows not a multiple of 4, a single row
    for N in (1, 3, 9, 17, 40):
        ws, b, x = make_group(K + N, shapes, K, N, [True, False, True, True])
        combos = [(0, 0)] + [(2, v) for v in range(1, i2s.i2s_kernel_variants(2) + 1)]
        if N <= 8:
            combos += [(1, v) for v in range(1, i2s.i2s_kernel_variants(1) + 1)]
        if N <= 4:
            combos += [(3, v) for v in range(0, i2s.i2s_kernel_variants(3) + 1)]
        if N <= 64:
            combos += [(4, v) for v in range(0, i2s.i2s_kernel_variants(4) + 1)]
        for kern, var in combos:
            check_group(ws, b, x, K, kernel=kern, variant=var)


@pytest.mark.parametrize("variant", [0, 16, 17, 18])
def test_group_paired_subtiles_with_bias(variant):
    """Resident GEMM variants that deal each wave two adjacent subtiles and
    store them as whole lines, with biases: at N = 512 each block of the
    2048-row projection holds 4 subtiles (waves 0 and 1 a pair each); the
    1030-row projection (rows % 4 != 0) takes the per-subtile stores with the
    same subtile deal and a ragged last subtile.  Every output checked."""
    ws, b, x = make_group(91, [2048, 1030], 256, 512, [True, True])
    check_group(ws, b, x, 256, kernel=2, variant=variant)


def test_bias_with_negative_zero_and_zero_rows():
    K, N = 256, 2
    rng = np.random.default_rng(53)
    ws = [workloads.ternary(rng, 12, K)]
    b = [rng.standard_normal(12).astype(np.float32)]
    b[0][3] = np.float32(-0.0)
    x = np.zeros((N, K), np.float32)
    x[1] = workloads.normal(rng, 1, K)[0]
    for kern in (0, 1, 2, 3, 4):
        check_group(ws, b, x, K, kernel=kern)


def test_group_with_an_empty_projection():
    ws, b, x = make_group(59, [16, 0, 8], 128, 2, [True, False, False])
    check_group(ws, b, x, 128)


def test_group_argument_errors():
    K, N = 128, 2
    x = dev(np.zeros((N, K), np.float32))
    p = i2s.i2s_pack(dev(np.zeros((4, K), np.int8)), 1.0)
    with pytest.raises(i2s.I2SError) as e:
        i2s.i2s_mul_mat_group([], K, x)
    assert e.value.status == i2s.I2S_EINVAL
    with pytest.raises(i2s.I2SError) as e:
        i2s.i2s_mul_mat_group([(p, 4)] * 9, K, x)
    assert e.value.status == i2s.I2S_EINVAL
    bias = torch.zeros(8, dtype=torch.float32, device=DEV)
    with pytest.raises(i2s.I2SError) as e:   # bias not 16-byte aligned
        i2s.i2s_mul_mat_group([(p, 4)], K, x, biases=[bias[1:5]])
    assert e.value.status == i2s.I2S_EINVAL
    with pytest.raises(i2s.I2SError) as e:   # the fused group kernel takes N <= 4
        i2s.i2s_mul_mat_group([(p, 4)], K, dev(np.zeros((5, K), np.float32)), kernel=3)
    assert e.value.status == i2s.I2S_EKERNEL
