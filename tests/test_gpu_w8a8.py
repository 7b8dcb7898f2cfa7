"""GPU parity of the per-channel W8A8 path against the CPU oracle, bit for bit:
both quantizers (the hand-worked rounding row, near ties, zero rows, ragged
K), the contraction on every tile variant with ragged shapes and full-scale
accumulators, the activation-resident kernel's full and short subtile groups,
and the whole op on the Qwen2-1.5B projection shapes; every output is
compared (the oracle runs over slices of the activation rows on the host
threads)."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from exact import near_tie_rows
from goldens import w8a8_rounding
from ternary_weight_integer_amd import i2s, i8s, w8a8

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


def check_quantizers(x, tag):
    say(f"w8a8 quantizers {tag} shape={x.shape}")
    wq, ws = w8a8.w8a8_quantize_weight(dev(x))
    aq, as_ = w8a8.w8a8_quantize_act(dev(x))
    rwq, rws = oracle.w8a8_quantize_weight(x)
    raq, ras = oracle.w8a8_quantize_act(x)
    assert np.array_equal(host(wq), rwq) and np.array_equal(bits(host(ws)), bits(rws))
    assert np.array_equal(host(aq), raq) and np.array_equal(bits(host(as_)), bits(ras))


def test_quantizers_hand_worked_row():
    g = w8a8_rounding()
    x = g["x"][None, :]
    check_quantizers(x, "hand-worked")
    assert np.array_equal(host(w8a8.w8a8_quantize_weight(dev(x))[0])[0], g["weight_q"])
    assert np.array_equal(host(w8a8.w8a8_quantize_act(dev(x))[0])[0], g["act_q"])


@pytest.mark.parametrize("rows,K", [(1, 1536), (37, 48), (5, 7), (3, 1000), (512, 1536), (8, 8960)])
def test_quantizers_random(rows, K):
    rng = np.random.default_rng(rows * 7 + K)
    x = rng.normal(0, 1, size=(rows, K)).astype(np.float32)
    x[:, rng.integers(0, K, size=max(1, K // 100))] *= 20
    if rows > 2:
        x[1] = 0
        x[2] *= 1e-12   # maxima below the 1e-9 start
    check_quantizers(x, "random")


# (rows, K) through every (float4s per thread, waves per row) instance of the
# register quantizer: four waves under 1024 rows (eight for K > 4096 and at
# most 64 rows), one wave from 1024 rows; ragged tails; and rows past the
# register limit of their wave count (the workgroup-per-row kernel).
ACT_REG_CASES = [(3, 512), (4, 2048), (3, 3000), (2, 4096), (70, 260), (65, 8960), (100, 6100), (200, 9000),
                 (70, 12000), (65, 36864), (2, 6000), (3, 9216), (2, 20000), (1, 36864), (2, 49152), (1, 73728),
                 (1, 73732), (66, 36868), (1024, 256), (1024, 1000), (1024, 1536), (1024, 2200), (1024, 3000),
                 (1024, 4600), (1024, 6000), (1024, 9216), (1030, 9220), (2, 18000), (70, 16000), (80, 24000)]


@pytest.mark.parametrize("rows,K", ACT_REG_CASES)
def test_act_quantizer_every_register_width(rows, K):
    rng = np.random.default_rng(K)
    x = rng.standard_t(3, size=(rows, K)).astype(np.float32)
    x[0, K - 1] = 1e3   # the maximum in the last float4 of the row
    say(f"w8a8 act quantizer rows={rows} K={K}")
    aq, as_ = w8a8.w8a8_quantize_act(dev(x))
    raq, ras = oracle.w8a8_quantize_act(x)
    assert np.array_equal(host(aq), raq) and np.array_equal(bits(host(as_)), bits(ras))


@pytest.mark.parametrize("x_off,q_off", [(1, 0), (0, 1), (2, 2)])
def test_act_quantizer_unaligned_buffers(x_off, q_off):
    rows, K = 9, 1536
    x = np.random.default_rng(x_off * 3 + q_off).normal(0, 2, size=(rows, K)).astype(np.float32)
    xb = torch.zeros(rows * K + x_off, dtype=torch.float32, device=DEV)
    xv = xb[x_off:].view(rows, K)
    xv.copy_(dev(x))
    qb = torch.zeros(rows * K + q_off, dtype=torch.int8, device=DEV)
    qv = qb[q_off:].view(rows, K)
    say(f"w8a8 act quantizer unaligned x+{4 * x_off} B q+{q_off} B")
    aq, as_ = w8a8.w8a8_quantize_act(xv, q=qv)
    raq, ras = oracle.w8a8_quantize_act(x)
    assert np.array_equal(host(aq), raq) and np.array_equal(bits(host(as_)), bits(ras))
    if q_off:
        assert not host(qb[:q_off]).any()   # nothing written before q


def test_quantizers_near_ties():
    for row in near_tie_rows((3.3, 0.77, 100.0)):
        check_quantizers(row[None, :], "near ties")


SHAPES = [(70, 128, 37), (64, 64, 64), (200, 96, 129), (16, 16, 1), (1, 48, 5), (130, 1152, 9), (256, 256, 300)]


def variant_takes(v: int, K: int) -> bool:
    """Variant 10 (activation-resident) takes K % 64 == 0 up to 2544;
    variant 11 (the fused decode kernel) quantizes F32 rows itself, so the
    contraction on quantized rows never takes it."""
    return v != 11 and (v != 10 or (K % 64 == 0 and K <= 2544))


@pytest.mark.parametrize("OC,K,M", SHAPES + [(2048, 1536, 256), (1536, 2496, 130), (513, 1600, 64), (4100, 640, 130),
                                           (4097, 576, 70)])
def test_matmul_every_variant(OC, K, M):
    rng = np.random.default_rng(OC + K + M)
    wq = rng.integers(-127, 128, size=(OC, K), dtype=np.int8)
    aq = rng.integers(-127, 128, size=(M, K), dtype=np.int8)
    ws = rng.uniform(1e-4, 0.05, size=OC).astype(np.float32)
    as_ = rng.uniform(1e-3, 0.2, size=M).astype(np.float32)
    rd, rc = oracle.w8a8_matmul(aq, as_, wq, ws, with_c=True)
    for v in range(2, w8a8.w8a8_variants() + 1):
        if not variant_takes(v, K):
            continue
        say(f"w8a8_matmul OC={OC} K={K} M={M} variant={v}")
        y, c = w8a8.w8a8_matmul(dev(wq), dev(ws), dev(aq), dev(as_), dot_out=True, variant=v)
        assert np.array_equal(host(c), rc)
        assert np.array_equal(bits(host(y)), bits(rd))


@pytest.mark.parametrize("seed", range(3))
def test_random_shapes_every_variant(seed):
    """Seeded random OC, K (a multiple of 16), M and scales through every
    contraction variant, against the oracle bit for bit."""
    rng = np.random.default_rng(4000 + seed)
    for _ in range(4):
        OC = int(rng.integers(1, 400))
        K = 16 * int(rng.integers(1, 100))
        M = int(rng.integers(1, 300))
        wq = rng.integers(-127, 128, size=(OC, K), dtype=np.int8)
        aq = rng.integers(-127, 128, size=(M, K), dtype=np.int8)
        ws = rng.uniform(1e-5, 0.05, size=OC).astype(np.float32)
        as_ = rng.uniform(1e-4, 0.2, size=M).astype(np.float32)
        rd, rc = oracle.w8a8_matmul(aq, as_, wq, ws, with_c=True)
        for v in [0] + list(range(2, w8a8.w8a8_variants() + 1)):
            if not variant_takes(v, K):
                with pytest.raises(i2s.I2SError) as ei:
                    w8a8.w8a8_matmul(dev(wq), dev(ws), dev(aq), dev(as_), variant=v)
                assert ei.value.status == i2s.I2S_EKERNEL
                continue
            say(f"w8a8_matmul random seed={seed} OC={OC} K={K} M={M} variant={v}")
            y, c = w8a8.w8a8_matmul(dev(wq), dev(ws), dev(aq), dev(as_), dot_out=True, variant=v)
            assert np.array_equal(host(c), rc)
            assert np.array_equal(bits(host(y)), bits(rd))


def test_matmul_full_scale():
    K = 8192
    wq = np.full((64, K), 127, np.int8)
    wq[1::2] = -127
    aq = np.full((16, K), 127, np.int8)
    aq[5] = -127
    ws, as_ = np.full(64, 0.001, np.float32), np.full(16, 0.002, np.float32)
    rd, rc = oracle.w8a8_matmul(aq, as_, wq, ws, with_c=True)
    for v in range(2, w8a8.w8a8_variants() + 1):
        if not variant_takes(v, K):
            continue
        y, c = w8a8.w8a8_matmul(dev(wq), dev(ws), dev(aq), dev(as_), dot_out=True, variant=v)
        assert np.array_equal(host(c), rc) and np.array_equal(bits(host(y)), bits(rd))


# Shapes for the activation-resident kernel (variant 10): a block of ms
# 16-channel subtiles is dealt to 8 waves, each working through its subtiles
# in groups of G (4 from 4096 channels, 3 below), the last group possibly
# short.  (ms, subtiles per wave) for each shape:
#   4100 x 2048 rows: ms 33 -> waves of 5 and 4 (a full group of 4, one of 1)
#   4097 x 2048: the same without 16-byte stores (OC % 4 != 0)
#   4100 x 4096: ms 65 -> waves of 9 and 8 (two full groups of 4, one of 1)
#   4100 x 4000: as above with a ragged last activation tile
#   3000 x 2048: ms 24 -> 3 per wave (one full group of 3)
#   3001 x 4096: ms 47 -> 6 or 5 per wave (two groups of 3, a short one), no 16-byte stores
#   8960 x 1024 at K 1536: ms 35 -> 5 or 4 per wave, the prefill's shape at twice the rows
RES_GROUP_SHAPES = [(4100, 128, 2048), (4097, 128, 2048), (4100, 128, 4096), (4100, 64, 4000), (3000, 128, 2048),
                    (3001, 192, 4096), (8960, 1536, 1024)]


@pytest.mark.parametrize("OC,K,M", RES_GROUP_SHAPES)
def test_resident_kernel_full_and_short_groups(OC, K, M):
    rng = np.random.default_rng(OC * 3 + K + M)
    wq = rng.integers(-127, 128, size=(OC, K), dtype=np.int8)
    aq = rng.integers(-127, 128, size=(M, K), dtype=np.int8)
    ws = rng.uniform(1e-4, 0.05, size=OC).astype(np.float32)
    as_ = rng.uniform(1e-3, 0.2, size=M).astype(np.float32)
    rd, rc = oracle.w8a8_matmul_sliced(aq, as_, wq, ws, with_c=True)
    say(f"w8a8_matmul resident groups OC={OC} K={K} M={M}")
    for v in (10, 0):
        y, c = w8a8.w8a8_matmul(dev(wq), dev(ws), dev(aq), dev(as_), dot_out=True, variant=v)
        y2 = w8a8.w8a8_matmul(dev(wq), dev(ws), dev(aq), dev(as_), variant=v)
        assert np.array_equal(host(c), rc), v
        assert np.array_equal(bits(host(y)), bits(rd)), v
        assert np.array_equal(bits(host(y2)), bits(rd)), (v, "without dot_out")


@pytest.mark.parametrize("name,OC,K,M", [("decode_up", 8960, 1536, 1), ("down_small_batch", 1536, 8960, 8),
                                        ("qkv_64", 256, 1536, 64), ("prefill_gate", 8960, 1536, 512)])
def test_whole_op_qwen2_shapes(name, OC, K, M):
    say(f"w8a8_mul_mat {name} OC={OC} K={K} M={M}")
    rng = np.random.default_rng(0)
    w = (rng.normal(0, 0.02, size=(OC, K))).astype(np.float32)
    x = rng.normal(0, 1, size=(M, K)).astype(np.float32)
    x[:, rng.integers(0, K, size=K // 100)] *= 20
    wq, ws = w8a8.w8a8_quantize_weight(dev(w))
    rwq, rws = oracle.w8a8_quantize_weight(w)
    assert np.array_equal(host(wq), rwq) and np.array_equal(bits(host(ws)), bits(rws))
    y = host(w8a8.w8a8_mul_mat(wq, ws, dev(x)))
    rd = oracle.w8a8_mul_mat_sliced(rwq, rws, x)
    assert np.array_equal(bits(y), bits(rd))


def test_whole_op_zero_rows_and_streams():
    rng = np.random.default_rng(3)
    w = rng.normal(0, 1, size=(96, 64)).astype(np.float32)
    x = rng.normal(0, 1, size=(20, 64)).astype(np.float32)
    x[4] = 0
    wq, ws = oracle.w8a8_quantize_weight(w)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        y = w8a8.w8a8_mul_mat(dev(wq), dev(ws), dev(x), stream=s)
    s.synchronize()
    yh = host(y)
    assert not yh[4].any()
    assert np.array_equal(bits(yh), bits(oracle.w8a8_mul_mat(wq, ws, x)))


@pytest.mark.parametrize("OC,K,M", [(8960, 1536, 64), (1536, 8960, 4)])
def test_graph_replay_matches_eager(OC, K, M):
    say(f"graph replay w8a8_mul_mat OC={OC} K={K} M={M}")
    rng = np.random.default_rng(M)
    wq, ws_ = w8a8.w8a8_quantize_weight(dev(rng.normal(0, 0.02, size=(OC, K)).astype(np.float32)))
    x = dev(rng.normal(0, 1, size=(M, K)).astype(np.float32))
    wsp = w8a8.new_workspace(M, K, DEV)
    y = torch.empty((M, OC), dtype=torch.float32, device=DEV)
    w8a8.w8a8_mul_mat(wq, ws_, x, workspace=wsp, y=y)
    eager = host(y).copy()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        w8a8.w8a8_mul_mat(wq, ws_, x, workspace=wsp, y=y)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        w8a8.w8a8_mul_mat(wq, ws_, x, workspace=wsp, y=y)
    for r in range(4):
        y.zero_()
        wsp.zero_()
        torch.cuda.synchronize()
        g.replay()
        assert np.array_equal(bits(host(y)), bits(eager)), f"replay {r}"


# The fused decode kernel (W8A8 variant 11: the rows quantized inside the
# contraction's launch, M <= 4): every K class of its launch configuration
# (up to 1536, 2048, 4096 and 9216), OC ragged against its 16-, 8- and 4-row
# workgroups, K not a multiple of 64, and every M from 1 to 4.
FUSED_SHAPES = [(8960, 1536, 1), (37, 16, 1), (513, 48, 2), (1000, 2048, 3), (257, 4096, 4), (100, 2064, 1),
                (65, 9216, 2), (1536, 8960, 4), (17, 1552, 3),
                # 48-row workgroups (8192 < OC <= 12288, K <= 1536): a ragged last
                # workgroup, a short row, exactly 256 workgroups, and just past the range
                (8193, 1536, 4), (9000, 64, 3), (12288, 1520, 2), (12289, 1536, 1)]


def check_fused(wq, ws, x, tag):
    """The fused path (automatic and forced) against the oracle: y and C bit
    for bit, and the codes and scales where the quantizer would leave them."""
    OC, K = wq.shape
    M = x.shape[0]
    rq, rs = oracle.w8a8_quantize_act(x)
    rd, rc = oracle.w8a8_matmul(rq, rs, wq, ws, with_c=True)
    assert w8a8.w8a8_mul_mat_variant(OC, K, M) == 11
    for v in (0, 11):
        say(f"w8a8_mul_mat_ex fused {tag} OC={OC} K={K} M={M} variant={v}")
        wsp = w8a8.new_workspace(M, K, DEV)
        y, c = w8a8.w8a8_mul_mat_ex(dev(wq), dev(ws), dev(x), workspace=wsp, dot_out=True, variant=v)
        assert np.array_equal(host(c), rc), v
        assert np.array_equal(bits(host(y)), bits(rd)), v
        wh = host(wsp)
        assert np.array_equal(wh[: M * K].view(np.int8).reshape(M, K), rq), v
        so = -(-M * K // 256) * 256
        assert np.array_equal(wh[so: so + 4 * M].view(np.uint32), bits(rs)), v
    y2 = w8a8.w8a8_mul_mat(dev(wq), dev(ws), dev(x))
    assert np.array_equal(bits(host(y2)), bits(rd)), "without dot_out"


@pytest.mark.parametrize("OC,K,M", FUSED_SHAPES)
def test_fused_decode(OC, K, M):
    rng = np.random.default_rng(OC + 7 * K + M)
    wq = rng.integers(-127, 128, size=(OC, K), dtype=np.int8)
    ws = rng.uniform(1e-4, 0.05, size=OC).astype(np.float32)
    x = rng.normal(0, 1, size=(M, K)).astype(np.float32)
    x[:, rng.integers(0, K, size=max(1, K // 100))] *= 20
    check_fused(wq, ws, x, "random")


def test_fused_decode_near_ties_and_full_scale():
    rows = near_tie_rows((3.3, 0.77, 100.0))
    K = -(-max(r.size for r in rows) // 16) * 16
    x = np.zeros((3, K), np.float32)
    for i, r in enumerate(rows):
        x[i, : r.size] = r
    rng = np.random.default_rng(11)
    wq = rng.integers(-127, 128, size=(300, K), dtype=np.int8)
    check_fused(wq, rng.uniform(1e-4, 0.05, size=300).astype(np.float32), x, "near ties")
    # the largest accumulators: every product 127 * 127 (or its negative)
    K = 8192
    wq = np.full((64, K), 127, np.int8)
    wq[1::2] = -127
    x = np.full((2, K), 3.0, np.float32)
    x[1] = -3.0
    check_fused(wq, np.full(64, 0.001, np.float32), x, "full scale")


def test_fused_decode_refusals():
    wq = torch.zeros((64, 64), dtype=torch.int8, device=DEV)
    ws = torch.ones(64, dtype=torch.float32, device=DEV)
    for M, K in [(5, 64), (1, 9232)]:
        w = torch.zeros((64, K), dtype=torch.int8, device=DEV)
        with pytest.raises(i2s.I2SError) as ei:
            w8a8.w8a8_mul_mat_ex(w, ws, torch.zeros((M, K), dtype=torch.float32, device=DEV), variant=11)
        assert ei.value.status == i2s.I2S_EKERNEL
    aq = torch.zeros((1, 64), dtype=torch.int8, device=DEV)
    with pytest.raises(i2s.I2SError) as ei:
        w8a8.w8a8_matmul(wq, ws, aq, torch.ones(1, dtype=torch.float32, device=DEV), variant=11)
    assert ei.value.status == i2s.I2S_EKERNEL


def test_fused_decode_zero_row_on_a_stream():
    """A zero activation row through the fused launch: its maximum is the
    1e-9 floor, every code 0, every output +0; on a side stream."""
    rng = np.random.default_rng(5)
    w = rng.normal(0, 1, size=(200, 320)).astype(np.float32)
    x = rng.normal(0, 1, size=(3, 320)).astype(np.float32)
    x[1] = 0
    wq, ws = oracle.w8a8_quantize_weight(w)
    assert w8a8.w8a8_mul_mat_variant(200, 320, 3) == 11
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        y = w8a8.w8a8_mul_mat(dev(wq), dev(ws), dev(x), stream=s)
    s.synchronize()
    yh = host(y)
    assert not bits(yh[1]).any()
    assert np.array_equal(bits(yh), bits(oracle.w8a8_mul_mat(wq, ws, x)))
