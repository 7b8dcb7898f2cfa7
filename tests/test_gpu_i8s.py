"""GPU parity of the I8_S type and mul_mat_add(_relu) against the CPU oracle,
byte for byte (int8 payload, the in-band scale's bits and the slot's padding)
and, for the contraction, the int32 accumulators: the hand-worked fixture,
every variant on ragged shapes with and without bias and ReLU, the encoder's
block shapes, full-scale accumulators, and the degenerate cases."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from goldens import i8s_mul_mat_add
from ternary_weight_integer_amd import i2s, i8s

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


def rand_i8s(rng, rows, cols, scale, full=False):
    q = rng.integers(-127, 128, size=(rows, cols), dtype=np.int8)
    if full and q.size:
        q.flat[rng.integers(0, q.size)] = 127
    return oracle.i8s_make(q, np.float32(scale))


def run_mm(W, OC, IC, X, N, bias, relu, variant):
    out, dot = i8s.i8s_mul_mat_add_ex(dev(W), OC, IC, dev(X), N, None if bias is None else dev(bias), relu,
                                      dot_out=True, variant=variant)
    return host(out), host(dot)


def check_mm(W, OC, IC, X, N, bias, relu, variant, tag=""):
    say(f"mul_mat_add OC={OC} IC={IC} N={N} relu={relu} bias={bias is not None} variant={variant} {tag}")
    ref, ref_dot = oracle.i8s_mul_mat_add(W, OC, IC, X, N, bias, relu, with_dot=True)
    out, dot = run_mm(W, OC, IC, X, N, bias, relu, variant)
    assert np.array_equal(dot.reshape(N, OC), ref_dot), "int32 accumulators differ"
    assert out.tobytes() == ref.tobytes(), (
        f"payload mismatches {np.count_nonzero(out[:N * OC] != ref[:N * OC])}, "
        f"scale {out[N * OC:N * OC + 4].view('<f4')} vs {ref[N * OC:N * OC + 4].view('<f4')}")


# --- I8_S quantize / dequantize ---------------------------------------------

@pytest.mark.parametrize("n", [0, 1, 15, 16, 17, 255, 4099, 65536, (1 << 20) + 7])
def test_quantize_matches_oracle(n):
    say(f"i8s_quantize n={n}")
    rng = np.random.default_rng(n)
    x = rng.normal(0, 1, size=n).astype(np.float32)
    if n:
        x[rng.integers(0, n, size=max(1, n // 100))] *= 20
    got = host(i8s.i8s_quantize(dev(x)))
    assert got.tobytes() == oracle.i8s_quantize(x).tobytes()


def test_quantize_degenerate_and_ties():
    say("i8s_quantize zeros and ties")
    z = np.zeros(1000, np.float32)
    assert host(i8s.i8s_quantize(dev(z))).tobytes() == oracle.i8s_quantize(z).tobytes()
    # s = 1 exactly; halves round away from zero.
    t = np.array([127, 2.5, -2.5, 0.5, -0.5, 126.5, -127, 1.5] * 5, np.float32)
    assert host(i8s.i8s_quantize(dev(t))).tobytes() == oracle.i8s_quantize(t).tobytes()


@pytest.mark.parametrize("n", [0, 3, 16, 1000, 100003])
def test_dequantize_matches_oracle(n):
    say(f"i8s_dequantize n={n}")
    rng = np.random.default_rng(7 + n)
    t = rand_i8s(rng, 1, n, 0.0137)
    got = host(i8s.i8s_dequantize(dev(t), n))
    assert np.array_equal(got.view(np.uint32), oracle.i8s_dequantize(t, n).view(np.uint32))


# --- mul_mat_add / mul_mat_add_relu -----------------------------------------

@pytest.mark.parametrize("name", ["pos", "pos_relu", "neg", "neg_relu", "dead_relu"])
def test_hand_worked_cases(name):
    sh, cases = i8s_mul_mat_add()
    case = next(c for c in cases if c["name"] == name)
    OC, IC, N = sh["OC"], sh["IC"], sh["N"]
    w = sh["w"].reshape(OC, IC)
    x = sh["x"].reshape(N, IC)
    # IC = 4 runs on the plain kernel; zero-padding IC to 64 (the same sums)
    # runs the same case on every MFMA tile.
    wp = np.zeros((OC, 64), np.int8)
    xp = np.zeros((N, 64), np.int8)
    wp[:, :IC], xp[:, :IC] = w, x
    for v, (ww, xx, ic) in [(1, (w, x, IC))] + [(v, (wp, xp, 64)) for v in range(2, i8s.i8s_variants() + 1)]:
        out, dot = run_mm(oracle.i8s_make(ww, sh["ws"]), OC, ic, oracle.i8s_make(xx, sh["xs"]), N, case["bias"],
                          case["relu"], v)
        say(f"hand-worked {name} variant {v}")
        assert np.array_equal(dot.reshape(-1), sh["acc"])
        assert np.array_equal(out[:N * OC].view(np.int8), case["q"])
        assert int(out[N * OC:N * OC + 4].view("<u4")[0]) == case["scale_bits"]
        assert not out[N * OC + 4:N * OC + 32].any()


SHAPES = [(64, 64, 64), (70, 128, 37), (128, 32, 300), (48, 160, 77), (200, 96, 129), (256, 256, 130),
          (16, 16, 1), (1, 48, 5), (130, 1152, 9)]


@pytest.mark.parametrize("OC,IC,N", SHAPES)
def test_every_variant_ragged(OC, IC, N):
    rng = np.random.default_rng(OC * 7 + IC * 3 + N)
    W = rand_i8s(rng, OC, IC, 0.0123, full=True)
    X = rand_i8s(rng, N, IC, 0.0371)
    bias = rng.normal(0, 30, size=OC).astype(np.float32)
    for v in range(1, i8s.i8s_variants() + 1):
        for relu in (0, 1):
            check_mm(W, OC, IC, X, N, bias if relu else None, relu, v)
            check_mm(W, OC, IC, X, N, None if relu else bias, relu, v)


@pytest.mark.parametrize("seed", range(4))
def test_random_shapes_every_variant(seed):
    """Seeded random OC, IC (any, so the plain kernel is covered too), N,
    scales and biases through every variant that accepts them; refusals must
    be I2S_EKERNEL (an MFMA variant with IC % 16 != 0)."""
    rng = np.random.default_rng(3000 + seed)
    for _ in range(4):
        OC = int(rng.integers(1, 260))
        IC = int(rng.integers(1, 400))
        N = int(rng.integers(1, 300))
        W = rand_i8s(rng, OC, IC, float(rng.uniform(1e-4, 0.05)), full=True)
        X = rand_i8s(rng, N, IC, float(rng.uniform(1e-3, 0.1)))
        bias = rng.normal(0, float(rng.uniform(0.1, 50)), size=OC).astype(np.float32)
        relu = int(rng.integers(0, 2))
        for v in range(0, i8s.i8s_variants() + 1):
            if v >= 2 and IC % 16:
                with pytest.raises(i8s.I2SError) as ei:
                    run_mm(W, OC, IC, X, N, bias, relu, v)
                assert ei.value.status == i2s.I2S_EKERNEL
                continue
            check_mm(W, OC, IC, X, N, bias, relu, v, tag=f"random seed {seed}")


@pytest.mark.parametrize("OC,IC,N", [(3, 7, 5), (33, 40, 21), (8, 1, 3), (5, 100, 2)])
def test_plain_kernel_any_ic(OC, IC, N):
    rng = np.random.default_rng(IC)
    W = rand_i8s(rng, OC, IC, 0.5)
    X = rand_i8s(rng, N, IC, 0.25)
    bias = rng.normal(0, 100, size=OC).astype(np.float32)
    assert i8s.i8s_mul_mat_add_variant(OC, IC, N) == 1
    for relu in (0, 1):
        check_mm(W, OC, IC, X, N, bias, relu, 0)


# The encoder's ConvNeXt block MLPs at a 4-second 24 kHz input (stage lengths
# 96000 / 3200 * stride products), FC1 = C -> 4C with ReLU, FC2 = 4C -> C.
ENCODER = [(128, 32, 96000, 1), (32, 128, 96000, 0), (512, 128, 24000, 1), (1024, 256, 6000, 1),
           (256, 1024, 6000, 0), (2048, 512, 1200, 1), (8192, 2048, 30, 1), (2048, 8192, 30, 0),
           (1536, 1536, 30, 0)]


@pytest.mark.parametrize("OC,IC,N,relu", ENCODER)
def test_encoder_block_shapes(OC, IC, N, relu):
    rng = np.random.default_rng(OC + IC + N)
    W = rand_i8s(rng, OC, IC, 0.02, full=True)
    X = rand_i8s(rng, N, IC, 0.05)
    bias = rng.normal(0, 5, size=OC).astype(np.float32)
    check_mm(W, OC, IC, X, N, bias, relu, 0, tag=f"(auto variant {i8s.i8s_mul_mat_add_variant(OC, IC, N)})")


def test_full_scale_accumulators():
    OC, IC, N = 64, 8192, 16
    w = np.full((OC, IC), 127, np.int8)
    w[1::2] = -127
    x = np.full((N, IC), 127, np.int8)
    x[3] = -127
    W, X = oracle.i8s_make(w, 1.0), oracle.i8s_make(x, 1.0)
    for v in range(1, i8s.i8s_variants() + 1):
        check_mm(W, OC, IC, X, N, None, 0, v)


def test_degenerate_shapes():
    rng = np.random.default_rng(0)
    # Empty output: only the scale slot is written (s = 1e-5 / 127).
    for OC, IC, N in [(0, 64, 5), (8, 64, 0), (0, 0, 0)]:
        W = rand_i8s(rng, OC, IC, 0.1)
        X = rand_i8s(rng, N, IC, 0.1)
        for v in (1, 2):
            check_mm(W, OC, IC, X, N, None, 0, v)
    # IC = 0: every acc is 0 and f is the bias.
    W, X = oracle.i8s_make(np.zeros((40, 0), np.int8), 1.0), oracle.i8s_make(np.zeros((9, 0), np.int8), 1.0)
    b = rng.normal(0, 1, size=40).astype(np.float32)
    for v in (1, 2, 3):
        check_mm(W, 40, 0, X, 9, b, 0, v)
        check_mm(W, 40, 0, X, 9, b, 1, v)
    # Zero weights, scale 0: every f is +0; the floor keeps the scale finite.
    W = oracle.i8s_make(np.zeros((32, 64), np.int8), 0.0)
    X = rand_i8s(rng, 20, 64, 0.3)
    for v in (1, 2):
        check_mm(W, 32, 64, X, 20, None, 0, v)


def test_named_entry_points_and_streams():
    rng = np.random.default_rng(21)
    OC, IC, N = 96, 64, 50
    W = rand_i8s(rng, OC, IC, 0.01)
    X = rand_i8s(rng, N, IC, 0.02)
    bias = rng.normal(0, 0.5, size=OC).astype(np.float32)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        a = i8s.i8s_mul_mat_add(dev(W), OC, IC, dev(X), N, dev(bias), stream=s)
        b = i8s.i8s_mul_mat_add_relu(dev(W), OC, IC, dev(X), N, dev(bias), stream=s)
    s.synchronize()
    assert host(a).tobytes() == oracle.i8s_mul_mat_add(W, OC, IC, X, N, bias, 0).tobytes()
    assert host(b).tobytes() == oracle.i8s_mul_mat_add(W, OC, IC, X, N, bias, 1).tobytes()


def test_chained_block_mlp():
    # FC1 + ReLU feeding FC2, I8_S end to end on the device, as in a block.
    rng = np.random.default_rng(33)
    C, N = 256, 700
    x = rng.normal(0, 1, size=(N, C)).astype(np.float32)
    W1, W2 = rand_i8s(rng, 4 * C, C, 0.01), rand_i8s(rng, C, 4 * C, 0.01)
    b1, b2 = rng.normal(0, 0.1, size=4 * C).astype(np.float32), rng.normal(0, 0.1, size=C).astype(np.float32)
    X = i8s.i8s_quantize(dev(x))
    H = i8s.i8s_mul_mat_add_relu(dev(W1), 4 * C, C, X, N, dev(b1))
    Y = i8s.i8s_mul_mat_add(dev(W2), C, 4 * C, H, N, dev(b2))
    rX = oracle.i8s_quantize(x)
    rH = oracle.i8s_mul_mat_add(W1, 4 * C, C, rX, N, b1, 1)
    rY = oracle.i8s_mul_mat_add(W2, C, 4 * C, rH, N, b2, 0)
    assert host(X).tobytes() == rX.tobytes()
    assert host(H).tobytes() == rH.tobytes()
    assert host(Y).tobytes() == rY.tobytes()


def test_requantize_near_ties():
    # Zero activations make every accumulator 0, so f = bias[o] exactly; the
    # biases sit on and a few floats either side of (k + 1/2) * s for the
    # tensor scale s = f32(100 / 127) fixed by bias[0] = 100, where the
    # rounding of the division decides q.
    OC, IC, N = 1024, 64, 3
    s = np.float32(np.float32(100.0) / np.float32(127.0))
    vals = [np.float32(100.0)]
    rng = np.random.default_rng(2)
    while len(vals) < OC:
        k = int(rng.integers(-127, 127))
        c = np.float32((k + 0.5) * float(s))
        for d in range(-3, 4):
            v = c
            step = np.float32(np.inf) if d > 0 else np.float32(-np.inf)
            for _ in range(abs(d)):
                v = np.nextafter(v, step)
            vals.append(np.float32(v))
    bias = np.array(vals[:OC], np.float32)
    W = rand_i8s(rng, OC, IC, 0.01)
    X = oracle.i8s_make(np.zeros((N, IC), np.int8), 0.5)
    for v in range(1, i8s.i8s_variants() + 1):
        for relu in (0, 1):
            check_mm(W, OC, IC, X, N, bias, relu, v, tag="near ties")


@pytest.mark.parametrize("OC,IC,N,relu", [(1024, 256, 600, 1), (2048, 512, 30, 0)])
def test_graph_replay_matches_eager(OC, IC, N, relu):
    # Both passes captured in a HIP graph; every replay, with eager work and
    # synchronizations in between, must give the eager bytes (the partial
    # maxima are written by the kernels themselves, no memset is captured).
    say(f"graph replay mul_mat_add OC={OC} IC={IC} N={N}")
    rng = np.random.default_rng(OC + N)
    W, X = dev(rand_i8s(rng, OC, IC, 0.01)), dev(rand_i8s(rng, N, IC, 0.02))
    b = dev(rng.normal(0, 1, size=OC).astype(np.float32))
    ws = i8s.new_workspace(DEV)
    out = torch.empty(i8s.i8s_bytes(N * OC), dtype=torch.uint8, device=DEV)
    fn = i8s.i8s_mul_mat_add_relu if relu else i8s.i8s_mul_mat_add
    fn(W, OC, IC, X, N, b, out=out, workspace=ws)
    eager = host(out).copy()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn(W, OC, IC, X, N, b, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn(W, OC, IC, X, N, b, out=out, workspace=ws)
    for r in range(4):
        out.zero_()
        ws.fill_(0xFF)   # stale partial maxima must not leak into the next replay
        torch.cuda.synchronize()
        g.replay()
        assert host(out).tobytes() == eager.tobytes(), f"replay {r}"
