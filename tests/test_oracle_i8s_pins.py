"""Pins of the CPU oracle's I8_S type and mul_mat_add(_relu) against what the
pages and the mathematics fix: the hand-worked fixture, the exact-rational
model of tests/exact.py, numpy's integer matmul, closed forms and invariants.
A plausible slip in the oracle (ties to even, a reciprocal scale, a per-row
instead of a per-tensor requantization, ReLU after requantizing, the bias on
the wrong axis, a transposed operand, a missing floor) fails one of them.
CPU only.
"""

from __future__ import annotations

from fractions import Fraction

import numpy as np
import pytest

import oracle
from exact import AMAX_FLOOR, f32_bits, f32_mul, f32_round, frac, near_tie_rows, quantize_row
from goldens import i8s_mul_mat_add, quantize_cases


def _exact_mul_mat_add(w, ws, x, xs, bias, relu):
    """Exact-rational model: acc in Python integers; f = F32(F32(acc) * F32(ws*xs));
    + bias as one rounded add; ReLU; then quantize_row over the whole tensor."""
    OC, N = w.shape[0], x.shape[0]
    t = f32_mul(ws, xs)
    f = []
    for n in range(N):
        for o in range(OC):
            acc = sum(int(a) * int(b) for a, b in zip(w[o], x[n]))
            v = f32_mul(f32_round(Fraction(acc)), t)
            if bias is not None:
                v = f32_round(frac(v) + frac(bias[o]))
            if relu and not v > 0:
                v = np.float32(0.0)
            f.append(v)
    q, s, _ = quantize_row(f)
    return np.array(q, dtype=np.int8).reshape(N, OC), s


# --- the I8_S type -------------------------------------------------------------

@pytest.mark.parametrize("case", quantize_cases(), ids=lambda c: c["name"])
def test_i8s_quantize_of_one_row_is_the_hand_worked_vector(case):
    # A one-row tensor: the per-tensor amax is the row's, so the hand-worked
    # per-row vectors (rounding, ties, the 1e-5 floor) apply unchanged.
    t = oracle.i8s_quantize(case["x"])
    n = case["x"].size
    assert t.size == n + 32
    assert np.array_equal(oracle.i8s_payload(t, n), case["q"])
    assert f32_bits(oracle.i8s_scale(t, n)) == f32_bits(case["scale"])


def test_i8s_quantize_matches_exact_rational_over_whole_tensor():
    rng = np.random.default_rng(5)
    for shape in [(3, 50), (1, 7), (4, 33)]:
        x = rng.normal(0, 2, size=shape).astype(np.float32)
        x.flat[rng.integers(0, x.size)] *= 30
        t = oracle.i8s_quantize(x)
        q, s, _ = quantize_row(x.reshape(-1))
        assert np.array_equal(oracle.i8s_payload(t, x.size), np.array(q, dtype=np.int8))
        assert f32_bits(oracle.i8s_scale(t, x.size)) == f32_bits(s)
    # Near-tie values: the last bit of the division decides q.
    for row in near_tie_rows((3.3, 0.77)):
        t = oracle.i8s_quantize(row)
        q, s, _ = quantize_row(row)
        assert np.array_equal(oracle.i8s_payload(t, row.size), np.array(q, dtype=np.int8))


def test_i8s_scale_is_per_tensor_not_per_row():
    # Row 0 is small, row 1 large: one scale serves both, so row 0 quantizes
    # coarsely (a per-row scale would give it +-127).
    x = np.array([[0.5, -0.25, 0.125, 0.0], [127.0, -3.0, 2.5, 1.0]], dtype=np.float32)
    t = oracle.i8s_quantize(x)
    assert oracle.i8s_scale(t, 8) == np.float32(1.0)
    assert oracle.i8s_payload(t, 8).tolist() == [1, 0, 0, 0, 127, -3, 3, 1]


def test_i8s_round_trip_error_bound():
    rng = np.random.default_rng(11)
    x = rng.normal(0, 1, size=4099).astype(np.float32)
    t = oracle.i8s_quantize(x)
    s = frac(oracle.i8s_scale(t, x.size))
    y = oracle.i8s_dequantize(t, x.size)
    q = oracle.i8s_payload(t, x.size)
    assert np.abs(q.astype(int)).max() == 127 and np.abs(q.astype(int)).max() <= 127
    for xi, yi, qi in zip(x[:600], y[:600], q[:600]):
        assert frac(yi) == frac(f32_round(Fraction(int(qi)) * s))   # y = F32(q * s)
        assert abs(frac(xi) - Fraction(int(qi)) * s) <= s / 2 * (1 + Fraction(1, 1 << 20))


def test_i8s_degenerate_scale_gives_zero_not_nan():
    for n in (1, 128, 1000):
        t = oracle.i8s_quantize(np.zeros(n, np.float32))
        assert f32_bits(oracle.i8s_scale(t, n)) == 0x33A917DC == f32_bits(f32_round(frac(AMAX_FLOOR) / 127))
        assert not oracle.i8s_payload(t, n).any()
        y = oracle.i8s_dequantize(t, n)
        assert not np.isnan(y).any() and not y.any() and not np.signbit(y).any()


# --- mul_mat_add / mul_mat_add_relu -----------------------------------------

def _golden_inputs():
    sh, cases = i8s_mul_mat_add()
    OC, IC, N = sh["OC"], sh["IC"], sh["N"]
    W = oracle.i8s_make(sh["w"], sh["ws"])
    X = oracle.i8s_make(sh["x"], sh["xs"])
    return sh, cases, OC, IC, N, W, X


@pytest.mark.parametrize("name", ["pos", "pos_relu", "neg", "neg_relu", "dead_relu"])
def test_mul_mat_add_hand_worked(name):
    sh, cases, OC, IC, N, W, X = _golden_inputs()
    case = next(c for c in cases if c["name"] == name)
    out, acc = oracle.i8s_mul_mat_add(W, OC, IC, X, N, case["bias"], case["relu"], with_dot=True)
    assert np.array_equal(acc.reshape(-1), sh["acc"])
    assert np.array_equal(oracle.i8s_payload(out, N * OC), case["q"])
    assert f32_bits(oracle.i8s_scale(out, N * OC)) == case["scale_bits"]


@pytest.mark.parametrize("OC,IC,N,relu,with_bias", [(5, 32, 3, 0, True), (7, 16, 4, 1, True), (3, 48, 6, 0, False),
                                                    (9, 20, 2, 1, False)])
def test_mul_mat_add_matches_exact_rational(OC, IC, N, relu, with_bias):
    rng = np.random.default_rng(OC * 100 + IC + N)
    w = rng.integers(-127, 128, size=(OC, IC), dtype=np.int8)
    x = rng.integers(-127, 128, size=(N, IC), dtype=np.int8)
    ws, xs = np.float32(0.0123), np.float32(0.0371)
    bias = rng.normal(0, 20, size=OC).astype(np.float32) if with_bias else None
    out = oracle.i8s_mul_mat_add(oracle.i8s_make(w, ws), OC, IC, oracle.i8s_make(x, xs), N, bias, relu)
    q, s = _exact_mul_mat_add(w, ws, x, xs, bias, relu)
    assert np.array_equal(oracle.i8s_payload(out, N * OC).reshape(N, OC), q)
    assert f32_bits(oracle.i8s_scale(out, N * OC)) == f32_bits(s)


def test_mul_mat_add_integer_part_matches_numpy_at_full_scale():
    rng = np.random.default_rng(3)
    OC, IC, N = 37, 4096, 5
    w = rng.integers(-127, 128, size=(OC, IC), dtype=np.int8)
    x = rng.integers(-127, 128, size=(N, IC), dtype=np.int8)
    w[0] = 127
    x[0] = 127
    w[1] = -127
    _, acc = oracle.i8s_mul_mat_add(oracle.i8s_make(w, 1.0), OC, IC, oracle.i8s_make(x, 1.0), N, with_dot=True)
    ref = x.astype(np.int64) @ w.astype(np.int64).T
    assert ref[0, 0] == 127 * 127 * IC and ref[0, 1] == -127 * 127 * IC
    assert np.array_equal(acc.astype(np.int64), ref)


def test_mul_mat_add_power_of_two_scale_equivariance():
    # Doubling ws doubles every f exactly (no bias), hence amax and the
    # output scale; the int8 payload is unchanged.
    rng = np.random.default_rng(8)
    OC, IC, N = 11, 64, 7
    w = rng.integers(-127, 128, size=(OC, IC), dtype=np.int8)
    x = rng.integers(-127, 128, size=(N, IC), dtype=np.int8)
    X = oracle.i8s_make(x, 0.0371)
    a = oracle.i8s_mul_mat_add(oracle.i8s_make(w, 0.0123), OC, IC, X, N)
    b = oracle.i8s_mul_mat_add(oracle.i8s_make(w, 0.0246), OC, IC, X, N)
    assert np.array_equal(oracle.i8s_payload(a, N * OC), oracle.i8s_payload(b, N * OC))
    assert oracle.i8s_scale(b, N * OC) == 2 * oracle.i8s_scale(a, N * OC)


def test_mul_mat_add_channel_permutation_and_transpose():
    rng = np.random.default_rng(9)
    OC, IC, N = 6, 40, 4
    w = rng.integers(-127, 128, size=(OC, IC), dtype=np.int8)
    x = rng.integers(-127, 128, size=(N, IC), dtype=np.int8)
    bias = rng.normal(0, 30, size=OC).astype(np.float32)
    perm = np.array([3, 0, 5, 1, 4, 2])
    X = oracle.i8s_make(x, 0.05)
    a = oracle.i8s_mul_mat_add(oracle.i8s_make(w, 0.02), OC, IC, X, N, bias, 1)
    b = oracle.i8s_mul_mat_add(oracle.i8s_make(w[perm], 0.02), OC, IC, X, N, bias[perm], 1)
    qa = oracle.i8s_payload(a, N * OC).reshape(N, OC)
    qb = oracle.i8s_payload(b, N * OC).reshape(N, OC)
    assert np.array_equal(qa[:, perm], qb)
    assert oracle.i8s_scale(a, N * OC) == oracle.i8s_scale(b, N * OC)
    # Without a bias the op is symmetric in its operands up to a transpose
    # (ws * xs = xs * ws): swapping them transposes the output.
    c = oracle.i8s_mul_mat_add(oracle.i8s_make(w, 0.02), OC, IC, X, N)
    d = oracle.i8s_mul_mat_add(X, N, IC, oracle.i8s_make(w, 0.02), OC)
    assert np.array_equal(oracle.i8s_payload(c, N * OC).reshape(N, OC), oracle.i8s_payload(d, N * OC).reshape(OC, N).T)
    assert oracle.i8s_scale(c, N * OC) == oracle.i8s_scale(d, N * OC)


def test_mul_mat_add_relu_is_plain_when_every_value_is_positive():
    rng = np.random.default_rng(12)
    OC, IC, N = 8, 32, 5
    w = rng.integers(-127, 128, size=(OC, IC), dtype=np.int8)
    x = rng.integers(-127, 128, size=(N, IC), dtype=np.int8)
    W, X = oracle.i8s_make(w, 0.001), oracle.i8s_make(x, 0.001)
    bias = np.full(OC, 50.0, np.float32)   # |acc * 1e-6| < 0.52, so every f > 0
    a = oracle.i8s_mul_mat_add(W, OC, IC, X, N, bias, 0)
    b = oracle.i8s_mul_mat_add(W, OC, IC, X, N, bias, 1)
    assert np.array_equal(a, b)
    r = oracle.i8s_mul_mat_add(W, OC, IC, X, N, None, 1)
    assert (oracle.i8s_payload(r, N * OC) >= 0).all()


def test_mul_mat_add_on_ternary_weights_is_the_i2s_op_for_one_row():
    # One activation row: the per-tensor I8_S quantization of x is the per-row
    # activation quantization, and with ternary weights the pre-requantization
    # values of mul_mat_add (no bias) are the I2_S op's outputs bit for bit:
    # sum(w*q) = sum(code*q) - row_sum, times ws * s.
    rng = np.random.default_rng(4)
    rows, K = 24, 256
    w = rng.choice(np.array([-1, 0, 1], np.int8), size=(rows, K))
    x = rng.normal(0, 1, size=(1, K)).astype(np.float32)
    ws = np.float32(0.015)
    y = oracle.mul_mat(oracle.pack(w, ws), rows, K, x)
    X = oracle.i8s_quantize(x)
    q, s, _ = oracle.quantize_act(x)
    assert np.array_equal(oracle.i8s_payload(X, K), q[0]) and oracle.i8s_scale(X, K) == s[0]
    _, f = oracle.i8s_mul_mat_add(oracle.i8s_make(w, ws), rows, K, X, 1, with_f=True)
    assert np.array_equal(f.view(np.uint32), y.view(np.uint32))
