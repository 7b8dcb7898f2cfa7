"""Pins of the CPU oracle's per-channel W8A8 path (the NPU page's scheme)
against the hand-worked rounding row, an exact-rational model of each
quantizer and of the dequantization, numpy's integer matmul, and the
degenerate cases.  A slip in the oracle (ties to even for activations,
roundf for weights, a division instead of the reciprocal, the 1e-5 floor of
the I2_S path, aScale * (bScale * C)) fails one of them.  CPU only."""

from __future__ import annotations

from fractions import Fraction

import numpy as np
import pytest

import oracle
from exact import f32_bits, f32_mul, f32_round, frac
from goldens import w8a8_rounding

FLOOR = f32_round(Fraction(1, 10 ** 9))  # the binary32 literal 1e-9f


def _half_even(v) -> int:
    a = frac(v)
    fl = a.numerator // a.denominator
    rem = a - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return fl


def _exact_weight_row(w):
    mx = max([frac(FLOOR)] + [abs(frac(v)) for v in w])
    s = f32_round(mx / 127)
    q = [max(-127, min(127, _half_even(f32_round(frac(v) / frac(s))))) for v in w]
    return q, s


def _exact_act_row(x):
    mx = max([frac(FLOOR)] + [abs(frac(v)) for v in x])
    s = f32_round(mx / 127)
    inv = f32_round(127 / mx)
    q = []
    for v in x:
        p = f32_round(frac(v) * frac(inv))
        h = f32_round(frac(p) + (Fraction(1, 2) if np.signbit(p) == 0 else Fraction(-1, 2)))
        t = int(frac(h))  # truncation toward zero
        q.append(max(-127, min(127, t)))
    return q, s


def test_hand_worked_rounding_row():
    g = w8a8_rounding()
    x = g["x"][None, :]
    wq, ws = oracle.w8a8_quantize_weight(x)
    aq, as_ = oracle.w8a8_quantize_act(x)
    assert np.array_equal(wq[0], g["weight_q"]) and np.array_equal(aq[0], g["act_q"])
    assert ws[0] == g["scale"] and as_[0] == g["scale"]


def test_quantizers_match_exact_rational():
    rng = np.random.default_rng(6)
    x = rng.normal(0, 1, size=(5, 96)).astype(np.float32)
    x[1, 7] *= 40
    x[3] *= 1e-3
    wq, ws = oracle.w8a8_quantize_weight(x)
    aq, as_ = oracle.w8a8_quantize_act(x)
    for r in range(x.shape[0]):
        q, s = _exact_weight_row(x[r])
        assert wq[r].tolist() == q and f32_bits(ws[r]) == f32_bits(s)
        q, s = _exact_act_row(x[r])
        assert aq[r].tolist() == q and f32_bits(as_[r]) == f32_bits(s)


def test_quantizers_on_near_ties():
    # Values on and next to (k + 1/2) * s for a scale that is not a power of
    # two: the last bit of the division (weights) or of the product with the
    # reciprocal (activations) decides.
    mx = np.float32(3.3)
    s = f32_round(frac(mx) / 127)
    vals = [mx]
    for m in range(-126, 126, 5):
        c = np.float32(float((Fraction(m) + Fraction(1, 2)) * frac(s)))
        vals += [np.nextafter(c, np.float32(-1e9)), c, np.nextafter(c, np.float32(1e9))]
    row = np.array(vals, np.float32)[None, :]
    wq, _ = oracle.w8a8_quantize_weight(row)
    aq, _ = oracle.w8a8_quantize_act(row)
    assert wq[0].tolist() == _exact_weight_row(row[0])[0]
    assert aq[0].tolist() == _exact_act_row(row[0])[0]


def test_floor_gives_zero_not_nan():
    z = np.zeros((3, 32), np.float32)
    wq, ws = oracle.w8a8_quantize_weight(z)
    aq, as_ = oracle.w8a8_quantize_act(z)
    expect = f32_bits(f32_round(frac(FLOOR) / 127))
    assert not wq.any() and not aq.any()
    assert all(f32_bits(v) == expect for v in ws) and all(f32_bits(v) == expect for v in as_)
    rng = np.random.default_rng(1)
    w = rng.normal(0, 1, size=(4, 32)).astype(np.float32)
    d = oracle.w8a8_mul_mat(*oracle.w8a8_quantize_weight(w), z)
    assert not np.isnan(d).any() and not d.any()


@pytest.mark.parametrize("M,OC,K", [(3, 5, 64), (7, 2, 32), (1, 9, 160)])
def test_dequantization_is_left_to_right(M, OC, K):
    rng = np.random.default_rng(M * 31 + OC)
    a = rng.integers(-127, 128, size=(M, K), dtype=np.int8)
    w = rng.integers(-127, 128, size=(OC, K), dtype=np.int8)
    as_ = rng.uniform(1e-3, 0.1, size=M).astype(np.float32)
    ws = rng.uniform(1e-3, 0.1, size=OC).astype(np.float32)
    d, c = oracle.w8a8_matmul(a, as_, w, ws, with_c=True)
    assert np.array_equal(c.astype(np.int64), a.astype(np.int64) @ w.astype(np.int64).T)
    for m in range(M):
        for n in range(OC):
            e = f32_mul(f32_mul(as_[m], ws[n]), f32_round(Fraction(int(c[m, n]))))
            assert f32_bits(d[m, n]) == f32_bits(e)


def test_dequantization_order_is_observable():
    # (0.1f * 0.3f) * 7 and 0.1f * (0.3f * 7) differ in the last bit: the
    # oracle must give the first.
    a = np.full((1, 16), 0, np.int8)
    w = np.full((1, 16), 0, np.int8)
    a[0, 0], w[0, 0] = 1, 7
    as_, ws = np.array([0.1], np.float32), np.array([0.3], np.float32)
    left = f32_mul(f32_mul(as_[0], ws[0]), np.float32(7))
    right = f32_mul(as_[0], f32_mul(ws[0], np.float32(7)))
    assert f32_bits(left) != f32_bits(right)
    d = oracle.w8a8_matmul(a, as_, w, ws)
    assert f32_bits(d[0, 0]) == f32_bits(left)


def test_full_scale_integer_part():
    K = 8192
    a = np.full((2, K), 127, np.int8)
    w = np.full((3, K), -127, np.int8)
    w[1] = 127
    _, c = oracle.w8a8_matmul(a, np.ones(2, np.float32), w, np.ones(3, np.float32), with_c=True)
    assert c[0, 0] == -127 * 127 * K and c[1, 1] == 127 * 127 * K


def test_sliced_oracle_is_the_whole_call():
    """The row-sliced W8A8 oracle calls give the whole calls' bits."""
    rng = np.random.default_rng(78)
    for OC, K, M, threads in ((33, 96, 19, 4), (7, 64, 3, 16), (40, 48, 1, 0)):
        w = rng.normal(0, 0.05, size=(OC, K)).astype(np.float32)
        x = rng.normal(0, 1, size=(M, K)).astype(np.float32)
        wq, ws = oracle.w8a8_quantize_weight(w)
        d, c = oracle.w8a8_mul_mat(wq, ws, x, with_c=True)
        d2, c2 = oracle.w8a8_mul_mat_sliced(wq, ws, x, with_c=True, threads=threads)
        assert np.array_equal(c2, c) and np.array_equal(d2.view(np.uint32), d.view(np.uint32))
        aq, as_ = oracle.w8a8_quantize_act(x)
        d3, c3 = oracle.w8a8_matmul_sliced(aq, as_, wq, ws, with_c=True, threads=threads)
        assert np.array_equal(c3, c) and np.array_equal(d3.view(np.uint32), d.view(np.uint32))
