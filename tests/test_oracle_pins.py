"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: bytes worked
by hand from the layout sentence, exact rational arithmetic, Python-integer
brute force with signed weights, closed forms and invariants.  Chosen so that
a plausible slip in the oracle (a wrong shift or slice, a reciprocal instead of
a division, ties-to-even rounding, a forgotten row-sum correction, swapped
scales) fails at least one of them.  CPU only.
"""

from __future__ import annotations

import itertools

import numpy as np
import pytest

import oracle
from exact import AMAX_FLOOR, epilogue, f32_bits, f32_round, frac, near_tie_rows, quantize_row, round_half_away
from goldens import bias_add, headroom, pack_cases, quantize_cases
from ternary_weight_integer_amd import workloads


# --- packing -----------------------------------------------------------------

@pytest.mark.parametrize("case", pack_cases(), ids=lambda c: c["name"])
def test_pack_matches_hand_worked_bytes(case):
    rows, K = case["w"].shape
    p = oracle.pack(case["w"], case["ws"])
    assert p.size == rows * K // 4 + 32
    assert p[: rows * K // 4].tobytes() == case["bytes"]
    # The in-band scale: F32 little-endian right after the payload.
    assert p[rows * K // 4: rows * K // 4 + 4].tobytes() == case["scale"]


def _hand_decode_group(group_bytes: bytes) -> list[int]:
    """Codes of one 32-byte group, read slice by slice: slice s is the bit
    pair at shift 6-2s of bytes 0..31, giving positions 32s .. 32s+31."""
    codes = []
    for s in range(4):
        codes += [(b >> (6 - 2 * s)) & 3 for b in group_bytes]
    return codes


def test_pack_slices_line_up_and_row_stride():
    """Each row is K/4 bytes and decodes on its own; the four bit-pair lanes of
    a group are four consecutive 32-value slices of the row."""
    rng = np.random.default_rng(7)
    for rows, K in [(3, 128), (5, 384), (2, 1152)]:
        w = workloads.ternary(rng, rows, K)
        p = oracle.pack(w, 1.0)
        for r in range(rows):
            row = p[r * K // 4:(r + 1) * K // 4].tobytes()
            assert len(row) == K // 4
            codes = []
            for g in range(K // 128):
                codes += _hand_decode_group(row[32 * g: 32 * g + 32])
            assert codes == [int(v) + 1 for v in w[r]]


def test_pack_rejects_k_not_multiple_of_128():
    with pytest.raises(ValueError):
        oracle.pack(np.zeros((2, 96), np.int8), 1.0)


# --- activation quantization ---------------------------------------------------

@pytest.mark.parametrize("case", quantize_cases(), ids=lambda c: c["name"])
def test_quantize_matches_hand_worked_vector(case):
    q, s, rs = oracle.quantize_act(case["x"][None, :])
    assert q[0].tolist() == case["q"].tolist()
    assert f32_bits(s[0]) == f32_bits(case["scale"])
    assert int(rs[0]) == case["row_sum"]


def test_quantize_matches_exact_rational_on_near_ties():
    found_recip_flip = 0
    found_tie = 0
    for x in near_tie_rows():
        q, s, rs = oracle.quantize_act(x[None, :])
        eq, es, ers = quantize_row(x)
        assert f32_bits(s[0]) == f32_bits(es)
        assert q[0].tolist() == eq
        assert int(rs[0]) == ers
        # Teeth: the set must hold values where the P4-style reciprocal
        # (x * (127/amax)) or ties-to-even would give another q.
        inv = f32_round(127 / max(abs(frac(v)) for v in x))
        for v, qe in zip(x, eq):
            v_div = f32_round(frac(v) / frac(es))
            if round_half_away(f32_round(frac(v) * frac(inv))) != qe:
                found_recip_flip += 1
            if abs(frac(v_div)) % 1 == frac(0.5):
                found_tie += 1
    assert found_recip_flip > 0
    assert found_tie > 0


def test_quantize_random_rows_exact_rational():
    rng = np.random.default_rng(3)
    x = np.concatenate([
        workloads.normal(rng, 3, 256),
        workloads.with_outliers(rng, workloads.normal(rng, 2, 256)),
        workloads.relu(workloads.normal(rng, 2, 256, 0.5)),
        (workloads.normal(rng, 1, 256) * np.float32(1e-7)).astype(np.float32),  # below the amax floor
    ])
    q, s, rs = oracle.quantize_act(x)
    for n in range(x.shape[0]):
        eq, es, ers = quantize_row(x[n])
        assert q[n].tolist() == eq, n
        assert f32_bits(s[n]) == f32_bits(es)
        assert int(rs[n]) == ers


def test_quantize_floor_and_symmetry():
    assert f32_bits(AMAX_FLOOR) == 0x3727C5AC
    rng = np.random.default_rng(11)
    x = workloads.normal(rng, 4, 384)
    q, s, rs = oracle.quantize_act(x)
    qn, sn, rsn = oracle.quantize_act(-x)
    assert np.array_equal(qn, -q)
    assert np.array_equal(sn.view(np.uint32), s.view(np.uint32))
    assert np.array_equal(rsn, -rs)
    assert np.all(np.abs(q) <= 127)


# --- contraction and epilogue: brute force with signed weights ---------------

def _brute(w, ws, x):
    """y[N][rows] and sum(w*q)[N][rows] from signed weights, no codes, no packing."""
    N, rows = x.shape[0], w.shape[0]
    y = np.empty((N, rows), np.float32)
    swq = np.empty((N, rows), np.int64)
    for n in range(N):
        q, s, _ = quantize_row(x[n])
        for o in range(rows):
            t = sum(int(a) * b for a, b in zip(w[o], q))
            swq[n, o] = t
            y[n, o] = epilogue(t, ws, s)
    return y, swq


@pytest.mark.parametrize("rows,K,N,ws", [(3, 128, 2, 0.02), (5, 256, 3, 0.015), (2, 384, 1, 0.7), (4, 128, 4, 0.0)])
def test_mul_mat_matches_python_int_brute_force(rows, K, N, ws):
    rng = np.random.default_rng(rows * 1000 + K + N)
    w = workloads.ternary(rng, rows, K)
    x = workloads.normal(rng, N, K)
    p = oracle.pack(w, ws)
    y, dot = oracle.mul_mat(p, rows, K, x, with_dot=True)
    yb, swq = _brute(w, ws, x)
    _, _, rs = oracle.quantize_act(x)
    # The unsigned-code identity: sum(code*q) = sum(w*q) + sum(q).
    assert np.array_equal(dot.astype(np.int64), swq + rs[:, None].astype(np.int64))
    assert np.array_equal(y.view(np.uint32), yb.view(np.uint32))


GRID_K = (128, 1024, 1152)
GRID_DIM = (1, 2, 64, 70, 100)


@pytest.mark.parametrize("K", GRID_K)
def test_mul_mat_test_grid(K):
    """K in {128, 1024, 1152} x out in {1,2,64,70,100} x N in {1,2,64,70,100},
    against an int64 matmul of signed weights and the exact-rational epilogue."""
    rng = np.random.default_rng(K)
    wmax = workloads.ternary(rng, max(GRID_DIM), K)
    xmax = workloads.normal(rng, max(GRID_DIM), K)
    q_all, s_all, rs_all = oracle.quantize_act(xmax)
    # quantization pinned on a few rows against exact rationals
    for n in (0, 63, 99):
        assert q_all[n].tolist() == quantize_row(xmax[n])[0]
    swq_all = q_all.astype(np.int64) @ wmax.astype(np.int64).T  # [N][rows]
    for rows, N in itertools.product(GRID_DIM, GRID_DIM):
        w, x = wmax[:rows], xmax[:N]
        p = oracle.pack(w, 0.015)
        y, dot = oracle.mul_mat(p, rows, K, x, with_dot=True)
        assert np.array_equal(dot.astype(np.int64), swq_all[:N, :rows] + rs_all[:N, None])
        for n in range(0, N, max(1, N // 7)):
            for o in range(0, rows, max(1, rows // 7)):
                ye = epilogue(int(swq_all[n, o]), 0.015, s_all[n])
                assert f32_bits(y[n, o]) == f32_bits(ye), (rows, N, n, o)


# --- closed forms, degenerate cases, invariants ------------------------------

def test_headroom_closed_form():
    h = headroom()
    K = h["K"]
    w = np.ones((3, K), np.int8)
    x = np.full((2, K), 127.0, np.float32)
    p = oracle.pack(w, h["ws"])
    assert (p[: 3 * K // 4] == 0xAA).all()
    q, s, rs = oracle.quantize_act(x)
    assert f32_bits(s[0]) == f32_bits(h["scale"]) and int(rs[0]) == h["row_sum"]
    y, dot = oracle.mul_mat(p, 3, K, x, with_dot=True)
    assert (dot == h["dot"]).all()
    assert (y.view(np.uint32) == h["y_bits"]).all()


def test_degenerate_scales_give_zero_not_nan():
    rng = np.random.default_rng(5)
    K = 256
    # all-zero weights with weight scale 0
    w0 = np.zeros((6, K), np.int8)
    x = workloads.normal(rng, 3, K)
    y = oracle.mul_mat(oracle.pack(w0, 0.0), 6, K, x)
    assert not np.isnan(y).any() and (y == 0).all()
    # a zero activation row gives +0.0 exactly, for any weights and scale
    w = workloads.ternary(rng, 6, K)
    x[1] = 0.0
    y = oracle.mul_mat(oracle.pack(w, 0.02), 6, K, x)
    assert (y[1].view(np.uint32) == 0).all()
    # weight scale 0 with nonzero weights: zeros (either sign), never NaN
    y = oracle.mul_mat(oracle.pack(w, 0.0), 6, K, x)
    assert not np.isnan(y).any() and (y == 0).all()


def test_all_zero_ternary_row_sum_correction():
    """All codes 1: sum(code*q) equals the row sum, so y is +0.0 for any x."""
    rng = np.random.default_rng(9)
    K = 384
    x = workloads.normal(rng, 5, K)
    y, dot = oracle.mul_mat(oracle.pack(np.zeros((4, K), np.int8), 0.5), 4, K, x, with_dot=True)
    _, _, rs = oracle.quantize_act(x)
    assert np.array_equal(dot, np.repeat(rs[:, None], 4, axis=1))
    assert (y.view(np.uint32) == 0).all()


def test_sign_invariants():
    rng = np.random.default_rng(13)
    rows, K, N = 16, 512, 3
    w = workloads.ternary(rng, rows, K)
    x = workloads.normal(rng, N, K)
    y = oracle.mul_mat(oracle.pack(w, 0.015), rows, K, x)
    yw = oracle.mul_mat(oracle.pack(-w, 0.015), rows, K, x)
    yx = oracle.mul_mat(oracle.pack(w, 0.015), rows, K, -x)
    nz = y != 0
    assert np.array_equal(yw[nz].view(np.uint32), (-y[nz]).view(np.uint32))
    assert np.array_equal(yx[nz].view(np.uint32), (-y[nz]).view(np.uint32))
    assert (yw[~nz] == 0).all() and (yx[~nz] == 0).all()


def test_quantization_error_bound():
    """|y - ws*sum(w*x)| <= ws*s*sum|w|/2 plus rounding of the two multiplies:
    the int8 step is s, so each |x - s*q| <= s/2."""
    rng = np.random.default_rng(17)
    rows, K, N, ws = 32, 1024, 4, 0.015
    w = workloads.ternary(rng, rows, K)
    x = workloads.with_outliers(rng, workloads.normal(rng, N, K))
    y = oracle.mul_mat(oracle.pack(w, ws), rows, K, x).astype(np.float64)
    _, s, _ = oracle.quantize_act(x)
    exact = np.float64(np.float32(ws)) * (x.astype(np.float64) @ w.astype(np.float64).T)
    bound = np.float64(np.float32(ws)) * s.astype(np.float64)[:, None] * np.abs(w).sum(1)[None, :] / 2
    bound = bound * (1 + 1e-6) + np.abs(exact) * 2.0 ** -22
    assert (np.abs(y - exact) <= bound).all()


def test_dot_on_row_slice_equals_full():
    """Groups never straddle rows, so a row slice of the payload is itself a
    valid I2_S payload (row stride K/4)."""
    rng = np.random.default_rng(19)
    rows, K = 10, 256
    w = workloads.ternary(rng, rows, K)
    p = oracle.pack(w, 1.0)
    q, _, _ = oracle.quantize_act(workloads.normal(rng, 2, K))
    full = oracle.dot(p, rows, K, q)
    part = oracle.dot(p[3 * K // 4:], 4, K, q)
    assert np.array_equal(part, full[:, 3:7])


# --- bias add (grouped decoder projections) ----------------------------------

def _bits_to_f32(b: int) -> np.float32:
    return np.array([b], dtype=np.uint32).view(np.float32)[0]


def test_bias_add_on_headroom_is_exact():
    g, h = bias_add(), headroom()
    K = h["K"]
    p = oracle.pack(np.ones((3, K), np.int8), h["ws"])
    y = oracle.mul_mat(p, 3, K, np.full((2, K), 127.0, np.float32))
    yb = oracle.add_bias(y, np.full(3, _bits_to_f32(g["headroom_bias_hex"]), np.float32))
    assert (yb.view(np.uint32) == g["headroom_y_bias_hex"]).all()


def test_bias_added_once_after_the_rounded_epilogue():
    """The worked case tells the plain reading (round the epilogue product,
    then one F32 add) from a fused multiply-add, whose result differs."""
    g = bias_add()
    K = 128
    x = np.zeros((1, K), np.float32)
    x[0, 0], x[0, 1] = 127.0, 3.0
    w = np.zeros((1, K), np.int8)
    w[0, 1] = 1
    p = oracle.pack(w, _bits_to_f32(g["fma_ws_hex"]))
    y, dot = oracle.mul_mat(p, 1, K, x, with_dot=True)
    assert int(dot[0, 0]) == 133
    assert int(y.view(np.uint32)[0, 0]) == g["fma_y_hex"]
    yn = oracle.add_bias(y, np.array([_bits_to_f32(g["fma_bias_neg_hex"])], np.float32))
    assert int(yn.view(np.uint32)[0, 0]) == g["fma_y_neg_hex"]
    assert g["fma_y_neg_hex"] != g["fma_fused_would_be_hex"]
    yt = oracle.add_bias(y, np.array([_bits_to_f32(g["fma_bias_tiny_hex"])], np.float32))
    assert int(yt.view(np.uint32)[0, 0]) == g["fma_y_tiny_hex"]


def test_bias_on_zero_activation_row():
    """y = +0 for an all-zero activation row, so y + b = b bitwise, and
    +0 + (-0) = +0."""
    rng = np.random.default_rng(29)
    rows, K = 6, 256
    p = oracle.pack(workloads.ternary(rng, rows, K), 0.015)
    y = oracle.mul_mat(p, rows, K, np.zeros((2, K), np.float32))
    assert (y.view(np.uint32) == 0).all()
    b = rng.standard_normal(rows).astype(np.float32)
    b[2] = np.float32(-0.0)
    yb = oracle.add_bias(y, b)
    expect = b.view(np.uint32).copy()
    expect[2] = 0
    assert (yb.view(np.uint32) == expect[None, :]).all()


def test_group_is_each_projection_on_the_same_activation():
    """A group is its projections one by one (quantization depends on x
    alone), each followed by its own bias if it has one."""
    rng = np.random.default_rng(31)
    K, N = 256, 3
    x = workloads.normal(rng, N, K)
    ws = [oracle.pack(workloads.ternary(rng, r, K), 0.02) for r in (8, 4)]
    b0 = rng.standard_normal(8).astype(np.float32)
    ys, ds = oracle.mul_mat_group([(ws[0], 8, b0), (ws[1], 4, None)], K, x, with_dot=True)
    y0, d0 = oracle.mul_mat(ws[0], 8, K, x, with_dot=True)
    y1, d1 = oracle.mul_mat(ws[1], 4, K, x, with_dot=True)
    assert np.array_equal(ds[0], d0) and np.array_equal(ds[1], d1)
    assert np.array_equal(ys[1].view(np.uint32), y1.view(np.uint32))
    assert np.array_equal(ys[0].view(np.uint32), (y0 + b0[None, :]).astype(np.float32).view(np.uint32))


def test_batched_is_the_same_rows_reindexed():
    """Quantization is per activation row, so a 3-D batch equals the 2-D op on
    its N*B rows, reshaped (the batched test's indexing, "ggml-cpu: ternary
    I2_S matmul kernel (VibeASR, 3/4)", Tests)."""
    rng = np.random.default_rng(37)
    rows, K, B, N = 9, 256, 3, 4
    p = oracle.pack(workloads.ternary(rng, rows, K), 0.02)
    x = workloads.normal(rng, B * N, K).reshape(B, N, K)
    yb, db = oracle.mul_mat_batched(p, rows, K, x, with_dot=True)
    y2, d2 = oracle.mul_mat(p, rows, K, x.reshape(B * N, K), with_dot=True)
    assert yb.shape == (B, N, rows)
    assert np.array_equal(db.reshape(B * N, rows), d2)
    assert np.array_equal(yb.reshape(B * N, rows).view(np.uint32), y2.view(np.uint32))


def test_sliced_oracle_is_the_whole_call():
    """mul_mat_sliced (output features split over threads) gives mul_mat's
    bits: every slice is a valid packed tensor and rows are independent."""
    rng = np.random.default_rng(77)
    for rows, K, N, threads in ((97, 384, 5, 4), (16, 128, 3, 16), (5, 1152, 2, 7), (300, 256, 1, 0)):
        w = workloads.ternary(rng, rows, K)
        x = workloads.normal(rng, N, K)
        p = oracle.pack(w, 0.0125)
        y, d = oracle.mul_mat(p, rows, K, x, with_dot=True)
        ys, ds = oracle.mul_mat_sliced(p, rows, K, x, with_dot=True, threads=threads)
        assert np.array_equal(ds, d)
        assert np.array_equal(ys.view(np.uint32), y.view(np.uint32))
