"""GPU parity: the HIP library against the CPU oracle, bit for bit.

Packed bytes, int8 activations, activation-scale bits, row sums, int32 dots and
F32 outputs must all be identical to the oracle's (the integer steps are exact
and the three F32 operations are single IEEE round-to-nearest operations in a
fixed order, so there is exactly one correct bit pattern).  Every case goes
through the C ABI (via the ctypes binding) on the same seeded inputs the
oracle gets.  Every output of every workload is compared, full-size shapes
included: the oracle runs over slices of the output features on the host
threads (oracle.mul_mat_sliced), which is the same computation split by
weight row.
"""

from __future__ import annotations

import itertools
import sys

import numpy as np
import pytest
import torch

import oracle
from exact import near_tie_rows, tie_margin_rows
from ternary_weight_integer_amd import i2s, workloads

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # only reachable when gpu tests are selected on a host without a GPU
    pytest.skip("no GPU visible", allow_module_level=True)

DEV = torch.device("cuda:0")


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def bits(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def gpu_pack(w: np.ndarray, ws: float) -> torch.Tensor:
    return i2s.i2s_pack(dev(w), ws)


def check_mul_mat(case: workloads.Case, kernel=0, variant=0, packed_gpu=None, packed_np=None, expected=None):
    """The whole op through the C ABI against the oracle on every output:
    int32 dots and F32 bits; `expected` = (y, dot) of the oracle when a
    caller checks several kernels against one oracle run."""
    rows, K, N = case.rows, case.K, case.N
    say(f"[parity] {case.name} rows={rows} K={K} N={N} kernel={kernel} variant={variant}")
    if packed_np is None:
        packed_np = oracle.pack(case.w, case.ws)
    if packed_gpu is None:
        packed_gpu = gpu_pack(case.w, case.ws)
    x = dev(case.x)
    y, d = i2s.i2s_mul_mat_ex(packed_gpu, rows, K, x, dot_out=True, kernel=kernel, variant=variant)
    # The same call without dot_out may take other store paths: it must give the same y.
    y_only = i2s.i2s_mul_mat_ex(packed_gpu, rows, K, x, kernel=kernel, variant=variant)
    y, d, y_only = host(y), host(d), host(y_only)
    assert np.array_equal(bits(y), bits(y_only)), "y differs with and without dot_out"
    if expected is None:
        expected = oracle.mul_mat_sliced(packed_np, rows, K, case.x, with_dot=True)
    ye, de = expected
    assert np.array_equal(d, de), f"dot mismatch at {np.argwhere(d != de)[:5]}"
    assert np.array_equal(bits(y), bits(ye)), f"y mismatch at {np.argwhere(bits(y) != bits(ye))[:5]}"
    return y


# --- pack ---------------------------------------------------------------------

@pytest.mark.parametrize("rows,K", [(1, 128), (3, 256), (64, 256), (70, 1152), (8960, 1536), (1536, 8960), (256, 1536)])
def test_pack_bytes_match_oracle(rows, K):
    say(f"[pack] rows={rows} K={K}")
    rng = np.random.default_rng(rows + K)
    w = workloads.ternary(rng, rows, K)
    p = host(gpu_pack(w, 0.015))
    pe = oracle.pack(w, 0.015)
    assert p.shape == pe.shape
    assert np.array_equal(p, pe)


def test_pack_maps_other_values_by_sign():
    rng = np.random.default_rng(1)
    w = rng.integers(-128, 128, size=(5, 384), dtype=np.int8)
    assert np.array_equal(host(gpu_pack(w, 2.0)), oracle.pack(w, 2.0))


# --- quantize -------------------------------------------------------------------

def _quant_inputs():
    out = [("small", workloads.small_case().x), ("decode_up", workloads.decode_up_case().x),
           ("down_relu", workloads.down_small_batch_case().x[:, :]),
           ("prefill", workloads.prefill_gate_case().x)]
    ties = near_tie_rows()
    L = max(r.size for r in ties)
    out.append(("near_ties", np.stack([np.pad(r, (0, L - r.size)) for r in ties])))
    margins = tie_margin_rows()
    L = max(r.size for r in margins)
    out.append(("tie_margins", np.stack([np.pad(r, (0, L - r.size)) for r in margins])))
    z = np.zeros((3, 256), np.float32)
    z[1] = np.float32(1e-7)
    z[2, 5] = np.float32(-3e-6)
    out.append(("zero_and_tiny", z))
    out.append(("headroom", np.full((2, 8960), 127.0, np.float32)))
    out.append(("long_k", workloads.normal(np.random.default_rng(6), 3, 10240)))  # the two-pass kernel (K > 9216)
    out.append(("mid_k", workloads.normal(np.random.default_rng(7), 5, 3072)))
    return out


@pytest.mark.parametrize("name,x", _quant_inputs(), ids=lambda v: v if isinstance(v, str) else "")
def test_quantize_matches_oracle(name, x):
    say(f"[quantize] {name} shape={x.shape}")
    q, s, rs = i2s.i2s_quantize_act(dev(x))
    qe, se, rse = oracle.quantize_act(x)
    assert np.array_equal(host(q), qe)
    assert np.array_equal(bits(host(s)), bits(se))
    assert np.array_equal(host(rs), rse)


@pytest.mark.parametrize("rows_of", [near_tie_rows, tie_margin_rows], ids=["on_ties", "at_margin"])
def test_near_ties_through_every_kernel(rows_of):
    """Activation rows on and around the .5 boundaries of x/s (on_ties), and
    just outside the 2^-14 band in which the kernels' quantizer switches from
    a reciprocal product to the quotient (at_margin), quantized inside each
    contraction path (the fused kernels quantize for themselves): any q off
    by one shows in dot (random codes over 96 weight rows) and y."""
    ties = rows_of()
    K = max(r.size for r in ties)
    x = np.stack([np.pad(r, (0, K - r.size)) for r in ties])
    N = x.shape[0]
    rng = np.random.default_rng(17)
    w = workloads.ternary(rng, 96, K)
    pnp = oracle.pack(w, 0.015)
    pg = gpu_pack(w, 0.015)
    ye, de = oracle.mul_mat(pnp, 96, K, x, with_dot=True)
    xg = dev(x)
    for kern in (0, 1, 2, 3, 4):
        for var in range(0 if kern == 0 else 1, (1 if kern == 0 else i2s.i2s_kernel_variants(kern)) + 1):
            try:
                y, d = i2s.i2s_mul_mat_ex(pg, 96, K, xg, dot_out=True, kernel=kern, variant=var)
            except i2s.I2SError as e:
                assert e.status == i2s.I2S_EKERNEL
                continue
            say(f"[{rows_of.__name__}] K={K} N={N} kernel={kern} variant={var}")
            assert np.array_equal(host(d), de), (kern, var)
            assert np.array_equal(bits(host(y)), bits(ye)), (kern, var)


# --- the five workloads, through the automatic dispatch that the benchmark uses -------

def test_small_case():
    check_mul_mat(workloads.small_case())


def test_decode_up_gemv_full():
    check_mul_mat(workloads.decode_up_case())


def test_down_small_batch_full():
    check_mul_mat(workloads.down_small_batch_case())


def test_prefill_gate_gemm_full():
    """The 512-row prefill on the gate shape, every one of its 512 x 8960
    outputs, through the automatic choice (the schedule the benchmark times)
    and through every GEMM variant."""
    case = workloads.prefill_gate_case()
    pnp = oracle.pack(case.w, case.ws)
    pg = gpu_pack(case.w, case.ws)
    exp = oracle.mul_mat_sliced(pnp, case.rows, case.K, case.x, with_dot=True)
    check_mul_mat(case, packed_gpu=pg, packed_np=pnp, expected=exp)
    for v in range(1, i2s.i2s_kernel_variants(2) + 1):
        check_mul_mat(case, kernel=2, variant=v, packed_gpu=pg, packed_np=pnp, expected=exp)


@pytest.mark.parametrize("case", workloads.layer_sweep_cases(), ids=lambda c: c.name)
def test_layer_sweep(case):
    check_mul_mat(case)


# --- every launch geometry gives the same bits (the M2 grid) -------------------------

GRID_K = (128, 1024, 1152)
GRID_DIM = (1, 2, 64, 70, 100)


@pytest.mark.parametrize("K", GRID_K)
def test_grid_all_kernels_and_variants(K):
    rng = np.random.default_rng(K + 5)
    wmax = workloads.ternary(rng, max(GRID_DIM), K)
    xmax = workloads.normal(rng, max(GRID_DIM), K)
    nv1, nv2 = i2s.i2s_kernel_variants(1), i2s.i2s_kernel_variants(2)
    for rows in GRID_DIM:
        w = wmax[:rows]
        pnp = oracle.pack(w, 0.015)
        pg = gpu_pack(w, 0.015)
        assert np.array_equal(host(pg), pnp)
        for N in GRID_DIM:
            x = xmax[:N]
            ye, de = oracle.mul_mat(pnp, rows, K, x, with_dot=True)
            combos = [(0, 0)] + [(2, v) for v in range(1, nv2 + 1)]
            if N <= 8:
                combos += [(1, v) for v in range(1, nv1 + 1)]
            if N <= 4:
                combos += [(3, v) for v in range(1, i2s.i2s_kernel_variants(3) + 1)]
            if N <= 64:
                combos += [(4, v) for v in range(0, i2s.i2s_kernel_variants(4) + 1)]
            say(f"[grid] K={K} rows={rows} N={N} combos={len(combos)}")
            xg = dev(x)
            for kern, var in combos:
                y, d = i2s.i2s_mul_mat_ex(pg, rows, K, xg, dot_out=True, kernel=kern, variant=var)
                y2 = i2s.i2s_mul_mat_ex(pg, rows, K, xg, kernel=kern, variant=var)
                y, d, y2 = host(y), host(d), host(y2)
                assert np.array_equal(d, de), (K, rows, N, kern, var)
                assert np.array_equal(bits(y), bits(ye)), (K, rows, N, kern, var)
                assert np.array_equal(bits(y2), bits(ye)), (K, rows, N, kern, var, "no dot_out")


# Longest K of each fused configuration (64 * lanes per row * chunk batches).
FUSED_MAX_K = {1: 1536, 2: 2048, 3: 2048, 4: 12288, 5: 10240, 6: 1536, 7: 1536, 8: 2048}


@pytest.mark.parametrize("N", [1, 2, 4])
def test_all_fused_variants_decode_shapes(N):
    """Fused quantize + GEMV variants on the decoder shapes (K = 1536 and the
    K = 8960 down projection); variants whose K limit is exceeded are refused."""
    for rows, K in ((8960, 1536), (1536, 1536), (256, 1536), (1536, 8960)):
        case = workloads.random_case(23, rows, K, N)
        pnp = oracle.pack(case.w, case.ws)
        pg = gpu_pack(case.w, case.ws)
        exp = oracle.mul_mat_sliced(pnp, rows, K, case.x, with_dot=True)
        for v in range(1, i2s.i2s_kernel_variants(3) + 1):
            if K > FUSED_MAX_K[v]:
                with pytest.raises(i2s.I2SError):
                    i2s.i2s_mul_mat_ex(pg, rows, K, dev(case.x), kernel=3, variant=v)
                continue
            check_mul_mat(case, kernel=3, variant=v, packed_gpu=pg, packed_np=pnp, expected=exp)


@pytest.mark.parametrize("rows,K,N", [(8960, 2048, 1), (8200, 1664, 3), (12288, 2048, 2), (12289, 1920, 1),
                                        (8193, 2048, 3)])
def test_fused_48_row_range(rows, K, N):
    """The automatic fused choice for 8192 < rows <= 12288 at 1536 < K <= 2048
    (48-row workgroups; a ragged last one at 8200 and 8193 rows, exactly 256 at
    12288) and just past it, every output against the oracle."""
    assert i2s.i2s_mul_mat_variant(rows, K, N) == (8 if rows <= 12288 else 2)
    case = workloads.random_case(29 + N, rows, K, N)
    check_mul_mat(case)


@pytest.mark.parametrize("N", [1, 3, 8])
def test_all_gemv_variants_full_decode_shapes(N):
    """GEMV variants on the decoder shapes (K = 1536 and 8960) against the oracle."""
    for rows, K in [(8960, 1536), (1536, 8960), (256, 1536)]:
        case = workloads.random_case(21, rows, K, N)
        pnp = oracle.pack(case.w, case.ws)
        pg = gpu_pack(case.w, case.ws)
        exp = oracle.mul_mat_sliced(pnp, rows, K, case.x, with_dot=True)
        for v in range(1, i2s.i2s_kernel_variants(1) + 1):
            check_mul_mat(case, kernel=1, variant=v, packed_gpu=pg, packed_np=pnp, expected=exp)


@pytest.mark.parametrize("N", [16, 17, 32, 33, 48, 64])
def test_all_skinny_variants_decode_shapes(N):
    """Skinny MFMA variants at every activation-block count (N <= 16, 32, 64)
    on the decoder shapes against the oracle, with a ragged weight-row count
    (not a multiple of 16 or of 4) for the scalar store path."""
    for rows, K in [(8960, 1536), (1536, 8960), (256, 1536), (1501, 1536)]:
        case = workloads.random_case(29 + N, rows, K, N)
        pnp = oracle.pack(case.w, case.ws)
        pg = gpu_pack(case.w, case.ws)
        exp = oracle.mul_mat_sliced(pnp, rows, K, case.x, with_dot=True)
        for v in range(1, i2s.i2s_kernel_variants(4) + 1):
            check_mul_mat(case, kernel=4, variant=v, packed_gpu=pg, packed_np=pnp, expected=exp)


def test_all_gemm_variants_prefill_shape():
    case = workloads.prefill_gate_case(N=200)
    pnp = oracle.pack(case.w, case.ws)
    pg = gpu_pack(case.w, case.ws)
    exp = oracle.mul_mat_sliced(pnp, case.rows, case.K, case.x, with_dot=True)
    for v in range(1, i2s.i2s_kernel_variants(2) + 1):
        check_mul_mat(case, kernel=2, variant=v, packed_gpu=pg, packed_np=pnp, expected=exp)


def test_gemm_variants_many_groups_per_wave():
    """N = 2048 on the gate shape: 9 subtiles per wave, so every resident
    variant runs several groups and a short last one (groups of 2, 3 and 4;
    16-18 with each wave's first two subtiles paired for whole-line stores,
    and cached stores because the waves hold several groups); every output
    checked."""
    case = workloads.prefill_gate_case(seed=5, N=2048)
    pnp = oracle.pack(case.w, case.ws)
    pg = gpu_pack(case.w, case.ws)
    exp = oracle.mul_mat_sliced(pnp, case.rows, case.K, case.x, with_dot=True)
    for v in (0, 11, 12, 13, 14, 16, 17, 18):
        check_mul_mat(case, kernel=2, variant=v, packed_gpu=pg, packed_np=pnp, expected=exp)


# --- edge cases -----------------------------------------------------------------------

@pytest.mark.parametrize("N", [1, 8, 64])
def test_headroom(N):
    case = workloads.headroom_case(N)
    y = check_mul_mat(case)
    assert y.shape == (N, 1536)
    assert (bits(y) == 0x46855999).all()  # every output: the closed form


@pytest.mark.parametrize("N,row", [(1, 0), (64, 17)])
def test_zero_activation_row(N, row):
    case = workloads.zero_row_case(N, row)
    y = check_mul_mat(case)
    assert y.shape == (N, 8960)
    assert (bits(y[row]) == 0).all()  # all 8960 features of the zero row are +0
    assert not np.isnan(y).any()


def test_zero_weights_zero_scale():
    rng = np.random.default_rng(4)
    for N in (1, 5, 33):
        case = workloads.Case("zero_w", np.zeros((96, 1024), np.int8), 0.0, workloads.normal(rng, N, 1024))
        y = check_mul_mat(case)
        assert not np.isnan(y).any() and (y == 0).all()


@pytest.mark.parametrize("rows,K,N", [(1, 128, 1), (17, 384, 9), (33, 640, 3), (130, 1152, 17), (8961 - 16, 1536, 2),
                                      (5, 8960, 100), (1000, 256, 300), (50, 10240, 3), (70, 3072, 6)])
def test_ragged_shapes(rows, K, N):
    case = workloads.random_case(rows + N, rows, K, N, ws=0.031)
    exp = oracle.mul_mat_sliced(oracle.pack(case.w, case.ws), rows, K, case.x, with_dot=True)
    check_mul_mat(case, expected=exp)
    if N <= 8:
        check_mul_mat(case, kernel=2, variant=1, expected=exp)


@pytest.mark.parametrize("seed", range(6))
def test_random_shapes_every_kernel(seed):
    """Seeded random shapes (rows 1..600, K a multiple of 128 up to 2560,
    N 1..80) through every kernel and variant that accepts them, against the
    oracle, bit for bit; every refusal must be I2S_EKERNEL."""
    rng = np.random.default_rng(1000 + seed)
    for _ in range(5):
        rows = int(rng.integers(1, 601))
        K = 128 * int(rng.integers(1, 21))
        N = int(rng.integers(1, 81))
        case = workloads.random_case(int(rng.integers(1 << 30)), rows, K, N, ws=float(rng.uniform(0.001, 0.1)))
        pnp = oracle.pack(case.w, case.ws)
        pg = gpu_pack(case.w, case.ws)
        ye, de = oracle.mul_mat(pnp, rows, K, case.x, with_dot=True)
        xg = dev(case.x)
        combos = [(0, 0)] + [(k, v) for k in (1, 2, 3, 4) for v in range(1, i2s.i2s_kernel_variants(k) + 1)]
        say(f"[random] seed={seed} rows={rows} K={K} N={N} combos={len(combos)}")
        ran = 0
        for kern, var in combos:
            try:
                y, d = i2s.i2s_mul_mat_ex(pg, rows, K, xg, dot_out=True, kernel=kern, variant=var)
            except i2s.I2SError as e:
                assert e.status == i2s.I2S_EKERNEL, (rows, K, N, kern, var, e.status)
                continue
            ran += 1
            assert np.array_equal(host(d), de), (rows, K, N, kern, var)
            assert np.array_equal(bits(host(y)), bits(ye)), (rows, K, N, kern, var)
        assert ran >= 2


def test_empty_inputs_are_noops():
    pg = gpu_pack(np.zeros((4, 128), np.int8), 1.0)
    y = torch.full((1, 4), 7.0, device=DEV)
    i2s.i2s_mul_mat(pg, 4, 128, torch.empty((0, 128), device=DEV), y=y)  # N == 0
    assert (host(y) == 7.0).all()
    yy = torch.full((3, 1), 5.0, device=DEV)
    i2s.i2s_mul_mat(gpu_pack(np.zeros((0, 128), np.int8), 1.0), 0, 128, torch.zeros((3, 128), device=DEV), y=yy)
    assert (host(yy) == 5.0).all()  # rows == 0


def test_error_codes_through_binding():
    pg = gpu_pack(np.zeros((4, 128), np.int8), 1.0)
    x = torch.zeros((2, 128), device=DEV)
    with pytest.raises(i2s.I2SError) as e:
        i2s.i2s_mul_mat(pg, 4, 128, x, workspace=torch.empty(64, dtype=torch.uint8, device=DEV))
    assert e.value.status == i2s.I2S_EWORKSPACE
    with pytest.raises(i2s.I2SError) as e:
        i2s.i2s_mul_mat_ex(pg, 4, 128, torch.zeros((9, 128), device=DEV), kernel=1)
    assert e.value.status == i2s.I2S_EKERNEL


def test_non_default_stream_and_reuse():
    """Calls on a side stream, reusing one workspace, in order."""
    case = workloads.random_case(8, 512, 1024, 12)
    pnp = oracle.pack(case.w, case.ws)
    pg = gpu_pack(case.w, case.ws)
    ye = oracle.mul_mat(pnp, 512, 1024, case.x)
    s = torch.cuda.Stream()
    ws = i2s.new_workspace(12, 1024, DEV)
    x = dev(case.x)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        outs = [i2s.i2s_mul_mat(pg, 512, 1024, x[: n], workspace=ws, stream=s) for n in (12, 3, 12)]
    s.synchronize()
    assert np.array_equal(bits(host(outs[0])), bits(ye))
    assert np.array_equal(bits(host(outs[1])), bits(ye[:3]))
    assert np.array_equal(bits(host(outs[2])), bits(ye))


def test_shared_workspace_feeds_several_weights():
    """One i2s_quantize_act_ws, then i2s_mul_mat_ws against q, k and v shaped
    weights: each result equals the oracle's."""
    rng = np.random.default_rng(30)
    K = 1536
    for N in (1, 16):
        x = workloads.normal(rng, N, K)
        ws = i2s.new_workspace(N, K, DEV)
        i2s.i2s_quantize_act_ws(dev(x), ws)
        for rows in (1536, 256, 256):
            w = workloads.ternary(rng, rows, K)
            pnp = oracle.pack(w, 0.015)
            y, d = i2s.i2s_mul_mat_ws(gpu_pack(w, 0.015), rows, K, N, ws, dot_out=True)
            ye, de = oracle.mul_mat(pnp, rows, K, x, with_dot=True)
            assert np.array_equal(host(d), de)
            assert np.array_equal(bits(host(y)), bits(ye))


@pytest.mark.parametrize("rows,K,N", [(8960, 1536, 1), (1536, 8960, 1), (1536, 8960, 8), (2048, 1536, 100)])
def test_graph_replay_matches_eager(rows, K, N):
    """i2s_mul_mat captured in a HIP graph: every replay, with eager work and
    synchronizations in between, gives the eager bits (and the oracle's)."""
    case = workloads.random_case(40 + N, rows, K, N)
    pg = gpu_pack(case.w, case.ws)
    x = dev(case.x)
    ws = i2s.new_workspace(N, K, DEV)
    y = torch.empty((N, rows), device=DEV)
    y_eager = host(i2s.i2s_mul_mat(pg, rows, K, x, workspace=ws)).copy()
    ye = oracle.mul_mat_sliced(oracle.pack(case.w, case.ws), rows, K, case.x)
    assert np.array_equal(bits(y_eager), bits(ye))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        i2s.i2s_mul_mat(pg, rows, K, x, workspace=ws, y=y)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        i2s.i2s_mul_mat(pg, rows, K, x, workspace=ws, y=y)
    for rep in range(4):
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(host(y)), bits(y_eager)), rep
        i2s.i2s_mul_mat(pg, rows, K, x, workspace=ws)  # eager work between replays
        torch.cuda.synchronize()
