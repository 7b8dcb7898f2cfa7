"""Host-side checks of the work deals the contraction kernels rely on: every
output tile (I8_S / W8A8 MFMA contraction) and every 16-row weight subtile
(I2_S activation-resident GEMM) is taken by exactly one workgroup or wave.

The functions below restate the launcher's grid choice and the kernels'
index arithmetic (csrc/i8s.hip: launch_mfma and the tile cursor of
i8s_mm_mfma_kernel; csrc/i2s.hip: the subtile deal of gemm_res_kernel) in
Python, over many shapes, including empty and ragged ones.  They run on the
CPU; the GPU parity tests check the kernels' outputs themselves.
"""

from __future__ import annotations

import itertools

import pytest

XCDS = 8
RESIDENT_GROUPS = 512
MAP_STRIDE, MAP_XLOCAL, MAP_WLOCAL = 0, 1, 2


def mfma_grid(OC: int, N: int, TM: int, TN: int, cap: int = RESIDENT_GROUPS):
    """(map, rep, grid) as launch_mfma chooses them."""
    tiles_o, tiles_n = -(-OC // TM), -(-N // TN)
    x_larger = N >= OC
    if x_larger and tiles_o >= 1 and tiles_n >= XCDS and XCDS * tiles_o <= cap:
        r = min(-(-tiles_n // XCDS), cap // (XCDS * tiles_o))
        return MAP_XLOCAL, r, XCDS * tiles_o * r
    if not x_larger and tiles_n >= 1 and tiles_o >= XCDS and XCDS * tiles_n <= cap:
        r = min(-(-tiles_o // XCDS), cap // (XCDS * tiles_n))
        return MAP_WLOCAL, r, XCDS * tiles_n * r
    prod = tiles_o * tiles_n
    g = (prod if prod > 0 else 1) if prod < cap else cap
    if 1 <= tiles_o <= cap:
        per = tiles_n if tiles_n < cap // tiles_o else cap // tiles_o
        g = tiles_o * (per if per > 0 else 1)
    return MAP_STRIDE, 1, g


def mfma_tiles_of(b: int, G: int, tiles_o: int, tiles_n: int, mp: int, rep: int):
    """The (channel block, row block) tiles workgroup b walks, as its cursor steps."""
    tiles = tiles_o * tiles_n
    if tiles == 0:
        return []
    if mp == MAP_STRIDE:
        ob, nb = b % tiles_o, b // tiles_o
        step_o, step_n = G % tiles_o, G // tiles_o
        mine = (tiles - b + G - 1) // G if b < tiles else 0
    else:
        xcd, sl, stride = b % XCDS, b // XCDS, XCDS * rep
        fixed_n = tiles_o if mp == MAP_XLOCAL else tiles_n
        fixed, start = sl % fixed_n, xcd + XCDS * (sl // fixed_n)
        local_n = tiles_n if mp == MAP_XLOCAL else tiles_o
        mine = (local_n - start + stride - 1) // stride if start < local_n else 0
        if mp == MAP_XLOCAL:
            ob, nb, step_o, step_n = fixed, start, 0, stride
        else:
            ob, nb, step_o, step_n = start, fixed, stride, 0
    out = []
    for _ in range(mine):
        out.append((ob, nb))
        ob += step_o
        nb += step_n
        if mp == MAP_STRIDE and ob >= tiles_o:
            ob -= tiles_o
            nb += 1
    return out


TILE_SHAPES = [(128, 64), (64, 64), (128, 128), (64, 128)]
DIMS = [0, 1, 63, 64, 65, 127, 128, 129, 256, 300, 513, 1024, 1536, 2048, 4100, 6000, 8960, 12000]


@pytest.mark.parametrize("TM,TN", TILE_SHAPES)
def test_mfma_contraction_visits_every_tile_once(TM, TN):
    checked = 0
    for OC, N in itertools.product(DIMS, DIMS):
        mp, rep, g = mfma_grid(OC, N, TM, TN)
        tiles_o, tiles_n = -(-OC // TM), -(-N // TN)
        assert 1 <= g <= RESIDENT_GROUPS, (OC, N, g)
        seen = {}
        for b in range(g):
            for t in mfma_tiles_of(b, g, tiles_o, tiles_n, mp, rep):
                assert 0 <= t[0] < tiles_o and 0 <= t[1] < tiles_n, (OC, N, mp, b, t)
                assert t not in seen, (OC, N, mp, b, t, seen[t])
                seen[t] = b
        assert len(seen) == tiles_o * tiles_n, (OC, N, mp, len(seen))
        if mp != MAP_STRIDE:  # an XCD-local deal keeps each block of the local operand on one XCD
            for (ob, nb), b in seen.items():
                local = nb if mp == MAP_XLOCAL else ob
                assert b % XCDS == local % XCDS, (OC, N, mp, ob, nb, b)
        checked += 1
    assert checked == len(DIMS) ** 2


def gemm_res_deal(msub: int, waves: int, pair: bool):
    """Per wave, the block-local subtiles it holds, in order, as
    gemm_res_kernel deals them: round-robin, or (pair) its first two adjacent
    and the rest round-robin from 2 * waves."""
    out = []
    for w in range(waves):
        if pair:
            mine = (2 * w < msub) + (2 * w + 1 < msub) + (
                (msub - 2 * waves - w + waves - 1) // waves if msub > 2 * waves + w else 0)
            local = [2 * w + i if i < 2 else 2 * waves + w + waves * (i - 2) for i in range(mine)]
        else:
            mine = (msub - w + waves - 1) // waves if msub > w else 0
            local = [w + waves * i for i in range(mine)]
        out.append(local)
    return out


@pytest.mark.parametrize("pair", [False, True])
def test_resident_gemm_deals_every_subtile_once(pair):
    for waves in (4, 8):
        for msub in range(0, 8 * waves + 3):
            deal = gemm_res_deal(msub, waves, pair)
            flat = [s for local in deal for s in local]
            assert sorted(flat) == list(range(msub)), (waves, msub, pair, deal)
            for local in deal:
                assert local == sorted(local)  # a wave's subtiles below msub are a prefix of its list
            if pair:
                for w, local in enumerate(deal):
                    if len(local) >= 2:  # the first two are adjacent: their outputs share 128-byte lines
                        assert local[:2] == [2 * w, 2 * w + 1]
            counts = [len(local) for local in deal]
            assert max(counts) - min(counts) <= (1 if not pair else 3), (waves, msub, pair, counts)


def test_prefill_block_deal():
    """The 8960 x 1536, N = 512 prefill: 18 subtiles per block over 8 waves;
    with pairing, waves 0 and 1 hold three (a pair and subtile 16 or 17), the
    others a pair, so every SIMD (waves w and w + 4) carries 5 or 4."""
    deal = gemm_res_deal(18, 8, True)
    assert deal[0] == [0, 1, 16] and deal[1] == [2, 3, 17]
    assert all(len(deal[w]) == 2 for w in range(2, 8))
    assert [len(deal[s]) + len(deal[s + 4]) for s in range(4)] == [5, 5, 4, 4]
