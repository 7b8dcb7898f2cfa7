"""Exact-arithmetic helpers for pinning the oracle (test side only).

Everything here is computed with Python integers and ``fractions.Fraction``:
an IEEE binary32 operation is modelled as "exact rational result, then round
to the nearest binary32, ties to even", written out below from the IEEE 754
definition.  None of it calls the oracle or the GPU library, so agreement
between these helpers and the oracle is evidence about the oracle, not a
re-run of it.
"""

from __future__ import annotations

from fractions import Fraction

import numpy as np

_F32_MANT = 23
_F32_EMIN = -126
_F32_EMAX = 127


def f32_round(q: Fraction) -> np.float32:
    """Nearest binary32 to the exact rational q (ties to even)."""
    if q == 0:
        return np.float32(0.0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    # e = floor(log2(a)), exactly.
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    if e < _F32_EMIN:
        quantum = Fraction(2) ** (_F32_EMIN - _F32_MANT)   # subnormal spacing
    else:
        quantum = Fraction(2) ** (e - _F32_MANT)
    m = a / quantum
    lo = m.numerator // m.denominator
    rem = m - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    val = lo * quantum
    if val >= Fraction(2) ** (_F32_EMAX + 1):
        return np.float32(sign * np.inf)
    return np.float32(sign * float(val))  # float(val) is exact: val is a binary32 value


def frac(v) -> Fraction:
    return Fraction(float(v))


def round_half_away(v: np.float32) -> int:
    """Exact round-half-away-from-zero of a finite float to an integer."""
    a = abs(frac(v))
    r = int(a + Fraction(1, 2))  # floor(a + 1/2) for a >= 0
    return -r if v < 0 else r


AMAX_FLOOR = f32_round(Fraction(1, 100000))  # the binary32 literal 1e-5f


def quantize_row(x) -> tuple[list[int], np.float32, int]:
    """(q, s, row_sum) of one F32 row: amax floored at 1e-5f, s = f32(amax/127),
    q = clamp(round_half_away(f32(x/s)), -127, 127)."""
    amax = max((abs(frac(v)) for v in x), default=Fraction(0))
    if amax < frac(AMAX_FLOOR):
        amax = frac(AMAX_FLOOR)
    s = f32_round(amax / 127)
    q = []
    for v in x:
        r = round_half_away(f32_round(frac(v) / frac(s)))
        q.append(max(-127, min(127, r)))
    return q, s, sum(q)


def f32_mul(a, b) -> np.float32:
    """IEEE binary32 product of two finite binary32 values: the exact product
    rounded to nearest; a zero result takes the XOR of the operands' signs."""
    r = f32_round(frac(a) * frac(b))
    if r == 0 and (np.signbit(np.float32(a)) != np.signbit(np.float32(b))):
        return np.float32(-0.0)
    return r


def epilogue(sum_wq: int, ws: float, s: np.float32) -> np.float32:
    """F32(F32(sum_wq) * F32(ws * s)): the two rounded multiplies."""
    t = f32_mul(np.float32(ws), s)
    d = f32_round(Fraction(sum_wq))
    return f32_mul(d, t)


def f32_bits(v) -> int:
    return int(np.asarray(v, dtype=np.float32).view(np.uint32))


def near_tie_rows(amaxes=(100.0, 3.3, 0.77, 12345.678)) -> list[np.ndarray]:
    """F32 rows (length a multiple of 128) whose values sit on, or one or two
    floats either side of, each .5 boundary of x/s, for scales s that are not
    powers of two, so that the last bit of the division decides q."""
    rows = []
    for amax in (np.float32(a) for a in amaxes):
        s = f32_round(frac(amax) / 127)
        vals = [amax]
        for m in range(-126, 127):
            centre = np.float32(float((frac(m) + Fraction(1, 2)) * frac(s)))
            up, down = np.float32(np.inf), np.float32(-np.inf)
            u1 = np.nextafter(centre, up)
            d1 = np.nextafter(centre, down)
            vals += [np.nextafter(d1, down), d1, centre, u1, np.nextafter(u1, up)]
        row = np.array([v for v in vals if abs(v) <= amax], dtype=np.float32)
        pad = (-row.size) % 128
        rows.append(np.concatenate([row, np.zeros(pad, np.float32)]))
    return rows


def tie_margin_rows(amaxes=(100.0, 3.3, 0.77, 12345.678)) -> list[np.ndarray]:
    """F32 rows whose values put x/s at 1.25, 2 and 4 times 2^-14 either side
    of each .5 boundary (and none nearer): a quantizer that rounds a product
    x * (1/s) instead of the quotient, and switches to the quotient only for
    values within 2^-14 of a boundary, takes its fast path on every value of
    these rows, at the edge of its error margin."""
    rows = []
    for amax in (np.float32(a) for a in amaxes):
        s = f32_round(frac(amax) / 127)
        vals = [amax]
        for m in range(-126, 127):
            for k in (Fraction(5, 4), Fraction(2), Fraction(4)):
                for sign in (-1, 1):
                    vals.append(np.float32(float((frac(m) + Fraction(1, 2) + sign * k / 2**14) * frac(s))))
        row = np.array([v for v in vals if abs(v) <= amax], dtype=np.float32)
        pad = (-row.size) % 128
        rows.append(np.concatenate([row, np.zeros(pad, np.float32)]))
    return rows
