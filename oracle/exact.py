"""The NVFP4 quantizer in exact rational arithmetic (oracle; test
infrastructure only).

A brute-force twin of ``oracle.quantize`` for tiny tensors: every quantity is
a ``fractions.Fraction``, every rounding picks the nearest representable value
by direct comparison, and the format tables are rebuilt here from the bit
definitions rather than imported.  The float64 quantizer is checked against it
bit for bit.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

# E2M1 magnitudes, index 0..7 (bit 3 of a code is the sign)
E2M1_MAGS = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2),
             Fraction(2), Fraction(3), Fraction(4), Fraction(6)]


def e4m3_value(byte: int) -> Fraction:
    """Exact value of a finite non-negative E4M3FN code 0..126."""
    e, m = (byte >> 3) & 0xF, byte & 7
    if e == 0:
        return Fraction(m, 2 ** 9)
    return Fraction(2) ** (e - 7) * (1 + Fraction(m, 8))


E4M3_FINITE = [e4m3_value(b) for b in range(127)]


def nearest_even(q: Fraction, values) -> int:
    """Index of the value nearest to q in the increasing list ``values``; on an
    exact tie the even index; values beyond the last saturate to it."""
    if q >= values[-1]:
        return len(values) - 1
    best = 0
    for i in range(1, len(values)):
        if values[i] >= q:
            lo, hi = values[i - 1], values[i]
            d_lo, d_hi = q - lo, hi - q
            if d_lo < d_hi:
                best = i - 1
            elif d_hi < d_lo:
                best = i
            else:
                best = i - 1 if (i - 1) % 2 == 0 else i
            break
    return best


def round_to_f32(q: Fraction) -> Fraction:
    """Exact round-to-nearest-even of a non-negative rational onto float32
    (normal and subnormal range; q is far below the overflow threshold here)."""
    if q == 0:
        return Fraction(0)
    # find e with 2^e <= q < 2^(e+1)
    e = q.numerator.bit_length() - q.denominator.bit_length()
    if Fraction(2) ** e > q:
        e -= 1
    elif Fraction(2) ** (e + 1) <= q:
        e += 1
    e = max(e, -126)                       # subnormals share the 2^-149 step
    ulp = Fraction(2) ** (e - 23)
    n = q / ulp
    k = n.numerator // n.denominator
    rem = n - k
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and k % 2 == 1):
        k += 1
    return k * ulp


def f32_fraction(v: np.float32) -> Fraction:
    return Fraction(float(np.float32(v)))


def quantize_rows_exact(x: np.ndarray, s_t: Fraction):
    """Row-wise NVFP4 quantization with exact arithmetic.  x: float32 [R, C].
    Returns (unpacked codes int [R, C], scale codes int [R, C/16])."""
    rows, cols = x.shape
    codes = np.zeros((rows, cols), dtype=np.int64)
    scales = np.zeros((rows, cols // 16), dtype=np.int64)
    for r in range(rows):
        for b in range(cols // 16):
            blk = [Fraction(float(v)) for v in x[r, 16 * b:16 * b + 16]]
            amax_b = max(abs(v) for v in blk)
            if s_t == 0:
                sb = 0
            else:
                sb = nearest_even(amax_b / (6 * s_t), E4M3_FINITE)
            scales[r, b] = sb
            step = E4M3_FINITE[sb] * s_t
            for j, v in enumerate(blk):
                sign = 8 if np.signbit(x[r, 16 * b + j]) else 0
                idx = 0 if step == 0 else nearest_even(abs(v) / step, E2M1_MAGS)
                codes[r, 16 * b + j] = sign | idx
    return codes, scales


def quantize_exact(x: np.ndarray):
    """Both layouts of float32 x with one exact tensor scale.
    Returns (row codes, row scales, col codes, col scales, s_t as Fraction)."""
    amax = max((abs(Fraction(float(v))) for v in x.reshape(-1)), default=Fraction(0))
    s_t = round_to_f32(amax / 2688)
    rc, rs = quantize_rows_exact(x, s_t)
    cc, cs = quantize_rows_exact(np.ascontiguousarray(x.T), s_t)
    return rc, rs, cc, cs, s_t


def dot_exact(a_vals, b_vals) -> Fraction:
    return sum((Fraction(float(p)) * Fraction(float(q)) for p, q in zip(a_vals, b_vals)), Fraction(0))
