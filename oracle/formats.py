"""E2M1 and E4M3 number formats (oracle; test infrastructure only).

NVFP4 is named, not defined, by the pages ([FS4 §1], [FS4 §2.1]).  Reading
taken: OCP E2M1 element codes and E4M3 "FN" scales.

E2M1 code (4 bits): bit 3 is the sign, bits 2..0 index the magnitudes
    0, 0.5, 1, 1.5, 2, 3, 4, 6
No infinities, no NaN.

E4M3FN byte: bit 7 sign, bits 6..3 exponent (bias 7), bits 2..0 mantissa.
    exponent 0:  value = mantissa * 2**-9            (subnormal)
    otherwise:   value = 2**(exponent-7) * (1 + mantissa/8)
    0x7F / 0xFF: NaN (no infinities); largest finite value 448 (0x7E).
"""
from __future__ import annotations

import numpy as np

E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)

# Midpoints between neighbouring grid magnitudes; a value exactly on a
# midpoint goes to the neighbour whose code index is even.
_E2M1_MIDS = (E2M1_GRID[:-1] + E2M1_GRID[1:]) / 2.0          # 0.25 .. 5.0
_E2M1_TIE_UP = np.array([(i + 1) % 2 == 0 for i in range(7)])  # upper index even?

E2M1_MAX = 6.0
E4M3_MAX = 448.0
E4M3_MAX_CODE = 0x7E
TENSOR_SCALE_DIVISOR = E2M1_MAX * E4M3_MAX  # 2688


def e2m1_decode(code) -> np.ndarray:
    """4-bit code(s) -> float64 value(s)."""
    c = np.asarray(code, dtype=np.int64)
    mag = E2M1_GRID[c & 7]
    return np.where((c & 8) != 0, -mag, mag)


def e2m1_rne_index(v) -> np.ndarray:
    """Magnitude index (0..7) of round-to-nearest-even of v >= 0 onto the E2M1
    grid, saturating at 6.

    Counts the midpoints v lies above; on a midpoint the even index wins.
    ``v`` is compared as given (float64 or exact), so callers pass a value whose
    side of every midpoint is the exact one.
    """
    v = np.asarray(v, dtype=np.float64)
    idx = np.zeros(v.shape, dtype=np.int64)
    for mid, up in zip(_E2M1_MIDS, _E2M1_TIE_UP):
        idx += (v > mid)
        if up:
            idx += (v == mid)
    return idx


def _e4m3_table() -> np.ndarray:
    vals = np.empty(256, dtype=np.float64)
    for b in range(256):
        e = (b >> 3) & 0xF
        m = b & 7
        if e == 0:
            mag = m * 2.0 ** -9
        else:
            mag = 2.0 ** (e - 7) * (1.0 + m / 8.0)
        if (b & 0x7F) == 0x7F:
            mag = np.nan
        vals[b] = -mag if (b & 0x80) else mag
    return vals


E4M3_VALUES = _e4m3_table()
_E4M3_POS = E4M3_VALUES[:E4M3_MAX_CODE + 1]          # codes 0..126, increasing
_E4M3_MIDS = (_E4M3_POS[:-1] + _E4M3_POS[1:]) / 2.0  # exact in fp64 (5 significant bits)


def e4m3_decode(byte) -> np.ndarray:
    """E4M3FN byte(s) -> float64 value(s) (NaN for 0x7F/0xFF)."""
    return E4M3_VALUES[np.asarray(byte, dtype=np.int64) & 0xFF]


def e4m3_rne_satfinite(q) -> np.ndarray:
    """Non-negative value(s) -> E4M3FN code of round-to-nearest-even, with
    values above 448 mapped to 448 ("satfinite").

    Reading: the scale uses the same round-to-nearest-even as the elements;
    saturation keeps every scale finite (without it, values from 464 up would
    round to the NaN code).

    Nearest of the 127 finite non-negative values; a value exactly halfway
    between two of them takes the one with the even code.
    """
    q0 = np.asarray(q, dtype=np.float64)
    if np.any(~(q0 >= 0)):
        raise ValueError("e4m3_rne_satfinite expects finite non-negative input")
    q = np.atleast_1d(q0)
    # number of midpoints strictly below q, plus ties resolved to the even code
    below = np.searchsorted(_E4M3_MIDS, q, side="left")       # mids < q
    at = np.searchsorted(_E4M3_MIDS, q, side="right") - below  # q == mid (0 or 1)
    code = below.copy()
    tie = at > 0
    # on a tie between code `below` and `below + 1`, pick the even one
    code[tie] = np.where(below[tie] % 2 == 0, below[tie], below[tie] + 1)
    return np.minimum(code, E4M3_MAX_CODE).astype(np.uint8).reshape(q0.shape)


def tensor_scale_from_amax(amax: float) -> np.float32:
    """FP32 per-tensor decode scale s_t = RNE_fp32(amax / (6 * 448)).

    Reading: the tensor scale is chosen so that the block holding the tensor's
    largest magnitude gets the largest E4M3 scale (448) and its largest element
    the largest E2M1 magnitude (6).

    amax is a float32 value (24 significant bits); the fp64 quotient is then
    rounded once to fp32.  The quotient amax/2688 is never an fp32 rounding
    midpoint unless it is exact, and its distance to one is far above the fp64
    rounding error, so this equals the exactly rounded real quotient (the exact
    twin in ``oracle.exact`` checks it).
    """
    return np.float32(float(amax) / TENSOR_SCALE_DIVISOR)
