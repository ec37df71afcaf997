"""Two-level NVFP4 block quantizer (oracle; test infrastructure only).

What it computes ([FS4 §2.1]: the residual W_res is held in NVFP4; [FS4 §2.3]:
the Newton-Schulz products run on NVFP4 operands; the format itself is the
reading stated in ``oracle.formats``):

1. amax_t = max |x| over the whole tensor; s_t = RNE_fp32(amax_t / 2688).
2. For every block of 16 consecutive elements along the blocked dimension:
   amax_b = max |x| over the block;
   s_b    = E4M3 round-to-nearest-even, satfinite, of amax_b / (6 s_t)
            (0 when s_t = 0).
3. Every element: code = sign(x) | E2M1 RNE index of |x| / (s_b s_t), the
   division taken exactly (as a real number).  When s_b s_t = 0 the code is
   the signed zero.  The sign is the IEEE sign bit, so -0.0 and negatives that
   round to zero give code 8.
4. Packing: byte j of a row holds code 2j in its low nibble and code 2j+1 in
   its high nibble.

Layouts
-------
row-wise:    blocks of 16 along the last (contiguous) dimension of x [R, C];
             codes [R, C/2], scales [R, C/16].
column-wise: the row-wise quantization of x^T: blocks of 16 along R;
             codes [C, R/2], scales [C, R/16].  Different blocks, so a
             different quantization, not a transpose of the row-wise codes.
Both layouts share the one tensor scale.

Exactness of the float64 steps (inputs are float32 values):
* 6 s_t and s_b s_t are products of <= 24-bit and <= 4-bit significands, exact.
* amax_b / (6 s_t): an E4M3 midpoint has 5 significant bits, so a quotient that
  is not a midpoint sits at least ~2^-32 (relative) away from it, far above the
  2^-53 rounding of the fp64 division; a quotient that is a midpoint is
  representable and comes out exact.  Same argument for |x| / (s_b s_t) against
  the E2M1 midpoints.  ``oracle.exact`` redoes all of it in rationals.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .formats import (TENSOR_SCALE_DIVISOR, e2m1_decode, e2m1_rne_index, e4m3_decode,
                      e4m3_rne_satfinite, tensor_scale_from_amax)

BLOCK = 16


@dataclass
class NVFP4:
    """One NVFP4 view: the blocked (contraction) dimension is ``cols``."""
    codes: np.ndarray    # uint8 [rows, cols/2]
    scales: np.ndarray   # uint8 [rows, cols/16], raw E4M3FN bytes
    tscale: np.float32   # per-tensor decode scale
    rows: int
    cols: int


def _as_f32(x) -> np.ndarray:
    x = np.asarray(x)
    if x.dtype != np.float32:
        raise TypeError("oracle quantizer takes float32 values (widen bf16 exactly first)")
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite input")
    return x


def tensor_amax(x) -> np.float32:
    x = _as_f32(x)
    return np.float32(np.max(np.abs(x))) if x.size else np.float32(0.0)


def tensor_scale(x) -> np.float32:
    return tensor_scale_from_amax(tensor_amax(x))


def quantize_rows(x, s_t) -> NVFP4:
    """Row-wise quantization of float32 x [R, C] (C % 16 == 0) with the given
    tensor decode scale s_t."""
    x = _as_f32(x)
    if x.ndim != 2 or x.shape[1] % BLOCK:
        raise ValueError("x must be 2-D with a multiple of 16 columns")
    rows, cols = x.shape
    s_t64 = float(np.float32(s_t))
    blocks = x.astype(np.float64).reshape(rows, cols // BLOCK, BLOCK)
    mag = np.abs(blocks)
    amax_b = mag.max(axis=2)
    if s_t64 > 0.0:
        sb_code = e4m3_rne_satfinite(amax_b / (6.0 * s_t64))
    else:
        sb_code = np.zeros(amax_b.shape, dtype=np.uint8)
    step = e4m3_decode(sb_code) * s_t64                    # s_b s_t, exact
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(step[..., None] > 0, mag / step[..., None], 0.0)
    idx = e2m1_rne_index(ratio)
    idx = np.where(step[..., None] > 0, idx, 0)
    sign = np.signbit(blocks).astype(np.int64) << 3
    codes = (idx | sign).reshape(rows, cols)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return NVFP4(packed, sb_code, np.float32(s_t64), rows, cols)


def quantize(x, rowwise: bool = True, colwise: bool = True):
    """Quantize float32 x [R, C] with one tensor scale.

    Returns (row_view or None, col_view or None, s_t).
    """
    x = _as_f32(x)
    s_t = tensor_scale(x)
    row = quantize_rows(x, s_t) if rowwise else None
    col = quantize_rows(np.ascontiguousarray(x.T), s_t) if colwise else None
    return row, col, s_t


def unpack_codes(packed) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8).astype(np.int64)
    out = np.empty((p.shape[0], p.shape[1] * 2), dtype=np.int64)
    out[:, 0::2] = p & 0xF
    out[:, 1::2] = p >> 4
    return out


def block_values(v: NVFP4) -> np.ndarray:
    """Block-level dequantized values e2m1(code) * e4m3(s_b) in float64 (exact),
    without the tensor scale."""
    codes = unpack_codes(v.codes)
    scale = np.repeat(e4m3_decode(v.scales), BLOCK, axis=1)
    return e2m1_decode(codes) * scale


def dequantize(v: NVFP4) -> np.ndarray:
    """x_hat = e2m1(code) * e4m3(s_b) * s_t, float64 (exact)."""
    return block_values(v) * float(v.tscale)


__all__ = ["NVFP4", "BLOCK", "tensor_amax", "tensor_scale", "quantize_rows", "quantize",
           "unpack_codes", "block_values", "dequantize", "TENSOR_SCALE_DIVISOR"]
