"""Q-AdamW second-moment state codec (oracle; test infrastructure only).

[FS4 §2.2]: the AdamW second moment v_t is stored in NVFP4 after three
steps: a square root that shortens its heavy tail, the removal of a tile
mean (the common positive part, kept in BF16) that leaves a roughly
zero-mean residual, and a Hadamard transform that spreads the residual's
localized energy.  Reconstruction inverts the transform and the mean, then
squares.  The pages fix none of the sizes or orders; the readings taken:

* v is fp32 [R, C] (R, C multiples of 16), non-negative.
* Tiles are 16 x 16; the mean of s = sqrt(v) over a tile is kept as BF16
  (fp64 -> fp32 -> BF16, each round-to-nearest-even), and the residual uses
  that rounded mean: r = s - mu.
* The transform is the orthonormal 16-point Hadamard matrix H/4 (Sylvester
  order) along each row's 16-element groups, the same groups as the NVFP4
  blocks; it is its own inverse.
* The transformed residual h, rounded to fp32, is quantized row-wise with the
  two-level NVFP4 quantizer (one tensor scale).
* Decode: h_hat = dequantized codes, r_hat = H/4 h_hat, s_hat = r_hat + mu,
  v_hat = fp32(s_hat^2).

All arithmetic before a rounding to fp32 or BF16 is fp64 in a fixed order
(the butterflies below, the tile sum as the sum of its 16 row-group sums in
row order), so that an implementation following the same order reaches the
same fp32 values, and the quantizer the same codes.
"""
from __future__ import annotations

import numpy as np

from .lora import bf16_rne
from .quantize import NVFP4, dequantize, quantize

TILE = 16


def fwht16(x) -> np.ndarray:
    """Unnormalised Walsh-Hadamard transform (Sylvester order) of each
    16-element group along the last axis, in float64, as butterflies
    (a, b) -> (a + b, a - b) with strides 1, 2, 4, 8."""
    y = np.array(x, dtype=np.float64, copy=True)
    shp = y.shape
    y = y.reshape(-1, 16)
    h = 1
    while h < 16:
        y = y.reshape(-1, 16 // (2 * h), 2, h)
        a, b = y[:, :, 0, :].copy(), y[:, :, 1, :].copy()
        y[:, :, 0, :] = a + b
        y[:, :, 1, :] = a - b
        y = y.reshape(-1, 16)
        h *= 2
    return y.reshape(shp)


def hadamard16(x) -> np.ndarray:
    """The orthonormal transform H/4 on each 16-element group (float64)."""
    return fwht16(x) * 0.25


def tile_means(s64) -> np.ndarray:
    """BF16 means (as float64) of the 16 x 16 tiles of s64 [R, C]: each
    row-group sum is the butterflies' first output, the tile sum adds the 16
    row-groups in row order."""
    r, c = s64.shape
    g = fwht16(s64)[:, 0::16]                          # row-group sums [R, C/16]
    g = g.reshape(r // TILE, TILE, c // TILE)
    tot = np.zeros((r // TILE, c // TILE))
    for i in range(TILE):
        tot = tot + g[:, i, :]
    return bf16_rne(tot / (TILE * TILE))


def vstate_encode(v):
    """Returns (NVFP4 row view of h, means float64 [R/16, C/16] holding BF16
    values, h float32)."""
    v = np.asarray(v, dtype=np.float32)
    r, c = v.shape
    if r % TILE or c % TILE:
        raise ValueError("v must be [R, C] with R and C multiples of 16")
    s = np.sqrt(v.astype(np.float64))
    mu = tile_means(s)
    res = s - np.repeat(np.repeat(mu, TILE, axis=0), TILE, axis=1)
    h = hadamard16(res).astype(np.float32)
    view, _, _ = quantize(h, rowwise=True, colwise=False)
    return view, mu, h


def vstate_decode(view: NVFP4, mu) -> np.ndarray:
    """v_hat float32 [R, C] from the stored view and BF16 tile means."""
    h_hat = dequantize(view)
    s_hat = hadamard16(h_hat) + np.repeat(np.repeat(np.asarray(mu, np.float64), TILE, axis=0), TILE, axis=1)
    return (s_hat * s_hat).astype(np.float32)
