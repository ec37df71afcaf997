"""Q-AdamW optimizer-state codecs (oracle; test infrastructure only): the
second moment below, the first moment at the end of the module.

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


# ---------------------------------------------------------------------------
# First moment, [FS4 §2.2]: Hadamard mixing, then stochastic rounding and
# adaptive 4/6 quantization.  Readings:
#
# * h = fp32(H/4 m) on each 16-element row group (as for v, no root, no mean);
#   one tensor scale s_t = RNE_fp32(amax(h) / 2688) as in NVFP4.
# * Adaptive 4/6 ("four over six"): each block tries the E4M3 scale that maps
#   its amax to 6 and the one that maps it to 4, s_k = E4M3(amax_b / (k s_t)),
#   quantizes the block to nearest with each, and keeps the one with the
#   smaller sum of squared errors (6 on a tie).
# * Stochastic rounding with the kept scale: y = |h| / (s_b s_t); at or above
#   6 the code saturates; otherwise y lies in [g_lo, g_hi) between two E2M1
#   magnitudes and rounds up exactly when u < (y - g_lo) / (g_hi - g_lo),
#   u = r * 2^-32 for a caller-supplied uint32 r per element.
# * Decode: m_hat = fp32(H/4 dequant).
# All of it in fp64 with the divisions and comparisons stated.

from .formats import E2M1_GRID, e2m1_rne_index, e4m3_decode, e4m3_rne_satfinite
from .quantize import tensor_scale


def _sse_rne(mag, step):
    """Sum over the last axis of squared errors of round-to-nearest E2M1 at
    the given step (float64; zero step gives the magnitudes' own squares)."""
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(step[..., None] > 0, mag / step[..., None], 0.0)
    val = E2M1_GRID[e2m1_rne_index(ratio)] * step[..., None]
    err = (mag - val) ** 2
    tot = np.zeros(err.shape[:-1])
    for k in range(err.shape[-1]):          # the elements of a block in order
        tot = tot + err[..., k]
    return tot


def mstate_encode(m, rnd):
    """First-moment codec.  m fp32 [R, C] (C % 16 == 0), rnd uint32 [R, C].
    Returns (NVFP4 row view, h float32)."""
    m = np.asarray(m, dtype=np.float32)
    rows, cols = m.shape
    h = hadamard16(m.astype(np.float64)).astype(np.float32)
    s_t = tensor_scale(h)
    st64 = float(s_t)
    blocks = h.astype(np.float64).reshape(rows, cols // 16, 16)
    mag = np.abs(blocks)
    amax_b = mag.max(axis=2)
    if st64 > 0.0:
        s6 = e4m3_rne_satfinite(amax_b / (6.0 * st64))
        s4 = e4m3_rne_satfinite(amax_b / (4.0 * st64))
    else:
        s6 = s4 = np.zeros(amax_b.shape, dtype=np.uint8)
    e6 = _sse_rne(mag, e4m3_decode(s6) * st64)
    e4 = _sse_rne(mag, e4m3_decode(s4) * st64)
    sb = np.where(e4 < e6, s4, s6).astype(np.uint8)
    step = e4m3_decode(sb) * st64
    with np.errstate(divide="ignore", invalid="ignore"):
        y = np.where(step[..., None] > 0, mag / step[..., None], 0.0)
    lo = np.searchsorted(E2M1_GRID, y, side="right") - 1          # largest grid value <= y
    lo = np.clip(lo, 0, 7)
    hi = np.minimum(lo + 1, 7)
    g_lo, g_hi = E2M1_GRID[lo], E2M1_GRID[hi]
    with np.errstate(divide="ignore", invalid="ignore"):
        p = np.where(hi > lo, (y - g_lo) / (g_hi - g_lo), 0.0)
    u = np.asarray(rnd, dtype=np.uint32).astype(np.float64).reshape(y.shape) * 2.0 ** -32
    idx = np.where(u < p, hi, lo)
    idx = np.where(step[..., None] > 0, idx, 0)
    sign = np.signbit(blocks).astype(np.int64) << 3
    codes = (idx | sign).reshape(rows, cols)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return NVFP4(packed, sb, np.float32(st64), rows, cols), h


def mstate_decode(view: NVFP4) -> np.ndarray:
    return hadamard16(dequantize(view)).astype(np.float32)
