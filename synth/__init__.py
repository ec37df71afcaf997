"""Seeded synthetic inputs shared by the CPU oracle and the HIP path.

This module draws random tensors and rounds them to their storage types; it
holds none of the NVFP4 arithmetic (no scaling, no rounding onto E2M1/E4M3,
no GEMM).  Both sides receive the exact same bytes from it.

Storage conventions
-------------------
* bf16 tensors are numpy ``uint16`` arrays of raw bfloat16 bits.  ``bf16_to_f32``
  widens them exactly to float32 for the oracle; the GPU side reinterprets the
  same bits as ``torch.bfloat16``.
* fp32 tensors are numpy ``float32`` arrays.

Rounding to bf16 goes fp64 -> fp32 (numpy, round-to-nearest-even) -> bf16
(round-to-nearest-even on the fp32 bits, below).  The double rounding only
defines which bf16 values are drawn; nothing downstream depends on it.

Workloads (the shapes of the linear layers of the 3B-parameter run the pages
train; the pages never print the model's hidden sizes, so K = 3072, N = 8192
and 8192 tokens per step are the chosen stand-ins):

=====  ==========================================================================
seed   workload
=====  ==========================================================================
1      tiny linear: X 64x256 ~N(0,1); W 256x256 ~N(0,0.02) with 4 input columns
       scaled x20; rank-8 low-rank factors
2      quantizer: 4096x4096 ~N(0,1) with 0.1% of entries multiplied by 50
3      3B-shape linear: X 8192x3072 ~N(0,1); W 8192x3072 ~N(0,0.02) with 1% of
       entries replaced by 0.02 * Student-t(3); rank-32 factors
4      3B-shape backward: dY 8192x8192 ~N(0,1e-3) (X, W from seed 3)
5      Newton-Schulz: G 3072x8192 ~N(0,1)
=====  ==========================================================================

The second parameter of N(mu, sigma) is the standard deviation.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_round", "bf16_to_f32", "rng_for", "normal_bf16", "tiny_linear",
    "quantizer_input", "linear3b", "linear3b_dy", "ns_input", "lowrank_split",
    "randomized_lowrank_split",
]


def rng_for(seed: int) -> np.random.Generator:
    """PCG64 generator for one workload."""
    return np.random.default_rng(seed)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """fp64/fp32 array -> raw bf16 bits (uint16), round-to-nearest-even.

    Inputs must be finite.
    """
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    u = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return u.astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """Raw bf16 bits (uint16) -> float32, exact."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    return bf16_round(rng.standard_normal(shape) * std)


def lowrank_split(w: np.ndarray, r: int):
    """Split a weight into rank-r factors and a residual, W = U V + R.

    U = U_r diag(sqrt(S_r)) and V = diag(sqrt(S_r)) V_r^T from the exact SVD of
    W (fp64), each rounded to bf16; R = fp32(W - U V) with U V formed in fp64
    from the bf16 factors.  This is input preparation: the hot path and the
    oracle both take (U, V, R) as given.
    """
    w64 = np.asarray(w, dtype=np.float64)
    u, s, vt = np.linalg.svd(w64, full_matrices=False)
    return _factors_from_svd(w64, u[:, :r], s[:r], vt[:r])


def randomized_lowrank_split(w: np.ndarray, r: int, seed: int, oversample: int = 32,
                             power_iters: int = 2):
    """Same split as ``lowrank_split`` with a seeded randomized range finder
    (Gaussian sketch, ``power_iters`` subspace iterations, QR re-orthonormalised
    each time), for the large workloads where a full SVD is slow."""
    w64 = np.asarray(w, dtype=np.float64)
    rng = np.random.default_rng(seed)
    omega = rng.standard_normal((w64.shape[1], r + oversample))
    y = w64 @ omega
    for _ in range(power_iters):
        q, _ = np.linalg.qr(y)
        z = w64.T @ q
        q2, _ = np.linalg.qr(z)
        y = w64 @ q2
    q, _ = np.linalg.qr(y)
    ub, s, vt = np.linalg.svd(q.T @ w64, full_matrices=False)
    return _factors_from_svd(w64, (q @ ub)[:, :r], s[:r], vt[:r])


def _factors_from_svd(w64, ur, sr, vtr):
    root = np.sqrt(sr)
    u_b = bf16_round(ur * root[None, :])
    v_b = bf16_round(root[:, None] * vtr)
    uv = bf16_to_f32(u_b).astype(np.float64) @ bf16_to_f32(v_b).astype(np.float64)
    res = (w64 - uv).astype(np.float32)
    return u_b, v_b, res


def tiny_linear(seed: int = 1):
    """X 64x256 ~N(0,1); W 256x256 ~N(0,0.02) with 4 seeded input columns x20;
    rank 8.  Returns dict of X (bf16 bits), W (bf16 bits), U, V (bf16 bits),
    R (fp32)."""
    rng = rng_for(seed)
    m, k, n, r = 64, 256, 256, 8
    x = normal_bf16(rng, (m, k))
    w64 = rng.standard_normal((n, k)) * 0.02
    cols = rng.choice(k, size=4, replace=False)
    w64[:, cols] *= 20.0
    w = bf16_round(w64)
    u, v, res = lowrank_split(bf16_to_f32(w), r)
    return {"X": x, "W": w, "U": u, "V": v, "R": res, "outlier_cols": np.sort(cols), "r": r}


def quantizer_input(seed: int = 2, rows: int = 4096, cols: int = 4096):
    """rows x cols ~N(0,1) with 0.1% of positions (uniform, no replacement) x50."""
    rng = rng_for(seed)
    x = rng.standard_normal((rows, cols))
    n_out = (rows * cols) // 1000
    idx = rng.choice(rows * cols, size=n_out, replace=False)
    x.reshape(-1)[idx] *= 50.0
    return bf16_round(x)


def linear3b(seed: int = 3, m: int = 8192, k: int = 3072, n: int = 8192, r: int = 32):
    """X m x k ~N(0,1); W n x k ~N(0,0.02) with 1% of positions replaced by
    0.02 * t_3; rank-r factors via the randomized split."""
    rng = rng_for(seed)
    x = normal_bf16(rng, (m, k))
    w64 = rng.standard_normal((n, k)) * 0.02
    n_out = (n * k) // 100
    idx = rng.choice(n * k, size=n_out, replace=False)
    w64.reshape(-1)[idx] = 0.02 * rng.standard_t(3, size=n_out)
    w = bf16_round(w64)
    u, v, res = randomized_lowrank_split(bf16_to_f32(w), r, seed=seed + 1000)
    return {"X": x, "W": w, "U": u, "V": v, "R": res, "r": r}


def linear3b_dy(seed: int = 4, m: int = 8192, n: int = 8192):
    """dY m x n ~N(0, 1e-3)."""
    return normal_bf16(rng_for(seed), (m, n), std=1e-3)


def ns_input(seed: int = 5, m: int = 3072, n: int = 8192):
    """Momentum G m x n ~N(0,1)."""
    return normal_bf16(rng_for(seed), (m, n))
