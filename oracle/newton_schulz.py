"""Newton-Schulz orthogonalisation with NVFP4 operands (oracle; test
infrastructure only).

[FS4 §2.3]: the Root/Muon optimizer's Newton-Schulz matrix products run
directly on NVFP4 operands rather than on a mixed-precision path.  The pages
tune (a, b, c) per aspect ratio and clip outliers at the 99th percentile but
print neither the coefficients nor where the clip applies.  Readings: the
caller passes (a, b, c), by default the fixed quintic used by Muon,
(a, b, c) = (3.4445, -4.7750, 2.0315); with clipping on (clip_q, e.g. 0.99),
the iterate X is clipped at the nearest-rank clip_q quantile of |X| before
each of its quantizations, and only that quantized copy is clipped (the
float32 state and the a X term keep the outliers).  A and B are quantized
unclipped: A = X X^T carries its largest entries on the diagonal by
construction.

Iteration on X [m, n], m <= n:

    X_0     = G / (||G||_F + eps)                   (eps = 1e-7)
    A       = Q(X) Q(X)^T                           X row-wise (blocks along n)
    B       = b A + c Q(A) Q(A^T)^T                 A row- and column-wise
    X_next  = a X + Q(B) Q(X^T)^T                   B row-wise, X column-wise

Reading: the state X and the products A, B are float32 tensors (they are the
operands the quantizer sees); every GEMM is exact in float64 over the
dequantized operands and then rounded to float32; only GEMM operands are
quantized (b A and a X use the float32 values).
"""
from __future__ import annotations

import numpy as np

from .linear import gemm_nt, gemm_nt_abs
from .quantize import quantize

MUON_ABC = (3.4445, -4.7750, 2.0315)
NS_EPS = 1e-7


def ns_normalize(g, eps: float = NS_EPS):
    """X_0 = G / (||G||_F + eps), Frobenius norm in float64, X_0 rounded to
    float32.  Returns (X_0 float32, X_0 float64)."""
    g64 = np.asarray(g, dtype=np.float64)
    x64 = g64 / (np.sqrt(np.sum(g64 * g64)) + eps)
    return x64.astype(np.float32), x64


def abs_quantile(x, q: float) -> np.float32:
    """Nearest-rank q-quantile of |x|: the k-th smallest magnitude, k =
    ceil(q n) computed in float64 (1 <= k <= n), as float32."""
    mag = np.abs(np.asarray(x, dtype=np.float32)).reshape(-1)
    n = mag.size
    k = int(np.ceil(float(q) * n))
    k = min(max(k, 1), n)
    return np.float32(np.partition(mag, k - 1)[k - 1])


def clip_abs(x, p) -> np.ndarray:
    """Clips float32 values to magnitude p, keeping each value's sign."""
    x = np.asarray(x, dtype=np.float32)
    p = np.float32(p)
    return np.where(np.abs(x) > p, np.copysign(p, x), x).astype(np.float32)


def ns_step(x, a: float, b: float, c: float, clip_q: float | None = None):
    """One quantized Newton-Schulz step from float32 X (X clipped at the
    clip_q quantile of |X| for its quantization when clip_q is given).

    Returns dict: A, B, X (float32 results), A64, B64, X64 (float64 before
    rounding), the error normalisers A_D, B_D, X_D, and P, the clip value
    (None without clipping).
    """
    x = np.asarray(x, dtype=np.float32)
    p = None
    xq = x
    if clip_q is not None:
        p = abs_quantile(x, clip_q)
        xq = clip_abs(x, p)
    x_row, x_col, _ = quantize(xq, rowwise=True, colwise=True)
    a64 = gemm_nt(x_row, x_row)
    a_d = gemm_nt_abs(x_row, x_row)
    a32 = a64.astype(np.float32)
    a_row, a_col, _ = quantize(a32, rowwise=True, colwise=True)
    aa = gemm_nt(a_row, a_col)
    b64 = b * a32.astype(np.float64) + c * aa
    b_d = abs(b) * np.abs(a32.astype(np.float64)) + abs(c) * gemm_nt_abs(a_row, a_col)
    b32 = b64.astype(np.float32)
    b_row, _, _ = quantize(b32, rowwise=True, colwise=False)
    bx = gemm_nt(b_row, x_col)
    x64 = a * x.astype(np.float64) + bx
    x_d = abs(a) * np.abs(x.astype(np.float64)) + gemm_nt_abs(b_row, x_col)
    return {"A": a32, "A64": a64, "A_D": a_d, "B": b32, "B64": b64, "B_D": b_d,
            "X": x64.astype(np.float32), "X64": x64, "X_D": x_d, "P": p}


def newton_schulz(g, steps: int = 5, abc=MUON_ABC, eps: float = NS_EPS, normalize: bool = True,
                  clip_q: float | None = None):
    """Quantized NS from G.  Returns the list of float32 iterates X_0..X_steps
    and the list of per-step dicts from ``ns_step``."""
    a, b, c = abc
    x0 = ns_normalize(g, eps)[0] if normalize else np.asarray(g, dtype=np.float32)
    xs, steps_out = [x0], []
    for _ in range(steps):
        st = ns_step(xs[-1], a, b, c, clip_q)
        steps_out.append(st)
        xs.append(st["X"])
    return xs, steps_out


def newton_schulz_fp64(g, steps: int = 5, abc=MUON_ABC, eps: float = NS_EPS):
    """The same iteration without quantization, all in float64."""
    a, b, c = abc
    x = ns_normalize(g, eps)[1]
    for _ in range(steps):
        am = x @ x.T
        bm = b * am + c * (am @ am)
        x = a * x + bm @ x
    return x


# ---- shape-dependent coefficients (Q-Root) ----------------------------------------
# [FS4 §2.3] stabilises the NVFP4 iteration with (a, b, c) "optimised for the
# matrix aspect ratio" but prints neither the coefficients nor the criterion.
# Reading: for an m x n momentum (m <= n) the coefficients minimise the mean
# squared distance of the 5-step quintic's singular values to 1 (the polar
# factor's), averaged over the singular-value law of a Frobenius-normalised
# m x n Gaussian matrix, which the Marchenko-Pastur law gives in closed form:
# the eigenvalues lam of G G^T / n, y = m / n, have density
#     f(lam) = sqrt((lam_+ - lam)(lam - lam_-)) / (2 pi y lam),
#     lam_(+/-) = (1 +/- sqrt(y))^2,
# and since ||G||_F^2 ~ m n, the normalised singular values are
# sigma = sqrt(lam / m).  The minimisation starts from Muon's quintic.


def mp_density(lam, y: float) -> np.ndarray:
    """Marchenko-Pastur density of the eigenvalues of G G^T / n for an m x n
    (m <= n, y = m / n) matrix of independent N(0, 1) entries."""
    lam = np.asarray(lam, dtype=np.float64)
    lo, hi = (1.0 - np.sqrt(y)) ** 2, (1.0 + np.sqrt(y)) ** 2
    inside = (lam > lo) & (lam < hi)
    out = np.zeros_like(lam)
    out[inside] = np.sqrt((hi - lam[inside]) * (lam[inside] - lo)) / (2.0 * np.pi * y * lam[inside])
    return out


def mp_nodes(m: int, n: int, points: int = 400):
    """Quadrature nodes and weights over the normalised singular values of an
    m x n Gaussian matrix: Gauss-Chebyshev (second kind) in lam on
    [lam_-, lam_+], which absorbs the square-root edges of the density."""
    y = m / n
    lo, hi = (1.0 - np.sqrt(y)) ** 2, (1.0 + np.sqrt(y)) ** 2
    k = np.arange(1, points + 1)
    t = np.cos(k * np.pi / (points + 1))                    # nodes of U_points in (-1, 1)
    w_t = np.pi / (points + 1) * np.sin(k * np.pi / (points + 1)) ** 2
    lam = 0.5 * (hi + lo) + 0.5 * (hi - lo) * t
    # integral of g(lam) sqrt((hi-lam)(lam-lo)) dlam = ((hi-lo)/2)^2 sum w_t g(lam)
    w = ((hi - lo) / 2.0) ** 2 * w_t / (2.0 * np.pi * y * lam)
    return np.sqrt(lam / m), w


def quintic_power(sigma, abc, steps: int = 5) -> np.ndarray:
    """p applied `steps` times to singular values, p(s) = a s + b s^3 + c s^5."""
    a, b, c = abc
    s = np.asarray(sigma, dtype=np.float64)
    for _ in range(steps):
        s = a * s + b * s ** 3 + c * s ** 5
    return s


def polar_distance(abc, m: int, n: int, steps: int = 5, points: int = 400) -> float:
    """Mean over the m x n spectrum of (p^steps(sigma) - 1)^2: the expected
    squared Frobenius distance per singular value between the unquantized
    iteration and the polar factor."""
    s, w = mp_nodes(m, n, points)
    return float(np.sum(w * (quintic_power(s, abc, steps) - 1.0) ** 2) / np.sum(w))


def shape_coefficients(m: int, n: int, steps: int = 5, start=MUON_ABC):
    """(a, b, c) for an m x n momentum (m <= n): the minimiser of
    polar_distance from Muon's quintic (Nelder-Mead, tight tolerances)."""
    from scipy.optimize import minimize
    if m > n:
        m, n = n, m
    f = lambda v: polar_distance(tuple(v), m, n, steps)
    res = minimize(f, np.asarray(start, dtype=np.float64), method="Nelder-Mead",
                   options={"xatol": 1e-10, "fatol": 1e-14, "maxiter": 20000, "maxfev": 40000})
    return tuple(float(v) for v in res.x)
