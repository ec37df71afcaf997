"""LoRA-SVD training-side steps (oracle; test infrastructure only): the
subspace-constrained low-rank gradients and the periodic realignment.

[FS4 §2.1], backward-pass paragraph: the update of the BF16 low-rank branch
L2 L1 is held to the principal subspace by a Cholesky-QR constraint, while the
residual's gradient goes to the NVFP4 component.  The pages print no formula;
the readings taken here are:

* Cholesky-QR of a tall matrix A [n, r] of full column rank: S = A^T A,
  S = L L^T (Cholesky, positive diagonal), Q = A L^{-T}.  Q has orthonormal
  columns spanning the columns of A, and A = Q L^T.
* The principal subspace is the column space of U = L2 [N, r] on the output
  side and the row space of V = L1 [r, K] on the input side.  With
  Q_U = CholQR(U) and Q_V = CholQR(V^T), the constrained gradients are the
  orthogonal projections

      dU_c = Q_U Q_U^T dU        [N, r]
      dV_c = dV Q_V Q_V^T        [r, K]

  so a step along them changes the coordinates of the branch inside its
  subspace and never rotates the subspace (that is left to the periodic
  realignment).
* The residual keeps the plain chain-rule gradient dW of the full weight.

Everything is float64; the inputs (BF16 factors, fp32 gradients) are exact in
float64.  np.linalg.cholesky and scipy's triangular solve are the library
steps.
"""
from __future__ import annotations

import numpy as np
from scipy.linalg import solve_triangular


def cholesky_qr(a):
    """Cholesky-QR of a [n, r] (n >= r, full column rank), in float64.

    Returns (Q, Rf) with Q [n, r] orthonormal columns and Rf = L^T [r, r]
    upper triangular with a positive diagonal, Q Rf = a.  Raises
    np.linalg.LinAlgError when a^T a is not positive definite.
    """
    a64 = np.asarray(a, dtype=np.float64)
    s = a64.T @ a64
    low = np.linalg.cholesky(s)                 # s = low low^T
    # Q = a low^{-T}  <=>  low Q^T = a^T
    q = solve_triangular(low, a64.T, lower=True).T
    return q, low.T


def subspace_project(u, v, du=None, dv=None):
    """Project the low-rank gradients onto the branch's principal subspace.

    u [N, r], v [r, K] (the BF16 factors, as float32 or float64);
    du [N, r] and dv [r, K] (either may be None).  Returns (du_c, dv_c) in
    float64, None where the input was None.
    """
    du_c = dv_c = None
    if du is not None:
        q_u, _ = cholesky_qr(u)
        du_c = q_u @ (q_u.T @ np.asarray(du, dtype=np.float64))
    if dv is not None:
        q_v, _ = cholesky_qr(np.asarray(v, dtype=np.float64).T)
        dv_c = (np.asarray(dv, dtype=np.float64) @ q_v) @ q_v.T
    return du_c, dv_c


# ---------------------------------------------------------------------------
# Periodic realignment, [FS4 §2.1] (realignment paragraph): every few
# thousand steps the subspace is reset with a randomized SVD.  Readings:
#
# * The full weight is W = beta U V + R, with R the residual's fp32 master
#   copy (it is re-quantized to NVFP4 every step).
# * Randomized SVD as published by Halko, Martinsson and Tropp (2011):
#   Y = W Omega^T for l Gaussian test vectors (the rows of Omega, passed in),
#   q power iterations re-orthonormalised each time (Y <- W orth(W^T orth(Y))),
#   Q = orth(Y), B = Q^T W, B = U_b S V_b^T.  The top r triplets
#   (s_i, Q U_b[:, i], V_b^T[i]) replace the branch:
#       U <- bf16(u_i sqrt(s_i / beta)),  V <- bf16(sqrt(s_i / beta) v_i^T)
#   (the singular values split evenly between the factors, as in the
#   initial split), and the residual takes the rest with the rounded
#   factors: R <- fp32(W - beta U V).
# np.linalg.qr and np.linalg.svd are the library steps.

def bf16_rne(x) -> np.ndarray:
    """Round float64 values to bfloat16 (nearest, ties to even), returned as
    float64: first to float32 (nearest even), then to 8 significant bits."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    b = f.view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16 << 16
    return b.astype(np.uint32).view(np.float32).astype(np.float64)


def lora_realign(u, v, res, beta: float, omega, power_iters: int = 1):
    """Randomized-SVD realignment of W = beta U V + R.

    u [N, r], v [r, K] (BF16 values), res [N, K] (fp32), omega [l, K] with
    r <= l.  Returns (u_new, v_new) as float64 arrays holding BF16 values,
    r_new (float32) and the top r singular values s (float64, descending) of
    Q Q^T W.
    """
    u64, v64 = np.asarray(u, np.float64), np.asarray(v, np.float64)
    w = beta * (u64 @ v64) + np.asarray(res, np.float64)
    om = np.asarray(omega, np.float64)
    r = u64.shape[1]
    y = w @ om.T
    for _ in range(power_iters):
        q, _ = np.linalg.qr(y)
        qz, _ = np.linalg.qr(w.T @ q)
        y = w @ qz
    q, _ = np.linalg.qr(y)
    b = q.T @ w
    ub, s, vt = np.linalg.svd(b, full_matrices=False)
    s_r = s[:r]
    root = np.sqrt(s_r / beta)
    u_new = bf16_rne((q @ ub[:, :r]) * root[None, :])
    v_new = bf16_rne(root[:, None] * vt[:r])
    r_new = (w - beta * (u_new @ v_new)).astype(np.float32)
    return u_new, v_new, r_new, s_r
