"""LoRA-SVD training-side steps (oracle; test infrastructure only).

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
