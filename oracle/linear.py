"""Block-scaled NT GEMM and the LoRA-SVD linear projection (oracle; test
infrastructure only).

[FS4 §2.1] parametrises a projection weight as W = W_res + beta L2 L1: the
rank-r subspace L2 L1 stays in BF16 and the residual W_res is held in NVFP4.
Notation here: U = L2 [N, r], V = L1 [r, K], R = W_res [N, K].  With
activations X [M, K]:

    forward   Y  = Q(X) Q(R)^T + beta (X V^T) U^T
    backward  dX = Q(dY) Q(R^T)^T + beta (dY U) V         (dY blocked along N)
              dW = Q(dY^T) Q(X^T)^T                      (both blocked along M)
              dU = beta dY^T T,   T = X V^T
              dV = beta (dY U)^T X

Every quantized product is quantized along its own contraction dimension.
Readings: beta = 1 unless given; the low-rank term uses the unquantized BF16
X; dW is the gradient of the full weight, i.e. the update of the residual;
dU and dV here are the plain chain-rule gradients (the pages' Cholesky-QR
constraint on them is a separate step, oracle.lora.subspace_project).

GEMMs are float64 BLAS over the exactly dequantized operands; the result is
rounded to float32 only where the method stores float32.
"""
from __future__ import annotations

import numpy as np

from .quantize import NVFP4, block_values, quantize


def gemm_nt(a: NVFP4, b: NVFP4) -> np.ndarray:
    """C[m, n] = s_tA s_tB sum_k A_hat[m, k] B_hat[n, k], float64.

    A_hat, B_hat are the block-level values e2m1(code) * e4m3(s_b), exact in
    float64; the contraction dimension is ``cols`` of both views.
    """
    if a.cols != b.cols:
        raise ValueError("contraction dims differ")
    acc = block_values(a) @ block_values(b).T
    return acc * (float(a.tscale) * float(b.tscale))


def gemm_nt_abs(a: NVFP4, b: NVFP4) -> np.ndarray:
    """Error normaliser s_tA s_tB sum_k |A_hat[m, k]| |B_hat[n, k]|."""
    acc = np.abs(block_values(a)) @ np.abs(block_values(b)).T
    return acc * (float(a.tscale) * float(b.tscale))


def rel_err(got, ref, denom) -> float:
    """max |got - ref| / denom over all outputs; where denom is 0 the outputs
    must agree exactly (else inf)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    denom = np.asarray(denom, dtype=np.float64)
    diff = np.abs(got - ref)
    zero = denom == 0
    if np.any(diff[zero] != 0):
        return float("inf")
    if not np.any(~zero):
        return 0.0
    return float(np.max(diff[~zero] / denom[~zero]))


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def linear_fwd(x, r_row: NVFP4, u, v, beta: float = 1.0):
    """LoRA-SVD forward with an NVFP4 residual.

    x: float32 [M, K] (BF16 values); r_row: NVFP4 view of R (rows N, cols K);
    u: float32 [N, r]; v: float32 [r, K] (BF16 values, r may be 0).
    Returns dict with Y (float32), Y64, D (normaliser), T64 = X V^T (float64),
    and the quantized views of X (row: blocks along K, col: blocks along M).
    """
    x_row, x_col, _ = quantize(x, rowwise=True, colwise=True)
    main = gemm_nt(x_row, r_row)
    denom = gemm_nt_abs(x_row, r_row)
    x64, u64, v64 = _f64(x), _f64(u), _f64(v)
    t64 = x64 @ v64.T if v64.size else np.zeros((x64.shape[0], 0))
    lr = beta * (t64 @ u64.T) if v64.size else 0.0
    lr_abs = abs(beta) * (np.abs(t64) @ np.abs(u64).T) if v64.size else 0.0
    y64 = main + lr
    return {"Y": y64.astype(np.float32), "Y64": y64, "D": denom + lr_abs, "T64": t64,
            "X_row": x_row, "X_col": x_col}


def linear_bwd(dy, x, r_col: NVFP4, u, v, t, beta: float = 1.0, x_col: NVFP4 | None = None):
    """LoRA-SVD backward.

    dy: float32 [M, N] (BF16 values); x: float32 [M, K]; r_col: NVFP4 view of
    R^T (rows K, cols N); u [N, r], v [r, K]; t = X V^T [M, r] (float32 or
    float64).  x_col: NVFP4 view of X^T (rows K, cols M); quantized from x
    when not given.
    Returns dict of dX, dW, dU, dV (float64) and their normalisers.
    """
    dy_row, dy_col, _ = quantize(dy, rowwise=True, colwise=True)
    if x_col is None:
        _, x_col, _ = quantize(x, rowwise=False, colwise=True)
    dy64, x64, u64, v64, t64 = _f64(dy), _f64(x), _f64(u), _f64(v), _f64(t)
    out = {"dY_row": dy_row, "dY_col": dy_col}
    dx = gemm_nt(dy_row, r_col)
    dx_d = gemm_nt_abs(dy_row, r_col)
    dw = gemm_nt(dy_col, x_col)
    dw_d = gemm_nt_abs(dy_col, x_col)
    if v64.size:
        p = dy64 @ u64                      # [M, r]
        p_abs = np.abs(dy64) @ np.abs(u64)
        dx = dx + beta * (p @ v64)
        dx_d = dx_d + abs(beta) * (p_abs @ np.abs(v64))
        du = beta * (dy64.T @ t64)
        du_d = abs(beta) * (np.abs(dy64).T @ np.abs(t64))
        dv = beta * (p.T @ x64)
        # |dV| <= |beta| sum_m |P[m, j]| |X[m, k]| with P itself a sum: use the
        # fully expanded bound sum_m sum_n |dY||U||X|
        dv_d = abs(beta) * (p_abs.T @ np.abs(x64))
        out.update(dU=du, dU_D=du_d, dV=dv, dV_D=dv_d)
    out.update(dX=dx, dX_D=dx_d, dW=dw, dW_D=dw_d)
    return out
