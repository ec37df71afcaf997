"""NVFP4 mixed-precision attention, Q-Attn (oracle; test infrastructure only).

[FS4 §2.4]: attention runs the products the pages call robust, Q K^T and the
ones taking dS, on NVFP4 operands and keeps the softmax-sensitive ones, P V,
P^T dO and dO V^T, in BF16; the quantized views of Q, K and V made in the
forward are reused by the backward.

Readings (the pages print no formulas):
* Q, K, V, dO are BF16 tensors [G, S, D]: G = batch x heads independent
  sequences of length S with head dimension D.  Causal attention (decoder
  pretraining), softmax scale 1/sqrt(D).
* Q and K are each quantized once, as the [G*S, D] matrix, with one tensor
  scale: the row-wise view (blocks of 16 along D) serves Q K^T, the
  column-wise view of each sequence (blocks of 16 along S, the same tensor
  scale) serves the dS products.  V stays BF16: both products that read V
  are in the BF16 list; its reused "view" is the BF16 tensor itself.
* Forward: S = s_Q s_K Q_hat K_hat^T / sqrt(D) (exact), masked above the
  diagonal; P = softmax(S) row by row; O = P V; LSE = log sum exp(S) per row.
  The BF16 path rounds P to BF16 before P V (its error is the tolerance of
  the GPU test); the oracle's O is the exact product.
* Backward: P recomputed from the same quantized Q and K; dV = P^T dO;
  dP = dO V^T; Delta = rowsum(dO * O); dS = P * (dP - Delta) (the softmax
  gradient); dS is quantized once as the [G*S, S] matrix with one tensor
  scale, row-wise (blocks along keys) for dQ = Q(dS) Q_col(K)^T / sqrt(D) and
  column-wise (blocks along queries) for dK = Q(dS^T) Q_col(Q)^T / sqrt(D).
  dS's quantization uses the exact dS here (float32-rounded, as a kernel
  stores it).
"""
from __future__ import annotations

import numpy as np

from .formats import tensor_scale_from_amax
from .quantize import NVFP4, block_values, quantize, quantize_rows, tensor_amax


def _views_per_sequence(x32, G, S, D):
    """One quantization of x [G*S, D]: its row-wise view, and the column-wise
    view of each sequence (x_g^T [D, S] blocked along S) with the same tensor
    scale."""
    row, _, s_t = quantize(x32.reshape(G * S, D), rowwise=True, colwise=False)
    cols = [quantize_rows(np.ascontiguousarray(x32[g].T), s_t) for g in range(G)]
    return row, cols, s_t


def _head_rows(view: NVFP4, g: int, S: int) -> NVFP4:
    return NVFP4(view.codes[g * S:(g + 1) * S], view.scales[g * S:(g + 1) * S], view.tscale, S, view.cols)


def causal_mask(S: int) -> np.ndarray:
    """True where key j may be attended by query i (j <= i)."""
    return np.tril(np.ones((S, S), dtype=bool))


def _probs(view_q: NVFP4, view_k: NVFP4, g: int, S: int, st: float, mask: np.ndarray):
    """P = softmax of sequence g's masked scores S = st Q_hat K_hat^T, row by
    row, with each row's max m and sum l of exp(S - m)."""
    s = st * (block_values(_head_rows(view_q, g, S)) @ block_values(_head_rows(view_k, g, S)).T)
    s = np.where(mask, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    return e / l, m, l


def _each(fn, seqs, threads: int):
    """fn(g) for every g in seqs, in order, on `threads` threads (the
    sequences are independent; each one's arithmetic is the same either
    way)."""
    if threads <= 1:
        return [fn(g) for g in seqs]
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(threads) as ex:
        return list(ex.map(fn, seqs))


def attention_fwd(q, k, v, causal: bool = True, seqs=None, keep_P: bool = True, threads: int = 1):
    """q, k, v float32 [G, S, D] holding BF16 values (the tensor scales are
    those of all G sequences; `seqs` limits the products to some of them,
    leaving the others' outputs unset).  Returns dict: O (float64), LSE
    (float64 [G, S]), P (float64 [G, S, S]; None with seqs or without
    keep_P), the O error normaliser O_D = P |V| (what the BF16 rounding of P
    can move O by, per unit of relative error), and the quantized views
    (Q_row, K_row, Q_col, K_col per sequence)."""
    G, S, D = q.shape
    q_row, q_cols, _ = _views_per_sequence(q, G, S, D)
    k_row, k_cols, _ = _views_per_sequence(k, G, S, D)
    scale = 1.0 / np.sqrt(D)
    st = float(q_row.tscale) * float(k_row.tscale) * scale
    mask = causal_mask(S) if causal else np.ones((S, S), dtype=bool)
    O = np.empty((G, S, D))
    O_D = np.empty((G, S, D))
    P_all = np.empty((G, S, S)) if seqs is None and keep_P else None
    LSE = np.empty((G, S))

    def one(g):
        p, m, l = _probs(q_row, k_row, g, S, st, mask)
        v64 = v[g].astype(np.float64)
        O[g] = p @ v64
        O_D[g] = p @ np.abs(v64)
        if P_all is not None:
            P_all[g] = p
        LSE[g] = (m + np.log(l))[:, 0]

    _each(one, range(G) if seqs is None else seqs, threads)
    return {"O": O, "O_D": O_D, "LSE": LSE, "P": P_all, "scale": scale, "st": st, "mask": mask,
            "seqs": None if seqs is None else sorted(seqs),
            "Q_row": q_row, "K_row": k_row, "Q_col": q_cols, "K_col": k_cols}


def softmax_grad(fwd, v, do, g: int):
    """The softmax gradient of sequence g: P (the forward's, or recomputed
    from the same views), dP = dO V^T, Delta = rowsum(dO * O) with the
    forward's O, and dS = P * (dP - Delta), all float64."""
    S = v.shape[1]
    P = fwd["P"][g] if fwd["P"] is not None else _probs(fwd["Q_row"], fwd["K_row"], g, S, fwd["st"], fwd["mask"])[0]
    do64, v64 = do[g].astype(np.float64), v[g].astype(np.float64)
    dP = do64 @ v64.T
    delta = np.sum(do64 * fwd["O"][g], axis=1, keepdims=True)
    return {"P": P, "dP": dP, "Delta": delta[:, 0], "dS": P * (dP - delta)}


def attention_bwd(q, k, v, do, fwd=None, causal: bool = True, seqs=None, on_seq=None, threads: int = 1):
    """The backward from dO float32 [G, S, D] (BF16 values), with the
    forward's quantized views (and its P when kept).  dS's tensor scale is
    that of all G sequences; `seqs` limits the outputs to some of them (the
    forward must then still cover all G, for every sequence's dS enters the
    tensor scale).  `on_seq(g, parts)`, if given, sees softmax_grad's parts
    of every sequence as they are formed (from several threads at once
    when threads > 1).  Returns dict of dQ, dK, dV
    (float64 [G, S, D]; rows outside `seqs` unset), dS (float64 [G, S, S]
    before its quantization; None with seqs, else per sequence in dS_seq),
    the normalisers dQ_D, dK_D (sum |a||b| of the NVFP4 products) and
    dV_D = P^T |dO|, and dS's tensor scale."""
    G, S, D = q.shape
    if fwd is None:
        fwd = attention_fwd(q, k, v, causal, keep_P=seqs is None)
    if fwd["seqs"] is not None:
        raise ValueError("the backward needs the forward of every sequence")
    scale = fwd["scale"]
    sel = list(range(G)) if seqs is None else sorted(seqs)
    dV = np.empty((G, S, D))
    dV_D = np.empty((G, S, D))
    ds_seq = {}

    def one(g):
        parts = softmax_grad(fwd, v, do, g)
        ds32 = parts["dS"].astype(np.float32)
        if on_seq is not None:
            on_seq(g, parts)
        if g in sel:
            do64 = do[g].astype(np.float64)
            dV[g] = parts["P"].T @ do64
            dV_D[g] = parts["P"].T @ np.abs(do64)
            ds_seq[g] = (parts["dS"], ds32)
        return tensor_amax(ds32)

    s_ds = tensor_scale_from_amax(max(_each(one, range(G), threads)))
    dQ = np.empty((G, S, D))
    dK = np.empty((G, S, D))
    dQ_D = np.empty((G, S, D))
    dK_D = np.empty((G, S, D))
    for g in sel:
        ds32 = ds_seq[g][1]
        a = block_values(quantize_rows(ds32, s_ds))                        # dS_g, blocks along keys
        at = block_values(quantize_rows(np.ascontiguousarray(ds32.T), s_ds))   # dS_g^T, blocks along queries
        kc = block_values(fwd["K_col"][g])                                 # K_g^T [D, S], blocks along keys
        qc = block_values(fwd["Q_col"][g])                                 # Q_g^T [D, S], blocks along queries
        sq = float(s_ds) * float(fwd["K_row"].tscale) * scale
        sk = float(s_ds) * float(fwd["Q_row"].tscale) * scale
        dQ[g] = sq * (a @ kc.T)
        dQ_D[g] = sq * (np.abs(a) @ np.abs(kc).T)
        dK[g] = sk * (at @ qc.T)
        dK_D[g] = sk * (np.abs(at) @ np.abs(qc).T)
    dS = np.stack([ds_seq[g][0] for g in range(G)]) if seqs is None else None
    return {"dQ": dQ, "dK": dK, "dV": dV, "dS": dS, "dS_seq": {g: ds_seq[g][0] for g in sel},
            "dQ_D": dQ_D, "dK_D": dK_D, "dV_D": dV_D, "dS_tscale": s_ds}
