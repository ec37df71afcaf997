"""Block-scaled GEMM and LoRA-SVD linear fwd/bwd parity vs the oracle.

GEMM outputs must be within a max relative error of 1e-3 normalised by
sum_k |a||b| (the error bound of the path).  The products of expanded
operands are exact and accumulate in fp32, so the observed error is ~1e-6;
the 1e-3 bar is the stated tolerance, and a tighter 1e-5 check guards
against silent precision loss (e.g. a BF16 low-rank term without its lo
part would sit near 4e-3).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import need_gpu, dev_bf16, dev_f32, print_case, f32, assert_view_equal
from oracle.quantize import quantize_rows, tensor_scale

pytestmark = pytest.mark.gpu

TOL = 1e-3
TIGHT = 1e-5


def _err(got, ref, denom):
    e = oracle.rel_err(got, ref, denom)
    return e


@pytest.mark.parametrize("M,N,K", [(64, 64, 128), (272, 400, 272), (128, 256, 384), (16, 16, 16),
                                   (300 // 16 * 16, 130 // 16 * 16, 1040)])
def test_gemm_nt(M, N, K):
    fs4 = need_gpu()
    print_case(test="gemm_nt", M=M, N=N, K=K)
    rng = np.random.default_rng(M + N + K)
    a = synth.bf16_round(rng.standard_normal((M, K)) * np.exp(rng.uniform(-2, 2, (M, 1))))
    b = (rng.standard_t(3, size=(N, K)) * 0.02).astype(np.float32)
    ar, _ = fs4.quantize(dev_bf16(a), colwise=False)
    br, _ = fs4.quantize(dev_f32(b), colwise=False)
    E = rng.standard_normal((M, N)).astype(np.float32)
    C = fs4.gemm_nt(ar, br, alpha=0.5, E=dev_f32(E), beta_e=-1.25).cpu().numpy()
    qa, _, _ = oracle.quantize(f32(a), colwise=False)
    qb, _, _ = oracle.quantize(b, colwise=False)
    ref = 0.5 * oracle.gemm_nt(qa, qb) - 1.25 * E.astype(np.float64)
    den = 0.5 * oracle.gemm_nt_abs(qa, qb) + 1.25 * np.abs(E.astype(np.float64))
    e = _err(C, ref, den)
    assert e <= TOL and e <= TIGHT, e


def test_gemm_zero_operand():
    fs4 = need_gpu()
    print_case(test="gemm_zero")
    z = np.zeros((64, 128), dtype=np.float32)
    rng = np.random.default_rng(1)
    b = rng.standard_normal((96, 128)).astype(np.float32)
    zr, _ = fs4.quantize(dev_f32(z), colwise=False)
    br, _ = fs4.quantize(dev_f32(b), colwise=False)
    C = fs4.gemm_nt(zr, br).cpu().numpy()
    assert not C.any()


def _tiny_inputs():
    d = synth.tiny_linear()
    rng = np.random.default_rng(11)
    dy = synth.normal_bf16(rng, (64, 256), std=1e-3)
    return d, dy


def _fwd_bwd_check(X, R, U, V, dY, beta=1.0, check_bwd=True, label=""):
    """Run the HIP fwd/bwd and the oracle on the same inputs; compare."""
    fs4 = need_gpu()
    M, K = X.shape
    N = R.shape[0]
    r = U.shape[1]
    x32, u32, v32 = f32(X), f32(U), f32(V)
    Xd = dev_bf16(X)
    Ud = dev_bf16(U) if r else None
    Vd = dev_bf16(V) if r else None
    R_row, R_col = fs4.quantize(dev_f32(R))
    fwd = fs4.linear_fwd(Xd, R_row, Ud, Vd, beta)
    # oracle
    ref_rr, ref_rc, _ = oracle.quantize(R)
    assert_view_equal(R_row, ref_rr, label + " R_row")
    assert_view_equal(R_col, ref_rc, label + " R_col")
    ref = oracle.linear_fwd(x32, ref_rr, u32, v32, beta)
    assert_view_equal(fwd.X_col, ref["X_col"], label + " X_col")
    e = _err(fwd.Y.cpu().numpy(), ref["Y64"], ref["D"])
    assert e <= TOL and e <= TIGHT, ("Y", e)
    if r:
        T_gpu = fwd.T.cpu().numpy()
        T_den = np.abs(x32.astype(np.float64)) @ np.abs(v32.astype(np.float64)).T
        e = _err(T_gpu, ref["T64"], T_den)
        assert e <= TIGHT, ("T", e)
    if not check_bwd:
        return
    # backward: both sides take the oracle's T (fp32) so that no HIP output
    # feeds the oracle
    T32 = ref["T64"].astype(np.float32)
    Td = dev_f32(T32) if r else None
    bwd = fs4.linear_bwd(dev_bf16(dY), Xd, fwd.X_col, R_col, Ud, Vd, Td, beta)
    rb = oracle.linear_bwd(f32(dY), x32, ref_rc, u32, v32, T32, beta, x_col=ref["X_col"])
    for name in ("dX", "dW") + (("dU", "dV") if r else ()):
        got = getattr(bwd, name).cpu().numpy()
        e = _err(got, rb[name], rb[name + "_D"])
        assert e <= TOL and e <= TIGHT, (name, e)


def test_tiny_linear_fwd_bwd():
    print_case(test="linear_tiny")
    d, dy = _tiny_inputs()
    _fwd_bwd_check(d["X"], d["R"], d["U"], d["V"], dy, label="tiny")


@pytest.mark.parametrize("M,K,N,r,beta", [(80, 272, 208, 5, 1.0), (64, 128, 96, 0, 1.0),
                                          (48, 64, 64, 64, 0.5), (272, 512, 400, 32, 1.0),
                                          (16, 16, 16, 1, 2.0),
                                          # several 512 x 512 blocks of dY with ragged edges
                                          # (P and dU from one read of dY), and r = 33 past it
                                          (1040, 128, 1552, 32, 0.75), (1552, 64, 528, 7, 1.0),
                                          (528, 96, 1040, 33, 1.0)])
def test_linear_ragged_shapes_and_ranks(M, K, N, r, beta):
    print_case(test="linear_ragged", M=M, K=K, N=N, r=r, beta=beta)
    rng = np.random.default_rng(M * 31 + K + N + r)
    X = synth.normal_bf16(rng, (M, K))
    W = synth.bf16_round(rng.standard_normal((N, K)) * 0.02)
    if r:
        U, V, R = synth.lowrank_split(f32(W), r)
    else:
        U, V, R = np.zeros((N, 0), np.uint16), np.zeros((0, K), np.uint16), f32(W)
    dY = synth.normal_bf16(rng, (M, N), std=1e-3)
    _fwd_bwd_check(X, R, U, V, dY, beta=beta, label="ragged")


def test_exactly_rank_r_weight_has_zero_residual():
    fs4 = need_gpu()
    print_case(test="linear_rank_r")
    rng = np.random.default_rng(3)
    M, K, N, r = 32, 64, 48, 8
    U = synth.bf16_round(rng.integers(-8, 9, (N, r)) / 8.0)
    V = synth.bf16_round(rng.integers(-8, 9, (r, K)) / 16.0)
    R = np.zeros((N, K), dtype=np.float32)
    X = synth.normal_bf16(rng, (M, K))
    R_row, _ = fs4.quantize(dev_f32(R), colwise=False)
    torch.cuda.synchronize()
    assert R_row.tscale.item() == 0.0 and not R_row.codes.any() and not R_row.scales.any()
    fwd = fs4.linear_fwd(dev_bf16(X), R_row, dev_bf16(U), dev_bf16(V))
    want = (f32(X).astype(np.float64) @ f32(V).T.astype(np.float64)) @ f32(U).T.astype(np.float64)
    den = np.abs(f32(X).astype(np.float64)) @ np.abs(f32(V).T.astype(np.float64)) @ np.abs(f32(U).T.astype(np.float64))
    e = _err(fwd.Y.cpu().numpy(), want, den)
    assert e <= TIGHT, e


def _sampled_gemm_check(got, a_rows_q, b_rows_q, pairs, extra=None):
    """got[i, j] vs s_tA s_tB <A_hat[i], B_hat[j]> (+ extra(i, j)) on sampled pairs."""
    errs = []
    for (i, j), (qa, qb) in zip(pairs, zip(a_rows_q, b_rows_q)):
        av = oracle.block_values(qa)[0]
        bv = oracle.block_values(qb)[0]
        s = float(qa.tscale) * float(qb.tscale)
        ref = s * np.dot(av, bv)
        den = s * np.dot(np.abs(av), np.abs(bv))
        if extra is not None:
            x, xd = extra(i, j)
            ref += x
            den += xd
        errs.append(abs(float(got[i, j]) - ref) / den if den else (0.0 if got[i, j] == ref else np.inf))
    return max(errs)


@pytest.mark.parametrize("M,N,K", [(4096, 4096, 1040), (8192, 3008, 1040)])
def test_gemm_large_tiles_ragged_k_sampled(M, N, K):
    """Shapes large enough for the wide tile configurations (4096 x 4096 takes
    256 x 256 tiles; 8192 x 3008 takes 256 x 192 tiles with a ragged last
    column of tiles), with K % 128 != 0 (the byte-wise staging path with a k
    tail); sampled outputs against the oracle's rows."""
    fs4 = need_gpu()
    print_case(test="gemm_large_ragged_k", M=M, N=N, K=K)
    rng = np.random.default_rng(21 + N)
    a = synth.bf16_round(rng.standard_normal((M, K)))
    b = (rng.standard_t(3, size=(N, K)) * 0.02).astype(np.float32)
    ar, _ = fs4.quantize(dev_bf16(a), colwise=False)
    br, _ = fs4.quantize(dev_f32(b), colwise=False)
    C = fs4.gemm_nt(ar, br).cpu().numpy()
    a32 = f32(a)
    s_a, s_b = tensor_scale(a32), tensor_scale(b)
    ms, ns_ = rng.integers(0, M, 64), rng.integers(0, N, 64)
    ms[:4] = [0, M - 1, 255, 256]
    ns_[:4] = [N - 1, 0, 192, 191]
    qa = [quantize_rows(a32[m:m + 1], s_a) for m in ms]
    qb = [quantize_rows(b[n:n + 1], s_b) for n in ns_]
    e = _sampled_gemm_check(C, qa, qb, list(zip(ms, ns_)))
    assert e <= TOL and e <= TIGHT, e
