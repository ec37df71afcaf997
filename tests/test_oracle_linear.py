"""Pins for the oracle's block-scaled GEMM and LoRA-SVD linear fwd/bwd."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import exact as X
from oracle.formats import e4m3_decode


def _exact_block_values(codes, scales):
    """Rational block values from the exact twin's unpacked codes/scales."""
    rows, cols = codes.shape
    out = [[None] * cols for _ in range(rows)]
    for r in range(rows):
        for k in range(cols):
            c = int(codes[r, k])
            mag = X.E2M1_MAGS[c & 7] * X.E4M3_FINITE[int(scales[r, k // 16])]
            out[r][k] = -mag if c & 8 else mag
    return out


@pytest.mark.parametrize("m,n,k", [(16, 16, 32), (48, 32, 64), (8, 24, 16)])
def test_gemm_nt_matches_rational_brute_force(m, n, k):
    rng = np.random.default_rng(m * 1000 + n + k)
    a = (rng.standard_normal((m, k)) * np.exp(rng.uniform(-2, 2, (m, 1)))).astype(np.float32)
    b = rng.standard_t(3, size=(n, k)).astype(np.float32)
    ra, _, _, _, sa = X.quantize_exact(a)
    rb, _, _, _, sb = X.quantize_exact(b)
    av = _exact_block_values(ra, X.quantize_rows_exact(a, sa)[1])
    bv = _exact_block_values(rb, X.quantize_rows_exact(b, sb)[1])
    qa, _, _ = oracle.quantize(a, colwise=False)
    qb, _, _ = oracle.quantize(b, colwise=False)
    got = oracle.gemm_nt(qa, qb)
    assert got.shape == (m, n)
    for i in range(m):
        for j in range(n):
            want = sa * sb * sum((av[i][t] * bv[j][t] for t in range(k)), Fraction(0))
            assert abs(Fraction(float(got[i, j])) - want) <= abs(want) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 200)


def _representable(rng, rows, cols, scale_exp):
    """Values g * 448 * 2^scale_exp, g on the E2M1 grid, with a +-6 in every
    16-block of rows AND of columns: every block of both layouts has amax
    6 * 448 * s_t, so every scale is 448 and quantization is exact both ways."""
    g = rng.choice(oracle.E2M1_GRID[:7], size=(rows, cols)) * rng.choice([-1.0, 1.0], size=(rows, cols))
    i, j = np.indices((rows, cols))
    g[(i + j) % 16 == 0] = 6.0 * rng.choice([-1.0, 1.0], size=((i + j) % 16 == 0).sum())
    return (g * 448.0 * 2.0 ** scale_exp).astype(np.float32)


def test_representable_inputs_quantize_exactly():
    rng = np.random.default_rng(0)
    x = _representable(rng, 32, 48, -9)
    row, col, s_t = oracle.quantize(x)
    assert float(s_t) == 2.0 ** -9
    assert np.array_equal(oracle.dequantize(row), x.astype(np.float64))
    assert np.array_equal(oracle.dequantize(col), x.T.astype(np.float64))


def test_linear_fwd_bwd_reduce_to_autograd_on_representable_inputs():
    """With quantization exact, the NVFP4 path is the plain bilinear map; its
    gradients must equal torch autograd's of <dY, Y> in float64."""
    rng = np.random.default_rng(1)
    m, k, n, r = 32, 48, 64, 4
    x = _representable(rng, m, k, -3)
    res = _representable(rng, n, k, -12)
    dy = _representable(rng, m, n, -10)
    u = synth.bf16_to_f32(synth.bf16_round(rng.standard_normal((n, r)) * 0.1))
    v = synth.bf16_to_f32(synth.bf16_round(rng.standard_normal((r, k)) * 0.1))
    beta = 0.75
    r_row, r_col, _ = oracle.quantize(res)
    fwd = oracle.linear_fwd(x, r_row, u, v, beta)
    bwd = oracle.linear_bwd(dy, x, r_col, u, v, fwd["T64"], beta)

    tx = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    tr = torch.tensor(res, dtype=torch.float64, requires_grad=True)
    tu = torch.tensor(u, dtype=torch.float64, requires_grad=True)
    tv = torch.tensor(v, dtype=torch.float64, requires_grad=True)
    y = tx @ (tr + beta * tu @ tv).T
    (y * torch.tensor(dy, dtype=torch.float64)).sum().backward()
    np.testing.assert_allclose(fwd["Y64"], y.detach().numpy(), rtol=1e-13, atol=0)
    np.testing.assert_allclose(bwd["dX"], tx.grad.numpy(), rtol=1e-12, atol=1e-300)
    np.testing.assert_allclose(bwd["dW"], tr.grad.numpy(), rtol=1e-12, atol=1e-300)
    np.testing.assert_allclose(bwd["dU"], tu.grad.numpy(), rtol=1e-12, atol=1e-300)
    np.testing.assert_allclose(bwd["dV"], tv.grad.numpy(), rtol=1e-12, atol=1e-300)


def test_zero_residual_when_weight_is_exactly_rank_r():
    rng = np.random.default_rng(2)
    m, k, n, r = 16, 64, 32, 8
    # bf16 factors on a coarse dyadic grid: U V is exact in fp32
    u = (rng.integers(-8, 9, (n, r)) / 8.0).astype(np.float32)
    v = (rng.integers(-8, 9, (r, k)) / 16.0).astype(np.float32)
    w = (u.astype(np.float64) @ v.astype(np.float64)).astype(np.float32)
    res = (w.astype(np.float64) - u.astype(np.float64) @ v.astype(np.float64)).astype(np.float32)
    assert not res.any()
    r_row, r_col, s_t = oracle.quantize(res)
    assert float(s_t) == 0.0 and not r_row.codes.any() and not r_row.scales.any()
    x = synth.bf16_to_f32(synth.normal_bf16(rng, (m, k)))
    fwd = oracle.linear_fwd(x, r_row, u, v)
    np.testing.assert_array_equal(fwd["Y64"], (x.astype(np.float64) @ v.T.astype(np.float64)) @ u.T.astype(np.float64))


def test_rank_zero_is_plain_nvfp4():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((16, 32)).astype(np.float32)
    res = rng.standard_normal((48, 32)).astype(np.float32)
    r_row, _, _ = oracle.quantize(res, colwise=False)
    fwd = oracle.linear_fwd(x, r_row, np.zeros((48, 0), np.float32), np.zeros((0, 32), np.float32))
    qx, _, _ = oracle.quantize(x, colwise=False)
    np.testing.assert_array_equal(fwd["Y64"], oracle.gemm_nt(qx, r_row))


def test_tiny_config_samples_match_rational_brute_force():
    d = synth.tiny_linear()
    x = synth.bf16_to_f32(d["X"])
    u, v = synth.bf16_to_f32(d["U"]), synth.bf16_to_f32(d["V"])
    r_row, _, _ = oracle.quantize(d["R"], colwise=False)
    fwd = oracle.linear_fwd(x, r_row, u, v)
    rx, _, _, _, sx = X.quantize_exact(x[:, :])
    xs = X.quantize_rows_exact(x, sx)[1]
    rr, _, _, _, sr = X.quantize_exact(d["R"])
    rs = X.quantize_rows_exact(d["R"], sr)[1]
    rng = np.random.default_rng(4)
    for i, j in zip(rng.integers(0, 64, 12), rng.integers(0, 256, 12)):
        xv = _exact_block_values(rx[i:i + 1], xs[i:i + 1])[0]
        wv = _exact_block_values(rr[j:j + 1], rs[j:j + 1])[0]
        main = sx * sr * sum((xv[t] * wv[t] for t in range(256)), Fraction(0))
        t_row = [sum((Fraction(float(x[i, q])) * Fraction(float(v[p, q])) for q in range(256)), Fraction(0))
                 for p in range(d["r"])]
        lr = sum((t_row[p] * Fraction(float(u[j, p])) for p in range(d["r"])), Fraction(0))
        want = main + lr
        assert abs(Fraction(float(fwd["Y64"][i, j])) - want) <= abs(want) * Fraction(1, 2 ** 48) + Fraction(1, 2 ** 100)


def test_lowrank_split_reconstructs_weight():
    d = synth.tiny_linear()
    w = synth.bf16_to_f32(d["W"]).astype(np.float64)
    uv = synth.bf16_to_f32(d["U"]).astype(np.float64) @ synth.bf16_to_f32(d["V"]).astype(np.float64)
    np.testing.assert_allclose(uv + d["R"].astype(np.float64), w, atol=1e-7)
    # the residual carries less energy than the weight (the outlier columns go to U V)
    assert np.linalg.norm(d["R"]) < 0.8 * np.linalg.norm(w)


def test_rel_err_metric():
    ref = np.array([1.0, 2.0, 0.0])
    d = np.array([10.0, 10.0, 0.0])
    assert oracle.rel_err([1.0, 2.5, 0.0], ref, d) == 0.05
    assert oracle.rel_err([1.0, 2.0, 1e-30], ref, d) == float("inf")


# ---- the error normalisers ------------------------------------------------------
# Every GEMM parity bar divides by a normaliser D = sum |a||b| over the terms of
# the output.  A mistake in D (a dropped term, a dropped tensor scale) would
# make those bars vacuous, so D is pinned on its own: against the exact twin,
# against |C| where no term can cancel, as an upper bound of |C|, and for its
# scaling with each operand's tensor scale.

def _nonneg_linear_inputs(rng, M, K, N, r):
    x = synth.bf16_to_f32(synth.bf16_round(np.abs(rng.standard_normal((M, K)))))
    u = synth.bf16_to_f32(synth.bf16_round(np.abs(rng.standard_normal((N, r))) * 0.1))
    v = synth.bf16_to_f32(synth.bf16_round(np.abs(rng.standard_normal((r, K))) * 0.1))
    w = np.abs(rng.standard_t(3, size=(N, K)) * 0.02).astype(np.float32)
    dy = synth.bf16_to_f32(synth.bf16_round(np.abs(rng.standard_normal((M, N))) * 1e-3))
    return x, u, v, w, dy


@pytest.mark.parametrize("m,n,k", [(16, 16, 32), (8, 24, 48)])
def test_gemm_nt_abs_matches_rational_brute_force(m, n, k):
    rng = np.random.default_rng(7 * m + n + k)
    a = (rng.standard_normal((m, k)) * np.exp(rng.uniform(-2, 2, (m, 1)))).astype(np.float32)
    b = rng.standard_t(3, size=(n, k)).astype(np.float32)
    ra, _, _, _, sa = X.quantize_exact(a)
    rb, _, _, _, sb = X.quantize_exact(b)
    av = _exact_block_values(ra, X.quantize_rows_exact(a, sa)[1])
    bv = _exact_block_values(rb, X.quantize_rows_exact(b, sb)[1])
    qa, _, _ = oracle.quantize(a, colwise=False)
    qb, _, _ = oracle.quantize(b, colwise=False)
    got = oracle.gemm_nt_abs(qa, qb)
    for i in range(m):
        for j in range(n):
            want = sa * sb * sum((abs(av[i][t]) * abs(bv[j][t]) for t in range(k)), Fraction(0))
            assert abs(Fraction(float(got[i, j])) - want) <= want * Fraction(1, 2 ** 50)


def test_gemm_nt_abs_bounds_and_equals_the_product_without_cancellation():
    rng = np.random.default_rng(3)
    a = rng.standard_normal((40, 96)).astype(np.float32)
    b = rng.standard_t(3, size=(24, 96)).astype(np.float32)
    qa, _, _ = oracle.quantize(a, colwise=False)
    qb, _, _ = oracle.quantize(b, colwise=False)
    c, d = oracle.gemm_nt(qa, qb), oracle.gemm_nt_abs(qa, qb)
    assert np.all(d >= np.abs(c)) and np.any(d > np.abs(c) * 1.5)
    qa2, _, _ = oracle.quantize(np.abs(a), colwise=False)
    qb2, _, _ = oracle.quantize(np.abs(b), colwise=False)
    c2, d2 = oracle.gemm_nt(qa2, qb2), oracle.gemm_nt_abs(qa2, qb2)
    np.testing.assert_allclose(d2, np.abs(c2), rtol=1e-14, atol=0)


@pytest.mark.parametrize("ja,jb", [(3, 0), (0, -5), (7, -11)])
def test_gemm_nt_abs_scales_with_each_tensor_scale(ja, jb):
    """x -> 2^j x leaves codes and block scales alone and scales s_t by 2^j,
    so D scales by 2^(ja + jb) exactly; a normaliser without the tensor
    scales would not move."""
    rng = np.random.default_rng(ja * 31 + jb + 100)
    a = rng.standard_normal((32, 64)).astype(np.float32)
    b = rng.standard_normal((16, 64)).astype(np.float32)
    q = lambda x: oracle.quantize(x, colwise=False)[0]
    d0 = oracle.gemm_nt_abs(q(a), q(b))
    d1 = oracle.gemm_nt_abs(q(a * np.float32(2.0 ** ja)), q(b * np.float32(2.0 ** jb)))
    assert np.array_equal(d1, d0 * 2.0 ** (ja + jb))


def test_linear_normalisers_equal_the_outputs_without_cancellation():
    """With every input non-negative no term of Y, dX, dW, dU, dV can cancel,
    so each normaliser equals its output's magnitude; a dropped term (the
    rank-r part, a tensor scale) or a wrong one breaks the equality."""
    rng = np.random.default_rng(5)
    M, K, N, r = 48, 64, 32, 4
    x, u, v, w, dy = _nonneg_linear_inputs(rng, M, K, N, r)
    r_row, r_col, _ = oracle.quantize(w)
    for beta in (1.0, 0.5):
        f = oracle.linear_fwd(x, r_row, u, v, beta)
        np.testing.assert_allclose(f["D"], np.abs(f["Y64"]), rtol=1e-13, atol=0)
        b = oracle.linear_bwd(dy, x, r_col, u, v, f["T64"], beta, x_col=f["X_col"])
        for name in ("dX", "dW", "dU", "dV"):
            np.testing.assert_allclose(b[name + "_D"], np.abs(b[name]), rtol=1e-13, atol=0, err_msg=name)
    # with signs the normalisers bound the outputs and exceed them somewhere
    xs = x * rng.choice([-1.0, 1.0], x.shape).astype(np.float32)
    f = oracle.linear_fwd(xs, r_row, u, v)
    assert np.all(f["D"] >= np.abs(f["Y64"]) * (1 - 1e-13)) and np.any(f["D"] > 1.5 * np.abs(f["Y64"]))
    # the rank-r part of D is |beta| sum_j |T||U|: it scales with beta
    f1, f2 = oracle.linear_fwd(x, r_row, u, v, 1.0), oracle.linear_fwd(x, r_row, u, v, -2.0)
    d_main = oracle.gemm_nt_abs(f1["X_row"], r_row)
    np.testing.assert_allclose(f2["D"] - d_main, 2.0 * (f1["D"] - d_main), rtol=1e-12)
