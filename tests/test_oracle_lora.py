"""Pins for the oracle's LoRA-SVD training-side steps (Cholesky-QR, the
subspace-constrained low-rank gradients, the randomized-SVD realignment)."""
import numpy as np
import pytest

from oracle.lora import cholesky_qr, subspace_project


def test_cholesky_qr_closed_forms():
    # one column: Q = a / |a|, Rf = |a|
    q, rf = cholesky_qr(np.array([[3.0], [4.0]]))
    assert np.allclose(q, [[0.6], [0.8]], rtol=0, atol=1e-15)
    assert np.allclose(rf, [[5.0]], rtol=0, atol=1e-15)
    # worked by hand: A = [[1,0],[1,1],[0,1]], A^T A = [[2,1],[1,2]],
    # L = [[sqrt2, 0], [1/sqrt2, sqrt(3/2)]]
    a = np.array([[1.0, 0.0], [1.0, 1.0], [0.0, 1.0]])
    q, rf = cholesky_qr(a)
    s2, s15 = np.sqrt(2.0), np.sqrt(1.5)
    want_q = np.array([[1 / s2, -0.5 / s15], [1 / s2, 0.5 / s15], [0.0, 1 / s15]])
    want_r = np.array([[s2, 1 / s2], [0.0, s15]])
    assert np.allclose(q, want_q, rtol=0, atol=1e-15)
    assert np.allclose(rf, want_r, rtol=0, atol=1e-15)


@pytest.mark.parametrize("n,r", [(64, 8), (300, 32), (1000, 64), (40, 40)])
def test_cholesky_qr_is_the_unique_positive_qr(n, r):
    rng = np.random.default_rng(n + r)
    a = rng.standard_normal((n, r)) * np.exp(rng.uniform(-1, 1, r))[None, :]
    q, rf = cholesky_qr(a)
    assert np.allclose(q.T @ q, np.eye(r), rtol=0, atol=1e-10)
    assert np.allclose(q @ rf, a, rtol=0, atol=1e-12 * np.abs(a).max())
    assert np.allclose(np.tril(rf, -1), 0.0)
    assert np.all(np.diag(rf) > 0)
    # Householder QR reaches the same factorisation once its diagonal signs
    # are made positive (the QR of a full-rank matrix with diag(R) > 0 is unique)
    qh, rh = np.linalg.qr(a)
    sg = np.sign(np.diag(rh))
    assert np.allclose(q, qh * sg[None, :], rtol=0, atol=1e-9)
    assert np.allclose(rf, rh * sg[:, None], rtol=0, atol=1e-9 * np.abs(rh).max())


def test_cholesky_qr_rejects_rank_deficient():
    a = np.ones((10, 2))
    with pytest.raises(np.linalg.LinAlgError):
        cholesky_qr(a)


def _factors(seed, n=96, k=80, r=6):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((n, r)), rng.standard_normal((r, k)), rng


def test_projection_keeps_the_subspace_and_drops_its_complement():
    u, v, rng = _factors(1)
    n, r = u.shape
    k = v.shape[1]
    c = rng.standard_normal((r, r))
    inside_u = u @ c                           # columns in span(U)
    inside_v = c @ v                           # rows in the row space of V
    du_c, dv_c = subspace_project(u, v, inside_u, inside_v)
    assert np.allclose(du_c, inside_u, rtol=0, atol=1e-12)
    assert np.allclose(dv_c, inside_v, rtol=0, atol=1e-12)
    # complements: remove the least-squares fit
    z = rng.standard_normal((n, r))
    perp_u = z - u @ np.linalg.lstsq(u, z, rcond=None)[0]
    z = rng.standard_normal((r, k))
    perp_v = z - (v.T @ np.linalg.lstsq(v.T, z.T, rcond=None)[0]).T
    du_c, dv_c = subspace_project(u, v, perp_u, perp_v)
    assert np.abs(du_c).max() < 1e-12
    assert np.abs(dv_c).max() < 1e-12


def test_projection_is_the_least_squares_fit_and_idempotent():
    u, v, rng = _factors(2, n=200, k=150, r=12)
    du = rng.standard_normal(u.shape)
    dv = rng.standard_normal(v.shape)
    du_c, dv_c = subspace_project(u, v, du, dv)
    # closest point of span(U) to each column of dU
    assert np.allclose(du_c, u @ np.linalg.lstsq(u, du, rcond=None)[0], rtol=0, atol=1e-12)
    # closest point of the row space of V to each row of dV
    assert np.allclose(dv_c, (v.T @ np.linalg.lstsq(v.T, dv.T, rcond=None)[0]).T, rtol=0, atol=1e-12)
    du_cc, dv_cc = subspace_project(u, v, du_c, dv_c)
    assert np.allclose(du_cc, du_c, rtol=0, atol=1e-12)
    assert np.allclose(dv_cc, dv_c, rtol=0, atol=1e-12)
    # the residual of the projection is orthogonal to the subspace
    assert np.abs(u.T @ (du - du_c)).max() < 1e-10
    assert np.abs((dv - dv_c) @ v.T).max() < 1e-10


def test_projection_depends_only_on_the_subspace():
    u, v, rng = _factors(3, n=64, k=48, r=5)
    m = rng.standard_normal((5, 5)) + 3 * np.eye(5)      # invertible
    du = rng.standard_normal(u.shape)
    dv = rng.standard_normal(v.shape)
    a_u, a_v = subspace_project(u, v, du, dv)
    b_u, b_v = subspace_project(u @ m, np.linalg.inv(m) @ v, du, dv)
    assert np.allclose(a_u, b_u, rtol=0, atol=1e-11)
    assert np.allclose(a_v, b_v, rtol=0, atol=1e-11)


def test_projection_sides_are_independent():
    u, v, rng = _factors(4)
    du = rng.standard_normal(u.shape)
    dv = rng.standard_normal(v.shape)
    both_u, both_v = subspace_project(u, v, du, dv)
    only_u, none_v = subspace_project(u, v, du, None)
    none_u, only_v = subspace_project(u, v, None, dv)
    assert none_u is None and none_v is None
    assert np.array_equal(both_u, only_u) and np.array_equal(both_v, only_v)


# ---- realignment ------------------------------------------------------------
from oracle.lora import bf16_rne, lora_realign


def test_bf16_rounding_matches_torch():
    import torch
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(5000) * np.exp(rng.uniform(-20, 20, 5000)),
                        [0.0, -0.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 65504.0, 1e-40]])
    want = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(bf16_rne(x), want)


def _split(w, r, rng, beta=1.0):
    """An arbitrary (not principal) split of w: random BF16 factors, R the rest."""
    n, k = w.shape
    u = bf16_rne(rng.standard_normal((n, r)) * 0.1)
    v = bf16_rne(rng.standard_normal((r, k)) * 0.1)
    return u, v, (w - beta * (u @ v)).astype(np.float32)


def test_realign_recovers_an_exactly_low_rank_weight():
    rng = np.random.default_rng(1)
    n, k, r, l = 120, 96, 6, 10
    w = (rng.standard_normal((n, r)) * [8, 5, 3, 2, 1, 0.5]) @ rng.standard_normal((r, k))
    w = w.astype(np.float32).astype(np.float64)
    u, v, res = _split(w, r, rng)
    w = u @ v + res.astype(np.float64)        # the weight the split holds (R is fp32)
    s_true = np.linalg.svd(w, compute_uv=False)[:r]
    for q in (0, 1, 2):
        u2, v2, r2, s = lora_realign(u, v, res, 1.0, rng.standard_normal((l, k)), q)
        assert np.allclose(s, s_true, rtol=1e-10, atol=0)
        # W is rank r to within fp32: the residual holds the BF16 rounding of
        # the factors
        assert np.abs(r2).max() <= 2 ** -7 * np.abs(w).max()
        assert np.abs(u2 @ v2 + r2 - w).max() <= 1e-6 * np.abs(w).max()


def test_realign_matches_the_truncated_svd_with_a_gap():
    rng = np.random.default_rng(2)
    n, k, r, l = 200, 160, 8, 16
    a, _ = np.linalg.qr(rng.standard_normal((n, n)))
    b, _ = np.linalg.qr(rng.standard_normal((k, k)))
    sig = np.concatenate([np.linspace(10, 5, r), 0.05 * np.exp(-np.arange(k - r) / 20)])
    w = (a[:, :k] * sig) @ b.T
    u, v, res = _split(w, r, rng)
    u2, v2, r2, s = lora_realign(u, v, res, 1.0, rng.standard_normal((l, k)), 2)
    assert np.allclose(s, sig[:r], rtol=1e-8)
    best = (a[:, :r] * sig[:r]) @ b[:, :r].T              # Eckart-Young
    assert np.abs(u2 @ v2 - best).max() <= 2 ** -7 * np.abs(best).max()
    # the residual's norm is the tail of the spectrum, up to the factors' rounding
    assert abs(np.linalg.norm(r2) - np.linalg.norm(sig[r:])) <= 2 ** -7 * np.linalg.norm(best)


def test_realign_depends_only_on_the_weight_and_splits_beta():
    rng = np.random.default_rng(3)
    n, k, r, l = 64, 80, 4, 8
    w = rng.standard_normal((n, k)) + 6 * np.outer(rng.standard_normal(n), rng.standard_normal(k))
    om = rng.standard_normal((l, k))
    u, v, res = _split(w, r, rng)
    u_b, v_b, res_b = _split(w, r, np.random.default_rng(33))
    out1 = lora_realign(u, v, res, 1.0, om, 1)
    out2 = lora_realign(u_b, v_b, res_b, 1.0, om, 1)
    # the two splits hold W to within the fp32 rounding of their residuals
    assert np.allclose(out1[3], out2[3], rtol=1e-6)
    assert np.abs(out1[0] @ out1[1] - out2[0] @ out2[1]).max() <= 2 ** -7 * np.abs(w).max()
    # beta: the same weight with beta = 4 gives factors half as large
    u4, v4, res4 = _split(w, r, rng, beta=4.0)
    o4 = lora_realign(u4, v4, res4, 4.0, om, 1)
    assert np.allclose(o4[3], out1[3], rtol=1e-6)
    assert np.abs(4.0 * o4[0] @ o4[1] - out1[0] @ out1[1]).max() <= 2 ** -7 * np.abs(w).max()
    assert np.abs(4.0 * (o4[0] @ o4[1]) + o4[2] - w).max() <= 1e-6 * np.abs(w).max()
