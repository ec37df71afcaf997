"""Pins for the oracle's LoRA-SVD training-side steps (Cholesky-QR and the
subspace-constrained low-rank gradients)."""
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
