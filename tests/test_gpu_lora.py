"""GPU parity of fs4_lora_project (subspace-constrained rank-r gradients)
against the oracle's Cholesky-QR projection.

The library computes the projections in fp64 from BF16 factors and fp32
gradients (both exact in fp64) and rounds the result to fp32 once; the oracle
computes them in fp64 through the explicit orthonormal bases.  The two differ
by the fp32 rounding (2^-24 relative) plus fp64 error amplified by the
condition of the Gram matrices (below 1e3 here), so the bar is
max |got - ref| <= 1e-6 max |ref| per tensor.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import dev_bf16, dev_f32, f32, need_gpu, print_case

pytestmark = pytest.mark.gpu
TOL = 1e-6


def _inputs(seed, N, K, r):
    rng = synth.rng_for(seed)
    u = synth.normal_bf16(rng, (N, r))
    v = synth.normal_bf16(rng, (r, K), std=0.5)
    du = rng.standard_normal((N, r)).astype(np.float32)
    dv = (rng.standard_normal((r, K)) * 3.0).astype(np.float32)
    return u, v, du, dv


def _run(fs4, u, v, du, dv):
    U, V = dev_bf16(u), dev_bf16(v)
    dU = dev_f32(du) if du is not None else None
    dV = dev_f32(dv) if dv is not None else None
    fs4.lora_project(U, V, dU, dV)
    torch.cuda.synchronize()
    return (dU.cpu().numpy() if dU is not None else None, dV.cpu().numpy() if dV is not None else None)


def _close(got, ref, what):
    assert got.shape == ref.shape, what
    assert np.all(np.isfinite(got)), what
    err = np.abs(got.astype(np.float64) - ref).max()
    assert err <= TOL * np.abs(ref).max(), (what, err, np.abs(ref).max())


@pytest.mark.parametrize("N,K,r", [(16, 16, 8), (100, 37, 5), (257, 1000, 64), (64, 64, 64),
                                   (4099, 130, 1), (1000, 4111, 32)])
def test_projection_matches_oracle(N, K, r):
    fs4 = need_gpu()
    print_case(test="lora_project", N=N, K=K, r=r)
    u, v, du, dv = _inputs(N + 7 * K + r, N, K, r)
    got_u, got_v = _run(fs4, u, v, du, dv)
    ref_u, ref_v = oracle.subspace_project(f32(u), f32(v), du, dv)
    _close(got_u, ref_u, "dU")
    _close(got_v, ref_v, "dV")


def test_projection_3b_factors_and_linear_bwd_gradients():
    """The 3B-shape factors (rank 32, N 8192, K 3072) with the gradients
    fs4_linear_bwd produces for them."""
    fs4 = need_gpu()
    print_case(test="lora_project_3b")
    d = synth.linear3b()
    dy = synth.linear3b_dy()
    X, U, V = dev_bf16(d["X"]), dev_bf16(d["U"]), dev_bf16(d["V"])
    Rw = dev_f32(d["R"])
    R_row, R_col = fs4.quantize(Rw)
    f = fs4.linear_fwd(X, R_row, U, V)
    b = fs4.linear_bwd(dev_bf16(dy), X, f.X_col, R_col, U, V, f.T)
    du = b.dU.cpu().numpy()
    dv = b.dV.cpu().numpy()
    fs4.lora_project(U, V, b.dU, b.dV)
    torch.cuda.synchronize()
    ref_u, ref_v = oracle.subspace_project(f32(d["U"]), f32(d["V"]), du, dv)
    _close(b.dU.cpu().numpy(), ref_u, "dU")
    _close(b.dV.cpu().numpy(), ref_v, "dV")


def test_subspace_members_are_kept_and_complements_dropped():
    fs4 = need_gpu()
    N, K, r = 512, 384, 16
    u, v, _, _ = _inputs(11, N, K, r)
    u64, v64 = f32(u).astype(np.float64), f32(v).astype(np.float64)
    rng = np.random.default_rng(5)
    c = rng.standard_normal((r, r))
    du_in = (u64 @ c).astype(np.float32)
    dv_in = (c @ v64).astype(np.float32)
    got_u, got_v = _run(fs4, u, v, du_in, dv_in)
    ref_u, ref_v = oracle.subspace_project(u64, v64, du_in, dv_in)
    _close(got_u, ref_u, "dU in span")
    _close(got_v, ref_v, "dV in row space")
    assert np.abs(got_u - du_in).max() <= 1e-5 * np.abs(du_in).max()
    z = rng.standard_normal((N, r))
    perp_u = (z - u64 @ np.linalg.lstsq(u64, z, rcond=None)[0]).astype(np.float32)
    z = rng.standard_normal((r, K))
    perp_v = (z - (v64.T @ np.linalg.lstsq(v64.T, z.T, rcond=None)[0]).T).astype(np.float32)
    got_u, got_v = _run(fs4, u, v, perp_u, perp_v)
    assert np.abs(got_u).max() <= 1e-5 * np.abs(perp_u).max()
    assert np.abs(got_v).max() <= 1e-5 * np.abs(perp_v).max()


def test_one_side_only_and_empty():
    fs4 = need_gpu()
    N, K, r = 300, 200, 12
    u, v, du, dv = _inputs(3, N, K, r)
    got_u, _ = _run(fs4, u, v, du, None)
    ref_u, _ = oracle.subspace_project(f32(u), f32(v), du, None)
    _close(got_u, ref_u, "dU alone")
    _, got_v = _run(fs4, u, v, None, dv)
    _, ref_v = oracle.subspace_project(f32(u), f32(v), None, dv)
    _close(got_v, ref_v, "dV alone")
    # N = 0: nothing to project on the U side, the V side still runs
    U0 = torch.empty((0, r), dtype=torch.bfloat16, device="cuda")
    dU0 = torch.empty((0, r), dtype=torch.float32, device="cuda")
    V, dV = dev_bf16(v), dev_f32(dv)
    fs4.lora_project(U0, V, dU0, dV)
    torch.cuda.synchronize()
    _close(dV.cpu().numpy(), ref_v, "dV with N = 0")


def test_rank_deficient_side_is_nan():
    fs4 = need_gpu()
    N, K, r = 128, 96, 6
    u, v, du, dv = _inputs(9, N, K, r)
    u = u.copy()
    u[:, 3] = u[:, 1]                      # two equal columns: U^T U is singular
    got_u, got_v = _run(fs4, u, v, du, dv)
    assert np.all(np.isnan(got_u))
    _, ref_v = oracle.subspace_project(f32(u), f32(v), None, dv)
    _close(got_v, ref_v, "dV beside a singular U")
