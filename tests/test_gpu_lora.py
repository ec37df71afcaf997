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


def test_projection_3b_factors_and_linear_bwd_gradients(linear3b_inputs):
    """The 3B-shape factors (rank 32, N 8192, K 3072) with the gradients
    fs4_linear_bwd produces for them."""
    fs4 = need_gpu()
    print_case(test="lora_project_3b")
    d, dy = linear3b_inputs
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


# ---- realignment ------------------------------------------------------------
# Same algorithm on both sides with the same test vectors; the library's
# products with W use fp32 operands (~16-bit products), so the basis it finds
# differs from the fp64 oracle's by ~1e-5, and BF16 rounding of the factors
# can then land one BF16 step apart.  Compared: the singular values (1e-4,
# or 1e-3 for the flat 3B spectrum), the reconstruction beta U V + R = W
# (strict: fp32 rounding only), the rank-r part beta U V (within two BF16
# steps of its largest entry), and the residual's norm.

def _realign_case(fs4, u, v, res, om, beta, q):
    U, V, R = dev_bf16(u), dev_bf16(v), dev_f32(res)
    sig = fs4.lora_realign(U, V, R, dev_f32(om), beta=beta, power_iters=q)
    torch.cuda.synchronize()
    ub = U.view(torch.int16).cpu().numpy().view(np.uint16)
    vb = V.view(torch.int16).cpu().numpy().view(np.uint16)
    return f32(ub).astype(np.float64), f32(vb).astype(np.float64), R.cpu().numpy(), sig.cpu().numpy()


def _check_realign(got, ref, w, beta, s_rtol):
    gu, gv, gr, gs = got
    ou, ov, orr, os_ = ref
    assert np.all(np.isfinite(gu)) and np.all(np.isfinite(gv)) and np.all(np.isfinite(gr))
    assert np.allclose(gs, os_, rtol=s_rtol, atol=0), (gs[:4], os_[:4])
    # the split holds W exactly up to fp32 rounding
    assert np.abs(beta * (gu @ gv) + gr - w).max() <= 1e-6 * np.abs(w).max()
    lr_g, lr_o = beta * (gu @ gv), beta * (ou @ ov)
    assert np.abs(lr_g - lr_o).max() <= 2 ** -7 * np.abs(lr_o).max()
    assert abs(np.linalg.norm(gr) - np.linalg.norm(orr)) <= 1e-3 * np.linalg.norm(orr)


def _bf16_bits(x):
    return synth.bf16_round(np.asarray(x, np.float64))


@pytest.mark.parametrize("N,K,r,l,q,beta", [(256, 192, 8, 16, 1, 1.0), (512, 160, 5, 13, 2, 0.5),
                                            (144, 304, 16, 24, 0, 2.0)])
def test_realign_matches_oracle_with_a_gap(N, K, r, l, q, beta):
    fs4 = need_gpu()
    print_case(test="lora_realign", N=N, K=K, r=r, l=l, q=q, beta=beta)
    rng = np.random.default_rng(N + K + r)
    a, _ = np.linalg.qr(rng.standard_normal((N, r + 30)))
    b, _ = np.linalg.qr(rng.standard_normal((K, r + 30)))
    sig = np.concatenate([np.linspace(4, 2, r), 0.02 * np.exp(-np.arange(30) / 8)])
    w_true = (a * sig) @ b.T
    u = _bf16_bits(rng.standard_normal((N, r)) * 0.05)
    v = _bf16_bits(rng.standard_normal((r, K)) * 0.05)
    res = (w_true - beta * f32(u).astype(np.float64) @ f32(v).astype(np.float64)).astype(np.float32)
    w = beta * f32(u).astype(np.float64) @ f32(v).astype(np.float64) + res.astype(np.float64)
    om = rng.standard_normal((l, K)).astype(np.float32)
    got = _realign_case(fs4, u, v, res, om, beta, q)
    ref = oracle.lora_realign(f32(u), f32(v), res, beta, om, q)
    _check_realign(got, ref, w, beta, 1e-4)


def test_realign_exactly_low_rank():
    fs4 = need_gpu()
    N, K, r, l = 320, 256, 6, 12
    rng = np.random.default_rng(21)
    w_true = (rng.standard_normal((N, r)) * [5, 4, 3, 2, 1, 0.5]) @ rng.standard_normal((r, K))
    u = _bf16_bits(rng.standard_normal((N, r)) * 0.1)
    v = _bf16_bits(rng.standard_normal((r, K)) * 0.1)
    res = (w_true - f32(u).astype(np.float64) @ f32(v).astype(np.float64)).astype(np.float32)
    w = f32(u).astype(np.float64) @ f32(v).astype(np.float64) + res.astype(np.float64)
    om = rng.standard_normal((l, K)).astype(np.float32)
    gu, gv, gr, gs = _realign_case(fs4, u, v, res, om, 1.0, 1)
    s_true = np.linalg.svd(w, compute_uv=False)[:r]
    assert np.allclose(gs, s_true, rtol=1e-5)
    assert np.abs(gr).max() <= 2 ** -7 * np.abs(w).max()      # only the factors' BF16 rounding
    assert np.abs(gu @ gv + gr - w).max() <= 1e-6 * np.abs(w).max()


def test_realign_3b_shapes(linear3b_inputs):
    """The 3B weight (N 8192, K 3072, rank 32), l = 40 test vectors, one
    power iteration."""
    fs4 = need_gpu()
    print_case(test="lora_realign_3b")
    d = linear3b_inputs[0]
    u, v, res = d["U"], d["V"], d["R"]
    rng = synth.rng_for(1234)
    om = rng.standard_normal((40, 3072)).astype(np.float32)
    w = f32(u).astype(np.float64) @ f32(v).astype(np.float64) + res.astype(np.float64)
    got = _realign_case(fs4, u, v, res, om, 1.0, 1)
    ref = oracle.lora_realign(f32(u), f32(v), res, 1.0, om, 1)
    _check_realign(got, ref, w, 1.0, 1e-3)
