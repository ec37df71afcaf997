"""NVFP4 Newton-Schulz parity vs the oracle.

The iteration amplifies NVFP4 noise once aX and BX start to cancel, so two
correct implementations that differ only in fp32 summation order drift apart
over several steps.  Parity is therefore checked one step at a time: the HIP
path is started (normalize=0, steps=1) from the oracle's own iterate X_k and
its A, B and X_{k+1} are compared with the oracle's step from the same X_k,
normalised by sum |a||b| (+ |b A| and |a X| for the elementwise terms), with
the allowance of tests/gpu_util.ns_step_bounds for B and X_{k+1}.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import need_gpu, dev_bf16, dev_f32, print_case, f32, ns_step_bounds, within
from oracle.newton_schulz import MUON_ABC, shape_coefficients

pytestmark = pytest.mark.gpu

TOL = 1e-3
TIGHT = 1e-5


@pytest.mark.parametrize("m,n", [(192, 512), (80, 208)])
def test_normalization(m, n):
    fs4 = need_gpu()
    print_case(test="ns_normalize", m=m, n=n)
    g = synth.ns_input(seed=5, m=m, n=n)
    X = fs4.newton_schulz(dev_bf16(g), steps=0).cpu().numpy()
    _, ref = oracle.ns_normalize(f32(g))
    # one fp32 rounding of an fp64 value on each side
    assert np.max(np.abs(X - ref) / np.maximum(np.abs(ref), 1e-30)) <= 2.0 ** -23


def test_zero_steps_without_normalization_is_a_copy():
    """steps=0, normalize=0 returns G as fp32 exactly (the iterate is held
    transposed inside; 80 x 208 leaves partial 64 x 64 tiles)."""
    fs4 = need_gpu()
    print_case(test="ns_copy", m=80, n=208)
    g = synth.ns_input(seed=6, m=80, n=208)
    X = fs4.newton_schulz(dev_bf16(g), steps=0, normalize=False).cpu().numpy()
    assert np.array_equal(X, f32(g))


def _f32_abc(abc):
    return tuple(float(np.float32(v)) for v in abc)


@pytest.mark.parametrize("m,n,coef", [(192, 512, "muon"), (768, 2048, "muon"), (768, 2048, "shape")])
def test_per_step_parity(m, n, coef):
    """Each step from the oracle's own iterate X_k: A within 1e-5 of its
    normaliser (both sides multiply the same bit-exact views of X_k); B and
    X' within the bounds of tests/gpu_util.ns_step_bounds, which add to the
    1e-5 bar what any A (then B) within that bar can change through its
    quantization (a decision on a tie may come out either way for two
    correct summation orders)."""
    fs4 = need_gpu()
    print_case(test="ns_step", m=m, n=n, coef=coef)
    # shape: the oracle's shape-dependent (a, b, c) (Q-Root reading), as the
    # float32 values both sides then use
    abc = _f32_abc(MUON_ABC if coef == "muon" else shape_coefficients(m, n))
    g = synth.ns_input(seed=5, m=m, n=n)
    xs, steps = oracle.newton_schulz(f32(g), 5, abc=abc)
    for k in range(5):
        X, tX, tA, tB = fs4.newton_schulz(dev_f32(xs[k]), steps=1, abc=abc, normalize=False, trace=True)
        st = steps[k]
        Ag, Bg, Xg = tA[0].cpu().numpy(), tB[0].cpu().numpy(), X.cpu().numpy()
        eps_a, eps_b, eps_x = ns_step_bounds(xs[k], st, *abc, tol=TIGHT)
        rA, rB, rX = within(Ag, st["A64"], eps_a), within(Bg, st["B64"], eps_b), within(Xg, st["X64"], eps_x)
        eB, eX = oracle.rel_err(Bg, st["B64"], st["B_D"]), oracle.rel_err(Xg, st["X64"], st["X_D"])
        print("step", k, "A %.2e B %.2e X %.2e of their bounds; errB %.2e errX %.2e" % (rA, rB, rX, eB, eX),
              flush=True)
        assert rA <= 1.0 and rB <= 1.0 and rX <= 1.0, (k, rA, rB, rX)


def test_full_size_first_product_sampled():
    """3072 x 8192 momentum: normalisation in full and the first product
    A = Q(X_0) Q(X_0)^T on sampled entries, plus the full 5-step run's
    iterate staying in the band the quantized iteration reaches."""
    fs4 = need_gpu()
    print_case(test="ns_3072x8192")
    g = synth.ns_input()
    X, tX, tA, tB = fs4.newton_schulz(dev_bf16(g), steps=5, trace=True)
    x0_ref32, x0_ref = oracle.ns_normalize(f32(g))
    x0 = tX[0].cpu().numpy()
    assert np.max(np.abs(x0 - x0_ref) / np.maximum(np.abs(x0_ref), 1e-30)) <= 2.0 ** -23
    from oracle.quantize import quantize_rows, tensor_scale
    s = tensor_scale(x0_ref32)
    rng = np.random.default_rng(1)
    A0 = tA[0]
    for i, j in zip(rng.integers(0, 3072, 24), rng.integers(0, 3072, 24)):
        qi = oracle.block_values(quantize_rows(x0_ref32[i:i + 1], s))[0]
        qj = oracle.block_values(quantize_rows(x0_ref32[j:j + 1], s))[0]
        ref = float(s) ** 2 * np.dot(qi, qj)
        den = float(s) ** 2 * np.dot(np.abs(qi), np.abs(qj))
        assert abs(A0[i, j].item() - ref) <= TOL * den
    assert torch.equal(X, tX[5])
    assert torch.isfinite(X).all()


@pytest.mark.parametrize("m,n,clip", [(208, 512, 0.0), (768, 2048, 0.0), (3072, 8192, 0.0), (208, 512, 0.99)])
def test_upper_triangle_path_equals_traced_path(m, n, clip):
    """Untraced, A and B keep only their upper triangle's tiles and the
    quantizer writes each lower block from its mirror image; traced, both
    are stored whole and quantized whole.  A and B are exactly symmetric, so
    the codes, and every iterate, must agree bit for bit (208 leaves partial
    64 x 64 and 128 x 128 tiles on the diagonal)."""
    fs4 = need_gpu()
    print_case(test="ns_upper_vs_traced", m=m, n=n, clip=clip)
    G = dev_bf16(synth.ns_input(seed=9, m=m, n=n))
    X1 = fs4.newton_schulz(G, steps=5, clip_q=clip).cpu().numpy()
    X2, tX, tA, tB = fs4.newton_schulz(G, steps=5, trace=True, clip_q=clip)
    assert np.array_equal(X1.view(np.uint32), X2.cpu().numpy().view(np.uint32))
    A = tA.cpu().numpy()
    assert np.array_equal(A, np.transpose(A, (0, 2, 1)))
