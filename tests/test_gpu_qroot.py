"""GPU parity of the Q-Root outlier clipping: the |x| quantile (bit-exact:
it is a selection, an element of |x|), the clipped quantizer (codes and
scales bit-exact, as for the plain quantizer), and Newton-Schulz with the
iterate clipped at its p99 (per step, within the GEMM tolerance of the
plain NS tests)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_view_equal, dev_bf16, dev_f32, f32, need_gpu, print_case
from oracle.newton_schulz import MUON_ABC, abs_quantile, clip_abs

pytestmark = pytest.mark.gpu
TOL = 1e-3


def _inputs(kind, n, seed):
    rng = np.random.default_rng(seed)
    if kind == "normal":
        return rng.standard_normal(n).astype(np.float32)
    if kind == "ties":                                   # few distinct magnitudes, many zeros
        v = np.round(rng.standard_normal(n) * 2).astype(np.float32)
        v[rng.random(n) < 0.4] = 0.0
        return v
    if kind == "heavy":                                  # Student-t(2) outliers, wide exponent range
        return (rng.standard_t(2, n) * np.exp(rng.uniform(-30, 30, n))).astype(np.float32)
    if kind == "tiny":                                   # fp32 subnormals and zeros
        v = (rng.standard_normal(n) * 1e-40).astype(np.float32)
        v[::3] = 0.0
        return v
    raise ValueError(kind)


@pytest.mark.parametrize("kind", ["normal", "ties", "heavy", "tiny"])
@pytest.mark.parametrize("n", [1, 7, 4099, 262147])
def test_abs_quantile_is_exact(kind, n):
    fs4 = need_gpu()
    print_case(test="abs_quantile", kind=kind, n=n)
    x = _inputs(kind, n, n)
    X = dev_f32(x)
    for q in (1e-9, 0.5, 0.9, 0.99, 1.0):
        got = fs4.abs_quantile(X, q).cpu().numpy()[0]
        want = abs_quantile(x, q)
        assert np.float32(got).tobytes() == want.tobytes(), (q, got, want)


def test_abs_quantile_bf16_and_full_ns_size():
    fs4 = need_gpu()
    print_case(test="abs_quantile_bf16_full")
    g = synth.ns_input()                                 # 3072 x 8192 bf16
    G = dev_bf16(g)
    x = f32(g)
    for q in (0.99, 0.5, 1.0):
        got = fs4.abs_quantile(G, q).cpu().numpy()[0]
        assert np.float32(got).tobytes() == abs_quantile(x, q).tobytes(), q
    # the fp32 iterate the clipped NS sees
    x0 = oracle.ns_normalize(x)[0]
    got = fs4.abs_quantile(dev_f32(x0), 0.99).cpu().numpy()[0]
    assert np.float32(got).tobytes() == abs_quantile(x0, 0.99).tobytes()


@pytest.mark.parametrize("rows,cols,bf16", [(48, 80, False), (272, 400, True), (1040, 208, False),
                                            (4096, 4096, True)])
def test_quantize_clipped_is_bit_exact(rows, cols, bf16):
    fs4 = need_gpu()
    print_case(test="quantize_clipped", rows=rows, cols=cols, bf16=bf16)
    if bf16 and rows == 4096:
        xb = synth.quantizer_input()                     # ~N(0,1) with 0.1% of entries x50
        x = f32(xb)
        X = dev_bf16(xb)
    else:
        rng = np.random.default_rng(rows + cols)
        x = (rng.standard_t(3, (rows, cols))).astype(np.float32)
        if bf16:
            xb = synth.bf16_round(x.astype(np.float64))
            x = f32(xb)
            X = dev_bf16(xb)
        else:
            X = dev_f32(x)
    row, col = fs4.quantize_clipped(X, 0.99)
    p = abs_quantile(x, 0.99)
    ref_row, ref_col, _ = oracle.quantize(clip_abs(x, p))
    assert_view_equal(row, ref_row, "row")
    assert_view_equal(col, ref_col, "col")


@pytest.mark.parametrize("m,n", [(192, 512), (768, 2048)])
def test_clipped_ns_per_step(m, n):
    """Each product of a clipped step is checked from the GPU's own input to
    it: A from the shared X_k, B from the GPU's A (re-quantized by the
    oracle), X_{k+1} from the GPU's B.  A last-bit difference in fp32 A can
    move one E4M3 block scale across a tie (the oracle alone reproduces it:
    recomputing A in another summation order flips one block scale and moves
    B by ~1e-2 of its normaliser at 768 x 2048), so the quantization
    decisions must be taken on the same values on both sides."""
    from oracle.linear import gemm_nt, gemm_nt_abs
    fs4 = need_gpu()
    print_case(test="ns_clip_step", m=m, n=n)
    g = synth.ns_input(seed=7, m=m, n=n)
    a, b, c = MUON_ABC
    xs, steps = oracle.newton_schulz(f32(g), 5, clip_q=0.99)
    for k in range(5):
        X, tX, tA, tB = fs4.newton_schulz(dev_f32(xs[k]), steps=1, normalize=False, trace=True, clip_q=0.99)
        st = steps[k]
        Ag, Bg, Xg = tA[0].cpu().numpy(), tB[0].cpu().numpy(), X.cpu().numpy()
        eA = oracle.rel_err(Ag, st["A64"], st["A_D"])
        ar, ac, _ = oracle.quantize(Ag)
        b_ref = b * Ag.astype(np.float64) + c * gemm_nt(ar, ac)
        b_d = abs(b) * np.abs(Ag.astype(np.float64)) + abs(c) * gemm_nt_abs(ar, ac)
        eB = oracle.rel_err(Bg, b_ref, b_d)
        br, _, _ = oracle.quantize(Bg, rowwise=True, colwise=False)
        _, xcol, _ = oracle.quantize(clip_abs(xs[k], st["P"]), rowwise=False, colwise=True)
        x64 = xs[k].astype(np.float64)
        x_ref = a * x64 + gemm_nt(br, xcol)
        x_d = abs(a) * np.abs(x64) + gemm_nt_abs(br, xcol)
        eX = oracle.rel_err(Xg, x_ref, x_d)
        print("step", k, "p %.4e errA %.2e errB %.2e errX %.2e" % (st["P"], eA, eB, eX), flush=True)
        assert eA <= TOL and eB <= TOL and eX <= TOL, (k, eA, eB, eX)


def test_clip_at_the_maximum_equals_plain_ns():
    fs4 = need_gpu()
    g = dev_bf16(synth.ns_input(seed=8, m=128, n=384))
    plain = fs4.newton_schulz(g, steps=3)
    full = fs4.newton_schulz(g, steps=3, clip_q=1.0)
    torch.cuda.synchronize()
    assert torch.equal(plain, full)
