"""GPU parity of the Q-Root outlier clipping: the |x| quantile (bit-exact:
it is a selection, an element of |x|), the clipped quantizer (codes and
scales bit-exact, as for the plain quantizer), and Newton-Schulz with the
iterate clipped at its p99 (per step, from the oracle's iterates)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_view_equal, dev_bf16, dev_f32, f32, need_gpu, ns_step_bounds, print_case, within
from oracle.newton_schulz import MUON_ABC, abs_quantile, clip_abs

pytestmark = pytest.mark.gpu
TIGHT = 1e-5


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
    """One clipped step at a time from the oracle's own iterate X_k: A (from
    the shared, bit-exact clipped views of X_k) within 1e-5 of its
    normaliser; B and X' against the oracle's own B and X' within the bounds
    of tests/gpu_util.ns_step_bounds.  A last-bit difference in the fp32 A
    (the MFMA's summation order against the oracle's rounded exact sum) can
    move an E4M3 block scale of Q(A) across a tie, which moves B by ~1e-2 of
    its normaliser at 768 x 2048 (a float32 summation on the CPU does the
    same); both results are correct, and the bounds admit what any A within
    the 1e-5 bar can change through its quantization, and no more.  Every
    expected value and bound comes from the oracle's values alone."""
    fs4 = need_gpu()
    print_case(test="ns_clip_step", m=m, n=n)
    g = synth.ns_input(seed=7, m=m, n=n)
    xs, steps = oracle.newton_schulz(f32(g), 5, clip_q=0.99)
    for k in range(5):
        X, tX, tA, tB = fs4.newton_schulz(dev_f32(xs[k]), steps=1, normalize=False, trace=True, clip_q=0.99)
        st = steps[k]
        eps_a, eps_b, eps_x = ns_step_bounds(xs[k], st, *MUON_ABC, tol=TIGHT, clip_p=st["P"])
        Ag, Bg, Xg = tA[0].cpu().numpy(), tB[0].cpu().numpy(), X.cpu().numpy()
        rA, rB, rX = within(Ag, st["A64"], eps_a), within(Bg, st["B64"], eps_b), within(Xg, st["X64"], eps_x)
        print("step", k, "p %.4e A %.2e B %.2e X %.2e of their bounds; errB %.2e errX %.2e" % (
            st["P"], rA, rB, rX, oracle.rel_err(Bg, st["B64"], st["B_D"]), oracle.rel_err(Xg, st["X64"], st["X_D"])),
            flush=True)
        assert rA <= 1.0 and rB <= 1.0 and rX <= 1.0, (k, rA, rB, rX)


def test_clip_at_the_maximum_equals_plain_ns():
    fs4 = need_gpu()
    g = dev_bf16(synth.ns_input(seed=8, m=128, n=384))
    plain = fs4.newton_schulz(g, steps=3)
    full = fs4.newton_schulz(g, steps=3, clip_q=1.0)
    torch.cuda.synchronize()
    assert torch.equal(plain, full)
