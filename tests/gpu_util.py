"""Helpers for the GPU parity tests: move synth arrays to the device, bring
NVFP4 views back, run the oracle on the same inputs."""
import numpy as np
import pytest
import torch

import oracle
import synth


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import precision_pretraining_amd as fs4   # raises ImportError if libfs4.so is missing
    return fs4


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def host_view(v):
    """(codes uint8, scales uint8, tscale float32) of a device NVFP4 view."""
    torch.cuda.synchronize()
    return v.codes.cpu().numpy(), v.scales.cpu().numpy(), np.float32(v.tscale.cpu().item())


def assert_view_equal(gpu_view, ref: "oracle.NVFP4", what=""):
    codes, scales, ts = host_view(gpu_view)
    assert ts.tobytes() == np.float32(ref.tscale).tobytes(), (what, ts, ref.tscale)
    bad_s = np.argwhere(scales != ref.scales)
    assert bad_s.size == 0, (what, "scales differ", bad_s[:5], scales[tuple(bad_s[0])], ref.scales[tuple(bad_s[0])])
    bad_c = np.argwhere(codes != ref.codes)
    assert bad_c.size == 0, (what, "codes differ", bad_c[:5], codes[tuple(bad_c[0])], ref.codes[tuple(bad_c[0])])


def f32(bits):
    return synth.bf16_to_f32(bits)


def print_case(**kw):
    print("CASE " + " ".join("%s=%s" % (k, v) for k, v in kw.items()), flush=True)


def quantize_chunked(x, rowwise=True, colwise=True, chunk=512, threads=8):
    """oracle.quantize(x) for large x: the same tensor scale, then the
    oracle's own row quantizer on chunks of rows (of x, or of x^T for the
    column-wise view) in a thread pool.  Rows are quantized independently, so
    the result is oracle.quantize's bit for bit (tests/test_oracle_quantize.py
    checks it); the chunks keep numpy's temporaries small."""
    import concurrent.futures as cf
    from oracle.quantize import NVFP4, quantize_rows, tensor_scale
    x = np.ascontiguousarray(x, dtype=np.float32)
    s_t = tensor_scale(x)

    def layout(src):
        rows = src.shape[0]
        spans = [(i, min(i + chunk, rows)) for i in range(0, rows, chunk)]
        with cf.ThreadPoolExecutor(threads) as ex:
            parts = list(ex.map(lambda sp: quantize_rows(np.ascontiguousarray(src[sp[0]:sp[1]]), s_t), spans))
        codes = np.concatenate([p.codes for p in parts]) if parts else np.zeros((0, src.shape[1] // 2), np.uint8)
        scales = np.concatenate([p.scales for p in parts]) if parts else np.zeros((0, src.shape[1] // 16), np.uint8)
        return NVFP4(codes, scales, np.float32(s_t), src.shape[0], src.shape[1])

    row = layout(x) if rowwise else None
    col = layout(x.T) if colwise else None
    return row, col, s_t


def gemm_full_check(got, qa, qb, alpha=1.0, extra=None, extra_abs=None, rows=1024):
    """max |got - ref| / D over every element of an NT product, where
    ref = alpha s_tA s_tB A_hat B_hat^T (+ extra) and D the matching sum of
    |a||b| (+ extra_abs), from the oracle's block values, processed in bands
    of rows to bound host memory."""
    from oracle.quantize import block_values
    bb = block_values(qb)
    bb_abs = np.abs(bb)
    s = alpha * float(qa.tscale) * float(qb.tscale)
    worst = 0.0
    for i0 in range(0, qa.rows, rows):
        i1 = min(i0 + rows, qa.rows)
        sub = type(qa)(qa.codes[i0:i1], qa.scales[i0:i1], qa.tscale, i1 - i0, qa.cols)
        ab = block_values(sub)
        ref = s * (ab @ bb.T)
        den = abs(s) * (np.abs(ab) @ bb_abs.T)
        if extra is not None:
            ref += extra(i0, i1)
            den += extra_abs(i0, i1)
        worst = max(worst, oracle.rel_err(got[i0:i1], ref, den))
    return worst


def _directed_f32(v64, up):
    """float64 -> float32 rounded away from zero (up) or toward zero."""
    v32 = v64.astype(np.float32)
    back = v32.astype(np.float64)
    mag, mag32 = np.abs(v64), np.abs(back)
    fix = (mag32 < mag) if up else (mag32 > mag)
    toward = np.where(np.signbit(v64), -np.inf, np.inf) if up else np.zeros_like(v64)
    v32 = np.where(fix, np.nextafter(v32, toward.astype(np.float32)), v32)
    return v32.astype(np.float32)


def quantization_allowance(x_ref, eps):
    """How far the dequantized NVFP4 views of any x' with |x' - x_ref| <= eps
    (elementwise) can lie from those of x_ref.

    Two correct implementations that sum in different orders give float32
    results a few ulps apart; a quantization decision whose input lies that
    close to a rounding boundary (tensor scale, block scale or element code)
    may then come out either way, and both are correct.  Every decision is
    monotone in the magnitudes it reads, so the extremes are reached by
    shrinking or growing every magnitude by eps (this bounds each element
    exactly while its block scale is stable; where the block scale itself is
    ambiguous it bounds the two scale candidates at the edges of the box).
    Returns (Q_row, Q_col, dQ_row, dQ_col): the dequantized row- and
    column-wise views of x_ref (float64, Q_col in x^T's layout) and the
    elementwise bounds of their change."""
    from oracle.quantize import dequantize
    x = np.asarray(x_ref, dtype=np.float32).astype(np.float64)
    e = np.asarray(eps, dtype=np.float64)
    mag = np.abs(x)
    sgn = np.where(np.signbit(x), -1.0, 1.0)
    lo = _directed_f32(sgn * np.maximum(mag - e, 0.0), up=False)
    hi = _directed_f32(sgn * (mag + e), up=True)
    ref = oracle.quantize(x.astype(np.float32))
    outs = [dequantize(ref[0]), dequantize(ref[1])]
    d = [np.zeros_like(outs[0]), np.zeros_like(outs[1])]
    for alt in (lo, hi):
        q = oracle.quantize(alt)
        for i in range(2):
            d[i] = np.maximum(d[i], np.abs(dequantize(q[i]) - outs[i]))
    return outs[0], outs[1], d[0], d[1]


def ns_step_bounds(x_k, st, a, b, c, tol, clip_p=None):
    """Per-element bounds for one NVFP4 Newton-Schulz step computed by another
    correct implementation from the same iterate x_k: its A within
    tol * A_D of the oracle's; B within tol * B_D plus what any A within that
    bound can change through the quantization of A; X' within tol * X_D plus
    what any such B can change through the quantization of B.  (The iterate's
    own views are bit-exact on both sides; clip_p is the clip value of its
    quantized copy when clipping is on.)"""
    from oracle.newton_schulz import clip_abs
    eps_a = tol * st["A_D"]
    qar, qac, dqar, dqac = quantization_allowance(st["A"], eps_a)
    allow_b = abs(b) * eps_a + abs(c) * (dqar @ (np.abs(qac) + dqac).T + np.abs(qar) @ dqac.T)
    eps_b = tol * st["B_D"] + allow_b
    _, _, dqbr, _ = quantization_allowance(st["B"], eps_b)
    xq = np.asarray(x_k, dtype=np.float32) if clip_p is None else clip_abs(x_k, clip_p)
    _, x_col, _ = oracle.quantize(xq, rowwise=False, colwise=True)
    from oracle.quantize import dequantize
    allow_x = dqbr @ np.abs(dequantize(x_col)).T
    return eps_a, eps_b, tol * st["X_D"] + allow_x


def within(got, ref, bound):
    """max |got - ref| / bound (0/0 counts as 0; a nonzero difference over a
    zero bound as inf)."""
    diff = np.abs(np.asarray(got, np.float64) - ref)
    bound = np.asarray(bound, np.float64)
    zero = bound == 0
    if np.any(diff[zero] != 0):
        return float("inf")
    return float(np.max(diff[~zero] / bound[~zero])) if np.any(~zero) else 0.0
