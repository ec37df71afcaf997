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


def _box(x, eps):
    """x float64 with every magnitude shrunk (lo) or grown (hi) by eps,
    rounded to float32 toward zero and away from it."""
    e = np.asarray(eps, dtype=np.float64)
    mag = np.abs(x)
    sgn = np.where(np.signbit(x), -1.0, 1.0)
    lo = _directed_f32(sgn * np.maximum(mag - e, 0.0), up=False)
    hi = _directed_f32(sgn * (mag + e), up=True)
    return lo, hi


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
    lo, hi = _box(x, eps)
    ref = oracle.quantize(x.astype(np.float32))
    outs = [dequantize(ref[0]), dequantize(ref[1])]
    d = [np.zeros_like(outs[0]), np.zeros_like(outs[1])]
    for alt in (lo, hi):
        q = oracle.quantize(alt)
        for i in range(2):
            d[i] = np.maximum(d[i], np.abs(dequantize(q[i]) - outs[i]))
    return outs[0], outs[1], d[0], d[1]


def box_amax(x, eps):
    """(amax of x, of x with every magnitude shrunk by eps, of it grown by
    eps), as float32, with _box's roundings."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    lo, hi = _box(x, eps)
    return (np.float32(np.abs(x).max()), np.float32(np.abs(lo).max()), np.float32(np.abs(hi).max()))


def quantization_interval(x_ref, eps, s_ref, s_lo, s_hi):
    """How far the row-wise NVFP4 dequantization of any x' with
    |x' - x_ref| <= eps (elementwise), quantized with any tensor scale in
    [s_lo, s_hi], can lie from x_ref's own at s_ref; x_ref may be a part of
    a larger tensor (whole 16-blocks along its rows) whose amax fixes the
    tensor scale.  A bound for every x' in the box, with no monotonicity
    assumed: each block's scale code lies between the codes its smallest
    and largest possible amax give at the largest and smallest tensor scale,
    and for each such code the element's grid index lies between the
    indices of its smallest magnitude over the largest step and its largest
    over the smallest step; an element within eps of zero may change sign.
    Returns (deq_ref float64, allow)."""
    from oracle.formats import E2M1_GRID, e2m1_rne_index, e4m3_decode, e4m3_rne_satfinite
    from oracle.quantize import dequantize, quantize_rows
    x32 = np.asarray(x_ref, dtype=np.float32)
    x = x32.astype(np.float64)
    rows, cols = x.shape
    e = np.broadcast_to(np.asarray(eps, dtype=np.float64), x.shape)
    ref = dequantize(quantize_rows(x32, s_ref))
    mag = np.abs(x)
    sgn = np.where(np.signbit(x), -1.0, 1.0)
    mlo = np.maximum(mag - e, 0.0)
    mhi = mag + e
    flip = mlo == 0.0
    a_lo = mlo.reshape(rows, cols // 16, 16).max(axis=2)
    a_hi = mhi.reshape(rows, cols // 16, 16).max(axis=2)
    s_lo, s_hi = float(s_lo), float(s_hi)
    c_lo = e4m3_rne_satfinite(a_lo / (6.0 * s_hi)).astype(np.int64) if s_hi > 0 else np.zeros(a_lo.shape, np.int64)
    c_hi = e4m3_rne_satfinite(a_hi / (6.0 * s_lo)).astype(np.int64) if s_lo > 0 else np.zeros(a_hi.shape, np.int64)
    # per 16-block rows of every array, so that each candidate code visits
    # only the blocks whose range reaches it
    nb = rows * cols // 16
    mlo_b, mhi_b = mlo.reshape(nb, 16), mhi.reshape(nb, 16)
    sgn_b, ref_b, flip_b = sgn.reshape(nb, 16), ref.reshape(nb, 16), flip.reshape(nb, 16)
    c_lo, c_hi = c_lo.reshape(nb), c_hi.reshape(nb)
    allow = np.zeros((nb, 16))
    for off in range(int((c_hi - c_lo).max()) + 1):
        blk = np.nonzero(c_hi - c_lo >= off)[0]
        sb = e4m3_decode(c_lo[blk] + off)[:, None]
        t_lo, t_hi = sb * s_lo, sb * s_hi
        m_lo, m_hi = mlo_b[blk], mhi_b[blk]
        with np.errstate(divide="ignore", invalid="ignore"):
            k_min = e2m1_rne_index(np.where(t_hi > 0, m_lo / t_hi * (1 - 2.0 ** -50), 0.0))
            k_max = e2m1_rne_index(np.where(t_lo > 0, m_hi / t_lo * (1 + 2.0 ** -50), 0.0))
        v_lo = np.where(t_lo > 0, E2M1_GRID[k_min] * t_lo, 0.0)
        v_hi = np.where(t_hi > 0, E2M1_GRID[k_max] * t_hi, 0.0)
        sg, rf = sgn_b[blk], ref_b[blk]
        d = np.maximum(np.abs(sg * v_lo - rf), np.abs(sg * v_hi - rf))
        d = np.where(flip_b[blk], np.maximum(d, np.abs(-sg * v_hi - rf)), d)
        allow[blk] = np.maximum(allow[blk], d)
    return ref, allow.reshape(rows, cols)


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


def gamma(n):
    """The float32 summation bound gamma_n = n u / (1 - n u), u = 2^-24:
    any order of n - 1 rounded additions errs by at most gamma_n sum |x|."""
    return n * 2.0 ** -24 / (1.0 - n * 2.0 ** -24)


class AttentionBwdBounds:
    """Per-element bounds for the Q-Attn backward computed by another correct
    implementation (float32 sums in its own order, exponentials to about
    one ulp) from an O and LSE within o_err and lse_err of the oracle
    forward's.  Called as the oracle
    backward's on_seq hook, it forms each sequence's dS allowance and the
    range of dS's amax over all sequences; bounds(g, ...) then gives the
    bounds of dS, dV, dQ and dK for a kept sequence.

    dS = P (dP - Delta): P moves by r_P P (the score sums over D exact
    products, the fp32 roundings of the exponent, the forward's LSE
    error), dP by gamma_D |dO||V|^T, Delta by the forward's O error
    times |dO| plus gamma_D |dO||O|.  dV = P^T dO with P rounded to BF16
    (2^-8 of itself) and fp32 sums over S.  dQ and dK multiply dS's NVFP4
    views, which may differ by quantization_interval at dS's allowance, plus fp32 sums over S and the 2^-22 of the final scaling."""

    def __init__(self, fwd, do, v, keep, o_err, lse_err):
        """o_err [G, S, D], lse_err [G, S]: how far the O and LSE the
        backward reads may lie from the oracle forward's."""
        from oracle.quantize import block_values
        self.fwd, self.do, self.v = fwd, do, v
        self.keep = set(keep)
        self.o_err, self.lse_err = o_err, lse_err
        self.bq = np.abs(block_values(fwd["Q_row"]))
        self.bk = np.abs(block_values(fwd["K_row"]))
        self.amax = [np.float32(0.0)] * 3
        self.kept = {}
        import threading
        self._lock = threading.Lock()

    def __call__(self, g, parts):
        fwd = self.fwd
        S, D = self.v.shape[1], self.v.shape[2]
        P, dP, delta = parts["P"], parts["dP"], parts["Delta"][:, None]
        n_qk = fwd["st"] * (self.bq[g * S:(g + 1) * S] @ self.bk[g * S:(g + 1) * S].T)   # >= |S_ij|
        lse = np.abs(fwd["LSE"][g])[:, None]
        r_p = gamma(D) * n_qk + 2.0 ** -20 * (n_qk + lse + 1.0) + self.lse_err[g][:, None]
        ado = np.abs(self.do[g].astype(np.float64))
        n_dv = ado @ np.abs(self.v[g].astype(np.float64)).T
        o_err = self.o_err[g]
        e_delta = np.sum(ado * o_err, axis=1) + gamma(D) * np.sum(ado * (np.abs(fwd["O"][g]) + o_err), axis=1)
        eps = P * ((1.0 + r_p) * (gamma(D) * n_dv + e_delta[:, None]) + (r_p + 2.0 ** -22) * np.abs(dP - delta))
        a = box_amax(parts["dS"].astype(np.float32), eps)
        with self._lock:
            self.amax = [max(x, y) for x, y in zip(self.amax, a)]
            if g in self.keep:
                self.kept[g] = (eps, r_p, P)

    def tscales(self):
        from oracle.formats import tensor_scale_from_amax
        return tuple(tensor_scale_from_amax(a) for a in self.amax)

    def bounds(self, g, ds_ref):
        """Bounds for sequence g; ds_ref the oracle's dS of g (float64)."""
        from oracle.quantize import dequantize
        fwd = self.fwd
        S = self.v.shape[1]
        eps, r_p, P = self.kept[g]
        s_ref, s_lo, s_hi = self.tscales()
        Qr, dQr = quantization_interval(ds_ref, eps, s_ref, s_lo, s_hi)
        Qc, dQc = quantization_interval(np.ascontiguousarray(ds_ref.T), np.ascontiguousarray(eps.T), s_ref, s_lo, s_hi)
        kc = np.abs(dequantize(fwd["K_col"][g]))
        qc = np.abs(dequantize(fwd["Q_col"][g]))
        scale, gs = fwd["scale"], gamma(S)
        mag_q = scale * ((np.abs(Qr) + dQr) @ kc.T)
        mag_k = scale * ((np.abs(Qc) + dQc) @ qc.T)
        dq = scale * (dQr @ kc.T) + (gs + 2.0 ** -22) * mag_q
        dk = scale * (dQc @ qc.T) + (gs + 2.0 ** -22) * mag_k
        ado = np.abs(self.do[g].astype(np.float64))
        dv = (P * (2.0 ** -8 + (1 + 2.0 ** -8) * r_p)).T @ ado + gs * (1 + 2.0 ** -8) * ((P * (1 + r_p)).T @ ado)
        return {"dS": eps, "dQ": dq, "dK": dk, "dV": dv}
