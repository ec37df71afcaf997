"""Pins for the bounds the Q-Attn backward's GPU parity test uses
(tests/gpu_util.AttentionBwdBounds), on the CPU.

Another correct implementation is emulated in float32 (its own summation
order through float32 BLAS, exponentials rounded once) and must fall within
the bounds, both from a forward whose O and LSE sit near the edge of the
forward test's bars and from the oracle forward's O and LSE rounded to
float32 (how the GPU test feeds the backward alone).  The same emulation
with one plausible mistake planted (a dropped Delta, exp2 in place of exp,
a transposed product, P rounded coarser than BF16, dS quantized with the
wrong tensor scale) must fall outside them.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import AttentionBwdBounds, within
from oracle.attention import attention_bwd, attention_fwd
from oracle.quantize import block_values, dequantize, quantize_rows, tensor_scale

O_TOL = 2.0 ** -8 + 2.0 ** -12
LSE_TOL = 2e-6


def _bf(rng, shape, std=1.0):
    return synth.bf16_to_f32(synth.bf16_round(rng.standard_normal(shape) * std))


def _emulate(q, k, v, do, fwd, causal, rng, plant=None, isolated=False):
    G, S, D = q.shape
    f32 = np.float32
    if isolated:
        O2 = fwd["O"].astype(f32).astype(np.float64)
        LSE2 = fwd["LSE"].astype(f32).astype(np.float64)
    else:
        O2 = fwd["O"] + rng.uniform(-0.9, 0.9, fwd["O"].shape) * O_TOL * fwd["O_D"]
        LSE2 = fwd["LSE"] + rng.uniform(-0.5, 0.5, fwd["LSE"].shape) * LSE_TOL
    bq = block_values(fwd["Q_row"]).astype(f32)
    bk = block_values(fwd["K_row"]).astype(f32)
    c = f32(fwd["st"])
    mask = np.tril(np.ones((S, S), bool)) if causal else np.ones((S, S), bool)
    dS = np.empty((G, S, S), f32)
    dV = np.empty((G, S, D), f32)
    for g in range(G):
        s = (bq[g * S:(g + 1) * S] @ bk[g * S:(g + 1) * S].T) * c
        P = np.where(mask, np.exp(s.astype(np.float64) - LSE2[g][:, None]), 0.0).astype(f32)
        if plant == "exp2_for_exp":
            P = np.where(mask, np.exp2(s.astype(np.float64) - LSE2[g][:, None]), 0.0).astype(f32)
        dP = do[g] @ v[g].T
        delta = np.sum(do[g] * O2[g].astype(f32), axis=1, dtype=f32)
        if plant == "no_delta":
            delta = np.zeros_like(delta)
        dS[g] = P * (dP - delta[:, None])
        Pb = synth.bf16_to_f32(synth.bf16_round(P.astype(np.float64)))
        if plant == "p_not_rounded_but_fp8":
            Pb = np.round(P * 16) / 16
        dV[g] = Pb.T @ do[g]
        if plant == "dv_transposed":
            dV[g] = Pb @ do[g]
    ds2 = dS.reshape(G * S, S)
    s_t = tensor_scale(ds2)
    if plant == "tensor_scale_per_sequence":
        s_t = tensor_scale(ds2[:S])
    dQ = np.empty((G, S, D))
    dK = np.empty((G, S, D))
    for g in range(G):
        a = dequantize(quantize_rows(dS[g], s_t)).astype(f32)
        at = dequantize(quantize_rows(np.ascontiguousarray(dS[g].T), s_t)).astype(f32)
        kc = dequantize(fwd["K_col"][g]).astype(f32)
        qc = dequantize(fwd["Q_col"][g]).astype(f32)
        dQ[g] = f32(fwd["scale"]) * (a @ kc.T)
        dK[g] = f32(fwd["scale"]) * (at @ qc.T)
    return {"dS": dS, "dV": dV, "dQ": dQ, "dK": dK}


def _ratios(G, S, D, causal, seed, plant=None, std=1.0, isolated=False):
    rng = np.random.default_rng(seed)
    q, k, v, do = (_bf(rng, (G, S, D), std if i < 2 else 1.0) for i in range(4))
    if plant == "tensor_scale_per_sequence":
        do[0] *= 0.25   # the first sequence's dS no longer holds the amax
    fwd = attention_fwd(q, k, v, causal)
    if isolated:
        o_err, lse_err = 2.0 ** -24 * np.abs(fwd["O"]), 2.0 ** -24 * np.abs(fwd["LSE"])
    else:
        o_err, lse_err = O_TOL * fwd["O_D"], LSE_TOL * np.maximum(1.0, np.abs(fwd["LSE"]))
    bb = AttentionBwdBounds(fwd, do, v, range(G), o_err, lse_err)
    ref = attention_bwd(q, k, v, do, fwd, causal, on_seq=bb)
    got = _emulate(q, k, v, do, fwd, causal, rng, plant, isolated)
    out = {}
    for g in range(G):
        b = bb.bounds(g, ref["dS"][g])
        for name in ("dS", "dV", "dQ", "dK"):
            r = ref["dS"][g] if name == "dS" else ref[name][g]
            out[name] = max(out.get(name, 0.0), within(got[name][g], r, b[name]))
    return out


@pytest.mark.parametrize("isolated", [False, True])
@pytest.mark.parametrize("G,S,D,causal,std", [(2, 128, 64, True, 1.0), (2, 96, 32, False, 1.0),
                                              (1, 128, 64, True, 2.0)])
def test_another_correct_implementation_is_within_the_bounds(G, S, D, causal, std, isolated):
    r = _ratios(G, S, D, causal, seed=S + D, std=std, isolated=isolated)
    print(r)
    assert all(v <= 1.0 for v in r.values()), r
    # the bounds are not vacuous: the emulation's own errors use some of them
    assert r["dV"] > 0.05 and r["dS"] > 1e-3, r


@pytest.mark.parametrize("isolated", [False, True])
@pytest.mark.parametrize("plant,caught_by", [
    ("no_delta", "dS"), ("exp2_for_exp", "dS"), ("p_not_rounded_but_fp8", "dV"),
    ("dv_transposed", "dV"), ("tensor_scale_per_sequence", "dQ")])
def test_planted_mistakes_fall_outside(plant, caught_by, isolated):
    r = _ratios(2, 128, 64, True, seed=11, plant=plant, isolated=isolated)
    assert r[caught_by] > 1.0, r
