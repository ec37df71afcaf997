"""GPU parity of the NVFP4 mixed-precision attention backward (Q-Attn)
against the oracle.

The bounds are tests/gpu_util.AttentionBwdBounds (their derivation is in its
docstring; tests/test_attention_bounds.py pins them on the CPU against an
emulated second implementation and planted mistakes).  Two ways in:
* the backward alone: the kernel reads the oracle forward's O and LSE,
  rounded to float32, so the bounds only allow the backward's own fp32
  sums, exponentials and the quantization decisions those can flip;
* the chain: the GPU forward's O and LSE, first checked against the forward
  test's bars, which then widen the bounds of Delta and P.
Every output is compared element by element: dS (fp32, before its
quantization), dV, dQ, dK; the column-wise NVFP4 views of Q and K that the
dS products read are compared bit for bit, and a second call that does not
keep dS (so the zeros above a causal diagonal are never written, nor read
by the quantizer) must return the same dQ, dK and dV bit for bit.
"""
import os

import numpy as np
import pytest
import torch

import synth
from gpu_util import AttentionBwdBounds, dev_bf16, need_gpu, print_case, within
from oracle.attention import attention_bwd, attention_fwd

pytestmark = pytest.mark.gpu

O_TOL = 2.0 ** -8 + 2.0 ** -12    # the forward test's bars
LSE_TOL = 2e-6


def _bf(rng, shape, std=1.0):
    return synth.bf16_round(rng.standard_normal(shape) * std)


def _col_slice_equal(view, ref, g, S, what):
    codes = view.codes.cpu().numpy()[:, g * S // 2:(g + 1) * S // 2]
    scales = view.scales.cpu().numpy()[:, g * S // 16:(g + 1) * S // 16]
    assert np.array_equal(codes, ref.codes), what + " codes"
    assert np.array_equal(scales, ref.scales), what + " scales"
    assert np.float32(view.tscale.cpu().numpy().reshape(-1)[0]) == np.float32(ref.tscale), what + " tscale"


def _run(G, S, D, causal, seed, seqs=None, std_qk=1.0, chain=False):
    fs4 = need_gpu()
    print_case(test="attention_bwd", G=G, S=S, D=D, causal=causal, chain=chain)
    threads = min(16, os.cpu_count() or 1)
    rng = np.random.default_rng(seed)
    qb, kb, vb, dob = (_bf(rng, (G, S, D), std_qk if i < 2 else 1.0) for i in range(4))
    Q, K, V, dO = (dev_bf16(x) for x in (qb, kb, vb, dob))
    q32, k32, v32, do32 = (synth.bf16_to_f32(x) for x in (qb, kb, vb, dob))
    sel = list(range(G)) if seqs is None else sorted(seqs)
    qv, kv = fs4.attention_quantize(Q), fs4.attention_quantize(K)
    fwd = attention_fwd(q32, k32, v32, causal, keep_P=seqs is None, threads=threads)
    if chain:
        f = fs4.attention_fwd(qv[0], kv[0], V, causal)
        O, LSE = f.O[sel].cpu().numpy(), f.LSE[sel].cpu().numpy()
        err_o = np.max(np.abs(O - fwd["O"][sel]) / fwd["O_D"][sel])
        err_l = np.max(np.abs(LSE - fwd["LSE"][sel]) / np.maximum(1.0, np.abs(fwd["LSE"][sel])))
        assert err_o <= O_TOL and err_l <= LSE_TOL, (err_o, err_l)
        o_err, lse_err = O_TOL * fwd["O_D"], LSE_TOL * np.maximum(1.0, np.abs(fwd["LSE"]))
    else:
        f = fs4.AttentionFwd(torch.from_numpy(fwd["O"].astype(np.float32)).to(V.device),
                             torch.from_numpy(fwd["LSE"].astype(np.float32)).to(V.device), None)
        o_err, lse_err = 2.0 ** -24 * np.abs(fwd["O"]), 2.0 ** -24 * np.abs(fwd["LSE"])
    b = fs4.attention_bwd(dO, V, f, qv, kv, causal, keep_dS=True)
    # without dS kept, the zeros above the diagonal are not written (the
    # quantizer skips those tiles): the results must not change by a bit
    b2 = fs4.attention_bwd(dO, V, f, qv, kv, causal, keep_dS=False)
    torch.cuda.synchronize()
    for name in ("dQ", "dK", "dV"):
        assert torch.equal(getattr(b, name), getattr(b2, name)), name
    for g in sel:
        _col_slice_equal(qv[1], fwd["Q_col"][g], g, S, "Q_col")
        _col_slice_equal(kv[1], fwd["K_col"][g], g, S, "K_col")
    bb = AttentionBwdBounds(fwd, do32, v32, sel, o_err, lse_err)
    ref = attention_bwd(q32, k32, v32, do32, fwd, causal, seqs=seqs, on_seq=bb, threads=threads)
    dS = b.dS.view(G, S, S)
    worst = {}
    for g in sel:
        bd = bb.bounds(g, ref["dS_seq"][g])
        got = {"dS": dS[g].cpu().numpy(), "dV": b.dV[g].cpu().numpy(), "dQ": b.dQ[g].cpu().numpy(),
               "dK": b.dK[g].cpu().numpy()}
        for name in got:
            r = ref["dS_seq"][g] if name == "dS" else ref[name][g]
            worst[name] = max(worst.get(name, 0.0), within(got[name], r, bd[name]))
    print("worst |got - ref| / bound:", {k: "%.3e" % v for k, v in worst.items()}, flush=True)
    assert all(v <= 1.0 for v in worst.values()), worst
    return worst


@pytest.mark.parametrize("G,S,D,causal", [(2, 256, 128, True), (3, 208, 64, True), (2, 192, 128, False),
                                          (1, 16, 128, True), (2, 80, 64, False), (1, 400, 128, True)])
def test_attention_bwd_parity(G, S, D, causal):
    _run(G, S, D, causal, seed=G * 1000 + S + D + 7)


@pytest.mark.parametrize("causal", [True, False])
def test_attention_bwd_after_gpu_forward(causal):
    _run(2, 320, 128, causal, seed=31, chain=True)


def test_attention_bwd_large_scores():
    """Scores of a few tens (Q, K ~ N(0, 2^2)): P is peaked, dS spans a wide
    range of magnitudes within its blocks."""
    _run(2, 512, 128, True, seed=6, std_qk=2.0)


@pytest.mark.timeout(900)
def test_attention_bwd_3b_shape_sampled_sequences():
    """The attention workload of the 3B-shape step: 4 sequences x 24 heads of
    2048 tokens, head dimension 128, causal, in the launch configuration the
    benchmark times; dS's tensor scale over all 96 sequences (the oracle
    forms every sequence's dS), the outputs compared in full on 4 of them
    (first, last and two drawn)."""
    rng = np.random.default_rng(19)
    seqs = sorted({0, 95, *rng.choice(np.arange(1, 95), 2, replace=False).tolist()})
    _run(96, 2048, 128, True, seed=97, seqs=seqs)
