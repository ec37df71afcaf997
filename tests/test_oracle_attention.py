"""Pins for the oracle's NVFP4 mixed-precision attention (Q-Attn).

Against what the pages and mathematics fix, not the oracle itself:
* with Q and K exactly representable in NVFP4 (quantization is the
  identity) the forward is plain causal attention: torch's fp64 scaled dot
  product attention, and the backward's dV and softmax gradient dS are
  torch autograd's;
* closed forms: Q = 0 gives uniform causal weights (O_i = mean of V_0..V_i,
  LSE_i = log(i + 1)); every row of dS sums to zero;
* the NVFP4 dS products dQ and dK stay within the error bound that the
  format alone fixes for the quantization of dS (one E2M1 step of its block,
  at most amax_b (1 + 2^-4) / 6) around autograd's exact dQ and dK.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle.attention import attention_bwd, attention_fwd

E2M1 = oracle.E2M1_GRID


def _bf(rng, shape, std=1.0):
    return synth.bf16_to_f32(synth.bf16_round(rng.standard_normal(shape) * std))


def _representable(rng, G, S, D, scale_exp):
    """Values g * 448 * 2^scale_exp (g on the E2M1 grid) with a +-6 in every
    16-block of rows and of columns of each sequence: every block scale is
    448 both ways, so both views quantize exactly; BF16 holds them too."""
    g = rng.choice(E2M1[:7], size=(G, S, D)) * rng.choice([-1.0, 1.0], size=(G, S, D))
    i, j = np.indices((S, D))
    on = (i + j) % 16 == 0
    g[:, on] = 6.0 * rng.choice([-1.0, 1.0], size=(G, int(on.sum())))
    return (g * 448.0 * 2.0 ** scale_exp).astype(np.float32)


def _torch_attention(q, k, v, do=None, causal=True):
    qt, kt, vt = (torch.from_numpy(x.astype(np.float64)).requires_grad_(do is not None) for x in (q, k, v))
    D = q.shape[-1]
    s = (qt @ kt.transpose(-1, -2)) / np.sqrt(D)
    if do is not None:
        s.retain_grad()
    if causal:
        S = q.shape[1]
        s = s.masked_fill(~torch.tril(torch.ones(S, S, dtype=torch.bool)), float("-inf"))
    p = torch.softmax(s, dim=-1)
    o = p @ vt
    lse = torch.logsumexp(s, dim=-1)
    if do is None:
        return o.detach().numpy(), lse.detach().numpy()
    o.backward(torch.from_numpy(do.astype(np.float64)))
    return o.detach().numpy(), lse.detach().numpy(), qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


@pytest.mark.parametrize("causal", [True, False])
def test_forward_with_representable_qk_is_plain_attention(causal):
    rng = np.random.default_rng(1)
    G, S, D = 2, 64, 32
    q, k = _representable(rng, G, S, D, -12), _representable(rng, G, S, D, -11)
    v = _bf(rng, (G, S, D))
    f = attention_fwd(q, k, v, causal)
    o, lse = _torch_attention(q, k, v, causal=causal)
    np.testing.assert_allclose(f["O"], o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(f["LSE"], lse, rtol=1e-12, atol=1e-12)


def test_zero_queries_give_uniform_causal_weights():
    rng = np.random.default_rng(2)
    G, S, D = 1, 48, 16
    q = np.zeros((G, S, D), np.float32)
    k, v = _bf(rng, (G, S, D)), _bf(rng, (G, S, D))
    f = attention_fwd(q, k, v)
    want = np.cumsum(v[0].astype(np.float64), axis=0) / np.arange(1, S + 1)[:, None]
    np.testing.assert_allclose(f["O"][0], want, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(f["LSE"][0], np.log(np.arange(1, S + 1)), rtol=1e-13)
    fn = attention_fwd(q, k, v, causal=False)
    np.testing.assert_allclose(fn["O"][0], np.broadcast_to(v[0].astype(np.float64).mean(axis=0), (S, D)), rtol=1e-12, atol=1e-13)


def test_backward_dv_and_softmax_gradient_match_autograd():
    rng = np.random.default_rng(3)
    G, S, D = 2, 64, 32
    q, k = _representable(rng, G, S, D, -12), _representable(rng, G, S, D, -11)
    v, do = _bf(rng, (G, S, D)), _bf(rng, (G, S, D))
    f = attention_fwd(q, k, v)
    b = attention_bwd(q, k, v, do, f)
    # autograd's gradient with respect to the scaled scores
    qt, kt = torch.from_numpy(q.astype(np.float64)), torch.from_numpy(k.astype(np.float64))
    s = ((qt @ kt.transpose(-1, -2)) / np.sqrt(D)).requires_grad_(True)
    sm = s.masked_fill(~torch.tril(torch.ones(S, S, dtype=torch.bool)), float("-inf"))
    o = torch.softmax(sm, dim=-1) @ torch.from_numpy(v.astype(np.float64))
    o.backward(torch.from_numpy(do.astype(np.float64)))
    np.testing.assert_allclose(b["dS"], s.grad.numpy(), rtol=1e-10, atol=1e-13)
    _, _, _, _, dv = _torch_attention(q, k, v, do)
    np.testing.assert_allclose(b["dV"], dv, rtol=1e-12, atol=1e-13)
    assert np.abs(b["dS"].sum(axis=2)).max() < 1e-12 * np.abs(b["dS"]).max() * S


def _ds_bound(ds, other, scale):
    """scale * sum_j e_ij |other_jd| with e_ij = amax of dS_ij's 16-block
    (1 + 2^-4) / 6 + |dS_ij| 2^-23: the quantization error of dS the format
    allows (one E2M1 step at a block scale within 2^-4 of amax/6, plus the
    float32 rounding of dS)."""
    G, S, _ = ds.shape
    amax = np.abs(ds).reshape(G, S, S // 16, 16).max(axis=3)
    e = np.repeat(amax, 16, axis=2) * (1 + 2.0 ** -4) / 6 + np.abs(ds) * 2.0 ** -23
    return scale * np.einsum("gij,gjd->gid", e, np.abs(other))


def test_ds_products_within_the_format_bound_of_autograd():
    rng = np.random.default_rng(4)
    G, S, D = 2, 64, 32
    q, k = _representable(rng, G, S, D, -12), _representable(rng, G, S, D, -11)
    v, do = _bf(rng, (G, S, D)), _bf(rng, (G, S, D))
    f = attention_fwd(q, k, v)
    b = attention_bwd(q, k, v, do, f)
    _, _, dq, dk, _ = _torch_attention(q, k, v, do)
    scale = 1.0 / np.sqrt(D)
    bq = _ds_bound(b["dS"], k.astype(np.float64), scale)
    bk = _ds_bound(np.transpose(b["dS"], (0, 2, 1)).copy(), q.astype(np.float64), scale)
    assert np.all(np.abs(b["dQ"] - dq) <= bq) and np.all(np.abs(b["dK"] - dk) <= bk)
    # the bound is not vacuous: the quantization moves dQ, and by far less
    # than the bound on average
    err = np.abs(b["dQ"] - dq)
    assert err.max() > 0 and np.mean(err) < 0.5 * np.mean(bq)
    # the normalisers bound the products themselves
    assert np.all(b["dQ_D"] >= np.abs(b["dQ"]) * (1 - 1e-12)) and np.all(b["dK_D"] >= np.abs(b["dK"]) * (1 - 1e-12))


def test_sampled_backward_equals_the_full_one():
    """The backward restricted to some sequences (the forward's P not kept,
    so recomputed from the same views) gives those sequences' outputs of the
    full backward exactly, with dS's tensor scale still over all of them;
    the per-sequence hook sees every sequence once, in order."""
    rng = np.random.default_rng(6)
    G, S, D = 4, 48, 32
    q, k, v, do = (_bf(rng, (G, S, D)) for _ in range(4))
    do[0] *= 4.0    # sequence 0, outside the sample, sets dS's amax
    full = attention_bwd(q, k, v, do, attention_fwd(q, k, v))
    seen = []
    part = attention_bwd(q, k, v, do, attention_fwd(q, k, v, keep_P=False), seqs=[1, 3],
                         on_seq=lambda g, parts: seen.append((g, np.abs(parts["dS"]).max())))
    assert [g for g, _ in seen] == list(range(G))
    assert part["dS_tscale"] == full["dS_tscale"]
    assert int(np.argmax([m for _, m in seen])) == 0
    for name in ("dQ", "dK", "dV", "dQ_D", "dK_D", "dV_D"):
        np.testing.assert_array_equal(part[name][[1, 3]], full[name][[1, 3]], err_msg=name)
    for g in (1, 3):
        np.testing.assert_array_equal(part["dS_seq"][g], full["dS"][g])
    with pytest.raises(ValueError):
        attention_bwd(q, k, v, do, attention_fwd(q, k, v, seqs=[1]), seqs=[1])
