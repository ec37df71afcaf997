"""GPU parity of the Q-AdamW second-moment codec against the oracle: the
encoder's codes, block scales, tensor scale and BF16 tile means bit for bit
(both sides reach the same fp32 h: fp64 arithmetic in one fixed order), and
the decoder's fp32 output bit for bit from the same stored state."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_view_equal, dev_f32, host_view, need_gpu, print_case
from oracle.adamw import hadamard16, tile_means, vstate_decode, vstate_encode
from oracle.quantize import quantize_rows, tensor_scale

pytestmark = pytest.mark.gpu


def _v(shape, seed):
    """A heavy-tailed second moment: squared Student-t(2) gradients, scaled
    per row over decades, with some exact zeros."""
    rng = np.random.default_rng(seed)
    v = rng.standard_t(2, shape) ** 2 * np.exp(rng.uniform(-6, 2, (shape[0], 1))) * 1e-8
    v[rng.random(shape) < 0.02] = 0.0
    return v.astype(np.float32)


def _means_bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _oracle_means_bits(mu):
    return (mu.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("R,C", [(16, 16), (48, 80), (272, 400), (1024, 3072)])
def test_encode_decode_bit_exact(R, C):
    fs4 = need_gpu()
    print_case(test="vstate", R=R, C=C)
    v = _v((R, C), R * 7 + C)
    q, means = fs4.vstate_encode(dev_f32(v))
    ref_q, ref_mu, _ = vstate_encode(v)
    assert np.array_equal(_means_bits(means), _oracle_means_bits(ref_mu))
    assert_view_equal(q, ref_q, "h")
    v_hat = fs4.vstate_decode(q, means).cpu().numpy()
    want = vstate_decode(ref_q, ref_mu)
    assert np.array_equal(v_hat.view(np.uint32), want.view(np.uint32))


def test_zero_state():
    fs4 = need_gpu()
    v = np.zeros((32, 64), dtype=np.float32)
    q, means = fs4.vstate_encode(dev_f32(v))
    _, _, ts = host_view(q)
    assert ts == 0.0 and not _means_bits(means).any()
    assert not fs4.vstate_decode(q, means).cpu().numpy().any()


def test_3b_weight_state_sampled():
    """v of the 8192 x 3072 projection weight: all tile means and the tensor
    scale, codes and decoded values on sampled rows."""
    fs4 = need_gpu()
    print_case(test="vstate_3b")
    R, C = 8192, 3072
    v = _v((R, C), 99)
    q, means = fs4.vstate_encode(dev_f32(v))
    s = np.sqrt(v.astype(np.float64))
    mu = tile_means(s)
    assert np.array_equal(_means_bits(means), _oracle_means_bits(mu))
    h = hadamard16(s - np.repeat(np.repeat(mu, 16, 0), 16, 1)).astype(np.float32)
    s_t = tensor_scale(h)
    codes, scales, ts = host_view(q)
    assert ts.tobytes() == s_t.tobytes()
    v_hat = fs4.vstate_decode(q, means).cpu().numpy()
    rows = np.random.default_rng(1).choice(R, 48, replace=False)
    for r in rows:
        ref = quantize_rows(h[r:r + 1], s_t)
        assert np.array_equal(codes[r], ref.codes[0]) and np.array_equal(scales[r], ref.scales[0]), r
        h_hat = oracle.dequantize(ref)[0]
        s_hat = hadamard16(h_hat) + np.repeat(mu[r // 16], 16)
        assert np.array_equal(v_hat[r].view(np.uint32), (s_hat * s_hat).astype(np.float32).view(np.uint32)), r


# ---- first moment ---------------------------------------------------------------
from oracle.adamw import mstate_decode, mstate_encode


def _m(shape, seed):
    rng = np.random.default_rng(seed)
    m = rng.standard_normal(shape) * np.exp(rng.uniform(-4, 1, (shape[0], 1))) * 1e-3
    m[:, ::37] *= 30.0                                   # outlier columns the Hadamard mixing spreads
    return m.astype(np.float32)


def _words(shape, seed):
    return np.random.default_rng(seed).integers(0, 2 ** 32, shape, dtype=np.uint64).astype(np.uint32)


@pytest.mark.parametrize("R,C", [(16, 16), (48, 80), (272, 400), (1024, 3072)])
def test_first_moment_bit_exact(R, C):
    fs4 = need_gpu()
    print_case(test="mstate", R=R, C=C)
    m = _m((R, C), R + C)
    w = _words((R, C), R * C)
    q = fs4.mstate_encode(dev_f32(m), torch.from_numpy(w.view(np.int32)).cuda())
    ref, _ = mstate_encode(m, w)
    assert_view_equal(q, ref, "m")
    got = fs4.mstate_decode(q).cpu().numpy()
    assert np.array_equal(got.view(np.uint32), mstate_decode(ref).view(np.uint32))


def test_first_moment_extreme_words():
    """All-zero words round every off-grid magnitude up, all-ones words down,
    as in the oracle."""
    fs4 = need_gpu()
    m = _m((64, 128), 5)
    for fill in (0, 0xFFFFFFFF):
        w = np.full(m.shape, fill, dtype=np.uint32)
        q = fs4.mstate_encode(dev_f32(m), torch.from_numpy(w.view(np.int32)).cuda())
        ref, _ = mstate_encode(m, w)
        assert_view_equal(q, ref, "fill %x" % fill)
