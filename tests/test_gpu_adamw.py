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


@pytest.mark.timeout(600)
def test_first_moment_3b_weight_state_full():
    """The 8192 x 3072 weight's first moment, every code, scale and decoded
    value.  At this size the encode grid (the workgroups resident at once)
    walks the 1.57 M groups of 16 in several grid-stride passes, which the
    smaller cases (one pass) do not reach."""
    fs4 = need_gpu()
    print_case(test="mstate_3b", R=8192, C=3072)
    m = _m((8192, 3072), 2024)
    w = _words(m.shape, 2025)
    q = fs4.mstate_encode(dev_f32(m), torch.from_numpy(w.view(np.int32)).cuda())
    got = fs4.mstate_decode(q).cpu().numpy()
    ref, _ = mstate_encode(m, w)
    assert_view_equal(q, ref, "m 8192x3072")
    assert np.array_equal(got.view(np.uint32), mstate_decode(ref).view(np.uint32))


def _m_on_and_near_grid(R, C, seed):
    """A first moment whose transformed values h = H/4 m sit on E2M1 grid
    points and within a few ulps of them.

    Every 16-group of h is g * m_b * 2^k with g on the E2M1 grid (one +-6 per
    group sets the block amax 6 m_b 2^k), m_b an E4M3 value >= 1, and one group
    holding 2688 * 2^k so that the tensor scale is exactly 2^k.  Those values
    are multiples of 2^(k-4) below 2^(k+16), so m = H h / 4 and the transform
    back are exact in fp32: the quotients |h| / (s_b s_t) land exactly on the
    grid for the 6-scale candidate.  In every other row each value is nudged
    by 0 to 2 ulps up or down before m is formed, so its quotient falls just
    beside a grid point (the transform's rounding keeps it within a few
    ulps)."""
    rng = np.random.default_rng(seed)
    k = -12
    e4m3_ge1 = np.array([2.0 ** e * (1 + mm / 8) for e in range(0, 9) for mm in range(8)
                         if 2.0 ** e * (1 + mm / 8) < 448])   # 448 only in the amax group
    grid = oracle.E2M1_GRID
    g = rng.choice(grid, size=(R, C // 16, 16)) * rng.choice([-1.0, 1.0], size=(R, C // 16, 16))
    pos = rng.integers(0, 16, size=(R, C // 16))
    np.put_along_axis(g, pos[..., None], 6.0 * rng.choice([-1.0, 1.0], size=(R, C // 16, 1)), axis=2)
    mb = rng.choice(e4m3_ge1, size=(R, C // 16, 1))
    mb[0, 0, 0] = 448.0
    g[0, 0, :] = np.abs(g[0, 0, :])
    g[0, 0, 0] = 6.0                                   # h = 2688 * 2^k: s_t = 2^k exactly
    h = (g * mb * 2.0 ** k).astype(np.float32)
    nudge = rng.integers(-2, 3, size=h.shape).astype(np.float32)
    odd = (np.arange(R) % 2 == 1)[:, None, None]
    h = np.where(odd & (h != 0), h + nudge * np.spacing(np.abs(h)) * np.sign(h), h).astype(np.float32)
    h = h.reshape(R, C)
    from oracle.adamw import hadamard16
    return hadamard16(h.astype(np.float64)).astype(np.float32)


def test_first_moment_on_and_near_grid_multi_pass():
    """Transformed values exactly on and a few ulps beside the E2M1 grid
    points, bit for bit, at 4096 x 1024 (262,144 groups: more than the
    encode grid holds, so the grid-stride loop runs a second pass)."""
    fs4 = need_gpu()
    print_case(test="mstate_grid", R=4096, C=1024)
    m = _m_on_and_near_grid(4096, 1024, 77)
    from oracle.adamw import hadamard16
    h = hadamard16(m.astype(np.float64))
    assert np.float32(np.abs(h).max()) == np.float32(2688 * 2.0 ** -12)
    for fill in (None, 0, 0xFFFFFFFF):
        w = _words(m.shape, 78) if fill is None else np.full(m.shape, fill, dtype=np.uint32)
        q = fs4.mstate_encode(dev_f32(m), torch.from_numpy(w.view(np.int32)).cuda())
        ref, _ = mstate_encode(m, w)
        assert_view_equal(q, ref, "grid words %s" % fill)
        got = fs4.mstate_decode(q).cpu().numpy()
        assert np.array_equal(got.view(np.uint32), mstate_decode(ref).view(np.uint32))
