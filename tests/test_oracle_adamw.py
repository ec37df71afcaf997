"""Pins for the oracle's Q-AdamW second-moment codec."""
import numpy as np

from oracle.adamw import TILE, fwht16, hadamard16, tile_means, vstate_decode, vstate_encode
from oracle.lora import bf16_rne
from oracle.quantize import dequantize


def _sylvester16():
    h = np.array([[1.0]])
    for _ in range(4):
        h = np.kron(np.array([[1.0, 1.0], [1.0, -1.0]]), h)
    return h


def test_butterflies_are_the_sylvester_matrix():
    h = _sylvester16()
    rng = np.random.default_rng(0)
    x = rng.standard_normal((7, 48))
    want = (x.reshape(-1, 16) @ h.T).reshape(7, 48)
    assert np.allclose(fwht16(x), want, rtol=0, atol=1e-12)
    q = hadamard16(np.eye(16))
    assert np.array_equal(q @ q, np.eye(16))                 # orthonormal and its own inverse
    assert np.array_equal(q, q.T)


def test_a_spike_spreads_evenly():
    x = np.zeros(16)
    x[5] = 8.0
    assert np.array_equal(np.abs(hadamard16(x)), np.full(16, 2.0))


def test_constant_tiles_round_trip_exactly():
    rng = np.random.default_rng(1)
    c = bf16_rne(np.exp(rng.uniform(-8, 2, (4, 6))))       # BF16-exact roots
    v = np.repeat(np.repeat(c * c, TILE, axis=0), TILE, axis=1).astype(np.float32)
    assert np.array_equal(v.astype(np.float64), np.repeat(np.repeat(c * c, TILE, 0), TILE, 1))
    view, mu, h = vstate_encode(v)
    assert np.array_equal(mu, c)
    assert not h.any() and float(view.tscale) == 0.0
    assert np.array_equal(vstate_decode(view, mu), v)


def test_means_and_parseval():
    rng = np.random.default_rng(2)
    v = (np.exp(rng.standard_normal((64, 96)) * 2.0) * 1e-6).astype(np.float32)   # heavy-tailed, positive
    view, mu, h = vstate_encode(v)
    s = np.sqrt(v.astype(np.float64))
    mu_full = np.repeat(np.repeat(mu, TILE, 0), TILE, 1)
    # the residual's tile means are zero up to the BF16 rounding of mu
    res_mean = (s - mu_full).reshape(4, TILE, 6, TILE).mean(axis=(1, 3))
    assert np.all(np.abs(res_mean) <= 2.0 ** -8 * mu)
    # the mean computed in the stated order equals the plain mean up to BF16 rounding
    plain = s.reshape(4, TILE, 6, TILE).mean(axis=(1, 3))
    assert np.array_equal(tile_means(s), bf16_rne(plain)) or np.abs(tile_means(s) - plain).max() <= 2.0 ** -8 * plain.max()
    # orthonormal transform: the error in s is the quantization error of h, group by group
    h_hat = dequantize(view)
    s_hat = hadamard16(h_hat) + mu_full
    e_s = np.linalg.norm((s_hat - s).reshape(-1, 16), axis=1)
    e_h = np.linalg.norm((h_hat - h.astype(np.float64)).reshape(-1, 16), axis=1)
    assert np.allclose(e_s, e_h, rtol=1e-6, atol=1e-6 * np.abs(s).max())
    # and decode squares the reconstruction
    assert np.array_equal(vstate_decode(view, mu), (s_hat * s_hat).astype(np.float32))


def test_codec_keeps_small_entries_of_a_heavy_tail():
    """An illustration of the method's point (not a pin of its arithmetic):
    on a heavy-tailed second moment, direct NVFP4 of v flushes the small
    entries that AdamW divides by (median relative error 1), while the codec
    keeps them."""
    from oracle.quantize import quantize
    rng = np.random.default_rng(3)
    v = (rng.standard_t(2, (256, 256)) ** 2 * 1e-8).astype(np.float32)
    view, mu, _ = vstate_encode(v)
    med_codec = np.median(np.abs(vstate_decode(view, mu) - v) / v)
    direct, _, _ = quantize(v, rowwise=True, colwise=False)
    med_direct = np.median(np.abs(dequantize(direct) - v) / v)
    assert med_direct > 0.9 and med_codec < 0.3, (med_codec, med_direct)
