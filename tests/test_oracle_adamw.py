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


# ---- first moment -------------------------------------------------------------
from oracle.adamw import mstate_decode, mstate_encode
from oracle.formats import E2M1_GRID, e4m3_decode
from oracle.quantize import unpack_codes

GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _m(shape, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal(shape) * np.exp(rng.uniform(-3, 1, (shape[0], 1))) * 1e-3).astype(np.float32)


def test_extreme_random_words_give_ceiling_and_floor():
    m = _m((8, 64), 0)
    view0, h = mstate_encode(m, np.zeros(m.shape, np.uint32))                 # u = 0: up whenever off-grid
    view1, _ = mstate_encode(m, np.full(m.shape, 0xFFFFFFFF, np.uint32))      # u ~ 1: never up
    step = np.repeat(e4m3_decode(view0.scales), 16, axis=1) * float(view0.tscale)
    assert np.array_equal(view0.scales, view1.scales)
    y = np.abs(h.astype(np.float64)) / step
    for (i, j), yy in np.ndenumerate(y):
        c0 = int(unpack_codes(view0.codes)[i, j]) & 7
        c1 = int(unpack_codes(view1.codes)[i, j]) & 7
        floor_i = max(k for k in range(8) if GRID[k] <= min(yy, 6.0))
        ceil_i = min(k for k in range(8) if GRID[k] >= min(yy, 6.0))
        assert c1 == floor_i and c0 == ceil_i, (yy, c0, c1)


def test_stochastic_rounding_is_unbiased():
    m = _m((4, 32), 1)
    rng = np.random.default_rng(2)
    acc = np.zeros(m.shape)
    n = 400
    for _ in range(n):
        view, h = mstate_encode(m, rng.integers(0, 2 ** 32, m.shape, dtype=np.uint64).astype(np.uint32))
        acc += oracle_dequant(view)
    mean_err = acc / n - h.astype(np.float64)
    step = np.repeat(e4m3_decode(view.scales), 16, axis=1) * float(view.tscale)
    # the standard error of the mean of n draws within one grid gap (<= 2 steps) is <= step / sqrt(n)
    assert np.all(np.abs(mean_err) <= 5 * 2 * step / np.sqrt(n) + 1e-30)


def oracle_dequant(view):
    from oracle.quantize import dequantize
    return dequantize(view)


def test_four_over_six_choice_by_brute_force():
    m = _m((16, 128), 3)
    view, h = mstate_encode(m, np.zeros(m.shape, np.uint32))
    st = float(view.tscale)
    from oracle.formats import e4m3_rne_satfinite
    blocks = np.abs(h.astype(np.float64)).reshape(16, 8, 16)
    n4 = 0
    for i in range(16):
        for b in range(8):
            mag = blocks[i, b]
            amax = mag.max()
            cands = []
            for k in (6.0, 4.0):
                sb = int(e4m3_rne_satfinite(np.array([amax / (k * st)]))[0])
                step = float(e4m3_decode(np.array([sb]))[0]) * st
                err = 0.0
                for x in mag:
                    best = min(GRID, key=lambda g: (abs(x - g * step), GRID.index(g) % 2))
                    err += (x - best * step) ** 2
                cands.append((err, sb))
            want = cands[1][1] if cands[1][0] < cands[0][0] else cands[0][1]
            assert view.scales[i, b] == want, (i, b)
            n4 += want != cands[0][1]
    assert n4 > 0                                  # some blocks do prefer the 4-scale


def test_first_moment_round_trip_parseval():
    m = _m((32, 64), 4)
    rng = np.random.default_rng(5)
    view, h = mstate_encode(m, rng.integers(0, 2 ** 32, m.shape, dtype=np.uint64).astype(np.uint32))
    m_hat = mstate_decode(view)
    from oracle.quantize import dequantize
    h_hat = dequantize(view)
    e_m = np.linalg.norm((m_hat.astype(np.float64) - m).reshape(-1, 16), axis=1)
    e_h = np.linalg.norm((h_hat - h).reshape(-1, 16), axis=1)
    assert np.allclose(e_m, e_h, rtol=1e-5, atol=1e-6 * np.abs(m).max())
