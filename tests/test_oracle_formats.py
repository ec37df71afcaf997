"""Pins for the oracle's number formats (E2M1, E4M3, FP32 tensor scale)."""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import exact as X


def test_e2m1_decode_all_codes():
    want = [0, .5, 1, 1.5, 2, 3, 4, 6]
    for c in range(16):
        v = F.e2m1_decode(c)
        assert abs(v) == want[c & 7]
        assert np.signbit(v) == bool(c & 8) or want[c & 7] == 0


def test_e2m1_grid_roundtrip():
    for i, g in enumerate(F.E2M1_GRID):
        assert F.e2m1_rne_index(g) == i


@pytest.mark.parametrize("mid,lo_idx", [(0.25, 0), (0.75, 1), (1.25, 2), (1.75, 3), (2.5, 4), (3.5, 5), (5.0, 6)])
def test_e2m1_midpoints_and_neighbours(mid, lo_idx):
    # exact tie -> even index
    even = lo_idx if lo_idx % 2 == 0 else lo_idx + 1
    assert F.e2m1_rne_index(mid) == even
    # one fp64 ulp either side lands on the near side
    assert F.e2m1_rne_index(np.nextafter(mid, 0)) == lo_idx
    assert F.e2m1_rne_index(np.nextafter(mid, 10)) == lo_idx + 1


def test_e2m1_saturates():
    assert F.e2m1_rne_index(6.0) == 7
    assert F.e2m1_rne_index(7.0) == 7
    assert F.e2m1_rne_index(1e30) == 7
    assert F.e2m1_rne_index(0.0) == 0


def test_e4m3_decode_matches_torch():
    b = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    t = b.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = F.e4m3_decode(np.arange(256))
    nan = np.isnan(t)
    assert np.array_equal(nan, np.isnan(ours))
    assert np.array_equal(t[~nan], ours[~nan])
    assert F.e4m3_decode(0x7E) == 448.0
    assert F.e4m3_decode(0x01) == 2.0 ** -9


def test_e4m3_decode_matches_exact_definition():
    for b in range(127):
        assert Fraction(float(F.e4m3_decode(b))) == X.e4m3_value(b)


def _torch_e4m3(vals_f32):
    return torch.from_numpy(vals_f32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_encode_matches_torch_random():
    # torch's cast is round-to-nearest-even for in-range values and NaN from
    # 464 up; compare on float32 values clamped to <= 448.
    rng = np.random.default_rng(123)
    v = np.concatenate([
        rng.uniform(0, 448, 400_000),
        np.exp(rng.uniform(np.log(2.0 ** -12), np.log(448.0), 600_000)),
    ]).astype(np.float32)
    ours = F.e4m3_rne_satfinite(v.astype(np.float64))
    assert np.array_equal(ours, _torch_e4m3(v))


def test_e4m3_encode_midpoints_match_torch():
    pos = F.e4m3_decode(np.arange(127))
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (pos[:-1] + pos[1:]) / 2)   # exact in fp32
    around = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9)),
                             pos.astype(np.float32)])
    ours = F.e4m3_rne_satfinite(around.astype(np.float64))
    assert np.array_equal(ours, _torch_e4m3(around))


def test_e4m3_satfinite():
    assert F.e4m3_rne_satfinite(448.0) == 0x7E
    assert F.e4m3_rne_satfinite(460.0) == 0x7E
    assert F.e4m3_rne_satfinite(470.0) == 0x7E      # torch gives NaN here
    assert F.e4m3_rne_satfinite(1e10) == 0x7E
    assert F.e4m3_rne_satfinite(2.0 ** -10) == 0     # tie between 0 and 2^-9 -> even code 0
    assert F.e4m3_rne_satfinite(1.5 * 2.0 ** -9) == 2


def test_e4m3_encode_matches_exact_twin():
    rng = np.random.default_rng(7)
    qs = np.exp(rng.uniform(np.log(2.0 ** -12), np.log(600.0), 3000))
    ours = F.e4m3_rne_satfinite(qs)
    for q, c in zip(qs, ours):
        assert X.nearest_even(Fraction(float(q)), X.E4M3_FINITE) == c


def test_tensor_scale_is_exactly_rounded():
    rng = np.random.default_rng(11)
    amax = np.concatenate([
        np.exp(rng.uniform(np.log(1e-40), np.log(1e30), 3000)).astype(np.float32),
        np.array([2688.0, 1.0, 6.0, 448.0, 2.0 ** -149, 2.0 ** -126, 3.4e38], dtype=np.float32),
    ])
    for a in amax:
        got = F.tensor_scale_from_amax(a)
        want = X.round_to_f32(Fraction(float(a)) / 2688)
        assert Fraction(float(got)) == want, a
    assert F.tensor_scale_from_amax(np.float32(2688.0)) == np.float32(1.0)
    assert F.tensor_scale_from_amax(np.float32(0.0)) == np.float32(0.0)


def test_round_to_f32_matches_numpy():
    # the exact twin's fp32 rounding is itself pinned to numpy's fp64->fp32 cast
    rng = np.random.default_rng(5)
    for v in np.exp(rng.uniform(np.log(1e-44), np.log(1e30), 2000)):
        assert Fraction(float(np.float32(v))) == X.round_to_f32(Fraction(float(v)))
