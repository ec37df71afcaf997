"""Pins for the oracle's NVFP4 quantizer."""
import os
from fractions import Fraction

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
from oracle import exact as X
from oracle.quantize import unpack_codes, quantize_rows
from oracle.formats import e4m3_decode

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "quantize_worked.txt")


def _load_golden():
    cases, cur = [], None
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, *rest = line.split()
        if key == "tensor":
            cur = {"name": rest[0], "shape": (int(rest[1]), int(rest[2]))}
            cases.append(cur)
        elif key == "x":
            cur["x"] = np.array([float(v) for v in rest], dtype=np.float32).reshape(cur["shape"])
        elif key == "tscale":
            cur["tscale"] = float(rest[0])
        else:
            cur[key] = np.array([int(v, 16) for v in rest], dtype=np.uint8)
    return cases


@pytest.mark.parametrize("case", _load_golden(), ids=lambda c: c["name"])
def test_hand_worked_examples(case):
    row, _, s_t = oracle.quantize(case["x"], rowwise=True, colwise=False)
    assert float(s_t) == case["tscale"]
    assert np.array_equal(row.scales.reshape(-1), case["scales"])
    assert np.array_equal(row.codes.reshape(-1), case["codes"])


def _representable_tensor(rng, rows, cols, s_t_exp):
    """x = g * m_b * s_t with g on the E2M1 grid, one +-6 per 16-block, an E4M3
    block scale m_b per block and s_t = 2^-k; one block uses m_b = 448 so that
    the tensor scale comes out as s_t exactly."""
    s_t = 2.0 ** s_t_exp
    grid = oracle.E2M1_GRID
    g = rng.choice(grid, size=(rows, cols)) * rng.choice([-1.0, 1.0], size=(rows, cols))
    nb = cols // 16
    pos = rng.integers(0, 16, size=(rows, nb))
    for r in range(rows):
        for b in range(nb):
            g[r, 16 * b + pos[r, b]] = 6.0 * rng.choice([-1.0, 1.0])
    mb = e4m3_decode(rng.integers(1, 127, size=(rows, nb)))
    mb[rng.integers(rows), rng.integers(nb)] = 448.0
    x = g * np.repeat(mb, 16, axis=1) * s_t
    return x.astype(np.float32), s_t


@pytest.mark.parametrize("s_t_exp", [0, -7, -20, 5])
def test_exact_roundtrip_of_representable_blocks(s_t_exp):
    rng = np.random.default_rng(100 + s_t_exp)
    x, s_t = _representable_tensor(rng, 8, 64, s_t_exp)
    assert np.array_equal(x.astype(np.float64) / s_t, np.round(x.astype(np.float64) / s_t, 12))
    row, _, got_st = oracle.quantize(x, rowwise=True, colwise=False)
    assert float(got_st) == s_t
    assert np.array_equal(oracle.dequantize(row), x.astype(np.float64))


def test_block_amax_maps_within_six_scales():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((64, 128)) * np.exp(rng.uniform(-6, 6, (64, 1)))).astype(np.float32)
    x[5, 7] *= 300
    row, col, s_t = oracle.quantize(x)
    for v, src in ((row, x), (col, x.T)):
        codes = unpack_codes(v.codes)
        assert np.all((codes & 7) <= 7)
        amax_b = np.abs(src.astype(np.float64)).reshape(v.rows, -1, 16).max(axis=2)
        step = e4m3_decode(v.scales) * float(s_t)
        # the block maximum lands on at most 6 steps after rounding ...
        top = np.take_along_axis(codes.reshape(v.rows, -1, 16) & 7,
                                 np.abs(src).reshape(v.rows, -1, 16).argmax(axis=2)[..., None], axis=2)[..., 0]
        assert np.all(oracle.E2M1_GRID[top] * step <= 6 * step)
        # ... and the scale is the E4M3 rounding of amax_b / 6 s_t: within one
        # E4M3 relative step (2^-4) of it for normal scales
        q = amax_b / (6 * float(s_t))
        normal = q >= 2.0 ** -6
        assert np.all(np.abs(e4m3_decode(v.scales)[normal] - q[normal]) <= q[normal] * 2.0 ** -4)
        # scales never exceed 448 and the tensor's largest block uses 448
        assert e4m3_decode(v.scales).max() == 448.0


def test_unit_scale_reduces_to_plain_e2m1_rounding():
    rng = np.random.default_rng(9)
    vals = np.concatenate([rng.uniform(0, 6, 200), [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]])
    x = np.zeros((1, 16 * 16), dtype=np.float32)
    chunks = np.array_split(vals, 15)
    for b, ch in enumerate(chunks):
        blk = np.zeros(16)
        blk[:len(ch[:15])] = ch[:15]
        blk[15] = 6.0                                   # block amax 6 -> s_b = 1
        x[0, 16 * b:16 * b + 16] = blk
    x[0, 16 * 15] = 2688.0                              # s_t = 1
    row, _, s_t = oracle.quantize(x, colwise=False)
    assert float(s_t) == 1.0
    codes = unpack_codes(row.codes)[0, :16 * 15]
    plain = []
    for v in x[0, :16 * 15].astype(np.float64):
        d = np.abs(oracle.E2M1_GRID - v)
        cand = np.flatnonzero(d == d.min())
        plain.append(cand[0] if len(cand) == 1 else cand[cand % 2 == 0][0])
    assert np.array_equal(codes & 7, np.array(plain))


def _check_against_exact(x):
    row, col, s_t = oracle.quantize(x)
    rc, rs, cc, cs, s_t_exact = X.quantize_exact(x)
    assert Fraction(float(s_t)) == s_t_exact
    assert np.array_equal(unpack_codes(row.codes), rc)
    assert np.array_equal(row.scales, rs)
    assert np.array_equal(unpack_codes(col.codes), cc)
    assert np.array_equal(col.scales, cs)


@pytest.mark.parametrize("seed", range(4))
def test_matches_exact_twin_random(seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((32, 48)) * np.exp(rng.uniform(-3, 3, (32, 1)))
    x[rng.random((32, 48)) < 0.05] *= 50
    x[rng.random((32, 48)) < 0.05] = 0.0
    x[0, :16] = 0.0                                      # an all-zero block
    x[1, 3] = -0.0
    _check_against_exact(x.astype(np.float32))


def test_matches_exact_twin_ties():
    # elements placed exactly on E2M1 midpoints of a non-trivial block step
    rng = np.random.default_rng(77)
    s_t = 2.0 ** -3
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    x = np.zeros((16, 32))
    for r in range(16):
        mb = float(e4m3_decode(rng.integers(1, 127)))
        x[r, :16] = rng.choice(mids, 16) * mb * s_t * rng.choice([-1, 1], 16)
        x[r, rng.integers(16)] = 6 * mb * s_t
        x[r, 16:] = rng.standard_normal(16)
    x[3, 20] = 6 * 448 * s_t
    _check_against_exact(x.astype(np.float32))


def test_matches_exact_twin_subnormal_tensor_scale():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((16, 32)) * 1e-41).astype(np.float32)   # fp32 subnormals
    assert np.any(x != 0)
    _check_against_exact(x)


@settings(max_examples=30, deadline=None)
@given(st.integers(0, 2 ** 32 - 1), st.sampled_from([(16, 16), (16, 32), (32, 16)]),
       st.floats(-30, 30))
def test_matches_exact_twin_property(seed, shape, log_scale):
    rng = np.random.default_rng(seed)
    x = rng.standard_t(3, size=shape) * np.exp(log_scale)
    x[rng.random(shape) < 0.1] = 0.0
    _check_against_exact(x.astype(np.float32))


def test_colwise_is_rowwise_of_transpose_with_shared_scale():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((32, 64)).astype(np.float32)
    x[:, 0] *= 100                                       # amax sits in column 0
    row, col, s_t = oracle.quantize(x)
    assert col.rows == 64 and col.cols == 32
    # the column layout of x^T would need its own amax; both layouts of x use
    # the one tensor scale of x
    assert float(row.tscale) == float(col.tscale) == float(s_t)
    ref = quantize_rows(np.ascontiguousarray(x.T), s_t)
    assert np.array_equal(ref.codes, col.codes) and np.array_equal(ref.scales, col.scales)


def test_zero_tensor():
    x = np.zeros((16, 16), dtype=np.float32)
    row, col, s_t = oracle.quantize(x)
    assert float(s_t) == 0.0
    assert not row.codes.any() and not row.scales.any()


def test_rejects_non_finite_and_bad_shapes():
    with pytest.raises(ValueError):
        oracle.quantize(np.full((16, 16), np.inf, dtype=np.float32))
    with pytest.raises(ValueError):
        quantize_rows(np.zeros((2, 20), dtype=np.float32), np.float32(1))
    with pytest.raises(TypeError):
        oracle.quantize(np.zeros((16, 16)))


def test_chunked_quantize_helper_equals_the_oracle():
    """The tests' chunked, threaded driver of the oracle's row quantizer (used
    at the full workload sizes) gives oracle.quantize's views bit for bit."""
    import sys
    import os
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    from gpu_util import quantize_chunked
    rng = np.random.default_rng(17)
    x = (rng.standard_t(3, size=(1040, 528)) * np.exp(rng.uniform(-3, 3, (1040, 1)))).astype(np.float32)
    want = oracle.quantize(x)
    got = quantize_chunked(x, chunk=96, threads=4)
    assert got[2] == want[2]
    for g, w in zip(got[:2], want[:2]):
        assert g.rows == w.rows and g.cols == w.cols and g.tscale == w.tscale
        assert np.array_equal(g.codes, w.codes) and np.array_equal(g.scales, w.scales)
