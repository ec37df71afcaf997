"""Quantizer parity: codes, scales and tensor scale bit-exact vs the oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import need_gpu, dev_bf16, dev_f32, assert_view_equal, host_view, print_case, f32, quantize_chunked

pytestmark = pytest.mark.gpu


def _run(x_dev, x_host_f32, rowwise=True, colwise=True, what=""):
    fs4 = need_gpu()
    row, col = fs4.quantize(x_dev, rowwise=rowwise, colwise=colwise)
    ref_row, ref_col, _ = oracle.quantize(x_host_f32, rowwise=rowwise, colwise=colwise)
    if rowwise:
        assert_view_equal(row, ref_row, what + " row")
    if colwise:
        assert_view_equal(col, ref_col, what + " col")


@pytest.mark.parametrize("shape", [(16, 16), (64, 64), (48, 80), (272, 400), (1040, 208)])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_random_shapes(shape, dtype):
    print_case(test="quantize_random", shape=shape, dtype=dtype)
    rng = np.random.default_rng(shape[0] * 7 + shape[1])
    x = rng.standard_t(3, size=shape) * np.exp(rng.uniform(-4, 4, (shape[0], 1)))
    x[rng.random(shape) < 0.02] = 0.0
    x[rng.random(shape) < 0.01] = -0.0
    if dtype == "bf16":
        b = synth.bf16_round(x)
        _run(dev_bf16(b), f32(b), what=dtype)
    else:
        x = x.astype(np.float32)
        _run(dev_f32(x), x, what=dtype)


def test_single_layouts():
    rng = np.random.default_rng(3)
    b = synth.bf16_round(rng.standard_normal((96, 160)))
    print_case(test="quantize_single_layouts")
    _run(dev_bf16(b), f32(b), rowwise=True, colwise=False, what="row only")
    _run(dev_bf16(b), f32(b), rowwise=False, colwise=True, what="col only")


def test_ties_and_representable_blocks():
    # elements exactly on E2M1 midpoints (ties) and on grid points times an
    # E4M3 scale, with a power-of-two tensor scale
    print_case(test="quantize_ties")
    rng = np.random.default_rng(5)
    s_t = 2.0 ** -4
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    grid = oracle.E2M1_GRID
    x = np.zeros((64, 128))
    for r in range(64):
        for blk in range(8):
            mb = float(oracle.e4m3_decode(rng.integers(1, 127)))
            vals = rng.choice(mids if (r + blk) % 2 else grid, 16) * rng.choice([-1, 1], 16)
            vals[rng.integers(16)] = 6.0
            x[r, 16 * blk:16 * blk + 16] = vals * mb * s_t
    x[7, 9] = 6 * 448 * s_t
    x = x.astype(np.float32)
    _run(dev_f32(x), x, what="ties")


def test_fp32_subnormal_and_tiny_tensor_scales():
    print_case(test="quantize_subnormal")
    rng = np.random.default_rng(6)
    for scale in (1e-41, 1e-36, 1e-30):
        x = (rng.standard_normal((32, 64)) * scale).astype(np.float32)
        _run(dev_f32(x), x, what="tiny %g" % scale)


def test_zero_and_negative_zero():
    print_case(test="quantize_zero")
    x = np.zeros((32, 32), dtype=np.float32)
    x[3, 5] = -0.0
    x[17, 0] = -0.0
    _run(dev_f32(x), x, what="zeros")


def test_empty_tensor_writes_zero_tensor_scale():
    fs4 = need_gpu()
    print_case(test="quantize_empty")
    x = torch.empty((0, 32), dtype=torch.bfloat16, device="cuda")
    ts = torch.full((1,), 7.0, device="cuda")
    rv = fs4.NVFP4(torch.empty(0, dtype=torch.uint8, device="cuda"),
                   torch.empty(0, dtype=torch.uint8, device="cuda"), ts, 0, 32)
    fs4.quantize(x, rowwise=True, colwise=False, out_row=rv)
    torch.cuda.synchronize()
    assert ts.item() == 0.0


def test_deterministic():
    fs4 = need_gpu()
    print_case(test="quantize_deterministic")
    b = synth.quantizer_input(seed=2, rows=512, cols=1024)
    x = dev_bf16(b)
    r1, c1 = fs4.quantize(x)
    r2, c2 = fs4.quantize(x)
    torch.cuda.synchronize()
    assert torch.equal(r1.codes, r2.codes) and torch.equal(c1.codes, c2.codes)
    assert torch.equal(r1.scales, r2.scales) and torch.equal(c1.scales, c2.scales)


def test_quantizer_workload_full_size():
    """4096 x 4096 bf16 ~N(0,1) with 0.1% x50 outliers, both layouts, all
    codes and scales compared."""
    print_case(test="quantize_4096", shape=(4096, 4096))
    b = synth.quantizer_input()
    _run(dev_bf16(b), f32(b), what="4096^2")


def test_3b_gradient_full(linear3b_inputs):
    """8192 x 8192 dY (the backward's largest quantization): both layouts bit
    for bit in full."""
    fs4 = need_gpu()
    print_case(test="quantize_dy_8192", shape=(8192, 8192))
    b = linear3b_inputs[1]
    row, col = fs4.quantize(dev_bf16(b))
    ref_r, ref_c, _ = quantize_chunked(f32(b))
    assert_view_equal(row, ref_r, "dY row")
    assert_view_equal(col, ref_c, "dY col")
