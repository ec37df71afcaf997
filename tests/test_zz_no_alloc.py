"""fs4_quantize_noalloc (the quantizer with the library's own per-device
scratch instead of a workspace) against fs4_quantize, through the C ABI:
codes, block scales and tensor scale bit for bit, on two calls in a row, the
second with a smaller input (the scratch keeps the first call's partials,
which the second must not read)."""
import ctypes

import numpy as np
import pytest
import torch

import synth
from gpu_util import need_gpu, print_case

pytestmark = pytest.mark.gpu


def _noalloc(fs4, x, rows, cols, code):
    dev = x.device
    row = fs4.NVFP4.empty(rows, cols, dev)
    col = fs4.NVFP4.empty(cols, rows, dev, row.tscale)
    rv, cv = row.c(), col.c()
    st = fs4._lib.fs4_quantize_noalloc(x.data_ptr(), code, rows, cols, ctypes.byref(rv), ctypes.byref(cv),
                                      torch.cuda.current_stream(dev).cuda_stream)
    assert st == 0, fs4.status_str(st)
    return row, col


def test_noalloc_quantize_equals_quantize_on_two_calls():
    fs4 = need_gpu()
    assert fs4._lib.fs4_quantize_noalloc_scratch_bytes() >= fs4._lib.fs4_quantize_workspace_bytes(1, 1)
    cases = [("bf16", 4096, 4096), ("fp32", 272, 400)]     # the second call smaller
    rng = np.random.default_rng(5)
    for dt, rows, cols in cases:
        print_case(test="quantize_noalloc", dtype=dt, rows=rows, cols=cols)
        if dt == "bf16":
            bits = synth.quantizer_input(rows=rows, cols=cols)
            x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
            code = fs4.FS4_BF16
        else:
            x = torch.from_numpy((rng.standard_t(3, (rows, cols)) * 1e-3).astype(np.float32)).cuda()
            code = fs4.FS4_FP32
        got_row, got_col = _noalloc(fs4, x, rows, cols, code)
        ref_row, ref_col = fs4.quantize(x)
        torch.cuda.synchronize()
        for got, ref, what in ((got_row, ref_row, "row"), (got_col, ref_col, "col")):
            assert torch.equal(got.codes, ref.codes), (dt, what, "codes")
            assert torch.equal(got.scales, ref.scales), (dt, what, "scales")
            assert torch.equal(got.tscale, ref.tscale), (dt, what, "tscale")
