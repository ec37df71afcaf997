"""Helpers for the GPU parity tests: move synth arrays to the device, bring
NVFP4 views back, run the oracle on the same inputs."""
import numpy as np
import pytest
import torch

import oracle
import synth


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import precision_pretraining_amd as fs4   # raises ImportError if libfs4.so is missing
    return fs4


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def host_view(v):
    """(codes uint8, scales uint8, tscale float32) of a device NVFP4 view."""
    torch.cuda.synchronize()
    return v.codes.cpu().numpy(), v.scales.cpu().numpy(), np.float32(v.tscale.cpu().item())


def assert_view_equal(gpu_view, ref: "oracle.NVFP4", what=""):
    codes, scales, ts = host_view(gpu_view)
    assert ts.tobytes() == np.float32(ref.tscale).tobytes(), (what, ts, ref.tscale)
    bad_s = np.argwhere(scales != ref.scales)
    assert bad_s.size == 0, (what, "scales differ", bad_s[:5], scales[tuple(bad_s[0])], ref.scales[tuple(bad_s[0])])
    bad_c = np.argwhere(codes != ref.codes)
    assert bad_c.size == 0, (what, "codes differ", bad_c[:5], codes[tuple(bad_c[0])], ref.codes[tuple(bad_c[0])])


def f32(bits):
    return synth.bf16_to_f32(bits)


def print_case(**kw):
    print("CASE " + " ".join("%s=%s" % (k, v) for k, v in kw.items()), flush=True)


def quantize_chunked(x, rowwise=True, colwise=True, chunk=512, threads=8):
    """oracle.quantize(x) for large x: the same tensor scale, then the
    oracle's own row quantizer on chunks of rows (of x, or of x^T for the
    column-wise view) in a thread pool.  Rows are quantized independently, so
    the result is oracle.quantize's bit for bit (tests/test_oracle_quantize.py
    checks it); the chunks keep numpy's temporaries small."""
    import concurrent.futures as cf
    from oracle.quantize import NVFP4, quantize_rows, tensor_scale
    x = np.ascontiguousarray(x, dtype=np.float32)
    s_t = tensor_scale(x)

    def layout(src):
        rows = src.shape[0]
        spans = [(i, min(i + chunk, rows)) for i in range(0, rows, chunk)]
        with cf.ThreadPoolExecutor(threads) as ex:
            parts = list(ex.map(lambda sp: quantize_rows(np.ascontiguousarray(src[sp[0]:sp[1]]), s_t), spans))
        codes = np.concatenate([p.codes for p in parts]) if parts else np.zeros((0, src.shape[1] // 2), np.uint8)
        scales = np.concatenate([p.scales for p in parts]) if parts else np.zeros((0, src.shape[1] // 16), np.uint8)
        return NVFP4(codes, scales, np.float32(s_t), src.shape[0], src.shape[1])

    row = layout(x) if rowwise else None
    col = layout(x.T) if colwise else None
    return row, col, s_t


def gemm_full_check(got, qa, qb, alpha=1.0, extra=None, extra_abs=None, rows=1024):
    """max |got - ref| / D over every element of an NT product, where
    ref = alpha s_tA s_tB A_hat B_hat^T (+ extra) and D the matching sum of
    |a||b| (+ extra_abs), from the oracle's block values, processed in bands
    of rows to bound host memory."""
    from oracle.quantize import block_values
    bb = block_values(qb)
    bb_abs = np.abs(bb)
    s = alpha * float(qa.tscale) * float(qb.tscale)
    worst = 0.0
    for i0 in range(0, qa.rows, rows):
        i1 = min(i0 + rows, qa.rows)
        sub = type(qa)(qa.codes[i0:i1], qa.scales[i0:i1], qa.tscale, i1 - i0, qa.cols)
        ab = block_values(sub)
        ref = s * (ab @ bb.T)
        den = abs(s) * (np.abs(ab) @ bb_abs.T)
        if extra is not None:
            ref += extra(i0, i1)
            den += extra_abs(i0, i1)
        worst = max(worst, oracle.rel_err(got[i0:i1], ref, den))
    return worst
