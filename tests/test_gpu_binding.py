"""The binding's argument checks on device tensors: every mismatch between
arguments (dtype, shape, layout, device) raises before the library is
called, so nothing is launched on a bad buffer."""
import pytest
import torch

from gpu_util import need_gpu, print_case

pytestmark = pytest.mark.gpu


def test_binding_rejects_mismatched_device_arguments():
    fs4 = need_gpu()
    print_case(test="binding_checks")
    d = torch.device("cuda")
    bf = lambda *s: torch.zeros(s, dtype=torch.bfloat16, device=d)
    f32 = lambda *s: torch.zeros(s, dtype=torch.float32, device=d)
    i32 = lambda *s: torch.zeros(s, dtype=torch.int32, device=d)
    A = fs4.NVFP4.empty(64, 128, d)
    B = fs4.NVFP4.empty(32, 128, d)
    B96 = fs4.NVFP4.empty(32, 96, d)
    cases = [
        (lambda: fs4.gemm_nt(A, B96), ValueError, "B must be a"),
        (lambda: fs4.gemm_nt(A, B, out=f32(64, 31)), ValueError, "out must have shape"),
        (lambda: fs4.gemm_nt(A, B, E=bf(64, 32), beta_e=1.0), TypeError, "E must have dtype"),
        (lambda: fs4.gemm_nt(A, B, out=f32(64, 64)[:, :32]), ValueError, "out must be contiguous"),
        (lambda: fs4.linear_fwd(bf(16, 128), B, bf(32, 8), bf(8, 64)), ValueError, "V must have shape"),
        (lambda: fs4.linear_fwd(bf(16, 128), B, bf(16, 8), bf(8, 128)), ValueError, "U must have shape"),
        (lambda: fs4.linear_fwd(bf(16, 128), B, f32(32, 8), bf(8, 128)), TypeError, "U must have dtype"),
        (lambda: fs4.linear_fwd(bf(16, 128), B, None, None, out=f32(16, 16)), ValueError, "out must have shape"),
        (lambda: fs4.linear_bwd(bf(16, 32), bf(16, 128), fs4.NVFP4.empty(128, 16, d), fs4.NVFP4.empty(128, 32, d),
                                bf(32, 8), bf(8, 128), f32(16, 4)), ValueError, "T must have shape"),
        (lambda: fs4.linear_bwd(bf(16, 32), f32(16, 128), fs4.NVFP4.empty(128, 16, d),
                                fs4.NVFP4.empty(128, 32, d), None, None, None), TypeError, "X must have dtype"),
        (lambda: fs4.linear_bwd(bf(16, 32), None, fs4.NVFP4.empty(128, 16, d), fs4.NVFP4.empty(128, 48, d),
                                None, None, None), ValueError, "R_col must be a"),
        (lambda: fs4.mstate_encode(f32(64, 64), i32(64, 32)), ValueError, "rnd must have shape"),
        (lambda: fs4.mstate_encode(f32(64, 64), torch.zeros((64, 64), dtype=torch.int16, device=d)), TypeError,
         "rnd must have dtype"),
        (lambda: fs4.vstate_decode(fs4.NVFP4.empty(64, 64, d), bf(4, 3)), ValueError, "means must have shape"),
        (lambda: fs4.lora_project(bf(64, 8), bf(8, 32), f32(64, 4), None), ValueError, "dU must have shape"),
        (lambda: fs4.lora_realign(bf(64, 8), bf(8, 32), f32(64, 32), f32(12, 16)), ValueError,
         "Omega must have shape"),
        (lambda: fs4.newton_schulz(bf(64, 128), out=f32(64, 64)), ValueError, "out must have shape"),
        (lambda: fs4.quantize(bf(64, 64), out_row=fs4.NVFP4.empty(64, 32, d)), ValueError, "out_row must be a"),
    ]
    if torch.cuda.device_count() > 1:   # pragma: no cover (one-GPU machines)
        cases.append((lambda: fs4.gemm_nt(A, fs4.NVFP4.empty(32, 128, torch.device("cuda:1"))), ValueError,
                      "B.codes is on"))
    for call, exc, match in cases:
        with pytest.raises(exc, match=match):
            call()
    torch.cuda.synchronize()
