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
