"""HIP graph capture of the library's calls.

The library never allocates, synchronises or writes memory with memset, so
a whole call can be captured into a HIP graph (bench.py times the step that
way).  Each captured graph is replayed several times, with the program's own
eager calls and synchronisations in between, and every replay must equal the
eager result bit for bit (all kernels are deterministic: fixed reduction
orders, and an order-independent max).
"""
import numpy as np
import pytest
import torch

import synth
from gpu_util import need_gpu, dev_bf16, print_case

pytestmark = pytest.mark.gpu


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = fn()
    torch.cuda.synchronize()
    return g, out


def test_linear_step_graph_replays_equal_eager():
    fs4 = need_gpu()
    print_case(test="graph_linear", M=320, K=256, N=384, r=16)
    rng = np.random.default_rng(11)
    M, K, N, r = 320, 256, 384, 16
    X = dev_bf16(synth.bf16_round(rng.standard_normal((M, K))))
    dY = dev_bf16(synth.bf16_round(rng.standard_normal((M, N)) * 1e-3))
    U = dev_bf16(synth.bf16_round(rng.standard_normal((N, r)) * 0.1))
    V = dev_bf16(synth.bf16_round(rng.standard_normal((r, K)) * 0.1))
    Rw = torch.from_numpy((rng.standard_t(3, size=(N, K)) * 0.02).astype(np.float32)).cuda()
    R_row = fs4.NVFP4.empty(N, K, torch.device("cuda"))
    R_col = fs4.NVFP4.empty(K, N, torch.device("cuda"), R_row.tscale)

    def step():
        fs4.quantize(Rw, out_row=R_row, out_col=R_col)
        f = fs4.linear_fwd(X, R_row, U, V)
        b = fs4.linear_bwd(dY, X, f.X_col, R_col, U, V, f.T)
        return f.Y, b.dX, b.dW, b.dU, b.dV

    ref = [t.clone() for t in step()]
    torch.cuda.synchronize()
    g, outs = _capture(step)
    for rep in range(3):
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, ref):
            assert torch.equal(o, e), rep
        step()                       # eager work between replays
        torch.cuda.synchronize()


def test_newton_schulz_graph_replays_equal_eager():
    fs4 = need_gpu()
    print_case(test="graph_ns", m=768, n=2048)
    G = dev_bf16(synth.ns_input(seed=7, m=768, n=2048))
    X = torch.empty((768, 2048), dtype=torch.float32, device="cuda")
    call = lambda: fs4.newton_schulz(G, steps=3, out=X)
    call()
    torch.cuda.synchronize()
    ref = X.clone()
    g, _ = _capture(call)
    for rep in range(3):
        X.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(X, ref), rep
        call()
        torch.cuda.synchronize()
