"""C-ABI checks that need no GPU: the library loads, exports every function
declared in include/fs4.h, and rejects bad arguments on the host before
launching anything (validation never touches the fake device pointers used
here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fs4.h")

fs4 = pytest.importorskip("precision_pretraining_amd", reason="libfs4.so not built")
lib = fs4._lib

OK, NULL, SHAPE, ALIGN, DTYPE, RANK, WORKSPACE, HIP, ARG = range(9)
A16 = 0x10000          # fake 16-byte aligned "device" address (never dereferenced)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fs4_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for want in ["fs4_quantize", "fs4_gemm_nt", "fs4_linear_fwd", "fs4_linear_bwd", "fs4_newton_schulz",
                 "fs4_workspace_bytes", "fs4_status_str"]:
        assert want in names


def test_library_exports_every_declared_symbol():
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert sorted(fs4.EXPORTS) == declared_functions()


def test_status_strings_and_version():
    for st in range(9):
        assert fs4.status_str(st).startswith("FS4")
    assert "gfx950" in fs4.version()


def view(rows, cols, codes=A16, scales=A16, tscale=A16):
    return fs4._View(codes, scales, tscale, rows, cols)


def q(x=A16, dt=0, rows=64, cols=64, rv="ok", cv="ok", ws=A16 * 16, wsb=1 << 20):
    r = view(rows, cols) if rv == "ok" else rv
    c = view(cols, rows) if cv == "ok" else cv
    return lib.fs4_quantize(x, dt, rows, cols, ctypes.byref(r) if r is not None else None,
                            ctypes.byref(c) if c is not None else None, ws, wsb, None)


def test_quantize_validation():
    assert q(dt=7) == DTYPE
    assert q(rows=-16) == SHAPE
    assert q(rv=None, cv=None) == NULL
    assert q(x=None) == NULL
    assert q(x=A16 + 4) == ALIGN
    assert q(rv=view(64, 48)) == SHAPE                     # view shape disagrees
    assert q(cols=40, rv=view(64, 40), cv=None) == SHAPE   # cols not a multiple of 16
    assert q(rows=40, rv=None, cv=view(64, 40)) == SHAPE   # rows blocked in the column view
    assert q(rv=view(64, 64, codes=None)) == NULL
    assert q(rv=view(64, 64, scales=A16 + 8)) == ALIGN
    assert q(wsb=16) == WORKSPACE
    assert q(ws=None) == NULL
    assert q(ws=A16 + 16) == ALIGN                         # workspace must be 256-byte aligned
    assert lib.fs4_quantize_workspace_bytes(64, 64) > 0


def test_gemm_validation():
    a, b = view(64, 128), view(32, 128)
    assert lib.fs4_gemm_nt(None, ctypes.byref(b), 1.0, None, 0.0, A16, None, 0, None) == NULL
    bad = view(32, 96)
    assert lib.fs4_gemm_nt(ctypes.byref(a), ctypes.byref(bad), 1.0, None, 0.0, A16, None, 0, None) == SHAPE
    assert lib.fs4_gemm_nt(ctypes.byref(a), ctypes.byref(b), 1.0, None, 0.0, None, None, 0, None) == NULL
    assert lib.fs4_gemm_nt(ctypes.byref(a), ctypes.byref(b), 1.0, A16 + 4, 0.0, A16, None, 0, None) == ALIGN
    odd = view(64, 40)
    assert lib.fs4_gemm_nt(ctypes.byref(odd), ctypes.byref(odd), 1.0, None, 0.0, A16, None, 0, None) == SHAPE


def fwd(X=A16, M=64, K=128, R="ok", U=A16, V=A16, r=8, Y=A16, T=None, xc=None, wsb=1 << 30):
    Rv = view(256, K) if R == "ok" else R
    return lib.fs4_linear_fwd(X, M, K, ctypes.byref(Rv) if Rv is not None else None, U, V, r, 1.0, Y, T,
                              ctypes.byref(xc) if xc is not None else None, A16 * 16, wsb, None)


def test_linear_fwd_validation():
    assert fwd(M=40) == SHAPE
    assert fwd(K=0) == SHAPE
    assert fwd(X=None) == NULL
    assert fwd(R=None) == NULL
    assert fwd(R=view(256, 64)) == SHAPE
    assert fwd(r=65) == RANK
    assert fwd(r=-1) == RANK
    assert fwd(U=None) == RANK
    assert fwd(Y=A16 + 8) == ALIGN
    assert fwd(xc=view(64, 128)) == SHAPE                  # must be rows = K, cols = M
    assert fwd(wsb=100) == WORKSPACE
    need = lib.fs4_linear_fwd_workspace_bytes(64, 128, 256, 8)
    assert need == lib.fs4_workspace_bytes(2, 64, 128, 256, 8)


def bwd(dY=A16, M=64, N=256, K=128, X=A16, xc="ok", rc="ok", U=A16, V=A16, r=8, T=A16, dX=A16, dW=A16,
        dU=A16, dV=A16, wsb=1 << 30):
    xcv = view(K, M) if xc == "ok" else xc
    rcv = view(K, N) if rc == "ok" else rc
    return lib.fs4_linear_bwd(dY, M, N, K, X, ctypes.byref(xcv) if xcv is not None else None,
                              ctypes.byref(rcv) if rcv is not None else None, U, V, r, 1.0, T, dX, dW, dU, dV,
                              A16 * 16, wsb, None)


def test_linear_bwd_validation():
    assert bwd(N=100) == SHAPE
    assert bwd(dY=None) == NULL
    assert bwd(xc=view(M := 64, 128)) == SHAPE
    assert bwd(rc=None) == NULL
    assert bwd(T=None) == RANK
    assert bwd(X=None) == NULL                             # dV requested needs X
    assert bwd(dX=None) == NULL
    assert bwd(dW=A16 + 4) == ALIGN
    assert bwd(wsb=1) == WORKSPACE


def ns(G=A16, dt=0, m=64, n=128, steps=5, X=A16 * 4, wsb=1 << 30, tX=None, clip=0.0):
    return lib.fs4_newton_schulz(G, dt, m, n, steps, 3.4445, -4.775, 2.0315, 1, 1e-7, clip, X, tX, None, None,
                                 A16 * 16, wsb, None)


def test_newton_schulz_validation():
    assert ns(dt=3) == DTYPE
    assert ns(m=256, n=128) == SHAPE                       # m <= n required
    assert ns(m=24) == SHAPE
    assert ns(steps=-1) == ARG
    assert ns(G=None) == NULL
    assert ns(X=A16 + 2) == ALIGN
    assert ns(wsb=1024) == WORKSPACE
    assert ns(X=A16) == ARG                                # X_out overlapping G (bf16 64 x 128)
    assert ns(X=A16 + 64 * 128 * 2 - 16) == ARG
    assert ns(X=A16 * 4 + 64 * 128 * 4 * 3, tX=A16 * 4) == ARG   # X_out inside trace_X
    assert ns(clip=1.5) == ARG
    assert ns(clip=-0.5) == ARG
    assert ns(clip=float("nan")) == ARG


def test_workspace_sizes_grow_with_shape():
    small = lib.fs4_linear_bwd_workspace_bytes(64, 64, 64, 8)
    big = lib.fs4_linear_bwd_workspace_bytes(8192, 8192, 3072, 32)
    assert big > small > 0
    assert lib.fs4_newton_schulz_workspace_bytes(3072, 8192) > 3072 * 8192 * 4
    assert lib.fs4_workspace_bytes(99, 1, 1, 1, 0) == 0


def lp(U=A16, V=A16 * 2, N=64, K=48, r=8, dU=A16 * 4, dV=A16 * 8, wsb=1 << 20):
    return lib.fs4_lora_project(U, V, N, K, r, dU, dV, A16 * 16, wsb, None)


def test_lora_project_validation():
    assert lp(r=65) == RANK
    assert lp(r=-1) == RANK
    assert lp(N=-1) == SHAPE
    assert lp(K=-16) == SHAPE
    assert lp(U=None) == NULL                              # dU given needs U
    assert lp(V=None) == NULL                              # dV given needs V
    assert lp(dU=A16 + 4) == ALIGN
    assert lp(V=A16 + 2) == ALIGN
    assert lp(wsb=1) == WORKSPACE
    # nothing to do: returns before any launch, whatever the pointers
    assert lp(r=0, U=None, V=None) == OK
    assert lp(dU=None, dV=None, U=None, V=None) == OK
    assert lp(N=0, dV=None, U=None) == OK


def test_lora_project_workspace():
    n = lib.fs4_lora_project_workspace_bytes(8192, 3072, 32)
    assert n > 0
    assert lib.fs4_workspace_bytes(fs4.FS4_OP_LORA_PROJECT, 8192, 3072, 0, 32) == n
    assert lib.fs4_lora_project_workspace_bytes(64, 64, 65) == 0
    assert lib.fs4_lora_project_workspace_bytes(8192, 8192, 64) >= n


def ra(N=64, K=48, r=8, l=12, beta=1.0, q=1, U=A16, V=A16 * 2, R=A16 * 3, Om=A16 * 5, sig=None, wsb=1 << 30):
    return lib.fs4_lora_realign(U, V, R, N, K, r, beta, Om, l, q, sig, A16 * 16, wsb, None)


def test_lora_realign_validation():
    assert ra(r=0) == RANK
    assert ra(l=7) == RANK                                 # l < r
    assert ra(l=65) == RANK
    assert ra(N=40) == SHAPE                               # not a multiple of 16
    assert ra(K=0) == SHAPE
    assert ra(N=16, l=17, r=8) == SHAPE                    # l > min(N, K)
    assert ra(q=-1) == ARG
    assert ra(q=17) == ARG
    assert ra(beta=0.0) == ARG
    assert ra(beta=float("nan")) == ARG
    assert ra(U=None) == NULL
    assert ra(Om=A16 + 8) == ALIGN
    assert ra(sig=A16 + 2) == ALIGN
    assert ra(wsb=1) == WORKSPACE
    assert lib.fs4_lora_realign_workspace_bytes(8192, 3072, 40) > 8192 * 3072 * 4
    assert lib.fs4_workspace_bytes(fs4.FS4_OP_LORA_REALIGN, 8192, 3072, 40, 0) == \
        lib.fs4_lora_realign_workspace_bytes(8192, 3072, 40)
    assert lib.fs4_lora_realign_workspace_bytes(8192, 3072, 65) == 0


def test_abs_quantile_validation():
    f = lambda x=A16, dt=1, n=100, q=0.99, out=A16 * 2, wsb=1 << 20: lib.fs4_abs_quantile(
        x, dt, n, q, out, A16 * 16, wsb, None)
    assert f(dt=5) == DTYPE
    assert f(n=0) == SHAPE
    assert f(n=(1 << 31) + 1) == SHAPE
    assert f(q=0.0) == ARG
    assert f(q=1.0000001) == ARG
    assert f(x=None) == NULL
    assert f(out=None) == NULL
    assert f(out=A16 + 2) == ALIGN
    assert f(x=A16 + 4) == ALIGN
    assert f(wsb=8) == WORKSPACE
    assert lib.fs4_abs_quantile_workspace_bytes(100) > 0


def test_quantize_clipped_validation():
    def qc(x=A16, dt=0, rows=64, cols=64, q=0.99, rv="ok", cv="ok", wsb=1 << 20):
        r = view(rows, cols) if rv == "ok" else rv
        c = view(cols, rows) if cv == "ok" else cv
        return lib.fs4_quantize_clipped(x, dt, rows, cols, q, ctypes.byref(r) if r is not None else None,
                                        ctypes.byref(c) if c is not None else None, A16 * 16, wsb, None)
    assert qc(q=0.0) == ARG
    assert qc(q=2.0) == ARG
    assert qc(dt=9) == DTYPE
    assert qc(rows=-16) == SHAPE
    assert qc(rv=None, cv=None) == NULL
    assert qc(rv=view(64, 48)) == SHAPE
    assert qc(wsb=16) == WORKSPACE
    assert lib.fs4_quantize_clipped_workspace_bytes(64, 64) > lib.fs4_quantize_workspace_bytes(64, 64)


def test_vstate_validation():
    enc = lambda R=64, C=48, v=A16, q="ok", mu=A16 * 3, wsb=1 << 30: lib.fs4_vstate_encode(
        v, R, C, ctypes.byref(view(R, C) if q == "ok" else q), mu, A16 * 16, wsb, None)
    assert enc(R=40) == SHAPE
    assert enc(C=0) == SHAPE
    assert enc(v=None) == NULL
    assert enc(v=A16 + 4) == ALIGN
    assert enc(q=view(64, 32)) == SHAPE
    assert enc(mu=None) == NULL
    assert enc(wsb=64) == WORKSPACE
    dec = lambda R=64, C=48, out=A16 * 5, mu=A16 * 3: lib.fs4_vstate_decode(
        ctypes.byref(view(R, C)), mu, R, C, out, None)
    assert dec(R=17) == SHAPE
    assert dec(out=None) == NULL
    assert dec(mu=A16 + 2) == ALIGN
    assert lib.fs4_vstate_encode_workspace_bytes(8192, 3072) >= 8192 * 3072 * 4
    assert lib.fs4_vstate_encode_workspace_bytes(8192, 3070) == 0


def test_mstate_validation():
    enc = lambda R=64, C=48, m=A16, rnd=A16 * 2, q="ok", wsb=1 << 30: lib.fs4_mstate_encode(
        m, rnd, R, C, ctypes.byref(view(R, C) if q == "ok" else q), A16 * 16, wsb, None)
    assert enc(R=8) == SHAPE
    assert enc(m=None) == NULL
    assert enc(rnd=None) == NULL
    assert enc(rnd=A16 + 4) == ALIGN
    assert enc(q=view(64, 16)) == SHAPE
    assert enc(wsb=4) == WORKSPACE
    assert lib.fs4_mstate_decode(ctypes.byref(view(64, 48)), 64, 48, None, None) == NULL
    assert lib.fs4_mstate_decode(ctypes.byref(view(64, 48)), 64, 40, A16, None) == SHAPE


# ---- the Python binding checks every tensor before calling the library ----------
torch = pytest.importorskip("torch")


def _cpu_view(rows, cols, dtype=None):
    return fs4.NVFP4(torch.zeros((rows, cols // 2), dtype=dtype or torch.uint8),
                     torch.zeros((rows, cols // 16), dtype=dtype or torch.uint8),
                     torch.zeros(1), rows, cols)


@pytest.mark.parametrize("call,exc,match", [
    # wrong dtypes
    (lambda: fs4.quantize(torch.zeros((64, 64), dtype=torch.float16)), TypeError, "x must have dtype"),
    (lambda: fs4.quantize(torch.zeros((64, 64), dtype=torch.int32)), TypeError, "x must have dtype"),
    (lambda: fs4.mstate_encode(torch.zeros((64, 64), dtype=torch.bfloat16),
                               torch.zeros((64, 64), dtype=torch.int32)), TypeError, "m must have dtype"),
    (lambda: fs4.vstate_encode(torch.zeros((64, 64), dtype=torch.float64)), TypeError, "v must have dtype"),
    (lambda: fs4.linear_fwd(torch.zeros((64, 64)), _cpu_view(32, 64), None, None), TypeError, "X must have dtype"),
    (lambda: fs4.gemm_nt(_cpu_view(64, 64, torch.int8), _cpu_view(32, 64)), TypeError, "A.codes must have dtype"),
    # wrong shapes
    (lambda: fs4.quantize(torch.zeros(64, dtype=torch.bfloat16)), ValueError, "x must be 2-D"),
    (lambda: fs4.linear_fwd(torch.zeros((64, 64), dtype=torch.bfloat16), _cpu_view(32, 48), None, None),
     ValueError, "must be on a CUDA device|R_row must be a"),
    (lambda: fs4.vstate_decode(_cpu_view(64, 64), torch.zeros((4, 3), dtype=torch.bfloat16)), ValueError,
     "q.codes must be on a CUDA device"),
    # a view whose tensors disagree with its rows/cols
    (lambda: fs4.gemm_nt(fs4.NVFP4(torch.zeros((64, 16), dtype=torch.uint8), torch.zeros((64, 4), dtype=torch.uint8),
                                   torch.zeros(1), 64, 64), _cpu_view(32, 64)), ValueError,
     r"A.codes must have shape \(64, 32\)"),
    (lambda: fs4.gemm_nt(_cpu_view(64, 40), _cpu_view(32, 40)), ValueError, "cols must be a non-negative multiple"),
    # non-contiguous
    (lambda: fs4.quantize(torch.zeros((64, 128), dtype=torch.bfloat16)[:, ::2]), ValueError, "x must be contiguous"),
    # right dtypes and shapes, but host memory
    (lambda: fs4.quantize(torch.zeros((64, 64), dtype=torch.bfloat16)), ValueError, "x must be on a CUDA device"),
    (lambda: fs4.mstate_encode(torch.zeros((64, 64)), torch.zeros((64, 64), dtype=torch.int32)), ValueError,
     "m must be on a CUDA device"),
    (lambda: fs4.abs_quantile(torch.zeros(100), 0.99), ValueError, "x must be on a CUDA device"),
    (lambda: fs4.newton_schulz(torch.zeros((64, 128), dtype=torch.bfloat16)), ValueError, "G must be on a CUDA"),
])
def test_binding_rejects_bad_tensors_before_calling_the_library(call, exc, match):
    """Host tensors can only reach the first argument's device check; the
    checks of later arguments against the first are exercised on the GPU
    (tests/test_gpu_binding.py)."""
    with pytest.raises(exc, match=match):
        call()


def test_tensor_check_order_dtype_shape_layout_device():
    """One argument's checks in order: dtype, shape, contiguity, device."""
    chk = fs4._tensor
    with pytest.raises(TypeError):
        chk(torch.zeros((4, 4), dtype=torch.float64), "t", (torch.float32,), (4, 4))
    with pytest.raises(ValueError, match="shape"):
        chk(torch.zeros((4, 5)), "t", (torch.float32,), (4, 4))
    with pytest.raises(ValueError, match="contiguous"):
        chk(torch.zeros((4, 8))[:, ::2], "t", (torch.float32,), (4, 4))
    with pytest.raises(ValueError, match="CUDA"):
        chk(torch.zeros((4, 4)), "t", (torch.float32,), (4, 4))
    with pytest.raises(TypeError, match="torch.Tensor"):
        chk(None, "t", (torch.float32,))


def test_binding_rejects_mismatched_factor_shapes():
    X = torch.zeros((64, 64), dtype=torch.bfloat16)
    U = torch.zeros((32, 8), dtype=torch.bfloat16)
    V = torch.zeros((4, 64), dtype=torch.bfloat16)     # rank disagrees with U
    with pytest.raises(ValueError):
        fs4.linear_fwd(X, _cpu_view(32, 64), U, V)
    with pytest.raises(ValueError):
        fs4.linear_fwd(X, _cpu_view(32, 64), U, None)


def test_quantize_noalloc_validation():
    """The no-workspace quantizer checks its arguments as fs4_quantize does,
    on the host, before it touches the device."""
    f = lambda x=A16, dt=0, rows=64, cols=64, rv="ok", cv="ok": lib.fs4_quantize_noalloc(
        x, dt, rows, cols, ctypes.byref(view(rows, cols)) if rv == "ok" else rv,
        ctypes.byref(view(cols, rows)) if cv == "ok" else cv, None)
    assert f(dt=7) == DTYPE
    assert f(rows=-16) == SHAPE
    assert f(rv=None, cv=None) == NULL
    assert f(x=None) == NULL
    assert f(x=A16 + 4) == ALIGN
    assert f(cols=40, cv=None) == SHAPE
    assert lib.fs4_quantize_noalloc_scratch_bytes() >= lib.fs4_quantize_workspace_bytes(64, 64)


def test_ns_shape_coefficients_match_the_oracle():
    """The library's shape-dependent Newton-Schulz coefficients (host code:
    its own Marchenko-Pastur quadrature and Nelder-Mead) agree with the
    oracle's (scipy) to 1e-5, and so do the minimised distances."""
    import numpy as np
    from oracle.newton_schulz import polar_distance, shape_coefficients
    for m, n in [(3072, 8192), (768, 2048), (192, 512), (1024, 1024), (8192, 3072)]:
        abc, d = fs4.ns_shape_coefficients(m, n)
        want = shape_coefficients(m, n)
        assert np.allclose(abc, want, rtol=1e-5, atol=1e-6), (m, n, abc, want)
        assert abs(d / polar_distance(want, min(m, n), max(m, n)) - 1.0) < 1e-4
    out = (ctypes.c_float * 3)()
    assert lib.fs4_ns_shape_coefficients(0, 16, 5, out, None) == ARG
    assert lib.fs4_ns_shape_coefficients(16, 16, 0, out, None) == ARG
    assert lib.fs4_ns_shape_coefficients(16, 16, 5, None, None) == NULL


def afwd(G=2, S=64, D=128, qr="ok", kr="ok", V=A16, O=A16 * 2, LSE=A16 * 3, Vt=A16 * 4, wsb=0):
    qv = view(G * S, D) if qr == "ok" else qr
    kv = view(G * S, D) if kr == "ok" else kr
    return lib.fs4_attention_fwd(ctypes.byref(qv) if qv is not None else None,
                                 ctypes.byref(kv) if kv is not None else None, V, G, S, D, 1, O, LSE, Vt,
                                 A16 * 16 if wsb else None, wsb, None)


def test_attention_fwd_validation():
    assert afwd(D=96) == SHAPE
    assert afwd(S=40) == SHAPE
    assert afwd(G=0) == SHAPE
    assert afwd(qr=view(2 * 64, 64)) == SHAPE
    assert afwd(kr=None) == NULL
    assert afwd(V=None) == NULL
    assert afwd(O=A16 + 8) == ALIGN
    assert afwd(LSE=A16 + 2) == ALIGN
    assert afwd(Vt=A16 + 8) == ALIGN
    # V^T is an optional side output and there is no workspace
    assert lib.fs4_attention_fwd_workspace_bytes(2, 64, 128) == 0
    assert lib.fs4_attention_fwd_workspace_bytes(2, 64, 96) == 0


def abwd(G=2, S=64, D=128, qr="ok", kr="ok", qc="ok", kc="ok", V=A16, dO=A16 * 2, O=A16 * 3, LSE=A16 * 4,
         dQ=A16 * 5, dK=A16 * 6, dV=A16 * 7, dS=None, wsb=1 << 30):
    views = []
    for v, shape in ((qr, (G * S, D)), (kr, (G * S, D)), (qc, (D, G * S)), (kc, (D, G * S))):
        views.append(view(*shape) if v == "ok" else v)
    refs = [ctypes.byref(v) if v is not None else None for v in views]
    return lib.fs4_attention_bwd(*refs, V, dO, O, LSE, G, S, D, 1, dQ, dK, dV, dS, A16 * 256, wsb, None)


def test_attention_bwd_validation():
    assert abwd(D=32) == SHAPE
    assert abwd(S=24) == SHAPE
    assert abwd(G=0) == SHAPE
    assert abwd(G=1 << 12, S=1 << 10) == SHAPE              # G S^2 = 2^32 elements of dS
    assert abwd(qc=view(128, 2 * 64 + 16)) == SHAPE
    assert abwd(S=96, kc=view(2 * 96, 128)) == SHAPE         # K's row view where its column view goes
    assert abwd(qr=None) == NULL
    assert abwd(dO=None) == NULL
    assert abwd(LSE=None) == NULL
    assert abwd(dV=A16 + 4) == ALIGN
    assert abwd(dS=A16 + 8) == ALIGN
    assert abwd(wsb=1024) == WORKSPACE
    need = lib.fs4_attention_bwd_workspace_bytes(2, 64, 128)
    assert need >= 2 * (2 * 64 * 64 * 9 // 16)   # at least dS's two NVFP4 views
    assert abwd(wsb=need - 1) == WORKSPACE
    assert lib.fs4_attention_bwd_workspace_bytes(2, 64, 96) == 0
    assert lib.fs4_attention_bwd_workspace_bytes(1 << 12, 1 << 10, 128) == 0
