"""Python binding of libfs4, the MI355X (gfx950) NVFP4 linear-projection
library of Full-Stack FP4.

Argument marshalling only: every step of the path runs in the HIP kernels of
libfs4.so.  PyTorch provides device memory and the current stream.  The
library must have been built (``python precision_pretraining_amd/build.py``);
importing this package without it raises ImportError.

Names follow the C ABI in include/fs4.h:

    quantize(x, rowwise=True, colwise=True)   -> (row view, col view)
    gemm_nt(A, B, alpha, E, beta_e)           -> C
    linear_fwd(X, R_row, U, V, beta)          -> LinearFwd(Y, T, X_col)
    linear_bwd(dY, X, X_col, R_col, U, V, T)  -> LinearBwd(dX, dW, dU, dV)
    newton_schulz(G, steps, abc, ...)         -> X (and traces)
    lora_project(U, V, dU, dV)                -> (dU, dV) projected in place
    lora_realign(U, V, R, Omega, ...)         -> sigma; U, V, R realigned in place
    vstate_encode(v) / vstate_decode(q, mu)   -> the Q-AdamW second-moment codec
    mstate_encode(m, rnd) / mstate_decode(q)  -> the Q-AdamW first-moment codec
"""
from __future__ import annotations

import atexit
import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfs4.so")

if not os.path.exists(LIB_PATH):
    raise ImportError("libfs4.so is not built; run `python precision_pretraining_amd/build.py` "
                      "(expected at %s)" % LIB_PATH)

_lib = ctypes.CDLL(LIB_PATH)

FS4_BF16, FS4_FP32 = 0, 1
FS4_OP_QUANTIZE, FS4_OP_GEMM, FS4_OP_LINEAR_FWD, FS4_OP_LINEAR_BWD, FS4_OP_NS, FS4_OP_LORA_PROJECT, \
    FS4_OP_LORA_REALIGN = range(7)
MUON_ABC = (3.4445, -4.7750, 2.0315)

EXPORTS = [
    "fs4_quantize_workspace_bytes", "fs4_quantize", "fs4_gemm_workspace_bytes", "fs4_gemm_nt",
    "fs4_linear_fwd_workspace_bytes", "fs4_linear_fwd", "fs4_linear_bwd_workspace_bytes",
    "fs4_linear_bwd", "fs4_newton_schulz_workspace_bytes", "fs4_newton_schulz",
    "fs4_lora_project_workspace_bytes", "fs4_lora_project",
    "fs4_lora_realign_workspace_bytes", "fs4_lora_realign",
    "fs4_abs_quantile_workspace_bytes", "fs4_abs_quantile",
    "fs4_quantize_clipped_workspace_bytes", "fs4_quantize_clipped",
    "fs4_vstate_encode_workspace_bytes", "fs4_vstate_encode", "fs4_vstate_decode",
    "fs4_mstate_encode_workspace_bytes", "fs4_mstate_encode", "fs4_mstate_decode",
    "fs4_workspace_bytes", "fs4_status_str", "fs4_version", "fs4_gemm_plan", "fs4_newton_schulz_plan",
    "fs4_quantize_noalloc", "fs4_quantize_noalloc_scratch_bytes", "fs4_ns_shape_coefficients",
    "fs4_attention_fwd_workspace_bytes", "fs4_attention_fwd",
    "fs4_attention_bwd_workspace_bytes", "fs4_attention_bwd",
]


class _View(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("tscale", ctypes.c_void_p),
                ("rows", ctypes.c_int64), ("cols", ctypes.c_int64)]


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_F = ctypes.c_float
_SZ = ctypes.c_size_t
_VP = ctypes.POINTER(_View)


def _sig(name, res, args):
    try:
        f = getattr(_lib, name)
    except AttributeError as e:
        raise ImportError("%s does not export %s: the library is older than this binding; rebuild it "
                          "with `python precision_pretraining_amd/build.py`" % (LIB_PATH, name)) from e
    f.restype = res
    f.argtypes = args
    return f


_sig("fs4_status_str", ctypes.c_char_p, [ctypes.c_int])
_sig("fs4_version", ctypes.c_char_p, [])
_sig("fs4_workspace_bytes", _SZ, [ctypes.c_int, _I64, _I64, _I64, ctypes.c_int])
_sig("fs4_quantize_workspace_bytes", _SZ, [_I64, _I64])
_sig("fs4_quantize", ctypes.c_int, [_P, ctypes.c_int, _I64, _I64, _VP, _VP, _P, _SZ, _P])
_sig("fs4_quantize_noalloc", ctypes.c_int, [_P, ctypes.c_int, _I64, _I64, _VP, _VP, _P])
_sig("fs4_quantize_noalloc_scratch_bytes", _SZ, [])
_sig("fs4_gemm_workspace_bytes", _SZ, [_I64, _I64, _I64])
_sig("fs4_gemm_nt", ctypes.c_int, [_VP, _VP, _F, _P, _F, _P, _P, _SZ, _P])
_sig("fs4_linear_fwd_workspace_bytes", _SZ, [_I64, _I64, _I64, ctypes.c_int])
_sig("fs4_linear_fwd", ctypes.c_int, [_P, _I64, _I64, _VP, _P, _P, ctypes.c_int, _F, _P, _P, _VP,
                                      _P, _SZ, _P])
_sig("fs4_linear_bwd_workspace_bytes", _SZ, [_I64, _I64, _I64, ctypes.c_int])
_sig("fs4_linear_bwd", ctypes.c_int, [_P, _I64, _I64, _I64, _P, _VP, _VP, _P, _P, ctypes.c_int, _F,
                                      _P, _P, _P, _P, _P, _P, _SZ, _P])
_sig("fs4_newton_schulz_workspace_bytes", _SZ, [_I64, _I64])
_sig("fs4_vstate_encode_workspace_bytes", _SZ, [_I64, _I64])
_sig("fs4_vstate_encode", ctypes.c_int, [_P, _I64, _I64, _VP, _P, _P, _SZ, _P])
_sig("fs4_vstate_decode", ctypes.c_int, [_VP, _P, _I64, _I64, _P, _P])
_sig("fs4_mstate_encode_workspace_bytes", _SZ, [_I64, _I64])
_sig("fs4_mstate_encode", ctypes.c_int, [_P, _P, _I64, _I64, _VP, _P, _SZ, _P])
_sig("fs4_mstate_decode", ctypes.c_int, [_VP, _I64, _I64, _P, _P])
_sig("fs4_lora_project_workspace_bytes", _SZ, [_I64, _I64, ctypes.c_int])
_sig("fs4_lora_project", ctypes.c_int, [_P, _P, _I64, _I64, ctypes.c_int, _P, _P, _P, _SZ, _P])
_sig("fs4_lora_realign_workspace_bytes", _SZ, [_I64, _I64, ctypes.c_int])
_sig("fs4_lora_realign", ctypes.c_int, [_P, _P, _P, _I64, _I64, ctypes.c_int, _F, _P, ctypes.c_int,
                                        ctypes.c_int, _P, _P, _SZ, _P])
_sig("fs4_newton_schulz", ctypes.c_int, [_P, ctypes.c_int, _I64, _I64, ctypes.c_int, _F, _F, _F,
                                         ctypes.c_int, _F, ctypes.c_double, _P, _P, _P, _P, _P, _SZ, _P])
_sig("fs4_abs_quantile_workspace_bytes", _SZ, [_I64])
_sig("fs4_abs_quantile", ctypes.c_int, [_P, ctypes.c_int, _I64, ctypes.c_double, _P, _P, _SZ, _P])
_sig("fs4_gemm_plan", ctypes.c_int, [_I64, _I64, _I64, ctypes.POINTER(_I64)])
_sig("fs4_ns_shape_coefficients", ctypes.c_int, [_I64, _I64, ctypes.c_int, ctypes.POINTER(_F),
                                                 ctypes.POINTER(ctypes.c_double)])
_sig("fs4_newton_schulz_plan", ctypes.c_int, [_I64, _I64, ctypes.POINTER(_I64)])
_sig("fs4_attention_fwd_workspace_bytes", _SZ, [_I64, _I64, _I64])
_sig("fs4_attention_fwd", ctypes.c_int, [_VP, _VP, _P, _I64, _I64, _I64, ctypes.c_int, _P, _P, _P, _P, _SZ, _P])
_sig("fs4_attention_bwd_workspace_bytes", _SZ, [_I64, _I64, _I64])
_sig("fs4_attention_bwd", ctypes.c_int, [_VP, _VP, _VP, _VP, _P, _P, _P, _P, _I64, _I64, _I64, ctypes.c_int,
                                         _P, _P, _P, _P, _P, _SZ, _P])
_sig("fs4_quantize_clipped_workspace_bytes", _SZ, [_I64, _I64])
_sig("fs4_quantize_clipped", ctypes.c_int, [_P, ctypes.c_int, _I64, _I64, ctypes.c_double, _VP, _VP, _P,
                                            _SZ, _P])


class FS4Error(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        super().__init__("%s: %s" % (call, _lib.fs4_status_str(status).decode()))


def _check(st: int, call: str):
    if st != 0:
        raise FS4Error(st, call)


def version() -> str:
    return _lib.fs4_version().decode()


def status_str(st: int) -> str:
    return _lib.fs4_status_str(st).decode()


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


# ---- argument checks ------------------------------------------------------------
# The C ABI sees raw device pointers and the sizes passed beside them, never
# the buffers' extents: a tensor of the wrong dtype or shape would make a
# kernel read or write past its allocation.  Every tensor is therefore checked
# here, before any call into the library.

_U32_LIKE = (torch.int32, torch.uint32) if hasattr(torch, "uint32") else (torch.int32,)


def _tensor(t, name: str, dtypes, shape=None, device=None) -> torch.Tensor:
    """Checks one tensor argument: dtype, exact shape, contiguity, a CUDA
    device (the same one as ``device`` when given)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor, got %s" % (name, type(t).__name__))
    if t.dtype not in dtypes:
        raise TypeError("%s must have dtype %s, got %s" % (name, " or ".join(str(d) for d in dtypes), t.dtype))
    if shape is not None and tuple(t.shape) != tuple(int(d) for d in shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(int(d) for d in shape), tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be on a CUDA device, got %s" % (name, t.device))
    if device is not None and t.device != torch.device(device):
        raise ValueError("%s is on %s, the call runs on %s" % (name, t.device, device))
    return t


def _opt_tensor(t, name, dtypes, shape, device):
    return None if t is None else _tensor(t, name, dtypes, shape, device)


def _matrix(t, name: str, dtypes, device=None):
    """A 2-D tensor of any shape; returns (rows, cols)."""
    if isinstance(t, torch.Tensor) and t.dim() != 2:
        raise ValueError("%s must be 2-D, got %d dimensions" % (name, t.dim()))
    _tensor(t, name, dtypes, None, device)
    return int(t.shape[0]), int(t.shape[1])


def _view(v, name: str, rows=None, cols=None, device=None):
    """Checks an NVFP4 view's three tensors against its rows/cols (and the
    expected rows/cols when given)."""
    if not isinstance(v, NVFP4):
        raise TypeError("%s must be an NVFP4 view, got %s" % (name, type(v).__name__))
    if rows is not None and v.rows != rows or cols is not None and v.cols != cols:
        raise ValueError("%s must be a %s x %s view, got %d x %d" % (name, rows, cols, v.rows, v.cols))
    if v.rows < 0 or v.cols < 0 or v.cols % 16:
        raise ValueError("%s: cols must be a non-negative multiple of 16, got %d x %d" % (name, v.rows, v.cols))
    empty = v.rows == 0 or v.cols == 0     # nothing is read or written but the tensor scale
    _tensor(v.codes, name + ".codes", (torch.uint8,), None if empty else (v.rows, v.cols // 2), device)
    _tensor(v.scales, name + ".scales", (torch.uint8,), None if empty else (v.rows, v.cols // 16), device)
    _tensor(v.tscale, name + ".tscale", (torch.float32,), None, v.codes.device)
    if v.tscale.numel() < 1:
        raise ValueError("%s.tscale must hold one float" % name)
    return v


_BF16 = (torch.bfloat16,)
_F32 = (torch.float32,)
_FLOAT = (torch.bfloat16, torch.float32)


_WS = {}


def _workspace(nbytes: int, device) -> torch.Tensor:
    """A cached device workspace (reused by calls ordered on one stream)."""
    key = (str(device), torch.cuda.current_stream(device).cuda_stream)
    ws = _WS.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        _WS[key] = ws
    return ws


def release_workspaces() -> None:
    """Waits for the work queued on the cached workspaces' devices, then
    drops the workspaces and returns torch's cached device memory.  Runs at
    interpreter exit, so that every device buffer is released while the HIP
    runtime (and any profiler attached to it) is still up, rather than during
    the C-level teardown that follows."""
    if not _WS:
        return
    devices = {k[0] for k in _WS}
    try:
        for d in devices:
            torch.cuda.synchronize(torch.device(d))
    finally:
        _WS.clear()
        try:
            torch.cuda.empty_cache()
        except RuntimeError:
            pass


atexit.register(release_workspaces)


@dataclass
class NVFP4:
    """One NVFP4 view on the device: codes [rows, cols/2] uint8, scales
    [rows, cols/16] uint8 (E4M3FN), tscale [1] float32; cols is the blocked
    (contraction) dimension."""
    codes: torch.Tensor
    scales: torch.Tensor
    tscale: torch.Tensor
    rows: int
    cols: int

    @staticmethod
    def empty(rows: int, cols: int, device, tscale: Optional[torch.Tensor] = None) -> "NVFP4":
        codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=device)
        scales = torch.empty((rows, cols // 16), dtype=torch.uint8, device=device)
        ts = tscale if tscale is not None else torch.empty(1, dtype=torch.float32, device=device)
        return NVFP4(codes, scales, ts, rows, cols)

    def c(self) -> _View:
        return _View(self.codes.data_ptr(), self.scales.data_ptr(), self.tscale.data_ptr(),
                     self.rows, self.cols)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return FS4_BF16
    if t.dtype == torch.float32:
        return FS4_FP32
    raise TypeError("fs4 takes bfloat16 or float32 tensors, got %s" % t.dtype)


def quantize(x: torch.Tensor, rowwise: bool = True, colwise: bool = True, out_row: Optional[NVFP4] = None,
             out_col: Optional[NVFP4] = None):
    """NVFP4-quantize a 2-D bf16/fp32 CUDA tensor; returns (row view, col view)
    (None for a layout not asked for).  Both views share one tscale tensor."""
    rows, cols = _matrix(x, "x", _FLOAT)
    dev = x.device
    ts = None
    if rowwise and out_row is None:
        out_row = NVFP4.empty(rows, cols, dev)
        ts = out_row.tscale
    if colwise and out_col is None:
        out_col = NVFP4.empty(cols, rows, dev, ts)
    if rowwise:
        _view(out_row, "out_row", rows, cols, dev)
    if colwise:
        _view(out_col, "out_col", cols, rows, dev)
    rv = out_row.c() if rowwise else None
    cv = out_col.c() if colwise else None
    nbytes = _lib.fs4_quantize_workspace_bytes(rows, cols)
    ws = _workspace(nbytes, dev)
    _check(_lib.fs4_quantize(x.data_ptr(), _dtype_code(x), rows, cols,
                             ctypes.byref(rv) if rv is not None else None,
                             ctypes.byref(cv) if cv is not None else None,
                             ws.data_ptr(), ws.numel(), _stream(dev)), "fs4_quantize")
    return (out_row if rowwise else None), (out_col if colwise else None)


def quantize_noalloc(x: torch.Tensor, out_row: Optional[NVFP4], out_col: Optional[NVFP4]):
    """quantize() into caller-given views with no workspace: the library's
    own per-device scratch array serves (calls that overlap on one GPU
    race).  Neither the binding nor the library allocates."""
    rows, cols = _matrix(x, "x", _FLOAT)
    dev = x.device
    if out_row is None and out_col is None:
        raise ValueError("quantize_noalloc needs at least one output view")
    if out_row is not None:
        _view(out_row, "out_row", rows, cols, dev)
    if out_col is not None:
        _view(out_col, "out_col", cols, rows, dev)
    rv = out_row.c() if out_row is not None else None
    cv = out_col.c() if out_col is not None else None
    _check(_lib.fs4_quantize_noalloc(x.data_ptr(), _dtype_code(x), rows, cols,
                                     ctypes.byref(rv) if rv is not None else None,
                                     ctypes.byref(cv) if cv is not None else None, _stream(dev)),
           "fs4_quantize_noalloc")
    return out_row, out_col


def gemm_nt(A: NVFP4, B: NVFP4, alpha: float = 1.0, E: Optional[torch.Tensor] = None, beta_e: float = 0.0,
            out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """C = alpha s_tA s_tB A_hat B_hat^T + beta_e E (fp32 [A.rows, B.rows])."""
    _view(A, "A")
    dev = A.codes.device
    _view(B, "B", None, A.cols, dev)
    _opt_tensor(E, "E", _F32, (A.rows, B.rows), dev)
    C = out if out is not None else torch.empty((A.rows, B.rows), dtype=torch.float32, device=dev)
    _tensor(C, "out", _F32, (A.rows, B.rows), dev)
    av, bv = A.c(), B.c()
    _check(_lib.fs4_gemm_nt(ctypes.byref(av), ctypes.byref(bv), alpha, _ptr(E), beta_e, C.data_ptr(),
                            None, 0, _stream(dev)), "fs4_gemm_nt")
    return C


@dataclass
class LinearFwd:
    Y: torch.Tensor
    T: Optional[torch.Tensor]
    X_col: Optional[NVFP4]


def linear_fwd(X: torch.Tensor, R_row: NVFP4, U: Optional[torch.Tensor], V: Optional[torch.Tensor],
               beta: float = 1.0, save_for_backward: bool = True, out: Optional[torch.Tensor] = None) -> LinearFwd:
    """Y = Q(X) Q(R)^T + beta (X V^T) U^T.  X bf16 [M, K]; U bf16 [N, r]; V bf16 [r, K]."""
    M, K = _matrix(X, "X", _BF16)
    dev = X.device
    _view(R_row, "R_row", None, K, dev)
    N = R_row.rows
    if (U is None) != (V is None):
        raise ValueError("U and V are given together or not at all")
    r = 0
    if U is not None:
        r = _matrix(U, "U", _BF16, dev)[1]
        _tensor(U, "U", _BF16, (N, r), dev)
        _tensor(V, "V", _BF16, (r, K), dev)
    Y = out if out is not None else torch.empty((M, N), dtype=torch.float32, device=dev)
    _tensor(Y, "out", _F32, (M, N), dev)
    T = torch.empty((M, r), dtype=torch.float32, device=dev) if (save_for_backward and r > 0) else None
    X_col = NVFP4.empty(K, M, dev) if save_for_backward else None
    rv = R_row.c()
    xc = X_col.c() if X_col is not None else None
    nbytes = _lib.fs4_linear_fwd_workspace_bytes(M, K, N, r)
    ws = _workspace(nbytes, dev)
    _check(_lib.fs4_linear_fwd(X.data_ptr(), M, K, ctypes.byref(rv), _ptr(U), _ptr(V), r, beta,
                               Y.data_ptr(), _ptr(T), ctypes.byref(xc) if xc is not None else None,
                               ws.data_ptr(), ws.numel(), _stream(dev)), "fs4_linear_fwd")
    return LinearFwd(Y, T, X_col)


@dataclass
class LinearBwd:
    dX: torch.Tensor
    dW: torch.Tensor
    dU: Optional[torch.Tensor]
    dV: Optional[torch.Tensor]


def linear_bwd(dY: torch.Tensor, X: Optional[torch.Tensor], X_col: NVFP4, R_col: NVFP4,
               U: Optional[torch.Tensor], V: Optional[torch.Tensor], T: Optional[torch.Tensor],
               beta: float = 1.0, need_factor_grads: bool = True) -> LinearBwd:
    """dX = Q(dY) Q(R^T)^T + beta (dY U) V; dW = Q(dY^T) Q(X^T)^T;
    dU = beta dY^T T; dV = beta (dY U)^T X."""
    M, N = _matrix(dY, "dY", _BF16)
    dev = dY.device
    _view(X_col, "X_col", None, M, dev)
    K = X_col.rows
    _view(R_col, "R_col", K, N, dev)
    if (U is None) != (V is None):
        raise ValueError("U and V are given together or not at all")
    r = 0
    if U is not None:
        r = _matrix(U, "U", _BF16, dev)[1]
        _tensor(U, "U", _BF16, (N, r), dev)
        _tensor(V, "V", _BF16, (r, K), dev)
        _tensor(T, "T", _F32, (M, r), dev)
    if X is not None or (r > 0 and need_factor_grads):
        _tensor(X, "X", _BF16, (M, K), dev)
    dX = torch.empty((M, K), dtype=torch.float32, device=dev)
    dW = torch.empty((N, K), dtype=torch.float32, device=dev)
    dU = torch.empty((N, r), dtype=torch.float32, device=dev) if (need_factor_grads and r > 0) else None
    dV = torch.empty((r, K), dtype=torch.float32, device=dev) if (need_factor_grads and r > 0) else None
    xc, rc = X_col.c(), R_col.c()
    nbytes = _lib.fs4_linear_bwd_workspace_bytes(M, N, K, r)
    ws = _workspace(nbytes, dev)
    _check(_lib.fs4_linear_bwd(dY.data_ptr(), M, N, K, _ptr(X), ctypes.byref(xc), ctypes.byref(rc),
                               _ptr(U), _ptr(V), r, beta, _ptr(T), dX.data_ptr(), dW.data_ptr(),
                               _ptr(dU), _ptr(dV), ws.data_ptr(), ws.numel(), _stream(dev)),
           "fs4_linear_bwd")
    return LinearBwd(dX, dW, dU, dV)


def newton_schulz(G: torch.Tensor, steps: int = 5, abc=MUON_ABC, normalize: bool = True, eps: float = 1e-7,
                  trace: bool = False, out: Optional[torch.Tensor] = None, clip_q: float = 0.0):
    """NVFP4 Newton-Schulz on G [m, n] (m <= n).  Returns X, or with
    trace=True (X, trace_X [steps+1, m, n], trace_A [steps, m, m],
    trace_B [steps, m, m]).  clip_q (e.g. 0.99): clip each quantized copy
    of the iterate at that quantile of its magnitudes (0: off)."""
    m, n = _matrix(G, "G", _FLOAT)
    dev = G.device
    X = out if out is not None else torch.empty((m, n), dtype=torch.float32, device=dev)
    _tensor(X, "out", _F32, (m, n), dev)
    tX = torch.empty((steps + 1, m, n), dtype=torch.float32, device=dev) if trace else None
    tA = torch.empty((max(steps, 1), m, m), dtype=torch.float32, device=dev) if trace else None
    tB = torch.empty((max(steps, 1), m, m), dtype=torch.float32, device=dev) if trace else None
    a, b, c = abc
    nbytes = _lib.fs4_newton_schulz_workspace_bytes(m, n)
    ws = _workspace(nbytes, dev)
    _check(_lib.fs4_newton_schulz(G.data_ptr(), _dtype_code(G), m, n, steps, a, b, c, int(normalize), eps,
                                  clip_q, X.data_ptr(), _ptr(tX), _ptr(tA), _ptr(tB), ws.data_ptr(), ws.numel(),
                                  _stream(dev)), "fs4_newton_schulz")
    if trace:
        return X, tX, tA, tB
    return X


def lora_project(U: torch.Tensor, V: torch.Tensor, dU: Optional[torch.Tensor] = None,
                 dV: Optional[torch.Tensor] = None):
    """Projects the rank-r gradients in place onto the branch's subspace:
    dU <- Q_U Q_U^T dU, dV <- dV Q_V Q_V^T (Q_U = CholQR(U), Q_V = CholQR(V^T)).
    U bf16 [N, r], V bf16 [r, K]; dU fp32 [N, r], dV fp32 [r, K] (either may
    be None).  Returns (dU, dV)."""
    N, r = _matrix(U, "U", _BF16)
    dev = U.device
    K = _matrix(V, "V", _BF16, dev)[1]
    _tensor(V, "V", _BF16, (r, K), dev)
    _opt_tensor(dU, "dU", _F32, (N, r), dev)
    _opt_tensor(dV, "dV", _F32, (r, K), dev)
    nbytes = _lib.fs4_lora_project_workspace_bytes(N, K, r)
    ws = _workspace(nbytes, dev)
    _check(_lib.fs4_lora_project(U.data_ptr(), V.data_ptr(), N, K, r, _ptr(dU), _ptr(dV), ws.data_ptr(),
                                 ws.numel(), _stream(dev)), "fs4_lora_project")
    return dU, dV


def lora_realign(U: torch.Tensor, V: torch.Tensor, R: torch.Tensor, Omega: torch.Tensor,
                 beta: float = 1.0, power_iters: int = 1) -> torch.Tensor:
    """Randomized-SVD realignment of W = beta U V + R, in place: U bf16
    [N, r], V bf16 [r, K], R fp32 [N, K]; Omega fp32 [l, K] Gaussian test
    vectors (r <= l <= 64).  Returns sigma, the r leading singular values."""
    N, r = _matrix(U, "U", _BF16)
    dev = U.device
    K = _matrix(V, "V", _BF16, dev)[1]
    _tensor(V, "V", _BF16, (r, K), dev)
    _tensor(R, "R", _F32, (N, K), dev)
    l = _matrix(Omega, "Omega", _F32, dev)[0]
    _tensor(Omega, "Omega", _F32, (l, K), dev)
    sigma = torch.empty(r, dtype=torch.float32, device=dev)
    nbytes = _lib.fs4_lora_realign_workspace_bytes(N, K, l)
    ws = _workspace(nbytes, dev)
    _check(_lib.fs4_lora_realign(U.data_ptr(), V.data_ptr(), R.data_ptr(), N, K, r, beta, Omega.data_ptr(),
                                 l, power_iters, sigma.data_ptr(), ws.data_ptr(), ws.numel(), _stream(dev)),
           "fs4_lora_realign")
    return sigma


def abs_quantile(x: torch.Tensor, q: float) -> torch.Tensor:
    """The nearest-rank q-quantile of |x| (a 1-element fp32 tensor)."""
    _tensor(x, "x", _FLOAT)
    out = torch.empty(1, dtype=torch.float32, device=x.device)
    ws = _workspace(_lib.fs4_abs_quantile_workspace_bytes(x.numel()), x.device)
    _check(_lib.fs4_abs_quantile(x.data_ptr(), _dtype_code(x), x.numel(), q, out.data_ptr(), ws.data_ptr(),
                                 ws.numel(), _stream(x.device)), "fs4_abs_quantile")
    return out


def quantize_clipped(x: torch.Tensor, q: float, rowwise: bool = True, colwise: bool = True):
    """quantize() of x clipped at the nearest-rank q-quantile of |x|."""
    rows, cols = _matrix(x, "x", _FLOAT)
    dev = x.device
    orow = NVFP4.empty(rows, cols, dev) if rowwise else None
    ocol = NVFP4.empty(cols, rows, dev, tscale=orow.tscale if orow is not None else None) if colwise else None
    rv = orow.c() if orow is not None else None
    cv = ocol.c() if ocol is not None else None
    ws = _workspace(_lib.fs4_quantize_clipped_workspace_bytes(rows, cols), dev)
    _check(_lib.fs4_quantize_clipped(x.data_ptr(), _dtype_code(x), rows, cols, q,
                                     ctypes.byref(rv) if rv is not None else None,
                                     ctypes.byref(cv) if cv is not None else None,
                                     ws.data_ptr(), ws.numel(), _stream(dev)), "fs4_quantize_clipped")
    return orow, ocol


def vstate_encode(v: torch.Tensor):
    """Q-AdamW second-moment codec: fp32 v [R, C] -> (NVFP4 view of the
    transformed residual, BF16 tile means [R/16, C/16])."""
    R, C = _matrix(v, "v", _F32)
    dev = v.device
    q = NVFP4.empty(R, C, dev)
    means = torch.empty((R // 16, C // 16), dtype=torch.bfloat16, device=dev)
    qv = q.c()
    ws = _workspace(_lib.fs4_vstate_encode_workspace_bytes(R, C), dev)
    _check(_lib.fs4_vstate_encode(v.data_ptr(), R, C, ctypes.byref(qv), means.data_ptr(), ws.data_ptr(),
                                  ws.numel(), _stream(dev)), "fs4_vstate_encode")
    return q, means


def vstate_decode(q: NVFP4, means: torch.Tensor) -> torch.Tensor:
    """The fp32 second moment back from vstate_encode's outputs."""
    _view(q, "q")
    _tensor(means, "means", _BF16, (q.rows // 16, q.cols // 16), q.codes.device)
    out = torch.empty((q.rows, q.cols), dtype=torch.float32, device=means.device)
    qv = q.c()
    _check(_lib.fs4_vstate_decode(ctypes.byref(qv), means.data_ptr(), q.rows, q.cols, out.data_ptr(),
                                  _stream(means.device)), "fs4_vstate_decode")
    return out


def mstate_encode(m: torch.Tensor, rnd: torch.Tensor) -> NVFP4:
    """Q-AdamW first-moment codec: fp32 m [R, C] and one random 32-bit word
    per element (int32 or uint32 tensor, bits used as given) -> NVFP4 view."""
    R, C = _matrix(m, "m", _F32)
    _tensor(rnd, "rnd", _U32_LIKE, (R, C), m.device)
    dev = m.device
    q = NVFP4.empty(R, C, dev)
    qv = q.c()
    ws = _workspace(_lib.fs4_mstate_encode_workspace_bytes(R, C), dev)
    _check(_lib.fs4_mstate_encode(m.data_ptr(), rnd.data_ptr(), R, C, ctypes.byref(qv), ws.data_ptr(),
                                  ws.numel(), _stream(dev)), "fs4_mstate_encode")
    return q


def mstate_decode(q: NVFP4) -> torch.Tensor:
    _view(q, "q")
    out = torch.empty((q.rows, q.cols), dtype=torch.float32, device=q.codes.device)
    qv = q.c()
    _check(_lib.fs4_mstate_decode(ctypes.byref(qv), q.rows, q.cols, out.data_ptr(), _stream(q.codes.device)),
           "fs4_mstate_decode")
    return out


def gemm_plan(M: int, N: int, K: int) -> dict:
    """The tile plan the GEMM launcher picks for an M x N x K product."""
    out = (_I64 * 4)()
    _check(_lib.fs4_gemm_plan(M, N, K, out), "fs4_gemm_plan")
    return {"tile": (out[0], out[1]), "tiles": out[2], "splits": out[3]}


def ns_shape_coefficients(m: int, n: int, steps: int = 5):
    """Shape-dependent quintic coefficients (a, b, c) for an m x n momentum
    (the Q-Root reading: minimum mean squared distance of `steps` steps to
    the polar factor over the Marchenko-Pastur spectrum), as float32 values
    for newton_schulz(abc=...).  Returns (abc, distance)."""
    abc = (_F * 3)()
    dist = ctypes.c_double()
    _check(_lib.fs4_ns_shape_coefficients(m, n, steps, abc, ctypes.byref(dist)), "fs4_ns_shape_coefficients")
    return (abc[0], abc[1], abc[2]), dist.value


def newton_schulz_plan(m: int, n: int) -> dict:
    """The tile plans of one Newton-Schulz step's products A, A^2 and the
    (transposed) update on an m x n iterate."""
    out = (_I64 * 12)()
    _check(_lib.fs4_newton_schulz_plan(m, n, out), "fs4_newton_schulz_plan")
    return {name: {"tile": (out[4 * i], out[4 * i + 1]), "tiles": out[4 * i + 2], "splits": out[4 * i + 3]}
            for i, name in enumerate(("A", "A2", "update"))}


@dataclass
class AttentionFwd:
    O: torch.Tensor
    LSE: torch.Tensor
    Vt: Optional[torch.Tensor]


def attention_quantize(x: torch.Tensor):
    """The NVFP4 views attention reuses for a BF16 [G, S, D] Q or K: one
    quantization of the [G*S, D] matrix; row-wise (blocks along D) for
    Q K^T, column-wise (blocks along the sequence) for the dS products."""
    if x.dim() != 3:
        raise ValueError("attention_quantize takes a [G, S, D] tensor")
    G, S, D = x.shape
    return quantize(x.reshape(G * S, D))


def attention_fwd(Q_row: NVFP4, K_row: NVFP4, V: torch.Tensor, causal: bool = True,
                  keep_vt: bool = False) -> AttentionFwd:
    """O = softmax(Q K^T / sqrt(D)) V with Q K^T on the NVFP4 views and P V
    in BF16.  V bf16 [G, S, D]; returns O fp32 [G, S, D], LSE fp32 [G, S]
    and, with keep_vt, V^T bf16 [G, D, S] as a side output."""
    if not isinstance(V, torch.Tensor) or V.dim() != 3:
        raise ValueError("V must be a [G, S, D] tensor")
    G, S, D = (int(v) for v in V.shape)
    dev = V.device
    _tensor(V, "V", _BF16, (G, S, D))
    _view(Q_row, "Q_row", G * S, D, dev)
    _view(K_row, "K_row", G * S, D, dev)
    O = torch.empty((G, S, D), dtype=torch.float32, device=dev)
    LSE = torch.empty((G, S), dtype=torch.float32, device=dev)
    Vt = torch.empty((G, D, S), dtype=torch.bfloat16, device=dev) if keep_vt else None
    qv, kv = Q_row.c(), K_row.c()
    _check(_lib.fs4_attention_fwd(ctypes.byref(qv), ctypes.byref(kv), V.data_ptr(), G, S, D, int(causal), O.data_ptr(),
                                  LSE.data_ptr(), _ptr(Vt), None, 0, _stream(dev)), "fs4_attention_fwd")
    return AttentionFwd(O, LSE, Vt)


@dataclass
class AttentionBwd:
    dQ: torch.Tensor
    dK: torch.Tensor
    dV: torch.Tensor
    dS: Optional[torch.Tensor]


def attention_bwd(dO: torch.Tensor, V: torch.Tensor, fwd: AttentionFwd, Q_views, K_views, causal: bool = True,
                  keep_dS: bool = False) -> AttentionBwd:
    """The backward of attention_fwd: dV = P^T dO and dP = dO V^T in BF16,
    dQ and dK on NVFP4 views of dS (one tensor scale over all sequences) and
    the forward's column-wise Q and K views.  dO, V bf16 [G, S, D];
    Q_views, K_views the (row, col) pairs attention_quantize returned; fwd
    the forward's outputs (O and LSE are read).  Returns dQ, dK, dV fp32
    [G, S, D] and, with keep_dS, dS fp32 [G*S, S] before its quantization."""
    if not isinstance(dO, torch.Tensor) or dO.dim() != 3:
        raise ValueError("dO must be a [G, S, D] tensor")
    G, S, D = (int(v) for v in dO.shape)
    dev = dO.device
    _tensor(dO, "dO", _BF16, (G, S, D))
    _tensor(V, "V", _BF16, (G, S, D), dev)
    _tensor(fwd.O, "O", _F32, (G, S, D), dev)
    _tensor(fwd.LSE, "LSE", _F32, (G, S), dev)
    (q_row, q_col), (k_row, k_col) = Q_views, K_views
    _view(q_row, "Q_row", G * S, D, dev)
    _view(k_row, "K_row", G * S, D, dev)
    _view(q_col, "Q_col", D, G * S, dev)
    _view(k_col, "K_col", D, G * S, dev)
    dQ, dK, dV = (torch.empty((G, S, D), dtype=torch.float32, device=dev) for _ in range(3))
    dS = torch.empty((G * S, S), dtype=torch.float32, device=dev) if keep_dS else None
    nbytes = _lib.fs4_attention_bwd_workspace_bytes(G, S, D)
    if nbytes == 0:
        raise ValueError("attention_bwd: unsupported shape G=%d S=%d D=%d" % (G, S, D))
    ws = _workspace(nbytes, dev)
    qr, kr, qc, kc = q_row.c(), k_row.c(), q_col.c(), k_col.c()
    _check(_lib.fs4_attention_bwd(ctypes.byref(qr), ctypes.byref(kr), ctypes.byref(qc), ctypes.byref(kc),
                                  V.data_ptr(), dO.data_ptr(), fwd.O.data_ptr(), fwd.LSE.data_ptr(), G, S, D,
                                  int(causal), dQ.data_ptr(), dK.data_ptr(), dV.data_ptr(), _ptr(dS),
                                  ws.data_ptr(), ws.numel(), _stream(dev)), "fs4_attention_bwd")
    return AttentionBwd(dQ, dK, dV, dS)


def workspace_bytes(op: int, d0: int, d1: int = 0, d2: int = 0, r: int = 0) -> int:
    return _lib.fs4_workspace_bytes(op, d0, d1, d2, r)


__all__ = ["NVFP4", "quantize", "quantize_noalloc", "gemm_nt", "linear_fwd", "LinearFwd", "linear_bwd", "LinearBwd",
           "newton_schulz", "lora_project", "lora_realign", "abs_quantile", "quantize_clipped",
           "vstate_encode", "vstate_decode", "mstate_encode", "mstate_decode", "workspace_bytes", "version", "status_str", "FS4Error", "LIB_PATH",
           "EXPORTS", "MUON_ABC",
           "release_workspaces", "gemm_plan", "newton_schulz_plan", "ns_shape_coefficients",
           "attention_quantize", "attention_fwd", "AttentionFwd", "attention_bwd", "AttentionBwd"]
