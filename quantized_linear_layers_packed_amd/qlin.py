"""ctypes binding of libqlin.so (argument marshalling only).

Every function has the name and argument order of the C entry point declared
in include/qlin.h.  Pointer arguments accept torch tensors (their data_ptr()),
numpy arrays (host pointers) or plain integers; ``stream=None`` means the
current torch stream of the current device.  A non-zero status raises
QlinError carrying the library's message.  The host pack calls additionally
allocate their numpy output arrays (sized by the matching *_sizes call) and
return them.

There is no fallback: if libqlin.so has not been built, importing this module
raises ImportError.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

# PyTorch ships its own HIP runtime.  Loading torch first makes libqlin.so bind to
# that same runtime (same SONAME), so tensors, streams and our kernels share one
# HIP context; loading the system runtime first would give the process two.
try:
    import torch  # noqa: F401
except ImportError:  # host-only use (pack calls) works without torch
    torch = None

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqlin.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with "
                      "`python -m quantized_linear_layers_packed_amd.build` (or __graft_entry__.build())")

_lib = C.CDLL(LIB_PATH)

QLIN_OK, QLIN_EINVAL, QLIN_EALIGN, QLIN_EUNSUPPORTED, QLIN_EHIP = range(5)
QLIN_F16, QLIN_BF16, QLIN_F32 = 1, 2, 3

EXPORTS = (
    "qlin_version", "qlin_status_str", "qlin_last_error",
    "qlin_w4_sizes", "qlin_w4_pack", "qlin_w4_forward", "qlin_w4_unpack",
    "spqr_sizes", "spqr_pack", "spqr_forward", "spqr_unpack",
    "sq_act_absmax", "sq_compute_smoothing", "sq_pack_weight", "sq_smooth_quant_act", "sq_int8_gemm",
    "qlin_stream_read", "qlin_stream_copy",
    "qlin_hessian", "qlin_w4_pack_gptq", "spqr_pack_hessian",
    "qlin_w4_pack_gptq_actorder", "qlin_w4_forward_perm",
    "qlin_w4_workspace_bytes", "sq_int8_gemm_workspace_bytes", "qlin_w4_forward_scratch",
    "qlin_mfma_peak", "spqr_workspace_bytes", "qlin_f16_gemm", "qlin_f16_gemm_workspace_bytes",
)

_vp, _i, _i64, _sz, _d = C.c_void_p, C.c_int, C.c_int64, C.c_size_t, C.c_double
_sigs = {
    "qlin_version": ([], _i),
    "qlin_status_str": ([_i], C.c_char_p),
    "qlin_last_error": ([], C.c_char_p),
    "qlin_w4_sizes": ([_i, _i, _i, _vp, _vp, _vp], _i),
    "qlin_w4_pack": ([_vp, _i, _i, _i, _vp, _vp, _vp], _i),
    "qlin_w4_forward": ([_vp, _i, _i, _i, _vp, _vp, _vp, _i, _i, _vp, _i, _vp, _sz, _vp], _i),
    "qlin_w4_workspace_bytes": ([_i, _i, _i, _i, _i, _i, _vp], _i),
    "qlin_w4_forward_scratch": ([_vp, _i, _i, _i, _vp, _vp, _vp, _i, _i, _vp, _i, _vp], _i),
    "qlin_w4_unpack": ([_vp, _vp, _i, _i, _i, _vp, _vp, _vp], _i),
    "spqr_sizes": ([_i, _i, _d, _vp, _vp, _vp, _vp], _i),
    "spqr_pack": ([_vp, _i, _i, _d, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp], _i),
    "spqr_forward": ([_vp, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i, _vp, _i, _vp, _sz, _vp], _i),
    "spqr_workspace_bytes": ([_i, _i, _i, _i, _vp], _i),
    "spqr_unpack": ([_vp, _vp, _i, _i, _vp, _vp, _vp, _vp], _i),
    "sq_act_absmax": ([_vp, _i, _i, _vp], _i),
    "sq_compute_smoothing": ([_vp, _vp, _i, _i, _d, _vp, _vp], _i),
    "sq_pack_weight": ([_vp, _vp, _i, _i, _vp, _vp], _i),
    "sq_smooth_quant_act": ([_vp, _vp, _i, _i, _vp, _vp, _vp], _i),
    "sq_int8_gemm": ([_vp, _vp, _vp, _vp, _i, _i, _i, _vp, _i, _vp, _vp, _sz, _vp], _i),
    "sq_int8_gemm_workspace_bytes": ([_i, _i, _i, _i, _vp], _i),
    "qlin_f16_gemm": ([_vp, _vp, _i, _i, _i, _vp, _i, _vp, _sz, _vp], _i),
    "qlin_f16_gemm_workspace_bytes": ([_i, _i, _i, _i, _vp], _i),
    "qlin_stream_read": ([_vp, _sz, _i, _i, _i, _vp, _vp], _i),
    "qlin_stream_copy": ([_vp, _vp, _sz, _vp], _i),
    "qlin_mfma_peak": ([_i, _i, _i, _vp, _vp], _i),
    "qlin_hessian": ([_vp, _i, _i, _vp], _i),
    "qlin_w4_pack_gptq": ([_vp, _i, _i, _i, _vp, _d, _vp, _vp, _vp], _i),
    "spqr_pack_hessian": ([_vp, _i, _i, _d, _vp, _d, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp], _i),
    "qlin_w4_pack_gptq_actorder": ([_vp, _i, _i, _i, _vp, _d, _i, _vp, _vp, _vp, _vp], _i),
    "qlin_w4_forward_perm": ([_vp, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _i, _i, _vp, _i, _vp, _sz, _vp], _i),
}
for _name, (_args, _res) in _sigs.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    _f.restype = _res


class QlinError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{status_str(status)}: {msg}")
        self.status = status


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if isinstance(x, np.ndarray):
        if not x.flags["C_CONTIGUOUS"]:
            raise ValueError("numpy argument must be C-contiguous")
        return x.ctypes.data
    if hasattr(x, "data_ptr"):
        if not x.is_contiguous():
            raise ValueError("tensor argument must be contiguous")
        return x.data_ptr()
    raise TypeError(f"cannot pass {type(x)} as a pointer")


def _stream(s):
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _nbytes(ws, nbytes):
    """Workspace size argument: the given count, else the buffer's own size."""
    if ws is None:
        return 0
    if nbytes is not None:
        return int(nbytes)
    if isinstance(ws, np.ndarray):
        return ws.nbytes
    if hasattr(ws, "untyped_storage"):
        return ws.numel() * ws.element_size()
    raise ValueError("pass workspace_bytes with an integer workspace pointer")


def _check(st: int):
    if st != QLIN_OK:
        raise QlinError(st, last_error())


def qlin_version() -> int:
    return _lib.qlin_version()


def status_str(st: int) -> str:
    return _lib.qlin_status_str(st).decode()


qlin_status_str = status_str


def last_error() -> str:
    return _lib.qlin_last_error().decode()


qlin_last_error = last_error


# ---------------------------------------------------------------------------
# W4

def qlin_w4_sizes(N, K, G):
    qb, sb, zb = C.c_size_t(), C.c_size_t(), C.c_size_t()
    _check(_lib.qlin_w4_sizes(N, K, G, C.byref(qb), C.byref(sb), C.byref(zb)))
    return qb.value, sb.value, zb.value


def qlin_w4_pack(W: np.ndarray, G: int = 128):
    W = np.ascontiguousarray(W, dtype=np.float32)
    N, K = W.shape
    qlin_w4_sizes(N, K, G)
    qw = np.zeros((N, K // 8), np.uint32)
    sc = np.zeros((N, K // G), np.uint16)
    qz = np.zeros((N, (K // G + 7) // 8), np.uint32)
    _check(_lib.qlin_w4_pack(_ptr(W), N, K, G, _ptr(qw), _ptr(sc), _ptr(qz)))
    return qw, sc.view(np.float16), qz


def qlin_hessian(X: np.ndarray):
    """H = (2/n) X^T X in fp64 from calibration rows X [n][K] (converted to fp32)."""
    X = np.ascontiguousarray(X, dtype=np.float32)
    n, K = X.shape
    H = np.zeros((K, K), np.float64)
    _check(_lib.qlin_hessian(_ptr(X), n, K, _ptr(H)))
    return H


def qlin_w4_pack_gptq(W: np.ndarray, G: int, H: np.ndarray, damp: float = 0.01):
    """Second-order (error-feedback) encode into the same storage as qlin_w4_pack."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    H = np.ascontiguousarray(H, dtype=np.float64)
    N, K = W.shape
    qlin_w4_sizes(N, K, G)
    qw = np.zeros((N, K // 8), np.uint32)
    sc = np.zeros((N, K // G), np.uint16)
    qz = np.zeros((N, (K // G + 7) // 8), np.uint32)
    _check(_lib.qlin_w4_pack_gptq(_ptr(W), N, K, G, _ptr(H), damp, _ptr(qw), _ptr(sc), _ptr(qz)))
    return qw, sc.view(np.float16), qz


def qlin_w4_pack_gptq_actorder(W: np.ndarray, G: int, H: np.ndarray, damp: float = 0.01,
                               static_groups: bool = True):
    """Act-order second-order encode; returns (qweight, scales, qzeros, perm)."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    H = np.ascontiguousarray(H, dtype=np.float64)
    N, K = W.shape
    qlin_w4_sizes(N, K, G)
    qw = np.zeros((N, K // 8), np.uint32)
    sc = np.zeros((N, K // G), np.uint16)
    qz = np.zeros((N, (K // G + 7) // 8), np.uint32)
    perm = np.zeros(K, np.int32)
    _check(_lib.qlin_w4_pack_gptq_actorder(_ptr(W), N, K, G, _ptr(H), damp, int(bool(static_groups)), _ptr(qw),
                                           _ptr(sc), _ptr(qz), _ptr(perm)))
    return qw, sc.view(np.float16), qz, perm


def qlin_w4_workspace_bytes(x_dtype, M, K, N, G, y_dtype):
    b = C.c_size_t()
    _check(_lib.qlin_w4_workspace_bytes(x_dtype, M, K, N, G, y_dtype, C.byref(b)))
    return b.value


def qlin_w4_forward_perm(X, x_dtype, M, K, perm, Xp, qweight, scales, qzeros, N, G, Y, y_dtype,
                         workspace=None, workspace_bytes=None, stream=None):
    _check(_lib.qlin_w4_forward_perm(_ptr(X), x_dtype, M, K, _ptr(perm), _ptr(Xp), _ptr(qweight), _ptr(scales),
                                     _ptr(qzeros), N, G, _ptr(Y), y_dtype, _ptr(workspace),
                                     _nbytes(workspace, workspace_bytes), _stream(stream)))


def qlin_w4_forward(X, x_dtype, M, K, qweight, scales, qzeros, N, G, Y, y_dtype,
                    workspace=None, workspace_bytes=None, stream=None):
    _check(_lib.qlin_w4_forward(_ptr(X), x_dtype, M, K, _ptr(qweight), _ptr(scales), _ptr(qzeros),
                                N, G, _ptr(Y), y_dtype, _ptr(workspace), _nbytes(workspace, workspace_bytes),
                                _stream(stream)))


def qlin_w4_forward_scratch(X, x_dtype, M, K, qweight, scales, qzeros, N, G, Y, y_dtype, stream=None):
    _check(_lib.qlin_w4_forward_scratch(_ptr(X), x_dtype, M, K, _ptr(qweight), _ptr(scales), _ptr(qzeros),
                                        N, G, _ptr(Y), y_dtype, _stream(stream)))


def qlin_w4_unpack(qweight, qzeros, N, K, G, codes, zeros, stream=None):
    _check(_lib.qlin_w4_unpack(_ptr(qweight), _ptr(qzeros), N, K, G, _ptr(codes), _ptr(zeros), _stream(stream)))


# ---------------------------------------------------------------------------
# SpQR

def spqr_sizes(N, K, outlier_frac):
    a, b, c, nnz = C.c_size_t(), C.c_size_t(), C.c_size_t(), C.c_int64()
    _check(_lib.spqr_sizes(N, K, outlier_frac, C.byref(a), C.byref(b), C.byref(c), C.byref(nnz)))
    return a.value, b.value, c.value, nnz.value


def spqr_pack(W: np.ndarray, outlier_frac: float = 0.01):
    W = np.ascontiguousarray(W, dtype=np.float32)
    N, K = W.shape
    _, _, _, nnz = spqr_sizes(N, K, outlier_frac)
    codes = np.zeros((N, K // 32, 3), np.uint32)
    s1 = np.zeros((N, K // 256, 3), np.uint32)
    s2 = np.zeros((N, K // 256, 4), np.uint16)
    rp = np.zeros(N + 1, np.int32)
    ci = np.zeros(max(nnz, 1), np.int32)
    vals = np.zeros(max(nnz, 1), np.uint16)
    out = C.c_int64()
    _check(_lib.spqr_pack(_ptr(W), N, K, outlier_frac, _ptr(codes), _ptr(s1), _ptr(s2), _ptr(rp),
                          _ptr(ci), _ptr(vals), nnz, C.byref(out)))
    n = out.value
    return dict(codes=codes, stats1=s1, stats2=s2.view(np.float16), row_ptr=rp,
                col_idx=ci[:n].copy(), val=vals[:n].view(np.float16).copy())


def spqr_pack_hessian(W: np.ndarray, outlier_frac: float, H: np.ndarray, damp: float = 0.01):
    """SpQR storage with outliers chosen by Hessian-weighted sensitivity (H fp64 [K][K])."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    H = np.ascontiguousarray(H, dtype=np.float64)
    N, K = W.shape
    _, _, _, nnz = spqr_sizes(N, K, outlier_frac)
    codes = np.zeros((N, K // 32, 3), np.uint32)
    s1 = np.zeros((N, K // 256, 3), np.uint32)
    s2 = np.zeros((N, K // 256, 4), np.uint16)
    rp = np.zeros(N + 1, np.int32)
    ci = np.zeros(max(nnz, 1), np.int32)
    vals = np.zeros(max(nnz, 1), np.uint16)
    out = C.c_int64()
    _check(_lib.spqr_pack_hessian(_ptr(W), N, K, outlier_frac, _ptr(H), damp, _ptr(codes), _ptr(s1), _ptr(s2),
                                  _ptr(rp), _ptr(ci), _ptr(vals), nnz, C.byref(out)))
    n = out.value
    return dict(codes=codes, stats1=s1, stats2=s2.view(np.float16), row_ptr=rp,
                col_idx=ci[:n].copy(), val=vals[:n].view(np.float16).copy())


def spqr_workspace_bytes(M, K, N, y_dtype=QLIN_F16):
    b = C.c_size_t()
    _check(_lib.spqr_workspace_bytes(M, K, N, y_dtype, C.byref(b)))
    return b.value


def spqr_forward(X, M, K, codes, stats1, stats2, row_ptr, col_idx, vals, nnz, N, Y, y_dtype=QLIN_F16,
                 workspace=None, workspace_bytes=None, stream=None):
    _check(_lib.spqr_forward(_ptr(X), M, K, _ptr(codes), _ptr(stats1), _ptr(stats2), _ptr(row_ptr),
                             _ptr(col_idx), _ptr(vals), nnz, N, _ptr(Y), y_dtype, _ptr(workspace),
                             _nbytes(workspace, workspace_bytes), _stream(stream)))


def spqr_unpack(codes, stats1, N, K, q, cs, cz, stream=None):
    _check(_lib.spqr_unpack(_ptr(codes), _ptr(stats1), N, K, _ptr(q), _ptr(cs), _ptr(cz), _stream(stream)))


# ---------------------------------------------------------------------------
# SmoothQuant

def sq_act_absmax(Xcal: np.ndarray):
    Xcal = np.ascontiguousarray(Xcal, dtype=np.float16)
    M, K = Xcal.shape
    out = np.zeros(K, np.float32)
    _check(_lib.sq_act_absmax(_ptr(Xcal), M, K, _ptr(out)))
    return out


def sq_compute_smoothing(amax: np.ndarray, W: np.ndarray, alpha: float):
    W = np.ascontiguousarray(W, dtype=np.float32)
    amax = np.ascontiguousarray(amax, dtype=np.float32)
    N, K = W.shape
    s = np.zeros(K, np.float32)
    inv = np.zeros(K, np.float32)
    _check(_lib.sq_compute_smoothing(_ptr(amax), _ptr(W), N, K, float(alpha), _ptr(s), _ptr(inv)))
    return s, inv


def sq_pack_weight(W: np.ndarray, s: np.ndarray):
    W = np.ascontiguousarray(W, dtype=np.float32)
    s = np.ascontiguousarray(s, dtype=np.float32)
    N, K = W.shape
    Wq = np.zeros((N, K), np.int8)
    ws = np.zeros(N, np.float32)
    _check(_lib.sq_pack_weight(_ptr(W), _ptr(s), N, K, _ptr(Wq), _ptr(ws)))
    return Wq, ws


def sq_smooth_quant_act(X, inv_s, M, K, Xq, x_scale, stream=None):
    _check(_lib.sq_smooth_quant_act(_ptr(X), _ptr(inv_s), M, K, _ptr(Xq), _ptr(x_scale), _stream(stream)))


def sq_int8_gemm_workspace_bytes(M, N, K, y_dtype=QLIN_F16):
    b = C.c_size_t()
    _check(_lib.sq_int8_gemm_workspace_bytes(M, N, K, y_dtype, C.byref(b)))
    return b.value


def sq_int8_gemm(Xq, x_scale, Wq, w_scale, M, N, K, Y, y_dtype=QLIN_F16, acc_out=None,
                 workspace=None, workspace_bytes=None, stream=None):
    _check(_lib.sq_int8_gemm(_ptr(Xq), _ptr(x_scale), _ptr(Wq), _ptr(w_scale), M, N, K, _ptr(Y), y_dtype,
                             _ptr(acc_out), _ptr(workspace), _nbytes(workspace, workspace_bytes), _stream(stream)))


# ---------------------------------------------------------------------------
# Dense fp16 layer

def qlin_f16_gemm_workspace_bytes(M, N, K, y_dtype=QLIN_F16):
    b = C.c_size_t()
    _check(_lib.qlin_f16_gemm_workspace_bytes(M, N, K, y_dtype, C.byref(b)))
    return b.value


def qlin_f16_gemm(X, W, M, N, K, Y, y_dtype=QLIN_F16, workspace=None, workspace_bytes=None, stream=None):
    _check(_lib.qlin_f16_gemm(_ptr(X), _ptr(W), M, N, K, _ptr(Y), y_dtype, _ptr(workspace),
                              _nbytes(workspace, workspace_bytes), _stream(stream)))


# ---------------------------------------------------------------------------
# Measurement aid

def qlin_stream_read(buf, nbytes, grid, unroll, nontemporal, out, stream=None):
    _check(_lib.qlin_stream_read(_ptr(buf), nbytes, grid, unroll, int(bool(nontemporal)), _ptr(out),
                                 _stream(stream)))


def qlin_mfma_peak(kind, iters, grid, out, stream=None):
    _check(_lib.qlin_mfma_peak(kind, iters, grid, _ptr(out), _stream(stream)))


def qlin_stream_copy(dst, src, nbytes, stream=None):
    _check(_lib.qlin_stream_copy(_ptr(dst), _ptr(src), nbytes, _stream(stream)))
