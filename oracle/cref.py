"""ctypes binding and build step of the plain C++ oracle forwards (qlin_oracle.cpp).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The C++ file is compiled on its own by the host compiler (g++ -O2, OpenMP,
floating-point contraction off) into oracle/libqlin_oracle.so; it shares no
source with the library.  ``build()`` compiles it every time it is called;
``lib()`` loads the built file and compiles it first only if it is missing.
The functions here marshal numpy arrays and return fp64 / int64 numpy arrays.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "qlin_oracle.cpp")
LIB = os.path.join(_HERE, "libqlin_oracle.so")
CXX_FLAGS = ["-O2", "-std=c++17", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]

_lib = None


def build(extra_flags=()):
    """Compile qlin_oracle.cpp into libqlin_oracle.so (always recompiles)."""
    tmp = LIB + ".tmp"
    cmd = ["g++", *CXX_FLAGS, *extra_flags, SRC, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        L = C.CDLL(LIB)
        vp, i = C.c_void_p, C.c_int
        L.oracle_max_threads.argtypes, L.oracle_max_threads.restype = [], i
        L.oracle_w4_forward.argtypes = [vp, i, i, i, vp, vp, vp, i, i, vp, i]
        L.oracle_w4_forward.restype = None
        L.oracle_spqr_forward.argtypes = [vp, i, i, vp, vp, vp, vp, vp, vp, i, vp, i]
        L.oracle_spqr_forward.restype = None
        L.oracle_sq_forward.argtypes = [vp, vp, vp, vp, i, i, i, vp, vp, i]
        L.oracle_sq_forward.restype = None
        _lib = L
    return _lib


def _p(a):
    return a.ctypes.data


def _x_bits(X):
    """(uint16 bits, is_bf16): fp16 arrays as fp16, uint16 arrays as bf16 patterns."""
    X = np.asarray(X)
    if X.dtype == np.float16:
        return np.ascontiguousarray(X).view(np.uint16), 0
    if X.dtype == np.uint16:
        return np.ascontiguousarray(X), 1
    raise TypeError("X must be float16 or uint16 (bf16 bits)")


def max_threads() -> int:
    return lib().oracle_max_threads()


def w4_forward(X, qweight, scales, qzeros, K: int, G: int = 128, threads: int = 0):
    """Y = X . W_hat^T in fp64 for the W4 storage (X fp16, or uint16 bf16 bits)."""
    xb, is_bf = _x_bits(X)
    M = xb.shape[0]
    qw = np.ascontiguousarray(qweight, dtype=np.uint32)
    sc = np.ascontiguousarray(np.asarray(scales, dtype=np.float16)).view(np.uint16)
    qz = np.ascontiguousarray(qzeros, dtype=np.uint32)
    N = qw.shape[0]
    assert xb.shape[1] == K and qw.shape[1] == K // 8 and sc.shape == (N, K // G)
    Y = np.empty((M, N), dtype=np.float64)
    lib().oracle_w4_forward(_p(xb), is_bf, M, K, _p(qw), _p(sc), _p(qz), N, G, _p(Y), threads)
    return Y


def spqr_forward(X, st, K: int, threads: int = 0):
    """Y = X . (W_dense + W_sparse)^T in fp64 for the SpQR storage dict (X fp16)."""
    xb, is_bf = _x_bits(X)
    assert not is_bf
    M = xb.shape[0]
    codes = np.ascontiguousarray(st["codes"], dtype=np.uint32)
    N = codes.shape[0]
    s1 = np.ascontiguousarray(st["stats1"], dtype=np.uint32)
    s2 = np.ascontiguousarray(np.asarray(st["stats2"], dtype=np.float16)).view(np.uint16)
    rp = np.ascontiguousarray(st["row_ptr"], dtype=np.int32)
    ci = np.ascontiguousarray(st["col_idx"], dtype=np.int32)
    vals = np.ascontiguousarray(np.asarray(st["val"], dtype=np.float16)).view(np.uint16)
    assert codes.size == N * (K // 32) * 3 and s1.size == N * (K // 256) * 3 and s2.size == N * (K // 256) * 4
    assert rp.shape == (N + 1,) and rp[0] == 0 and rp[-1] == ci.size == vals.size
    if ci.size:
        assert ci.min() >= 0 and ci.max() < K
    Y = np.empty((M, N), dtype=np.float64)
    # a zero-length CSR still needs valid pointers
    ci_ = ci if ci.size else np.zeros(1, np.int32)
    v_ = vals if vals.size else np.zeros(1, np.uint16)
    lib().oracle_spqr_forward(_p(xb), M, K, _p(codes), _p(s1), _p(s2), _p(rp), _p(ci_), _p(v_), N, _p(Y), threads)
    return Y


def sq_forward(Xq, x_scale, Wq, w_scale, threads: int = 0, want_y: bool = True):
    """(acc int64 [M][N], Y fp64 [M][N] or None) of the W8A8 integer product."""
    xq = np.ascontiguousarray(Xq, dtype=np.int8)
    wq = np.ascontiguousarray(Wq, dtype=np.int8)
    xs = np.ascontiguousarray(x_scale, dtype=np.float32)
    ws = np.ascontiguousarray(w_scale, dtype=np.float32)
    M, K = xq.shape
    N = wq.shape[0]
    assert wq.shape[1] == K and xs.shape == (M,) and ws.shape == (N,)
    acc = np.empty((M, N), dtype=np.int64)
    Y = np.empty((M, N), dtype=np.float64) if want_y else None
    lib().oracle_sq_forward(_p(xq), _p(xs), _p(wq), _p(ws), M, N, K, _p(acc), _p(Y) if want_y else None, threads)
    return acc, Y
