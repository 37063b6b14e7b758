"""Oracle for SmoothQuant W8A8: smoothing, per-token int8 X, per-channel int8 W.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the SmoothQuant bulletin fixes ("Makale Bülteni — SmoothQuant",
"İddia ve Gerçeklik"): an INT8 GEMM needs both operands in int8; some
activation channels carry outliers about 100x the rest; the layer is rewritten
as Y = (X diag(s)^-1)(diag(s) W) with a per-channel s that flattens the
activation peaks and is folded into the weights offline; then activations are
quantized per token and weights per channel and fed to a standard INT8 GEMM;
s comes from per-channel maxima found on about 512 calibration samples, with a
migration strength alpha of about 0.8-0.85.

In the page's equation W is in x out; here W is stored out x in ([N][K]) and
Y = X . W^T, so diag(s) . W becomes W . diag(s) (column j scaled by s_j).

Readings where the page is silent:

* s_j = max_m |Xcal[m, j]|^alpha / max_n |W[n, j]|^(1 - alpha) in fp64
  (s_j = 1 when either maximum is 0); stored as S32 = fp32(s_j), with
  inv_s = 1 / S32 in fp32;
* symmetric int8 in [-127, 127]; fp32 scales; rounding half-to-even;
  quantization multiplies by the fp32 value 127 / absmax;
* weights: W' = W * S32 (fp32), c_n = max_j |W'[n, j]|, dW_n = c_n / 127,
  Wq = clamp(rint(W' * (127 / c_n)), -127, 127); a zero row gives dW = 0, Wq = 0;
* activations: x~ = fp32(x) * inv_s_j, a_m = max_j |x~|, dX_m = a_m / 127,
  Xq = clamp(rint(x~ * (127 / a_m)), -127, 127); a zero row gives dX = 0, Xq = 0;
* acc = sum_j Xq * Wq exactly (int32 suffices: |acc| <= K * 127^2);
  Y = dX_m * dW_n * acc, here in fp64.
"""
from __future__ import annotations

import math

import numpy as np

F32 = np.float32


def act_absmax(Xcal):
    """Per-channel max |x| over the calibration rows (fp32 [K])."""
    return np.max(np.abs(np.asarray(Xcal).astype(F32)), axis=0)


def weight_absmax(W):
    """Per-input-channel max |w| over the output rows (fp32 [K])."""
    return np.max(np.abs(np.asarray(W, dtype=F32)), axis=0)


def smoothing(amax, W, alpha: float):
    """(S32 fp32 [K], inv_s fp32 [K]); the power law is evaluated with libm pow per channel."""
    a = np.asarray(amax, dtype=F32)
    b = weight_absmax(W)
    K = a.shape[0]
    s = np.empty(K, dtype=np.float64)
    for j in range(K):
        aj, bj = float(a[j]), float(b[j])
        if aj == 0.0 or bj == 0.0:
            s[j] = 1.0
        else:
            s[j] = math.pow(aj, alpha) / math.pow(bj, 1.0 - alpha)
    S32 = s.astype(F32)
    return S32, (F32(1.0) / S32).astype(F32)


def smoothing_f64(amax, W, alpha: float):
    """The same smoothing vector left in fp64 (for the identity check)."""
    a = np.asarray(amax, dtype=np.float64)
    b = weight_absmax(W).astype(np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        s = np.where((a == 0) | (b == 0), 1.0, a ** alpha / b ** (1.0 - alpha))
    return s


def quantize_weight(W, S32):
    """(Wq int8 [N][K], dW fp32 [N]) for W' = W . diag(S32)."""
    Wp = np.asarray(W, dtype=F32) * np.asarray(S32, dtype=F32)[None, :]
    c = np.max(np.abs(Wp), axis=1)
    zero = c == 0
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(zero, F32(0.0), F32(127.0) / c).astype(F32)
    q = np.clip(np.rint(Wp * r[:, None]), F32(-127.0), F32(127.0)).astype(np.int8)
    dW = np.where(zero, F32(0.0), c / F32(127.0)).astype(F32)
    return q, dW


def quantize_act(X, inv_s):
    """(Xq int8 [M][K], dX fp32 [M]) for x~ = X . diag(inv_s), per token."""
    Xt = np.asarray(X).astype(F32) * np.asarray(inv_s, dtype=F32)[None, :]
    a = np.max(np.abs(Xt), axis=1)
    zero = a == 0
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(zero, F32(0.0), F32(127.0) / a).astype(F32)
    q = np.clip(np.rint(Xt * r[:, None]), F32(-127.0), F32(127.0)).astype(np.int8)
    dX = np.where(zero, F32(0.0), a / F32(127.0)).astype(F32)
    return q, dX


def int_gemm(Xq, Wq):
    """acc[m][n] = sum_k Xq[m][k] * Wq[n][k], exact.

    Every partial sum is an integer below 2^53 in magnitude (K * 127^2), so the
    fp64 matrix product of the integer-valued arrays is exact in any order."""
    acc = np.asarray(Xq, dtype=np.float64) @ np.asarray(Wq, dtype=np.float64).T
    return acc.astype(np.int64)


def int_gemm_bruteforce(Xq, Wq):
    """The same sum with int64 arithmetic (small inputs only)."""
    a = np.asarray(Xq, dtype=np.int64)
    b = np.asarray(Wq, dtype=np.int64)
    return (a[:, None, :] * b[None, :, :]).sum(axis=2)


def dequant_output(acc, dX, dW):
    """Y = dX_m * dW_n * acc in fp64."""
    return (np.asarray(dX, np.float64)[:, None] * np.asarray(dW, np.float64)[None, :]
            * np.asarray(acc, np.float64))


def pack(W, Xcal, alpha: float):
    """Offline part: (S32, inv_s, Wq, dW) from fp32 W and the calibration rows."""
    S32, inv_s = smoothing(act_absmax(Xcal), W, alpha)
    Wq, dW = quantize_weight(W, S32)
    return S32, inv_s, Wq, dW


def forward(X, inv_s, Wq, dW):
    """Online part in the page's order: smooth + quantize X, int8 GEMM, rescale."""
    Xq, dX = quantize_act(X, inv_s)
    acc = int_gemm(Xq, Wq)
    return dequant_output(acc, dX, dW), Xq, dX, acc
