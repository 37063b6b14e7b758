"""Pins of the SmoothQuant oracle: the page's identity, hand-worked quantization
and smoothing values, exact integer accumulation against int64 brute force,
the s = 1 special case, the flattening invariant and 'smoothing helps'."""
import numpy as np
import pytest

import synth
from oracle import metrics
from oracle import smoothquant as sq


def test_identity_holds_in_fp64():
    """(X diag(s)^-1)(diag(s) W) = X W (the page's equation; W stored [N][K])."""
    X = synth.activations("sq_w8a8", 1, 512).astype(np.float64)
    W = synth.normal_f32((512, 4096), 0.02, "pin/sq/id")
    s = sq.smoothing_f64(sq.act_absmax(X), W, 0.85)
    lhs = (X / s[None, :]) @ (W.astype(np.float64) * s[None, :]).T
    rhs = X @ W.astype(np.float64).T
    assert metrics.rel_frob(lhs, rhs) <= 1e-12


def test_hand_worked_activation_quantization(golden):
    g = golden("sq_quant.json")["act"]
    X = np.array(g["X"], np.float16)
    Xq, dX = sq.quantize_act(X, np.array(g["inv_s"], np.float32))
    assert Xq.tolist() == g["Xq"]
    assert dX.tolist() == g["dX"]


def test_hand_worked_smoothing_factors(golden):
    g = golden("sq_quant.json")["smoothing"]
    S32, inv_s = sq.smoothing(np.array(g["amax"], np.float32), np.array(g["W"], np.float32), g["alpha"])
    expect = np.array(g["s"], np.float64)
    assert np.array_equal(S32, expect.astype(np.float32))
    assert np.array_equal(inv_s, (np.float32(1.0) / expect.astype(np.float32)))


def test_int_gemm_equals_int64_brute_force():
    r = np.random.default_rng(7)
    Xq = r.integers(-127, 128, size=(9, 4096)).astype(np.int8)
    Wq = r.integers(-127, 128, size=(13, 4096)).astype(np.int8)
    Xq[0] = 127
    Wq[0] = 127                                          # the largest |acc| possible
    Xq[1] = -127
    acc = sq.int_gemm(Xq, Wq)
    assert np.array_equal(acc, sq.int_gemm_bruteforce(Xq, Wq))
    assert acc[0, 0] == 4096 * 127 * 127 and acc[1, 0] == -4096 * 127 * 127


def test_unit_smoothing_is_plain_w8a8_rtn():
    """s = 1: per-channel weights and per-token activations are plain symmetric
    RTN; every value lies within half a step of the original."""
    W = synth.normal_f32((64, 4096), 0.02, "pin/sq/s1")
    X = synth.activations("sq_w8a8", 1, 256)
    one = np.ones(4096, np.float32)
    Wq, dW = sq.quantize_weight(W, one)
    Xq, dX = sq.quantize_act(X, one)
    assert np.all(np.abs(W - Wq * dW[:, None].astype(np.float64)) <= dW[:, None] * (0.5 + 1e-5))
    Xd = X.astype(np.float64)
    assert np.all(np.abs(Xd - Xq * dX[:, None].astype(np.float64)) <= dX[:, None] * (0.5 + 1e-5))
    assert np.all(np.abs(Wq).max(axis=1) == 127) and np.all(np.abs(Xq).max(axis=1) == 127)


def test_zero_rows_give_zero_scale():
    X = np.zeros((2, 64), np.float16)
    X[1, 3] = 2.0
    Xq, dX = sq.quantize_act(X, np.ones(64, np.float32))
    assert dX[0] == 0 and not np.any(Xq[0]) and Xq[1, 3] == 127
    W = np.zeros((2, 64), np.float32)
    Wq, dW = sq.quantize_weight(W, np.ones(64, np.float32))
    assert not np.any(dW) and not np.any(Wq)


def test_smoothing_balances_channel_maxima():
    """After smoothing, each channel's activation max times its weight max is
    unchanged (a_j b_j) and their ratio is (a_j b_j)^(1 - 2 alpha)."""
    Xc = synth.sq_calibration("sq_w8a8", 1)
    W = synth.normal_f32((4096, 4096), 0.02, "pin/sq/bal")
    a = sq.act_absmax(Xc).astype(np.float64)
    b = sq.weight_absmax(W).astype(np.float64)
    s = sq.smoothing_f64(a, W, 0.85)
    xa = a / s
    wb = b * s
    assert np.allclose(xa * wb, a * b, rtol=1e-12)
    assert np.allclose(xa / wb, (a * b) ** (1 - 2 * 0.85), rtol=1e-12)
    # the outlier channels (x100) are the ones pulled down hardest
    ch = synth.outlier_channels(4096, 0.01, "sq_w8a8/L1/channels")
    assert np.median(xa[ch]) < np.median(a[ch]) / 10


def test_smoothing_helps_on_outlier_channel_data():
    X = synth.activations("sq_w8a8", 1, 512)
    W = synth.normal_f32((1024, 4096), 0.02, "pin/sq/helps")
    Ytrue = X.astype(np.float64) @ W.astype(np.float64).T
    S32, inv_s, Wq, dW = sq.pack(W, X, 0.85)
    Y_sq = sq.forward(X, inv_s, Wq, dW)[0]
    one = np.ones(4096, np.float32)
    Wq1, dW1 = sq.quantize_weight(W, one)
    Y_plain = sq.forward(X, one, Wq1, dW1)[0]
    e_sq, e_plain = metrics.rel_frob(Y_sq, Ytrue), metrics.rel_frob(Y_plain, Ytrue)
    print("relFrob with smoothing", e_sq, "without", e_plain)
    assert e_sq < e_plain


@pytest.mark.parametrize("M", [256, 512])
def test_forward_decomposes_into_its_steps(M):
    X = synth.activations("sq_w8a8", 1, M)
    W = synth.normal_f32((128, 4096), 0.02, "pin/sq/steps")
    S32, inv_s, Wq, dW = sq.pack(W, synth.sq_calibration("sq_w8a8", 1), 0.85)
    Y, Xq, dX, acc = sq.forward(X, inv_s, Wq, dW)
    assert np.array_equal(acc[:, :7], sq.int_gemm_bruteforce(Xq, Wq[:7]))
    m, n = M - 1, 5
    assert Y[m, n] == float(dX[m]) * float(dW[n]) * float(acc[m, n])
