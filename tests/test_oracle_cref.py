"""Pins of the plain C++ oracle forwards (oracle/qlin_oracle.cpp via oracle.cref).

Each forward is checked against values fixed independently of it:
* W4: the hand-worked group of tests/golden/w4_rtn_group.json decoded through
  unit activation rows (the output is the dequantized weight itself, exactly);
  grid-point weights (every weight S (q - z) exactly) reproduced bit for bit;
  a brute-force Python sum; bf16 activations decoded as the top half of fp32;
* SpQR: the hand-worked single-code layout cases of tests/golden/spqr_layout.json
  read back through unit activations; grid-point layers reproduced exactly;
  the sparse-only case equal to a textbook CSR product (scipy); the dense +
  sparse reconstruction of the numpy oracle;
* W8A8: the int64 accumulator equal to a brute-force int64 matmul, and the
  output equal to dX_m dW_n acc evaluated left to right in fp64.
The thread count does not change any bit (one row per thread, fixed order).
"""
import numpy as np
import pytest
import scipy.sparse

import synth
from oracle import cref, smoothquant, spqr, w4

from test_oracle_spqr import _grid_layer
from test_oracle_w4 import _grid_weights


def _eye_f16(K):
    return np.eye(K, dtype=np.float16)


def test_w4_hand_worked_group_through_unit_rows(golden):
    g = golden("w4_rtn_group.json")
    K = G = g["G"]
    qw = np.array([g["qweight"]], np.uint32)
    S = np.array([[g["scale"]]], np.float16)
    assert int(S.view(np.uint16)[0, 0]) == g["scale_bits"]
    qz = np.array([g["qzeros"]], np.uint32)
    Y = cref.w4_forward(_eye_f16(K), qw, S, qz, K, G)
    want = g["scale"] * (np.array(g["q"], np.float64) - g["zero"])
    assert np.array_equal(Y[:, 0], want)


def test_w4_grid_points_exact():
    W, q, S, z = _grid_weights(16, 512, 128, seed=11)
    qw, S2, qz = w4.encode(W, 128)
    Y = cref.w4_forward(_eye_f16(512), qw, S2, qz, 512, 128)
    assert np.array_equal(Y.T, W.astype(np.float64))


def test_w4_brute_force_sum_and_numpy_oracle():
    N, K, G, M = 9, 256, 64, 3
    W = synth.normal_f32((N, K), 0.02, "pin/cref/w4")
    X = synth.x_f16(M, K, "pin/cref/w4x")
    qw, S, qz = w4.encode(W, G)
    Y = cref.w4_forward(X, qw, S, qz, K, G)
    q, z = w4.unpack(qw, qz, K, G)
    Sd = S.astype(np.float64)
    for m in range(M):
        for n in range(N):
            s = 0.0
            for k in range(K):
                s += float(X[m, k]) * (Sd[n, k // G] * (int(q[n, k]) - int(z[n, k // G])))
            assert Y[m, n] == s                      # same order, same fp64 arithmetic
    ref = w4.forward(X, qw, S, qz, K, G)
    assert np.max(np.abs(Y - ref)) <= 1e-13 * np.max(np.abs(ref))


def test_w4_bf16_activations():
    N, K = 20, 384
    W = synth.normal_f32((N, K), 0.02, "pin/cref/w4b")
    Xb = synth.x_bf16_bits(4, K, "pin/cref/w4bx")
    Xb[0, 0] = 0x47C3                                  # 99840.0: beyond the fp16 range
    Xb[1, 1] = 0x0001                                  # a bf16 subnormal
    qw, S, qz = w4.encode(W, 128)
    Y = cref.w4_forward(Xb, qw, S, qz, K, 128)
    xd = (Xb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert xd[0, 0] == 99840.0
    ref = xd @ w4.dequantize(qw, S, qz, K, 128).T
    assert np.max(np.abs(Y - ref)) <= 1e-13 * np.max(np.abs(ref))


def _unit_stats_row(nb):
    """stats1 / stats2 of one row whose every group decodes to s_hat = 1,
    z_hat = 0: c_s = 1, c_z = 0 (field value 1 at bit 6g of each block) and
    SS_s = 1, ZS_s = 0, SS_z = 1, ZS_z = 0."""
    stream = 0
    for gi in range(16):
        stream |= 1 << (6 * gi)
    words = [(stream >> (32 * j)) & 0xFFFFFFFF for j in range(3)]
    s1 = np.tile(np.array(words, np.uint32), (1, nb, 1))
    s2 = np.tile(np.array([1.0, 0.0, 1.0, 0.0], np.float16), (1, nb, 1))
    return s1, s2


def test_spqr_hand_worked_layout_cases(golden):
    g = golden("spqr_layout.json")
    K = 256
    s1, s2 = _unit_stats_row(1)
    for case in g["code_cases"]:
        codes = np.zeros((1, K // 32, 3), np.uint32)
        codes[0, 0] = case["words"]
        st = dict(codes=codes, stats1=s1, stats2=s2, row_ptr=np.zeros(2, np.int32),
                  col_idx=np.zeros(0, np.int32), val=np.zeros(0, np.float16))
        Y = cref.spqr_forward(_eye_f16(K), st, K)
        want = np.zeros(K)
        want[case["code"]] = case["value"]
        assert np.array_equal(Y[:, 0], want), case["why"]


def test_spqr_grid_points_exact():
    W, q, cs, cz, SS = _grid_layer(5, 512, seed=12)
    st = spqr.encode(W, p=0.0)
    Y = cref.spqr_forward(_eye_f16(512), st, 512)
    assert np.array_equal(Y.T, W.astype(np.float64))


def test_spqr_sparse_only_is_textbook_csr():
    N, K = 16, 512
    W = synth.student_t3_f32((N, K), 0.02, "pin/cref/sp")
    X = synth.x_f16(3, K, "pin/cref/spx")
    st = spqr.encode(W, 0.05)
    st0 = dict(st)
    st0["codes"] = np.zeros_like(st["codes"])
    s2 = st["stats2"].copy()
    s2[:, :, 2] = 0.0
    s2[:, :, 3] = 0.0
    st0["stats2"] = s2
    A = scipy.sparse.csr_matrix((st["val"].astype(np.float64), st["col_idx"], st["row_ptr"]), shape=(N, K))
    ref = (A @ X.astype(np.float64).T).T
    assert np.allclose(cref.spqr_forward(X, st0, K), ref, rtol=1e-14, atol=1e-14)


def test_spqr_matches_dense_plus_sparse_reconstruction():
    N, K = 24, 768
    W = synth.student_t3_f32((N, K), 0.02, "pin/cref/spd")
    X = synth.x_f16(4, K, "pin/cref/spdx")
    st = spqr.encode(W, 0.01)
    W_hat = (spqr.dequantize_dense(st["codes"], st["stats1"], st["stats2"], K)
             + spqr.sparse_dense(st["row_ptr"], st["col_idx"], st["val"], N, K))
    Y = cref.spqr_forward(X, st, K)
    ref = X.astype(np.float64) @ W_hat.T
    assert np.max(np.abs(Y - ref)) <= 1e-13 * np.max(np.abs(ref))
    # with unit rows the forward returns the reconstructed weights exactly
    assert np.array_equal(cref.spqr_forward(_eye_f16(K), st, K).T, W_hat)


def test_sq_int64_accumulator_and_output():
    r = np.random.default_rng(21)
    M, N, K = 7, 13, 320
    Xq = r.integers(-127, 128, size=(M, K)).astype(np.int8)
    Wq = r.integers(-127, 128, size=(N, K)).astype(np.int8)
    Xq[0] = 127
    Wq[0] = -127                                        # extreme products
    dX = r.random(M).astype(np.float32)
    dW = r.random(N).astype(np.float32)
    acc, Y = cref.sq_forward(Xq, dX, Wq, dW)
    assert np.array_equal(acc, smoothquant.int_gemm_bruteforce(Xq, Wq))
    assert acc[0, 0] == -127 * 127 * K
    want = np.empty((M, N))
    for m in range(M):
        for n in range(N):
            want[m, n] = float(dX[m]) * float(dW[n]) * float(acc[m, n])
    assert np.array_equal(Y, want)


@pytest.mark.parametrize("which", ["w4", "spqr", "sq"])
def test_thread_count_changes_no_bit(which):
    K = 512
    if which == "w4":
        W = synth.normal_f32((64, K), 0.02, "pin/cref/thr")
        X = synth.x_f16(2, K, "pin/cref/thrx")
        st = w4.encode(W, 128)
        a = cref.w4_forward(X, *st, K, 128, threads=1)
        b = cref.w4_forward(X, *st, K, 128, threads=4)
    elif which == "spqr":
        W = synth.student_t3_f32((64, K), 0.02, "pin/cref/thrs")
        X = synth.x_f16(2, K, "pin/cref/thrsx")
        st = spqr.encode(W, 0.01)
        a = cref.spqr_forward(X, st, K, threads=1)
        b = cref.spqr_forward(X, st, K, threads=4)
    else:
        r = np.random.default_rng(5)
        Xq = r.integers(-127, 128, size=(3, K)).astype(np.int8)
        Wq = r.integers(-127, 128, size=(64, K)).astype(np.int8)
        a = cref.sq_forward(Xq, np.ones(3, np.float32), Wq, np.ones(64, np.float32), threads=1)[1]
        b = cref.sq_forward(Xq, np.ones(3, np.float32), Wq, np.ones(64, np.float32), threads=4)[1]
    assert np.array_equal(a, b)
