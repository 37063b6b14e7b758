"""Pins of the 4-bit group-quantization oracle against facts that do not come
from the oracle itself: a hand-worked group, grid points that must round-trip
exactly, the RTN half-step bound, brute-force sums and special cases."""
import numpy as np
import pytest

import synth
from oracle import w4


def test_hand_worked_group(golden):
    g = golden("w4_rtn_group.json")
    W = np.array([g["W"]], dtype=np.float32)
    q, S, z = w4.quantize_rtn(W, G=g["G"])
    assert q[0].tolist() == g["q"]
    assert S.view(np.uint16)[0, 0] == g["scale_bits"]
    assert float(S[0, 0]) == g["scale"]
    assert int(z[0, 0]) == g["zero"]
    qw, S2, qz = w4.pack(q, S, z)
    assert qw[0].tolist() == g["qweight"]
    assert qz[0].tolist() == g["qzeros"]
    w_hat = w4.dequantize(qw, S2, qz, K=8, G=g["G"])
    assert np.array_equal(w_hat[0], g["scale"] * (np.array(g["q"], float) - g["zero"]))


def _grid_weights(N, K, G, seed):
    """Weights that sit exactly on the quantization grid: every group holds the
    codes 0 and 15, an fp16 scale and an integer zero in [0, 15]."""
    r = np.random.default_rng(seed)
    ng = K // G
    S = (2.0 ** r.integers(-12, -4, size=(N, ng)) * r.integers(1024, 2048, size=(N, ng)) / 1024)
    S = S.astype(np.float16)
    z = r.integers(0, 16, size=(N, ng)).astype(np.uint8)
    q = r.integers(0, 16, size=(N, ng, G)).astype(np.uint8)
    q[:, :, 0] = 0
    q[:, :, 1] = 15
    for n in range(N):                     # move the extremes around inside the group
        for gi in range(ng):
            r.shuffle(q[n, gi])
    W = S.astype(np.float32)[:, :, None] * (q.astype(np.float32) - z.astype(np.float32)[:, :, None])
    return W.reshape(N, K), q.reshape(N, K), S, z


def test_grid_points_are_reproduced_exactly():
    W, q, S, z = _grid_weights(32, 512, 128, seed=1)
    q2, S2, z2 = w4.quantize_rtn(W, 128)
    assert np.array_equal(q2, q)
    assert np.array_equal(S2.view(np.uint16), S.view(np.uint16))
    assert np.array_equal(z2, z)
    qw, S3, qz = w4.encode(W, 128)
    assert np.array_equal(w4.dequantize(qw, S3, qz, 512, 128), W.astype(np.float64))


def test_pack_unpack_round_trip_and_nibble_order():
    r = np.random.default_rng(2)
    q = r.integers(0, 16, size=(7, 11008)).astype(np.uint8)
    z = r.integers(0, 16, size=(7, 86)).astype(np.uint8)
    S = np.ones((7, 86), np.float16)
    qw, _, qz = w4.pack(q, S, z)
    assert qz.shape == (7, 11)                       # 86 zeros -> 11 words, 2 pad nibbles
    assert np.all((qz[:, -1] >> 24) == 0)
    q2, z2 = w4.unpack(qw, qz, 11008, 128)
    assert np.array_equal(q2, q) and np.array_equal(z2, z)
    seq = np.arange(1, 9, dtype=np.uint8)[None, :]  # codes 1..8 -> 0x87654321
    qw1, _, _ = w4.pack(seq, np.ones((1, 1), np.float16), np.zeros((1, 1), np.uint8))
    assert int(qw1[0, 0]) == 0x87654321


def test_rtn_half_step_bound():
    W = synth.normal_f32((64, 1024), 0.02, "pin/w4/rtn")
    q, S, z = w4.quantize_rtn(W, 128)
    s = S.astype(np.float64)
    w_hat = (s[:, :, None] * (q.reshape(64, 8, 128).astype(np.float64) - z[:, :, None])).reshape(64, 1024)
    inner = (q > 0) & (q < 15)
    step = np.repeat(s, 128, axis=1)
    err = np.abs(W.astype(np.float64) - w_hat)
    assert np.all(err[inner] <= step[inner] * (0.5 + 1e-6))
    # clamped entries can only be the group extremes, whose error is still below one step
    assert np.all(err <= step * (1.0 + 1e-6))


def test_forward_against_brute_force_sum():
    W = synth.normal_f32((5, 256), 0.02, "pin/w4/bf")
    X = synth.x_f16(3, 256, "pin/w4/bfx")
    qw, S, qz = w4.encode(W, 128)
    q, z = w4.unpack(qw, qz, 256, 128)
    Y = w4.forward(X, qw, S, qz, 256, 128)
    for m in range(3):
        for n in range(5):
            acc = 0.0
            for k in range(256):
                acc += float(X[m, k]) * float(S[n, k // 128]) * (int(q[n, k]) - int(z[n, k // 128]))
            assert abs(acc - Y[m, n]) <= 1e-12 * max(1.0, abs(acc))


def test_special_cases_single_group_single_row_and_batch_consistency():
    W = synth.normal_f32((4, 128), 0.02, "pin/w4/sc")
    X = synth.x_f16(4, 128, "pin/w4/scx")
    st = w4.encode(W, 128)                          # K = G: one group per row
    Y4 = w4.forward(X, *st, 128, 128)
    for m in range(4):                              # M = 1 equals one row of M = 4
        assert np.array_equal(w4.forward(X[m:m + 1], *st, 128, 128)[0], Y4[m])
    st1 = w4.encode(W[2:3], 128)                    # N = 1 encodes row 2 identically
    assert np.array_equal(st1[0][0], st[0][2]) and st1[1][0] == st[1][2]


def test_constant_zero_group_gets_unit_scale():
    W = np.zeros((1, 256), np.float32)
    W[0, 128:] = synth.normal_f32((1, 128), 0.02, "pin/w4/zero")
    q, S, z = w4.quantize_rtn(W, 128)
    assert float(S[0, 0]) == 1.0 and z[0, 0] == 0 and np.all(q[0, :128] == 0)


@pytest.mark.parametrize("K,G", [(1024, 128), (4096, 128), (11008, 128)])
def test_storage_sizes(K, G):
    W = synth.normal_f32((3, K), 0.02, f"pin/w4/size{K}")
    qw, S, qz = w4.encode(W, G)
    assert qw.shape == (3, K // 8) and S.shape == (3, K // G) and qz.shape == (3, (K // G + 7) // 8)
