"""Pins of the dense fp16 oracle: explicit loops on tiny inputs, unit rows that
select weight rows, a hand-worked product, exact small-integer products at
every size used on the GPU, and a transposed-operand check that fails if X and
W trade places."""
import numpy as np

from oracle import dense


def test_matches_explicit_loops_on_tiny_inputs():
    g = np.random.default_rng(1)
    X = (g.standard_normal((3, 5))).astype(np.float16)
    W = (g.standard_normal((4, 5))).astype(np.float16)
    Y = dense.forward(X, W)
    for m in range(3):
        for n in range(4):
            s = 0.0
            for k in range(5):
                s += float(X[m, k]) * float(W[n, k])
            assert abs(Y[m, n] - s) <= 1e-12 * max(1.0, abs(s))


def test_hand_worked_product():
    X = np.array([[1, 2], [-0.5, 4]], np.float16)
    W = np.array([[3, -1], [0.25, 0.5], [2, 2]], np.float16)
    # row 0: [1*3 + 2*-1, 1*0.25 + 2*0.5, 1*2 + 2*2] = [1, 1.25, 6]
    # row 1: [-1.5 - 4, -0.125 + 2, -1 + 8]        = [-5.5, 1.875, 7]
    assert dense.forward(X, W).tolist() == [[1.0, 1.25, 6.0], [-5.5, 1.875, 7.0]]


def test_unit_rows_select_weight_rows():
    g = np.random.default_rng(2)
    W = g.standard_normal((7, 64)).astype(np.float16)
    X = np.zeros((3, 64), np.float16)
    X[0, 5] = 1
    X[1, 63] = 1
    X[2, 0] = -2
    Y = dense.forward(X, W)
    assert np.array_equal(Y[0], W[:, 5].astype(np.float64))
    assert np.array_equal(Y[1], W[:, 63].astype(np.float64))
    assert np.array_equal(Y[2], -2 * W[:, 0].astype(np.float64))


def test_not_transposed():
    """A square product where X W^T != W X^T: swapping the operands fails."""
    X = np.array([[1, 0], [0, 0]], np.float16)
    W = np.array([[0, 0], [1, 0]], np.float16)
    assert dense.forward(X, W).tolist() == [[0.0, 1.0], [0.0, 0.0]]


def test_small_integers_are_exact():
    g = np.random.default_rng(3)
    X = g.integers(-3, 4, (9, 320)).astype(np.float16)
    W = g.integers(-3, 4, (11, 320)).astype(np.float16)
    ref = X.astype(np.int64) @ W.astype(np.int64).T
    assert np.array_equal(dense.forward(X, W), ref.astype(np.float64))


def test_column_subset():
    g = np.random.default_rng(4)
    X = g.standard_normal((2, 64)).astype(np.float16)
    W = g.standard_normal((10, 64)).astype(np.float16)
    cols = [0, 3, 9]
    assert np.array_equal(dense.forward_cols(X, W, cols), dense.forward(X, W)[:, cols])
