"""Pins of the second-order encoders in the oracle (CPU).

GPTQ bulletin, "İddia ve Gerçeklik": second-order error model with the inverse
Hessian from the input covariance, Cholesky for stability, column-by-column
error feedback.  SpQR bulletin, "İddia ve Gerçeklik": outliers by Hessian-based
sensitivity.  Each pin below checks the oracle against something other than
its own formulas: round-to-nearest (H proportional to I), the Optimal Brain
Surgeon update written with explicit inverses of the not-yet-quantized block,
the calibration error the method exists to reduce, and hand-worked groups.
"""
import numpy as np
import pytest
import scipy.linalg

from oracle import gptq, spqr, w4

F32 = np.float32


def _weights(N, K, seed, sigma=0.02):
    return (np.random.default_rng(seed).standard_normal((N, K)) * sigma).astype(F32)


def _correlated_x(n, K, seed):
    g = np.random.default_rng(seed)
    A = g.standard_normal((K, K)) * 0.3 + np.eye(K)
    return (g.standard_normal((n, K)) @ A).astype(F32)


def test_hessian_of_orthogonal_rows_and_of_one_row():
    K = 64
    Hd = scipy.linalg.hadamard(K).astype(F32)          # rows orthogonal, X^T X = K I
    assert np.array_equal(gptq.hessian(Hd), 2.0 * np.eye(K))
    x = np.arange(1, 9, dtype=F32)[None, :]
    assert np.array_equal(gptq.hessian(x), 2.0 * np.outer(x[0], x[0]).astype(np.float64))


@pytest.mark.parametrize("G", [32, 128])
@pytest.mark.parametrize("kind", ["hadamard", "scaled_identity", "zero"])
def test_identity_hessian_reduces_to_round_to_nearest(G, kind):
    """With H proportional to I, U is diagonal, no error is fed forward and the
    encode is round-to-nearest bit for bit (scales, zeros and codes)."""
    N, K = 24, 256
    W = _weights(N, K, 1)
    if kind == "hadamard":
        H = gptq.hessian(scipy.linalg.hadamard(K).astype(F32))
    elif kind == "scaled_identity":
        H = 3.7 * np.eye(K)
    else:
        H = np.zeros((K, K))                           # no calibration signal: H = I
    q, S, z = gptq.quantize_w4(W, H, G)
    q0, S0, z0 = w4.quantize_rtn(W, G)
    assert np.array_equal(q, q0)
    assert np.array_equal(S.view(np.uint16), S0.view(np.uint16))
    assert np.array_equal(z, z0)


def test_cholesky_form_equals_sequential_obs_with_explicit_inverses():
    """Brute force: quantize column j, then move the not-yet-quantized weights F
    by the Optimal Brain Surgeon update -(w_j - w_hat_j) [H_F^-1][:, j] /
    [H_F^-1][j, j], with H_F^-1 the explicit inverse of the damped H restricted
    to F = {j, ..., K-1}, recomputed at every step.  The oracle's Cholesky form
    must give the same codes and scales."""
    N, K, G = 5, 128, 32
    W = _weights(N, K, 2)
    H = gptq.hessian(_correlated_x(200, K, 3))
    Hd = gptq.damped(H)
    q_ref = np.zeros((N, K), np.uint8)
    S_ref = np.zeros((N, K // G), np.float16)
    for n in range(N):
        w = W[n].astype(np.float64)
        for j in range(K):
            if j % G == 0:
                S_ref[n, j // G], s, z = gptq._group_rule(w[j:j + G].astype(F32))
            qj = np.clip(np.rint(F32(w[j]) / s) + z, F32(0), F32(15))
            q_ref[n, j] = np.uint8(qj)
            w_hat = np.float64(s) * (np.float64(qj) - np.float64(z))
            Finv = np.linalg.inv(Hd[j:, j:])
            w[j:] -= (w[j] - w_hat) * Finv[:, 0] / Finv[0, 0]
    q, S, _ = gptq.quantize_w4(W, H, G)
    assert np.array_equal(S.view(np.uint16), S_ref.view(np.uint16))
    assert np.array_equal(q, q_ref)


@pytest.mark.parametrize("seed,G", [(4, 128), (5, 64), (6, 32)])
def test_error_feedback_reduces_the_calibration_error(seed, G):
    """The point of the method: on correlated calibration inputs the layer
    output error ||X (W_hat - W)^T|| is clearly below round-to-nearest's."""
    N, K = 48, 256
    W = _weights(N, K, seed)
    X = _correlated_x(400, K, seed + 100)
    H = gptq.hessian(X)

    def err(st):
        return np.linalg.norm(X.astype(np.float64) @ (w4.dequantize(*st, K, G) - W.astype(np.float64)).T)

    e_gptq = err(gptq.encode_w4(W, H, G))
    e_rtn = err(w4.encode(W, G))
    assert e_gptq < 0.85 * e_rtn, (e_gptq, e_rtn)


def _fixture_layer():
    """One row of 256 weights (16 groups of 16), hand-worked:

    group 0 = 0..6, 0..6, 63, 70: full min/max quantization has s = 10 and
      squared errors 71 + 71 + 9 + 0 = 151; without the 70, s = 9 and the
      rest costs 110, so its sensitivity is 41 (without the 63 it is 9);
    group 1 = 5 * (0..7, 0..6), 70: s = 10 and squared errors
      25 * (4 + 3) = 175; without the 70 every value sits on the grid of
      step 5 (error 0), so the 70 of group 1 has sensitivity 175;
    groups 2..15 = 0 (no error, sensitivity 0).
    """
    w = np.zeros((1, 256), F32)
    w[0, 0:14] = list(range(7)) * 2
    w[0, 14], w[0, 15] = 63, 70
    w[0, 16:31] = [5 * v for v in list(range(8)) + list(range(7))]
    w[0, 31] = 70
    return w


def test_sensitivity_hand_worked_groups():
    W = _fixture_layer()
    H = np.eye(256)                    # damped: every c_k = 1.01
    s = gptq.spqr_sensitivity(W, H)
    assert s[0, 15] == pytest.approx(41 * 1.01, rel=1e-12)
    assert s[0, 14] == pytest.approx(9 * 1.01, rel=1e-12)
    assert s[0, 31] == pytest.approx(175 * 1.01, rel=1e-12)
    assert np.all(s[0, 32:] == 0)
    # one outlier: magnitude takes the first 70 (lower index), sensitivity the second
    p = 1.0 / 256
    assert np.flatnonzero(spqr.select_outliers(W, 1)).tolist() == [15]
    assert np.flatnonzero(gptq.spqr_select_outliers(W, H, p)).tolist() == [31]


def test_sensitivity_follows_the_input_energy_of_the_column():
    """The same group in two places; the copy whose columns carry 4x the input
    energy (diagonal of H) is 4x as sensitive and is chosen first."""
    W = np.zeros((1, 256), F32)
    W[0, 16:32] = _fixture_layer()[0, 16:32]
    W[0, 64:80] = W[0, 16:32]
    c = np.ones(256)
    c[64:80] = 4.0
    H = np.diag(c)
    s = gptq.spqr_sensitivity(W, H)
    lam = 0.01 * np.mean(c)
    assert s[0, 31] == pytest.approx(175 * (1 + lam), rel=1e-12)
    assert s[0, 79] == pytest.approx(175 * (4 + lam), rel=1e-12)
    assert np.flatnonzero(gptq.spqr_select_outliers(W, H, 1.0 / 256)).tolist() == [79]


def test_sensitivity_is_invariant_to_the_scale_of_H():
    W = (np.random.default_rng(7).standard_t(3, (8, 256)) * 0.02).astype(F32)
    H = gptq.hessian(_correlated_x(100, 256, 8))
    m1 = gptq.spqr_select_outliers(W, H, 0.02)
    m2 = gptq.spqr_select_outliers(W, 1000.0 * H, 0.02)
    assert np.array_equal(m1, m2)
    assert m1.sum() == spqr.n_outliers(8, 256, 0.02)


def test_sensitivity_outliers_keep_the_storage_rules():
    """Outliers chosen by sensitivity leave the dense part exactly as the
    magnitude path does: the encode with that mask is the same function."""
    W = (np.random.default_rng(9).standard_t(3, (16, 512)) * 0.02).astype(F32)
    H = gptq.hessian(_correlated_x(100, 512, 10))
    mask = gptq.spqr_select_outliers(W, H, 0.01)
    st = gptq.encode_spqr(W, H, 0.01)
    ref = spqr.encode(W, 0.01, mask)
    for k in ref:
        assert np.array_equal(np.asarray(st[k]).view(np.uint8), np.asarray(ref[k]).view(np.uint8)), k
    rows = np.repeat(np.arange(16), np.diff(st["row_ptr"]))
    assert np.array_equal(np.flatnonzero(mask), rows * 512 + st["col_idx"])


def _energy_x(n, K, seed):
    """Correlated inputs whose channels carry very different energies (the case
    act-order is for)."""
    g = np.random.default_rng(seed)
    A = g.standard_normal((K, K)) * (3.0 / np.sqrt(K)) + np.eye(K)
    gain = np.exp(g.standard_normal(K) * 0.7)
    return ((g.standard_normal((n, K)) @ A) * gain).astype(F32)


@pytest.mark.parametrize("static_groups", [True, False])
def test_act_order_with_a_flat_diagonal_is_the_natural_order(static_groups):
    """diag(H) constant: the order is the natural one (ties to the lower index),
    so both act-order variants equal the natural-order encode."""
    N, K, G = 16, 256, 64
    W = _weights(N, K, 20)
    X = _correlated_x(300, K, 21)
    X /= np.sqrt(np.mean(X.astype(np.float64) ** 2, axis=0))[None, :].astype(F32)   # unit-energy columns
    H = gptq.hessian(X)
    H[np.diag_indices(K)] = 2.0                         # flat diagonal, same correlations
    q, S, z, perm = gptq.quantize_w4_actorder(W, H, G, static_groups=static_groups)
    assert np.array_equal(perm, np.arange(K))
    q0, S0, z0 = gptq.quantize_w4(W, H, G)
    if static_groups:
        # natural order, but statistics from the original weights
        assert np.array_equal(S.view(np.uint16), w4.quantize_rtn(W, G)[1].view(np.uint16))
    else:
        assert np.array_equal(q, q0) and np.array_equal(S.view(np.uint16), S0.view(np.uint16))
        assert np.array_equal(z, z0)


def test_static_groups_keep_round_to_nearest_statistics_and_match_brute_force():
    """Static groups: scales and zeros are round-to-nearest's bit for bit; the
    codes equal a brute-force Optimal Brain Surgeon pass in act-order that
    re-inverts the damped H on the not-yet-quantized columns at every step."""
    N, K, G = 4, 128, 32
    W = _weights(N, K, 22)
    H = gptq.hessian(_energy_x(300, K, 23))
    q, S, z, perm = gptq.quantize_w4_actorder(W, H, G, static_groups=True)
    q0, S0, z0 = w4.quantize_rtn(W, G)
    assert np.array_equal(S.view(np.uint16), S0.view(np.uint16)) and np.array_equal(z, z0)
    order = np.argsort(-np.diag(H), kind="stable")
    assert np.all(np.diff(np.diag(H)[order]) <= 0)
    Hd = gptq.damped(H[np.ix_(order, order)])
    s0 = S0.astype(F32)
    q_ref = np.zeros((N, K), np.uint8)
    for n in range(N):
        w = W[n, order].astype(np.float64)
        for t in range(K):
            j = order[t]
            s, zz = s0[n, j // G], F32(z0[n, j // G])
            qj = np.clip(np.rint(F32(w[t]) / s) + zz, F32(0), F32(15))
            q_ref[n, j] = np.uint8(qj)
            Finv = np.linalg.inv(Hd[t:, t:])
            w[t:] -= (w[t] - np.float64(s) * (np.float64(qj) - np.float64(zz))) * Finv[:, 0] / Finv[0, 0]
    assert np.array_equal(q, q_ref)


def test_act_order_forward_reads_the_activations_through_perm():
    """Closed form: X[:, perm] . W_stored^T = X . W_natural^T with the stored
    columns scattered back to their input columns."""
    N, K, G = 24, 256, 128
    W = _weights(N, K, 24)
    X = _energy_x(64, K, 25)
    st = gptq.encode_w4_actorder(W, gptq.hessian(X), G, static_groups=False)
    perm = st[3]
    assert sorted(perm.tolist()) == list(range(K))
    Wst = w4.dequantize(*st[:3], K, G)
    Wnat = np.empty_like(Wst)
    Wnat[:, perm] = Wst
    Xh = X.astype(np.float16)
    assert np.allclose(gptq.forward_perm(Xh, *st, K, G), Xh.astype(np.float64) @ Wnat.T, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("static_groups", [True, False])
def test_act_order_reduces_the_error_where_channel_energies_differ(static_groups):
    N, K, G = 48, 512, 128
    W = _weights(N, K, 26)
    X = _energy_x(600, K, 27)
    H = gptq.hessian(X)
    ex = X.astype(np.float64) @ W.astype(np.float64).T
    e_nat = np.linalg.norm(w4.forward(X.astype(np.float16), *gptq.encode_w4(W, H, G), K, G) - ex)
    st = gptq.encode_w4_actorder(W, H, G, static_groups=static_groups)
    Y = gptq.forward_perm(X.astype(np.float16), *st, K, G)
    e_act = np.linalg.norm(Y - ex)
    assert e_act < 0.9 * e_nat, (e_act, e_nat)
