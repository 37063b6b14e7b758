"""Library host encoders (second order) against the oracle, byte for byte (CPU).

The library's GPTQ-style encoder and its Hessian-sensitivity SpQR encoder are an
independent C++ implementation of the readings the oracle follows; given the
same Hessian both must produce identical storage."""
import numpy as np
import pytest

from oracle import gptq
from quantized_linear_layers_packed_amd import qlin

F32 = np.float32


def _correlated_x(n, K, seed):
    g = np.random.default_rng(seed)
    A = g.standard_normal((K, K)) * 0.3 + np.eye(K)
    return (g.standard_normal((n, K)) @ A).astype(F32)


def _same(a, b):
    a, b = np.asarray(a), np.asarray(b)
    return a.shape == b.shape and np.array_equal(a.view(np.uint8), b.view(np.uint8))


def test_hessian_matches():
    X = _correlated_x(300, 384, 1)
    H = qlin.qlin_hessian(X)
    Ho = gptq.hessian(X)
    assert np.array_equal(H, H.T)
    assert np.max(np.abs(H - Ho)) <= 1e-12 * np.max(np.abs(Ho))


@pytest.mark.parametrize("N,K,G", [(64, 256, 128), (96, 512, 64), (40, 512, 256), (33, 384, 32), (200, 1024, 128)])
def test_gptq_storage_identical(N, K, G):
    W = (np.random.default_rng(N + K).standard_normal((N, K)) * 0.02).astype(F32)
    H = gptq.hessian(_correlated_x(256, K, K))
    lib = qlin.qlin_w4_pack_gptq(W, G, H)
    ref = gptq.encode_w4(W, H, G)
    for a, b in zip(lib, ref):
        assert _same(a, b)


def test_gptq_with_identity_hessian_is_round_to_nearest():
    W = (np.random.default_rng(3).standard_normal((50, 512)) * 0.02).astype(F32)
    for H in (np.eye(512) * 2.5, np.zeros((512, 512))):
        for a, b in zip(qlin.qlin_w4_pack_gptq(W, 128, H), qlin.qlin_w4_pack(W, 128)):
            assert _same(a, b)


@pytest.mark.parametrize("N,K,p", [(48, 512, 0.01), (16, 256, 0.05), (20, 768, 0.0)])
def test_sensitivity_spqr_storage_identical(N, K, p):
    W = (np.random.default_rng(N * K).standard_t(3, (N, K)) * 0.02).astype(F32)
    H = gptq.hessian(_correlated_x(128, K, N))
    lib = qlin.spqr_pack_hessian(W, p, H)
    ref = gptq.encode_spqr(W, H, p)
    for k in ref:
        assert _same(lib[k], ref[k]), k


def test_second_order_calls_reject_bad_arguments():
    W = np.zeros((4, 256), F32)
    H = np.eye(256)
    Hasym = H.copy()
    Hasym[0, 1] = 1e-3
    Hnan = H.copy()
    Hnan[3, 3] = np.nan
    for bad, st in ((Hasym, qlin.QLIN_EINVAL), (Hnan, qlin.QLIN_EINVAL)):
        with pytest.raises(qlin.QlinError) as e:
            qlin.qlin_w4_pack_gptq(W, 128, bad)
        assert e.value.status == st
        with pytest.raises(qlin.QlinError) as e:
            qlin.spqr_pack_hessian(W, 0.01, bad)
        assert e.value.status == st
    # singular H with no damping cannot be inverted
    x = np.ones((3, 256), F32)
    with pytest.raises(qlin.QlinError) as e:
        qlin.qlin_w4_pack_gptq(W, 128, qlin.qlin_hessian(x), damp=0.0)
    assert e.value.status == qlin.QLIN_EINVAL and "positive definite" in str(e.value)
    with pytest.raises(qlin.QlinError):
        qlin.qlin_w4_pack_gptq(W, 128, H, damp=-1.0)
    with pytest.raises(qlin.QlinError):
        qlin.qlin_hessian(np.zeros((0, 8), F32))


@pytest.mark.parametrize("static_groups", [True, False])
@pytest.mark.parametrize("N,K,G", [(40, 512, 128), (33, 256, 32), (64, 1024, 256)])
def test_act_order_storage_identical(N, K, G, static_groups):
    g = np.random.default_rng(N + K + G)
    W = (g.standard_normal((N, K)) * 0.02).astype(F32)
    X = _correlated_x(256, K, K + 1) * np.exp(g.standard_normal(K) * 0.7).astype(F32)
    H = gptq.hessian(X)
    lib = qlin.qlin_w4_pack_gptq_actorder(W, G, H, static_groups=static_groups)
    ref = gptq.encode_w4_actorder(W, H, G, static_groups=static_groups)
    for a, b in zip(lib, ref):
        assert _same(a, b)
