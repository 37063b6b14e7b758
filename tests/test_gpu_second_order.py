"""Second-order encodes through the unchanged GPU kernels (C ABI).

The GPTQ-style and Hessian-sensitivity SpQR encoders write the same storage as
the round-to-nearest and magnitude encoders, so the forward kernels run
unchanged: their outputs must match the fp64 oracle's forward of that storage
within tolerance, and on the calibration inputs the GPTQ-encoded layer must
land closer to the unquantized product than the round-to-nearest one."""
import numpy as np
import pytest

from oracle import spqr as ospqr
from oracle import w4 as ow4
from quantized_linear_layers_packed_amd import qlin
from tests.gpu_util import check_close, dev, empty, host, say, spqr_ws, torch_cuda, w4_ws

pytestmark = pytest.mark.gpu

F16, F32 = qlin.QLIN_F16, qlin.QLIN_F32


def _calibration(n, K, seed):
    """fp16 activations with correlated channels (a random mixing of N(0,1))."""
    g = np.random.default_rng(seed)
    A = g.standard_normal((K, K)) * (0.5 / np.sqrt(K)) + np.eye(K)
    return (g.standard_normal((n, K)) @ A).astype(np.float16)


def _w4_gpu(X, packed, N, K, G):
    torch = torch_cuda()
    M = X.shape[0]
    Y = empty((M, N), torch.float32)
    qw, sc, qz = (dev(a) for a in packed)
    qlin.qlin_w4_forward(dev(X), F16, M, K, qw, sc, qz, N, G, Y, F32, workspace=w4_ws(F16, M, K, N, G, F32))
    return host(Y).astype(np.float64)


def test_gptq_encode_through_gemv_and_gemm():
    N, K, G = 1024, 2048, 128
    W = (np.random.default_rng(11).standard_normal((N, K)) * 0.02).astype(np.float32)
    Xc = _calibration(256, K, 12)
    H = qlin.qlin_hessian(Xc.astype(np.float32))
    gq = qlin.qlin_w4_pack_gptq(W, G, H)
    rtn = qlin.qlin_w4_pack(W, G)
    exact = Xc.astype(np.float64) @ W.astype(np.float64).T
    for M in (1, 8, 64, 256):
        say(f"gptq-encoded W4 N={N} K={K} M={M}")
        X = Xc[:M]
        y = _w4_gpu(X, gq, N, K, G)
        check_close(y, ow4.forward(X, *gq, K, G), f"gptq M={M}")
        if M == 256:
            e_g = np.linalg.norm(y - exact[:M])
            e_r = np.linalg.norm(_w4_gpu(X, rtn, N, K, G) - exact[:M])
            say(f"  calibration output error: gptq {e_g:.4e} vs round-to-nearest {e_r:.4e}")
            assert e_g < 0.9 * e_r


def test_sensitivity_spqr_encode_through_the_fused_kernel():
    N, K = 512, 2048
    W = (np.random.default_rng(13).standard_t(3, (N, K)) * 0.02).astype(np.float32)
    Xc = _calibration(128, K, 14)
    H = qlin.qlin_hessian(Xc.astype(np.float32))
    st = qlin.spqr_pack_hessian(W, 0.01, H)
    d = {k: dev(np.ascontiguousarray(v)) for k, v in st.items()}
    torch = torch_cuda()
    for M in (1, 4, 16):
        say(f"sensitivity-encoded SpQR N={N} K={K} M={M}")
        X = Xc[:M]
        Y = empty((M, N), torch.float32)
        nnz = len(st["val"])
        qlin.spqr_forward(dev(X), M, K, d["codes"], d["stats1"], d["stats2"], d["row_ptr"],
                          d["col_idx"], d["val"], nnz, N, Y, F32, workspace=spqr_ws(M, K, N, F32))
        check_close(host(Y).astype(np.float64), ospqr.forward(X, st, K), f"spqr M={M}")


@pytest.mark.parametrize("G", [128, 64])
def test_act_order_forward_through_the_gather(G):
    """Act-order storage without static groups runs through qlin_w4_forward_perm
    (gather of X by perm, then the regular kernels): parity with the oracle's
    X[:, perm] . W_stored^T at GEMV (M = 1, 3) and MFMA batch sizes; with static
    groups the storage is natural and runs through qlin_w4_forward; an identity
    perm gives qlin_w4_forward's result bit for bit."""
    from oracle import gptq as ogptq
    torch = torch_cuda()
    N, K = 640, 2048
    g = np.random.default_rng(15)
    W = (g.standard_normal((N, K)) * 0.02).astype(np.float32)
    Xc = (_calibration(256, K, 16).astype(np.float32) * np.exp(g.standard_normal(K) * 0.7)).astype(np.float16)
    H = qlin.qlin_hessian(Xc.astype(np.float32))
    dyn = qlin.qlin_w4_pack_gptq_actorder(W, G, H, static_groups=False)
    sta = qlin.qlin_w4_pack_gptq_actorder(W, G, H, static_groups=True)
    qw, sc, qz, perm = (dev(a) for a in dyn)
    ident = dev(np.arange(K, dtype=np.int32))
    for M in (1, 3, 8, 64):
        say(f"act-order W4 N={N} K={K} G={G} M={M}")
        X = Xc[:M]
        Xd = dev(X)
        Xp = empty((M, K), torch.float16)
        Y = empty((M, N), torch.float32)
        wsp = w4_ws(F16, M, K, N, G, F32)
        qlin.qlin_w4_forward_perm(Xd, F16, M, K, perm, Xp, qw, sc, qz, N, G, Y, F32, workspace=wsp)
        check_close(host(Y).astype(np.float64), ogptq.forward_perm(X, *dyn, K, G), f"dynamic groups M={M}")
        check_close(_w4_gpu(X, sta[:3], N, K, G), ow4.forward(X, *sta[:3], K, G), f"static groups M={M}")
        Y1 = empty((M, N), torch.float32)
        qlin.qlin_w4_forward_perm(Xd, F16, M, K, ident, Xp, qw, sc, qz, N, G, Y1, F32, workspace=wsp)
        Y2 = empty((M, N), torch.float32)
        qlin.qlin_w4_forward(Xd, F16, M, K, qw, sc, qz, N, G, Y2, F32, workspace=wsp)
        assert np.array_equal(host(Y1), host(Y2))
