"""GPU parity of SmoothQuant W8A8 against the oracle: int8 activations, their
scales and the int32 accumulators bit for bit; fp16 outputs within tolerance."""
import numpy as np
import pytest

import synth
from oracle import smoothquant as osq
from quantized_linear_layers_packed_amd import qlin
from tests.gpu_util import check_close, dev, empty, host, say, sq_ws, torch_cuda

pytestmark = pytest.mark.gpu

F16, F32 = qlin.QLIN_F16, qlin.QLIN_F32


def gpu_act(X, inv_s):
    torch = torch_cuda()
    M, K = X.shape
    Xq = empty((M, K), torch.int8)
    xs = empty((M,), torch.float32)
    qlin.sq_smooth_quant_act(dev(X), dev(inv_s), M, K, Xq, xs)
    return Xq, xs


def gpu_gemm(Xq_d, xs_d, Wq_d, ws_d, M, N, K, y_dtype=F16, want_acc=True):
    torch = torch_cuda()
    Y = empty((M, N), torch.float16 if y_dtype == F16 else torch.float32)
    acc = empty((M, N), torch.int32) if want_acc else None
    qlin.sq_int8_gemm(Xq_d, xs_d, Wq_d, ws_d, M, N, K, Y, y_dtype, acc, workspace=sq_ws(M, N, K, y_dtype))
    return host(Y).astype(np.float64), (host(acc) if want_acc else None)


def test_activation_quantization_is_bit_exact():
    X = synth.activations("sq_w8a8", 0, 2048)
    W = synth.layer_weight("sq_w8a8", 1)
    _, inv_s, _, _ = osq.pack(W, synth.sq_calibration("sq_w8a8", 1), 0.85)
    X = X.copy()
    X[5] = 0.0                                        # an all-zero token
    for M in (1, 3, 256, 512, 2048):
        say(f"sq act M={M}")
        Xq_d, xs_d = gpu_act(X[:M], inv_s)
        Xq_o, xs_o = osq.quantize_act(X[:M], inv_s)
        assert np.array_equal(host(Xq_d), Xq_o)
        assert host(xs_d).tobytes() == xs_o.tobytes()
    # rows longer than the values a thread keeps in registers (8192) are partly
    # read again in the quantize pass; rows shorter than one group per thread
    r = np.random.default_rng(5)
    for (M, K) in ((5, 11008), (3, 40), (2, 20000)):
        say(f"sq act M={M} K={K}")
        Xk = (r.standard_normal((M, K)) * 2).astype(np.float16)
        Xk[0, K // 3] = 300.0                          # an outlier channel value
        inv_k = r.uniform(0.2, 5.0, K).astype(np.float32)
        Xq_d, xs_d = gpu_act(Xk, inv_k)
        Xq_o, xs_o = osq.quantize_act(Xk, inv_k)
        assert np.array_equal(host(Xq_d), Xq_o)
        assert host(xs_d).tobytes() == xs_o.tobytes()


@pytest.mark.parametrize("layer", [0, 1])
def test_full_layer_end_to_end(layer):
    N, K = synth.WORKLOADS["sq_w8a8"]["layers"][layer]
    W = synth.layer_weight("sq_w8a8", layer)
    Xcal = synth.sq_calibration("sq_w8a8", layer)
    s, inv_s = qlin.sq_compute_smoothing(qlin.sq_act_absmax(Xcal), W, 0.85)
    Wq, ws = qlin.sq_pack_weight(W, s)
    S_o, inv_o, Wq_o, ws_o = osq.pack(W, Xcal, 0.85)
    assert inv_s.tobytes() == inv_o.tobytes() and Wq.tobytes() == Wq_o.tobytes() and ws.tobytes() == ws_o.tobytes()
    Wq_d, ws_d, inv_d = dev(Wq), dev(ws), dev(inv_s)
    cols = np.unique(np.r_[0, N - 1, np.random.default_rng(layer).choice(N, 510, replace=False)])
    for M in (256, 512, 2048):
        say(f"sq_w8a8 layer {layer} {N}x{K} M={M}")
        X = synth.activations("sq_w8a8", layer, M)
        Xq_d, xs_d = gpu_act(X, inv_s)
        Y, acc = gpu_gemm(Xq_d, xs_d, Wq_d, ws_d, M, N, K)
        Y_o, Xq_o, xs_o, acc_o = osq.forward(X, inv_o, Wq_o[cols], ws_o[cols])
        assert np.array_equal(host(Xq_d), Xq_o)
        assert np.array_equal(acc[:, cols], acc_o), "int32 accumulators differ"
        check_close(Y[:, cols], Y_o, f"{N}x{K} M={M}")


# (33, 64, 128) and (60, 3000, 512) reach the wave-grid kernel's 64 x 128 tiles (33..64
# tokens, K a multiple of 128); from (520, 1000, 1024) on, its tile sizes for more than 64
# tokens: 128 x 64 (ragged M and N, a single K step at K = 128, M = 65), 128 x 128
# (200 x 11000: 172 tiles) and 256 x 128 (600 x 8192: 192 tiles), and 8 output columns
# (every weight row past N clamped); the last shape (K % 128 = 64) and (300, 40, 320)
# fall back to the 32 TM x 128 kernel.
# Up to 2 tokens with rows up to 32768 the GEMV runs, with 1, 2, 4 or 8 waves per row of 1 to 4
# blocks of 1 KB each: (1, 100, 64) one wave of one block, (2, 333, 5120) 2 x 3, (1, 700, 11008)
# 4 x 3 (one block past the row end), (2, 90, 12352) 4 x 4, (1, 257, 20480) 8 x 3 and
# (2, 5000, 32768) 8 x 4; up to 4 tokens where K is not a multiple of 128: (3, 129, 192);
# (1, 64, 40000) falls back to the 32 TM x 128 kernel.  3..32 tokens with K a multiple of 128 run the small-batch kernel: one
# 16-column tile per workgroup (4 x 300, 5 x 1000, 9 x 5200), two (16 x 11008: 344 workgroups),
# four (8 x 19300: 302), and two 16-token tiles with one (24 x 77) or two column tiles (32 x 6000).
RAGGED = ((1, 100, 64), (3, 129, 192), (4, 300, 4096), (2, 5000, 32768), (1, 64, 40000),
          (2, 333, 5120), (1, 700, 11008), (2, 90, 12352), (1, 257, 20480),
          (5, 1000, 640), (9, 5200, 256), (16, 11008, 512), (8, 19300, 256), (24, 77, 1024), (32, 6000, 384),
          (33, 64, 128), (60, 3000, 512), (100, 257, 4096), (300, 40, 320),
          (520, 1000, 1024), (1100, 130, 128), (65, 16400, 256), (300, 6000, 512),
          (200, 11000, 384), (600, 8192, 256), (520, 8, 256), (513, 300, 4160))


def test_gemm_ragged_shapes():
    r = np.random.default_rng(11)
    for (M, N, K) in RAGGED:
        say(f"sq gemm M={M} N={N} K={K}")
        Xq = r.integers(-127, 128, size=(M, K)).astype(np.int8)
        Wq = r.integers(-127, 128, size=(N, K)).astype(np.int8)
        Xq[0, :] = 127
        Wq[0, :] = -127
        # scales sized like real ones (absmax / 127) so that |Y| stays inside fp16 range
        xs = r.uniform(1e-3, 1e-2, M).astype(np.float32)
        ws = r.uniform(1e-4, 1e-3, N).astype(np.float32)
        Y, acc = gpu_gemm(dev(Xq), dev(xs), dev(Wq), dev(ws), M, N, K, F32)
        acc_o = osq.int_gemm(Xq, Wq)
        assert np.array_equal(acc, acc_o)
        check_close(Y, osq.dequant_output(acc_o, xs, ws), "f32 out")
        Y16, _ = gpu_gemm(dev(Xq), dev(xs), dev(Wq), dev(ws), M, N, K, F16, want_acc=False)
        check_close(Y16, osq.dequant_output(acc_o, xs, ws), "f16 out")


def test_every_int8_kernel_gives_the_same_accumulators():
    """int32 accumulation is exact, so the int8 kernels agree bit for bit on the rows
    they share: prefixes of one batch through the GEMV (2 tokens), the small-batch
    kernel (5 and 24 tokens), the 64 x 128 wave-grid tiles (40), the larger wave-grid
    tiles (300) and, with K not a multiple of 128, the 32 TM x 128 kernel (the oracle
    checks the longest prefix)."""
    r = np.random.default_rng(21)
    for K in (2048, 2112):
        N = 1500
        Xq = r.integers(-127, 128, size=(300, K)).astype(np.int8)
        Wq = r.integers(-127, 128, size=(N, K)).astype(np.int8)
        xs = r.uniform(1e-3, 1e-2, 300).astype(np.float32)
        ws = r.uniform(1e-4, 1e-3, N).astype(np.float32)
        Wq_d, ws_d = dev(Wq), dev(ws)
        accs = {}
        for M in (2, 5, 24, 40, 300):
            say(f"sq int8 kernels K={K} M={M}")
            _, accs[M] = gpu_gemm(dev(Xq[:M]), dev(xs[:M]), Wq_d, ws_d, M, N, K, F32)
        assert np.array_equal(accs[300], osq.int_gemm(Xq, Wq))
        for M in (2, 5, 24, 40):
            assert np.array_equal(accs[M], accs[300][:M]), f"M={M} differs from the first rows of M=300"
