"""GPU parity of the dense fp16 GEMM (the 16-bit baseline layer) against the
fp64 oracle, through the C ABI."""
import numpy as np
import pytest

import synth
from oracle import dense as odense
from quantized_linear_layers_packed_amd import qlin
from tests.gpu_util import check_close, dev, empty, host, say, torch_cuda, workspace

pytestmark = pytest.mark.gpu

F16, BF16, F32 = qlin.QLIN_F16, qlin.QLIN_BF16, qlin.QLIN_F32

# single tiles, ragged rows / columns, several K steps, every tile size of the
# kernel choice (M <= 64, and 128 x 64 / 128 x 128 / 256 x 128 tiles above)
SHAPES = [(1, 37, 64), (3, 129, 128), (17, 200, 192), (64, 128, 640), (65, 257, 1024), (130, 300, 256),
          (257, 513, 2048), (600, 4096, 512), (1100, 4096, 256)]


def gpu_dense(X, W, y_dtype):
    torch = torch_cuda()
    M, K = X.shape
    N = W.shape[0]
    Y = empty((M, N), {F16: torch.float16, BF16: torch.bfloat16, F32: torch.float32}[y_dtype])
    qlin.qlin_f16_gemm(dev(X), dev(W), M, N, K, Y, y_dtype, workspace=workspace(
        qlin.qlin_f16_gemm_workspace_bytes(M, N, K, y_dtype)))
    return Y


@pytest.mark.parametrize("shape", SHAPES)
def test_small_integers_are_exact(shape):
    """Integers in [-3, 3]: every partial sum is an integer below 2^24, so the
    fp32 result is exact whatever the summation order."""
    M, N, K = shape
    say(f"dense f16 integers M={M} N={N} K={K}")
    g = np.random.default_rng(M * 7 + N)
    X = g.integers(-3, 4, (M, K)).astype(np.float16)
    W = g.integers(-3, 4, (N, K)).astype(np.float16)
    y = host(gpu_dense(X, W, F32)).astype(np.float64)
    assert np.array_equal(y, odense.forward(X, W))


@pytest.mark.parametrize("shape", SHAPES)
def test_random_values_within_tolerance(shape):
    M, N, K = shape
    say(f"dense f16 random M={M} N={N} K={K}")
    X = synth.x_f16(M, K, f"gpu/dense/x{M}_{K}")
    W = synth.normal_f32((N, K), 0.02, f"gpu/dense/w{N}_{K}").astype(np.float16)
    ref = odense.forward(X, W)
    y32 = host(gpu_dense(X, W, F32))
    check_close(y32.astype(np.float64), ref, "f32 out")
    check_close(host(gpu_dense(X, W, F16)).astype(np.float64), ref, "f16 out")
    # f16 / bf16 outputs are the fp32 result rounded once (nearest even)
    torch = torch_cuda()
    assert np.array_equal(host(gpu_dense(X, W, F16)), y32.astype(np.float16))
    yb = gpu_dense(X, W, BF16)
    assert torch.equal(yb.cpu(), torch.from_numpy(y32).to(torch.bfloat16))


@pytest.mark.parametrize("layer", [0, 1, 2])
def test_llama7b_layers_sampled_columns(layer):
    N, K = synth.WORKLOADS["w4_llama7b"]["layers"][layer]
    W = synth.layer_weight("w4_llama7b", layer).astype(np.float16)
    cols = np.unique(np.r_[0, N - 1, np.random.default_rng(layer).choice(N, 254, replace=False)])
    Wd = dev(W)
    torch = torch_cuda()
    for M in (1, 16, 256, 2048):
        say(f"dense f16 llama7b layer {layer} {N}x{K} M={M}")
        X = synth.x_f16(M, K, f"gpu/dense/l{layer}x{M}")
        Y = empty((M, N), torch.float16)
        qlin.qlin_f16_gemm(dev(X), Wd, M, N, K, Y, F16,
                           workspace=workspace(qlin.qlin_f16_gemm_workspace_bytes(M, N, K, F16)))
        check_close(host(Y)[:, cols].astype(np.float64), odense.forward_cols(X, W, cols), f"{N}x{K} M={M}")


def test_repeat_calls_are_bit_identical():
    """Tiles split over several workgroups sum their fp32 partials in K order,
    so repeated calls agree bit for bit."""
    torch = torch_cuda()
    M, N, K = 256, 4096, 4096
    X = dev(synth.x_f16(M, K, "gpu/dense/rep"))
    W = dev(synth.normal_f32((N, K), 0.02, "gpu/dense/repw").astype(np.float16))
    ws = workspace(qlin.qlin_f16_gemm_workspace_bytes(M, N, K, F32))
    outs = []
    for _ in range(3):
        Y = empty((M, N), torch.float32)
        qlin.qlin_f16_gemm(X, W, M, N, K, Y, F32, workspace=ws)
        outs.append(host(Y))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])
