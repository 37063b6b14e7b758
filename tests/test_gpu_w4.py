"""GPU parity of the W4 path (fused GEMV for M <= 16, MFMA GEMM above) against
the fp64 oracle, through the C ABI.  Integer unpacking is compared bit for bit;
float outputs within max|dY| <= 2e-3 max|Y| and relFrob <= 5e-4."""
import numpy as np
import pytest

import synth
from oracle import metrics
from oracle import w4 as ow4
from quantized_linear_layers_packed_amd import qlin
from tests.gpu_util import check_close, dev, empty, host, say, torch_cuda, w4_ws

pytestmark = pytest.mark.gpu

F16, BF16, F32 = qlin.QLIN_F16, qlin.QLIN_BF16, qlin.QLIN_F32


def _tdtype(code):
    torch = torch_cuda()
    return {F16: torch.float16, BF16: torch.bfloat16, F32: torch.float32}[code]


def gpu_w4(X, x_dtype, packed_dev, N, K, G, y_dtype):
    M = X.shape[0]
    qw, sc, qz = packed_dev
    Y = empty((M, N), _tdtype(y_dtype))
    qlin.qlin_w4_forward(dev(X), x_dtype, M, K, qw, sc, qz, N, G, Y, y_dtype,
                         workspace=w4_ws(x_dtype, M, K, N, G, y_dtype))
    y = host(Y)
    if y_dtype == BF16:
        return y                            # bit patterns
    return y.astype(np.float64)


def dev_pack(W, G):
    return tuple(dev(a) for a in qlin.qlin_w4_pack(W, G))


def f32_to_bf16_bits(a):
    return synth.f32_to_bf16_bits(np.asarray(a, np.float32))


def test_unpack_is_bit_exact():
    torch = torch_cuda()
    for (N, K, G) in ((1024, 1024, 128), (64, 11008, 128), (32, 512, 32)):
        say(f"w4 unpack N={N} K={K} G={G}")
        W = synth.normal_f32((N, K), 0.02, f"gpu/w4/unpack{K}")
        qw, sc, qz = qlin.qlin_w4_pack(W, G)
        codes = empty((N, K), torch.uint8)
        zeros = empty((N, K // G), torch.uint8)
        qlin.qlin_w4_unpack(dev(qw), dev(qz), N, K, G, codes, zeros)
        q_ref, z_ref = ow4.unpack(*ow4.encode(W, G)[::2], K, G)
        assert np.array_equal(host(codes), q_ref)
        assert np.array_equal(host(zeros), z_ref)


@pytest.mark.parametrize("M", [1, 4])
def test_small_layer(M):
    say(f"w4_1k M={M}")
    W = synth.layer_weight("w4_1k", 0)
    X = synth.activations("w4_1k", 0, M)
    Y = gpu_w4(X, F16, dev_pack(W, 128), 1024, 1024, 128, F16)
    check_close(Y, ow4.forward(X, *ow4.encode(W, 128), 1024, 128), f"w4_1k M={M}")


@pytest.mark.parametrize("layer", [0, 1, 2])
def test_llama7b_gemv_full_layer(layer):
    N, K = synth.WORKLOADS["w4_llama7b"]["layers"][layer]
    say(f"w4_llama7b layer {layer} {N}x{K} M=1")
    W = synth.layer_weight("w4_llama7b", layer)
    X = synth.activations("w4_llama7b", layer, 1)
    Y = gpu_w4(X, F16, dev_pack(W, 128), N, K, 128, F16)
    check_close(Y, ow4.forward(X, *ow4.encode(W, 128), K, 128), f"{N}x{K}")


@pytest.mark.parametrize("layer", [0, 1, 2])
def test_llama7b_small_batches_full_layer(layer):
    """The Llama-7B-shaped layers at the batch sizes of the crossover sweep that
    run the GEMV with two rows (M = 2) and the small-batch MFMA kernel (M = 8,
    16): all output columns against the oracle."""
    N, K = synth.WORKLOADS["w4_llama7b"]["layers"][layer]
    W = synth.layer_weight("w4_llama7b", layer)
    st = ow4.encode(W, 128)
    packed = dev_pack(W, 128)
    del W
    for M in (2, 8, 16):
        say(f"w4_llama7b layer {layer} {N}x{K} M={M}")
        X = synth.x_f16(M, K, f"gpu/w4/l7b{layer}x{M}")
        check_close(gpu_w4(X, F16, packed, N, K, 128, F16), ow4.forward(X, *st, K, 128), f"{N}x{K} M={M}")


@pytest.mark.parametrize("K", [3 * 256, 4096 + 512])
@pytest.mark.parametrize("G", [32, 64, 128, 256])
@pytest.mark.parametrize("x_dtype", [F16, BF16])
def test_gemv_ragged_shapes_and_dtypes(G, x_dtype, K):
    N = 37
    W = synth.normal_f32((N, K), 0.02, f"gpu/w4/rag{G}")
    packed = dev_pack(W, G)
    ref_st = ow4.encode(W, G)
    for M in (1, 2, 3, 5, 8, 13, 16):
        say(f"w4 gemv N={N} K={K} G={G} M={M} x={x_dtype}")
        if K > 1024 and M not in (1, 2, 16):
            continue
        if x_dtype == F16:
            X = synth.x_f16(M, K, f"gpu/w4/ragx{M}")
        else:
            X = synth.x_bf16_bits(M, K, f"gpu/w4/ragx{M}")
        ref = ow4.forward(X, *ref_st, K, G)
        y32 = gpu_w4(X, x_dtype, packed, N, K, G, F32)
        check_close(y32, ref, f"M={M} f32 out")
        check_close(gpu_w4(X, x_dtype, packed, N, K, G, F16), ref, f"M={M} f16 out")
        yb = gpu_w4(X, x_dtype, packed, N, K, G, BF16)
        assert np.array_equal(yb, f32_to_bf16_bits(y32)), "bf16 store is not RNE of the fp32 result"


@pytest.mark.parametrize("K", [14336, 16384, 16384 + 256])
@pytest.mark.parametrize("G", [32, 128])
def test_longest_gemv_rows_and_just_beyond(G, K):
    """The GEMV's widest instance (two waves per row, four blocks of 64 chunks
    per lane: 12288 < K <= 16384, the last block ragged at K = 14336) and the
    first K past the GEMV's range, which the MFMA kernels take at every batch."""
    N = 37
    W = synth.normal_f32((N, K), 0.02, f"gpu/w4/long{G}")
    packed = dev_pack(W, G)
    ref_st = ow4.encode(W, G)
    for M, x_dtype in ((1, F16), (2, BF16), (3, F16), (16, F16)):
        say(f"w4 long rows N={N} K={K} G={G} M={M} x={x_dtype}")
        X = synth.x_f16(M, K, f"gpu/w4/longx{M}") if x_dtype == F16 else synth.x_bf16_bits(M, K, f"gpu/w4/longx{M}")
        check_close(gpu_w4(X, x_dtype, packed, N, K, G, F32), ow4.forward(X, *ref_st, K, G), f"K={K} G={G} M={M}")


@pytest.mark.parametrize("M,N,K,G", [(20, 12800, 1024, 128), (40, 12800, 512, 256), (100, 2, 256, 128)])
def test_stream_k_tile_widths(M, N, K, G):
    """Shapes that put the stream-K GEMM on 128-column tiles: 32-row tiles with
    50 tiles of 256 columns, 64-row tiles with 50, and 128-row tiles on a
    two-row layer too small for the direct-load kernel."""
    W = synth.normal_f32((N, K), 0.015, f"gpu/w4/skw{N}")
    packed = dev_pack(W, G)
    st = ow4.encode(W, G)
    for x_dtype in (F16, BF16):
        say(f"w4 stream-K widths M={M} N={N} K={K} G={G} x={x_dtype}")
        X = (synth.x_bf16_bits if x_dtype == BF16 else synth.x_f16)(M, K, f"gpu/w4/skwx{M}")
        check_close(gpu_w4(X, x_dtype, packed, N, K, G, F32), ow4.forward(X, *st, K, G), f"M={M} N={N} K={K}")


def test_batch_rows_are_independent():
    """A row's result does not depend on the other rows of its batch, bit for
    bit within each kernel: the GEMV (M <= 3), the small-batch kernel
    (M = 4..16) and the stream-K GEMM (M = 17..32 share one split plan); across
    kernels the results agree within tolerance."""
    W = synth.normal_f32((256, 1024), 0.02, "gpu/w4/indep")
    packed = dev_pack(W, 128)
    X = synth.x_f16(32, 1024, "gpu/w4/indepx")

    def run(rows):
        return gpu_w4(np.ascontiguousarray(X[rows]), F16, packed, 256, 1024, 128, F32)

    full3 = run(list(range(3)))
    for m in range(3):
        assert np.array_equal(run([m])[0], full3[m])
    full16 = run(list(range(16)))
    for m in (0, 5, 12):
        assert np.array_equal(run(list(range(m, m + 4)))[0], full16[m])
    full32 = run(list(range(32)))
    assert np.array_equal(run(list(range(17)))[:17], full32[:17])
    check_close(full3, full16[:3], "GEMV vs small-batch kernel")
    check_close(full16, full32[:16], "small-batch kernel vs GEMM")


@pytest.mark.parametrize("x_dtype", [BF16, F16])
def test_gemm_ragged_shapes(x_dtype):
    # (8, 128) and (37, 640): the last scale / zero chunks of the arrays, read
    # from clamped starts by the direct-load tile kernel (more than 64 rows)
    for (N, K, G) in ((200, 512, 128), (256, 1024, 64), (96, 256, 256), (130, 384, 32), (8, 128, 128),
                      (37, 640, 128)):
        W = synth.normal_f32((N, K), 0.015, f"gpu/w4/gemm{N}")
        packed = dev_pack(W, G)
        st = ow4.encode(W, G)
        for M in (17, 32, 33, 64, 100, 129, 256, 300):
            say(f"w4 gemm N={N} K={K} G={G} M={M} x={x_dtype}")
            X = (synth.x_bf16_bits if x_dtype == BF16 else synth.x_f16)(M, K, f"gpu/w4/gemmx{M}")
            ref = ow4.forward(X, *st, K, G)
            y32 = gpu_w4(X, x_dtype, packed, N, K, G, F32)
            check_close(y32, ref, f"M={M} f32")
            yb = gpu_w4(X, x_dtype, packed, N, K, G, BF16)
            assert np.array_equal(yb, f32_to_bf16_bits(y32))


@pytest.mark.parametrize("layer", [0, 1, 2])
def test_llama70b_gemm_full_layer_sampled_rows(layer):
    """Full 70B-shaped layers at M = 32, 64, 256 (bf16 in, bf16 out): the kernel's
    fp32 result meets the tolerance on 384 sampled output columns, and its bf16
    output is exactly the RNE rounding of that fp32 result everywhere."""
    N, K = synth.WORKLOADS["w4_llama70b"]["layers"][layer]
    W = synth.layer_weight("w4_llama70b", layer)
    packed = dev_pack(W, 128)
    rows = np.unique(np.r_[0, N - 1, np.random.default_rng(layer).choice(N, 382, replace=False)])
    st = ow4.encode(W[rows], 128)
    del W
    for M in (32, 64, 256):
        say(f"w4_llama70b layer {layer} {N}x{K} M={M}")
        X = synth.activations("w4_llama70b", layer, M)
        y32 = gpu_w4(X, BF16, packed, N, K, 128, F32)
        check_close(y32[:, rows], ow4.forward(X, *st, K, 128), f"{N}x{K} M={M}")
        yb = gpu_w4(X, BF16, packed, N, K, 128, BF16)
        assert np.array_equal(yb, f32_to_bf16_bits(y32))
        ref_b = metrics.bf16_bits_to_f64(f32_to_bf16_bits(ow4.forward(X, *st, K, 128)))
        mism = np.mean(yb[:, rows] != f32_to_bf16_bits(ref_b))
        say(f"  bf16 outputs differing from bf16(oracle): {mism:.2e}")


def test_small_batch_beyond_the_gemv_range_uses_the_gemm():
    """M <= 16 with K above the GEMV's single-pass range runs the small-batch
    MFMA kernel (K split over the waves of a workgroup), M = 1 included."""
    N, K = 64, 20480
    W = synth.normal_f32((N, K), 0.02, "gpu/w4/longk")
    packed = dev_pack(W, 128)
    st = ow4.encode(W, 128)
    for M in (1, 5):
        say(f"w4 long-K N={N} K={K} M={M}")
        X = synth.x_f16(M, K, f"gpu/w4/longkx{M}")
        check_close(gpu_w4(X, F16, packed, N, K, 128, F32), ow4.forward(X, *st, K, 128), f"M={M}")


@pytest.mark.parametrize("x_dtype", [F16, BF16])
def test_small_batches_on_wide_layers(x_dtype):
    """Batches of 4..16 rows on layers wide enough for the small-batch kernel to
    give a workgroup 2 tiles of 16 columns (N = 5200: 163 workgroups) or 4
    (N = 10300: 161 workgroups), both with a ragged last tile."""
    for (N, K, G) in ((5200, 1024, 128), (10300, 512, 256)):
        W = synth.normal_f32((N, K), 0.02, f"gpu/w4/wide{N}")
        packed = dev_pack(W, G)
        st = ow4.encode(W, G)
        for M in (4, 9, 16):
            say(f"w4 small-batch wide N={N} K={K} G={G} M={M} x={x_dtype}")
            X = (synth.x_bf16_bits if x_dtype == BF16 else synth.x_f16)(M, K, f"gpu/w4/widex{M}")
            ref = ow4.forward(X, *st, K, G)
            y32 = gpu_w4(X, x_dtype, packed, N, K, G, F32)
            check_close(y32, ref, f"M={M} f32 out")
            yb = gpu_w4(X, x_dtype, packed, N, K, G, BF16)
            assert np.array_equal(yb, f32_to_bf16_bits(y32)), "bf16 store is not RNE of the fp32 result"


@pytest.mark.parametrize("x_dtype", [F16, BF16])
def test_small_batches_through_the_mfma_kernels(x_dtype):
    """Batches of 2..24 rows on layers whose activations exceed the GEMV's LDS
    staging: 4..16 rows run the small-batch kernel (K split over the waves of a
    workgroup, 16 columns each, ragged N), 17 and more the stream-K GEMM with
    few output tiles, so every tile's K range is split over many workgroups and
    the fix-up sums only the accumulator registers that can hold rows below M.
    K = 10240 takes the small-batch kernel's shallower ring for long rows."""
    for (N, K, G) in ((512, 8192, 128), (300, 6144, 256), (130, 10240, 128)):
        W = synth.normal_f32((N, K), 0.02, f"gpu/w4/smallm{N}")
        packed = dev_pack(W, G)
        st = ow4.encode(W, G)
        for M in (2, 4, 5, 8, 9, 16, 17, 24):
            say(f"w4 small-batch N={N} K={K} G={G} M={M} x={x_dtype}")
            X = (synth.x_bf16_bits if x_dtype == BF16 else synth.x_f16)(M, K, f"gpu/w4/smallmx{M}")
            check_close(gpu_w4(X, x_dtype, packed, N, K, G, F32), ow4.forward(X, *st, K, G), f"M={M}")


@pytest.mark.parametrize("G", [128, 64])
def test_bf16_activations_beyond_the_fp16_range(G):
    """bf16 activations that fp16 cannot hold: entries up to +-1e5, bf16
    subnormals, a row of values around 1e-30, a row far above 65504 and an
    all-zero row, at M = 5 (small-batch kernel, G = 128), 17 and 256 (GEMMs).
    The MFMA paths take a row-scaled fp16 copy; each row's outputs are scaled
    back, so the whole output meets the tolerance, and so does every special
    row on its own (relative to that row)."""
    N, K = 320, 2048
    W = synth.normal_f32((N, K), 0.02, f"gpu/w4/bfrange{G}")
    packed = dev_pack(W, G)
    st = ow4.encode(W, G)
    r = np.random.default_rng(7)
    for M in (5, 17, 256):
        say(f"w4 bf16 range N={N} K={K} G={G} M={M}")
        X = synth.x_bf16_bits(M, K, f"gpu/w4/bfrangex{M}").copy()
        big = r.choice(M * K, size=8, replace=False)
        X.flat[big] = f32_to_bf16_bits(np.float32(1e5) * np.sign(r.standard_normal(8)).astype(np.float32))
        sub = r.choice(M * K, size=64, replace=False)
        X.flat[sub] = r.integers(1, 128, size=64).astype(np.uint16) | (r.integers(0, 2, 64) << 15).astype(np.uint16)
        X[1] = f32_to_bf16_bits(synth.normal_f32((K,), 1e-30, f"gpu/w4/bftiny{M}"))       # tiny row
        X[2] = f32_to_bf16_bits(synth.normal_f32((K,), 3e6, f"gpu/w4/bfhuge{M}"))         # huge row
        X[3] = 0                                                                           # zero row
        ref = ow4.forward(X, *st, K, G)
        y32 = gpu_w4(X, BF16, packed, N, K, G, F32)
        assert np.all(np.isfinite(y32))
        check_close(y32, ref, f"M={M} all rows")
        check_close(y32[1], ref[1], f"M={M} row of ~1e-30")
        check_close(y32[2], ref[2], f"M={M} row of ~3e6")
        assert not np.any(y32[3])
        yb = gpu_w4(X, BF16, packed, N, K, G, BF16)
        assert np.array_equal(yb, f32_to_bf16_bits(y32))
