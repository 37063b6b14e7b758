"""GPU parity of the SpQR path (dense 3-bit bi-level part + fused CSR outliers)
against the fp64 oracle, through the C ABI."""
import numpy as np
import pytest

import synth
from oracle import spqr as ospqr
from quantized_linear_layers_packed_amd import qlin
from tests.gpu_util import check_close, dev, empty, host, say, spqr_ws, torch_cuda

pytestmark = pytest.mark.gpu

F16, F32 = qlin.QLIN_F16, qlin.QLIN_F32


def dev_pack(st):
    return {k: dev(np.ascontiguousarray(v)) for k, v in st.items()}


def gpu_spqr(X, d, N, K, y_dtype=F16):
    torch = torch_cuda()
    M = X.shape[0]
    Y = empty((M, N), torch.float16 if y_dtype == F16 else torch.float32)
    nnz = int(d["col_idx"].numel())
    qlin.spqr_forward(dev(X), M, K, d["codes"], d["stats1"], d["stats2"], d["row_ptr"],
                      d["col_idx"] if nnz else 0, d["val"] if nnz else 0, nnz, N, Y, y_dtype,
                      workspace=spqr_ws(M, K, N, y_dtype))
    return host(Y).astype(np.float64)


def test_unpack_is_bit_exact():
    torch = torch_cuda()
    N, K = 96, 6656
    say(f"spqr unpack {N}x{K}")
    W = synth.student_t3_f32((N, K), 0.02, "gpu/spqr/unpack")
    st = qlin.spqr_pack(W, 0.01)
    q = empty((N, K), torch.uint8)
    cs = empty((N, K // 16), torch.uint8)
    cz = empty((N, K // 16), torch.uint8)
    qlin.spqr_unpack(dev(st["codes"]), dev(st["stats1"]), N, K, q, cs, cz)
    d = ospqr.quantize(W, 0.01)
    assert np.array_equal(host(q), d["q"])
    assert np.array_equal(host(cs), d["cs"])
    assert np.array_equal(host(cz), d["cz"])


@pytest.mark.parametrize("p", [0.0, 0.01, 0.05])
def test_ragged_shapes(p):
    # M = 1 runs the GEMV (the four-row kernel where K > 8192), 2..6 the
    # four-rows-per-wave kernel (one token group up to 4, two beyond), 7 the
    # four-row kernel where N > K (here 300 x 256) and else, like 16, the
    # matrix-core path (two column tiles per wave where K >= 2N, one where K < 2N)
    for (N, K) in ((37, 512), (16, 256), (50, 2560), (21, 26624), (133, 256), (600, 768), (1100, 2048),
                   (300, 256)):
        W = synth.student_t3_f32((N, K), 0.02, f"gpu/spqr/rag{N}")
        d = dev_pack(qlin.spqr_pack(W, p))
        st = ospqr.encode(W, p)
        for M in (1, 2, 3, 4, 5, 6, 7, 16):
            say(f"spqr N={N} K={K} p={p} M={M}")
            X = synth.x_f16(M, K, f"gpu/spqr/ragx{M}")
            ref = ospqr.forward(X, st, K)
            check_close(gpu_spqr(X, d, N, K, F32), ref, f"M={M} f32")
            check_close(gpu_spqr(X, d, N, K, F16), ref, f"M={M} f16")


@pytest.mark.parametrize("K", [4352, 5120, 6144, 8192])
def test_single_token_gemv_block_counts(K):
    """One token on rows of 4097..8192 values: three and four 64-chunk blocks
    per lane in the GEMV (the layer shapes above reach one, two and four)."""
    N = 41
    W = synth.student_t3_f32((N, K), 0.02, f"gpu/spqr/gemv{K}")
    d = dev_pack(qlin.spqr_pack(W, 0.01))
    st = ospqr.encode(W, 0.01)
    say(f"spqr gemv blocks N={N} K={K} M=1")
    X = synth.x_f16(1, K, "gpu/spqr/gemvx")
    check_close(gpu_spqr(X, d, N, K, F32), ospqr.forward(X, st, K), f"N={N} K={K} M=1")


@pytest.mark.parametrize("N,K,M", [(45, 8448, 1), (45, 7168, 3), (45, 4352, 2), (29, 4352, 6)])
def test_four_row_kernel_step_counts(N, K, M):
    """Row lengths that put the four-row kernel on the instances the layers
    above do not reach: one token with a single 8448-long slice (six steps of
    16 chunks per wave), a 4-token group over two 3584-long slices (two steps),
    two tokens with both row groups over one 4352-long slice (three steps), and
    six tokens (two groups) over two slices."""
    W = synth.student_t3_f32((N, K), 0.02, f"gpu/spqr/steps{K}")
    d = dev_pack(qlin.spqr_pack(W, 0.01))
    st = ospqr.encode(W, 0.01)
    say(f"spqr four-row steps N={N} K={K} M={M}")
    X = synth.x_f16(M, K, f"gpu/spqr/stepsx{M}")
    check_close(gpu_spqr(X, d, N, K, F32), ospqr.forward(X, st, K), f"N={N} K={K} M={M}")


def test_csr_part_alone_matches_sparse_product():
    """Dense part forced to zero (codes 0, z_hat = 0): the output is the CSR
    product alone, so every outlier entry must be consumed once at its column."""
    N, K = 64, 1024
    W = synth.student_t3_f32((N, K), 0.02, "gpu/spqr/csr")
    st = qlin.spqr_pack(W, 0.04)
    st["codes"][:] = 0
    s2 = st["stats2"].copy()
    s2[:, :, 2:] = 0.0
    st["stats2"] = s2
    d = dev_pack(st)
    for M in (1, 2, 4, 6, 8, 16):
        say(f"spqr csr-only M={M}")
        X = synth.x_f16(M, K, f"gpu/spqr/csrx{M}")
        ref = ospqr.forward(X, st, K)
        dense = np.zeros((N, K))
        rp = st["row_ptr"]
        for n in range(N):
            dense[n, st["col_idx"][rp[n]:rp[n + 1]]] = st["val"][rp[n]:rp[n + 1]]
        assert np.allclose(ref, X.astype(np.float64) @ dense.T, rtol=1e-12, atol=1e-12)
        check_close(gpu_spqr(X, d, N, K, F32), ref, f"csr-only M={M}")


@pytest.mark.parametrize("layer", [0, 1, 2])
def test_33b_full_layer_sampled_rows(layer):
    N, K = synth.WORKLOADS["spqr_33b"]["layers"][layer]
    W = synth.layer_weight("spqr_33b", layer)
    d = dev_pack(qlin.spqr_pack(W, 0.01))
    rows = np.unique(np.r_[0, N - 1, np.random.default_rng(layer).choice(N, 254, replace=False)])
    st = ospqr.encode_rows(W, 0.01, rows)
    del W
    for M in (1, 4, 6, 8, 16):
        say(f"spqr_33b layer {layer} {N}x{K} M={M}")
        X = synth.activations("spqr_33b", layer, M)
        Y = gpu_spqr(X, d, N, K, F16)
        check_close(Y[:, rows], ospqr.forward(X, st, K), f"{N}x{K} M={M}")


@pytest.mark.parametrize("N,K", [(48, 1024), (1100, 2048)])
def test_matrix_core_path_leaves_the_counter_slots_zero(N, K):
    """The prepass writes after the 16 KiB of split-K arrival counters (on both
    routes of the matrix-core path: K >= 2N and K < 2N), so a workspace shared
    with the W4 and int8 GEMMs still has them zero."""
    torch = torch_cuda()
    M = 12
    W = synth.student_t3_f32((N, K), 0.02, "gpu/spqr/wsctr")
    d = dev_pack(qlin.spqr_pack(W, 0.01))
    need = qlin.spqr_workspace_bytes(M, K, N, F32)
    assert need > 16384
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    X = synth.x_f16(M, K, "gpu/spqr/wsctrx")
    Y = empty((M, N), torch.float32)
    nnz = int(d["col_idx"].numel())
    say(f"spqr workspace counters N={N} K={K} M={M}")
    qlin.spqr_forward(dev(X), M, K, d["codes"], d["stats1"], d["stats2"], d["row_ptr"], d["col_idx"], d["val"], nnz,
                      N, Y, F32, workspace=ws)
    torch.cuda.synchronize()
    assert not host(ws[:16384]).any()
    assert host(ws[16384:]).any()
