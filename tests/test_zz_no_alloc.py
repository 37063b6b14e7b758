"""The W4 forward that allocates nothing (qlin_w4_forward_scratch) against the
workspace forward (qlin_w4_forward), through the C ABI on the GPU.

Both run the same kernels with the same split plan, so the outputs must be
bit-identical; each is also within the float tolerance of the oracle.  Two
calls in a row, the second on a smaller input, for every path that uses
device scratch (split-K GEMM, bf16 row-scale copy) and for the GEMV, which
uses none.  Runs alone in a fresh process and after the other tests alike
(the scratch counters are cleared before each split-K call)."""
import numpy as np
import pytest

import synth
from oracle import w4 as ow4
from quantized_linear_layers_packed_amd import qlin
from tests.gpu_util import check_close, dev, empty, host, say, torch_cuda, w4_ws

pytestmark = pytest.mark.gpu

F16, BF16, F32 = qlin.QLIN_F16, qlin.QLIN_BF16, qlin.QLIN_F32


@pytest.mark.parametrize("x_dtype,shapes", [
    (F16, [(256, 2048, 4096), (64, 1024, 2048)]),     # split-K GEMM, then a smaller one
    (BF16, [(200, 1536, 2048), (8, 1024, 2048)]),     # row-scale copy + split-K, then the small-batch kernel
    (F16, [(3, 2048, 4096), (1, 512, 1024)]),         # GEMV (no scratch)
])
def test_scratch_forward_matches_the_workspace_forward(x_dtype, shapes):
    torch = torch_cuda()
    for call, (M, N, K) in enumerate(shapes):
        say(f"no-alloc W4 call {call}: M={M} N={N} K={K} x={'bf16' if x_dtype == BF16 else 'f16'}")
        W = synth.normal_f32((N, K), 0.02, f"gpu/noalloc/w{N}x{K}")
        st = ow4.encode(W, 128)
        qw, sc, qz = (dev(a) for a in qlin.qlin_w4_pack(W, 128))
        X = (synth.x_bf16_bits if x_dtype == BF16 else synth.x_f16)(M, K, f"gpu/noalloc/x{M}")
        Xd = dev(X)
        Y0 = empty((M, N), torch.float32)
        Y1 = empty((M, N), torch.float32)
        qlin.qlin_w4_forward(Xd, x_dtype, M, K, qw, sc, qz, N, 128, Y0, F32,
                             workspace=w4_ws(x_dtype, M, K, N, 128, F32))
        qlin.qlin_w4_forward_scratch(Xd, x_dtype, M, K, qw, sc, qz, N, 128, Y1, F32)
        y0, y1 = host(Y0), host(Y1)
        assert np.array_equal(y0, y1), "scratch forward differs from the workspace forward"
        check_close(y1.astype(np.float64), ow4.forward(X, *st, K, 128), f"call {call} vs oracle")


def test_scratch_forward_refuses_a_shape_beyond_its_size():
    need = qlin.qlin_w4_workspace_bytes(BF16, 4096, 16384, 8192, 128, F32)
    assert need > 80 << 20
    with pytest.raises(qlin.QlinError) as e:
        qlin.qlin_w4_forward_scratch(0x10000, BF16, 4096, 16384, 0x10000, 0x10000, 0x10000, 8192, 128, 0x10000, F32,
                                     stream=0)
    assert e.value.status == qlin.QLIN_EUNSUPPORTED and str(need) in str(e.value)
