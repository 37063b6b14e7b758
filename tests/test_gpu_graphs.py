"""Repeatability and graph capture through the C ABI (GPU).

Every forward is deterministic: the split-K GEMMs add their partial tiles in K
order whatever the arrival order of the workgroups, and their arrival counters
return to zero at the end of each call.  So a call repeated gives the same bits,
and a HIP graph that captured the calls gives, at every replay, the bits of
the eager calls (the workspace exists before capture, counters are never
cleared inside the graph)."""
import numpy as np
import pytest

import synth
from quantized_linear_layers_packed_amd import qlin
from tests.gpu_util import dev, empty, host, say, spqr_ws, sq_ws, torch_cuda, w4_ws

pytestmark = pytest.mark.gpu

F16, BF16, F32 = qlin.QLIN_F16, qlin.QLIN_BF16, qlin.QLIN_F32


def _calls():
    """Device inputs and a list of (name, callable writing its output, output tensor)."""
    torch = torch_cuda()
    out = []
    # W4: GEMV (M=1), small-batch kernel (M=8), stream-K GEMM (M=96, bf16 in)
    W = synth.normal_f32((1536, 2048), 0.02, "gpu/graph/w4")
    qw, sc, qz = (dev(a) for a in qlin.qlin_w4_pack(W, 128))
    for M, xd in ((1, F16), (8, F16), (96, BF16)):
        X = dev((synth.x_bf16_bits if xd == BF16 else synth.x_f16)(M, 2048, f"gpu/graph/x{M}"))
        Y = empty((M, 1536), torch.float32)
        wsp = w4_ws(xd, M, 2048, 1536, 128, F32)
        out.append((f"w4 M={M}", lambda X=X, Y=Y, M=M, xd=xd, wsp=wsp: qlin.qlin_w4_forward(
            X, xd, M, 2048, qw, sc, qz, 1536, 128, Y, F32, workspace=wsp), Y))
    # SpQR M=1 (GEMV) and 8 (prepass + matrix-core kernel)
    Ws = synth.student_t3_f32((512, 2048), 0.02, "gpu/graph/spqr")
    st = qlin.spqr_pack(Ws, 0.01)
    d = {k: dev(np.ascontiguousarray(v)) for k, v in st.items()}
    nnz = len(st["val"])
    for M in (1, 8):
        X = dev(synth.x_f16(M, 2048, f"gpu/graph/sx{M}"))
        Y = empty((M, 512), torch.float32)
        wsp = spqr_ws(M, 2048, 512, F32)
        out.append((f"spqr M={M}", lambda X=X, Y=Y, M=M, wsp=wsp: qlin.spqr_forward(
            X, M, 2048, d["codes"], d["stats1"], d["stats2"], d["row_ptr"], d["col_idx"], d["val"], nnz, 512, Y, F32,
            workspace=wsp), Y))
    # W8A8: activation kernel + int8 GEMM (stream-K), M=200
    Wf = synth.normal_f32((1024, 2048), 0.02, "gpu/graph/sq")
    Xc = synth.x_f16(200, 2048, "gpu/graph/sqx")
    s, inv = qlin.sq_compute_smoothing(qlin.sq_act_absmax(Xc), Wf, 0.85)
    Wq, ws = qlin.sq_pack_weight(Wf, s)
    Wq, ws, inv, X = dev(Wq), dev(ws), dev(inv), dev(Xc)
    Xq = empty((200, 2048), torch.int8)
    xs = empty((200,), torch.float32)
    Y = empty((200, 1024), torch.float32)
    acc = empty((200, 1024), torch.int32)

    ws200 = sq_ws(200, 1024, 2048, F32)

    def sq():
        qlin.sq_smooth_quant_act(X, inv, 200, 2048, Xq, xs)
        qlin.sq_int8_gemm(Xq, xs, Wq, ws, 200, 1024, 2048, Y, F32, acc, workspace=ws200)
    out.append(("w8a8 M=200", sq, Y))
    out.append(("w8a8 acc", lambda: None, acc))
    # W8A8 at M=600: the large-batch kernel (256 x 128 tiles, stream-K over 24 tiles)
    X6 = dev(synth.x_f16(600, 2048, "gpu/graph/sqx600"))
    Xq6 = empty((600, 2048), torch.int8)
    xs6 = empty((600,), torch.float32)
    Y6 = empty((600, 1024), torch.float16)
    acc6 = empty((600, 1024), torch.int32)

    ws600 = sq_ws(600, 1024, 2048, F16)

    def sq600():
        qlin.sq_smooth_quant_act(X6, inv, 600, 2048, Xq6, xs6)
        qlin.sq_int8_gemm(Xq6, xs6, Wq, ws, 600, 1024, 2048, Y6, F16, acc6, workspace=ws600)
    out.append(("w8a8 M=600", sq600, Y6))
    out.append(("w8a8 M=600 acc", lambda: None, acc6))
    return out, (qw, sc, qz, d, Wq)


def test_repeated_calls_give_identical_bits():
    calls, _keep = _calls()
    first = []
    for name, f, y in calls:
        f()
        first.append(host(y).copy())
    for rep in range(3):
        for (name, f, y), ref in zip(calls, first):
            f()
            assert np.array_equal(host(y), ref), f"{name}: repetition {rep} differs"
    say("  repeated calls: bit-identical")


def test_graph_replays_match_eager_calls():
    torch = torch_cuda()
    calls, _keep = _calls()
    eager = []
    for name, f, y in calls:
        f()
        eager.append(host(y).copy())
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            for name, f, y in calls:
                f()
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    for rep in range(3):
        for name, f, y in calls:
            y.zero_()
        graph.replay()
        torch.cuda.synchronize()
        for (name, f, y), ref in zip(calls, eager):
            assert np.array_equal(host(y), ref), f"{name}: replay {rep} differs from the eager call"
        # eager work between replays (the same calls, outside the graph)
        for name, f, y in calls:
            f()
        torch.cuda.synchronize()
    say("  graph replays: bit-identical to eager calls")


def test_first_call_of_a_shape_under_capture_and_growth_after_capture():
    """The library allocates nothing: the first call of a split-K shape can be
    captured (its workspace belongs to the caller), and a larger uncaptured call
    with another workspace afterwards leaves the graph's buffers untouched."""
    torch = torch_cuda()
    W = synth.normal_f32((1024, 2048), 0.02, "gpu/graph/first")
    qw, sc, qz = (dev(a) for a in qlin.qlin_w4_pack(W, 128))
    X = dev(synth.x_f16(80, 2048, "gpu/graph/firstx"))
    Y = empty((80, 1024), torch.float32)
    ws1 = torch.zeros(qlin.qlin_w4_workspace_bytes(F16, 80, 2048, 1024, 128, F32), dtype=torch.uint8,
                      device="cuda")
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            qlin.qlin_w4_forward(X, F16, 80, 2048, qw, sc, qz, 1024, 128, Y, F32, workspace=ws1)
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    first = host(Y).copy()
    eager = empty((80, 1024), torch.float32)
    qlin.qlin_w4_forward(X, F16, 80, 2048, qw, sc, qz, 1024, 128, eager, F32, workspace=ws1)
    assert np.array_equal(host(eager), first)
    # a larger shape, uncaptured, on its own workspace
    Xb = dev(synth.x_f16(600, 2048, "gpu/graph/firstxb"))
    Yb = empty((600, 1024), torch.float32)
    ws2 = torch.zeros(qlin.qlin_w4_workspace_bytes(F16, 600, 2048, 1024, 128, F32), dtype=torch.uint8,
                      device="cuda")
    qlin.qlin_w4_forward(Xb, F16, 600, 2048, qw, sc, qz, 1024, 128, Yb, F32, workspace=ws2)
    for _ in range(3):
        Y.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(Y), first)
    say("  first call captured; replays unchanged after a larger call")


def test_concurrent_split_k_calls_on_two_streams():
    """Two split-K GEMMs (W4 and int8) enqueued on two default-priority streams
    with their own workspaces run concurrently and give the bits of the same
    calls run one after the other."""
    torch = torch_cuda()
    W = synth.normal_f32((4096, 2048), 0.02, "gpu/graph/conc")
    qw, sc, qz = (dev(a) for a in qlin.qlin_w4_pack(W, 128))
    X = dev(synth.x_f16(256, 2048, "gpu/graph/concx"))
    Wf = synth.normal_f32((3072, 2048), 0.02, "gpu/graph/concsq")
    Xc = synth.x_f16(512, 2048, "gpu/graph/concsqx")
    s, inv = qlin.sq_compute_smoothing(qlin.sq_act_absmax(Xc), Wf, 0.85)
    Wq, wsc = qlin.sq_pack_weight(Wf, s)
    Wq, wsc, inv, Xd = dev(Wq), dev(wsc), dev(inv), dev(Xc)
    Xq = empty((512, 2048), torch.int8)
    xs = empty((512,), torch.float32)
    qlin.sq_smooth_quant_act(Xd, inv, 512, 2048, Xq, xs)
    wa = torch.zeros(qlin.qlin_w4_workspace_bytes(F16, 256, 2048, 4096, 128, F32), dtype=torch.uint8, device="cuda")
    wb = torch.zeros(qlin.sq_int8_gemm_workspace_bytes(512, 3072, 2048, F32), dtype=torch.uint8, device="cuda")
    Ya, Yb = empty((256, 4096), torch.float32), empty((512, 3072), torch.float32)
    Aa, Ab = empty((512, 3072), torch.int32), None

    def run_a(stream):
        qlin.qlin_w4_forward(X, F16, 256, 2048, qw, sc, qz, 4096, 128, Ya, F32, workspace=wa, stream=stream)

    def run_b(stream):
        qlin.sq_int8_gemm(Xq, xs, Wq, wsc, 512, 3072, 2048, Yb, F32, Aa, workspace=wb, stream=stream)

    torch.cuda.synchronize()
    run_a(None)
    run_b(None)
    ref_a, ref_b, ref_acc = host(Ya).copy(), host(Yb).copy(), host(Aa).copy()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for rep in range(4):
        Ya.zero_()
        Yb.zero_()
        Aa.zero_()
        torch.cuda.synchronize()
        for _ in range(3):
            run_a(s1)
            run_b(s2)
        torch.cuda.synchronize()
        assert np.array_equal(host(Ya), ref_a), f"W4 differs on concurrent run {rep}"
        assert np.array_equal(host(Yb), ref_b), f"int8 differs on concurrent run {rep}"
        assert np.array_equal(host(Aa), ref_acc)
    say("  concurrent split-K calls on two streams: bit-identical")
