#!/usr/bin/env python3
"""Benchmark of the packed quantized linear layer on one MI355X.

Headline (one JSON line on stdout): quantized-linear GB/s at M = 1 on the
Llama-7B-shaped 4-bit layers 4096x4096, 11008x4096, 4096x11008 (group 128,
fp16 in/out).  One step = one forward through the three layers.  Weights are
rotated over enough packed copies (>= 1 GiB) that every step streams them from
HBM rather than from the 256 MB last-level cache; the activations are resident.

The same run also times, each on its own workload (field "paths"):
  * SpQR 3-bit + 1% CSR outliers, 33B-shaped layers, M = 1       (GB/s)
  * W4 MFMA GEMM, 70B-shaped layers, M = 256, bf16 in/out          (TOPS)
  * SmoothQuant W8A8 int8 GEMM, 11008x4096 and 4096x4096, M = 256  (TOPS)
and the CPU oracle on a bounded sample ("cpu_baseline").

Timing uses HIP events on the stream the kernels run on: one event pair around
the K timed steps (replayed as a HIP graph) gives ms_per_step; each kernel's
average duration comes from a graph holding only that kernel's launches over the
weight rotation, timed the same way, and gives the roofline figures.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0, "i8": 5000.0}
ROTATE_BYTES = 1 << 30


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--no-paths", action="store_true", help="headline workload only")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--summarize", metavar="DIR",
                   help="summarize rocprofv3 csv output under DIR (trace/, fetch/, write/) and exit")
    p.add_argument("--calibrate", action="store_true",
                   help="first run a plain 256 MiB device copy (known traffic) 5 times, for counter scaling")
    p.add_argument("--sweep", choices=("batch", "outliers", "actorder"),
                   help="instead of the headline: batch crossover sweep M = 1..2048 (W4A16 vs W8A8 vs "
                        "dense fp16), SpQR outlier-fraction sweep 0-4%% at M = 1 and 4, or the act-order "
                        "penalty (gathered activations vs static groups) at M = 1, 8, 64")
    return p.parse_args()


# ---------------------------------------------------------------------------
# device helpers

def to_dev(torch, a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        return torch.from_numpy(a.view(np.int16)).view(torch.float16).cuda()
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda()
    if a.dtype == np.uint32:
        return torch.from_numpy(a.view(np.int32)).cuda()
    return torch.from_numpy(a).cuda()


def zeros_ws(torch, nbytes):
    """A zero-filled device workspace (None when none is needed)."""
    return torch.zeros(int(nbytes), dtype=torch.uint8, device="cuda") if nbytes else None


def copies_for(bytes_per_set):
    return max(2, -(-ROTATE_BYTES // max(1, bytes_per_set)))


def _graph(torch, body):
    """Capture body() into a HIP graph on a side stream; return the graph."""
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            body()
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    return graph


def _replay_ms(torch, graph, reps):
    """Average time of one replay, with events on the replaying stream."""
    graph.replay()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(reps):
        graph.replay()
    e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def time_steps(torch, step_fns, steps, warmup, copies):
    """Time ``steps`` steps; return (ms per step, per-kernel average ms list).

    step_fns: callables; step i runs every callable with argument i (i selects
    the weight copy).  The timed steps replay a HIP graph holding one full
    rotation (``copies`` steps), so host launch overhead stays out of the
    measurement.  Each kernel's average duration comes from a graph of that
    kernel alone over the same rotation, launched back to back (the events
    bracket ``copies`` launches on the stream they run on)."""
    for i in range(warmup):
        for f in step_fns:
            f(i)
    torch.cuda.synchronize()

    def whole():
        for i in range(copies):
            for f in step_fns:
                f(i)
    graph = _graph(torch, whole)
    reps = max(1, -(-steps // copies))
    ms_step = _replay_ms(torch, graph, reps) / copies
    del graph
    per = []
    for f in step_fns:
        g = _graph(torch, lambda f=f: [f(i) for i in range(copies)])
        per.append(_replay_ms(torch, g, reps) / copies)
        del g
    return ms_step, per


# ---------------------------------------------------------------------------
# workloads

def w4_layers(torch, qlin, synth, workload, M):
    cfg = synth.WORKLOADS[workload]
    G = cfg["G"]
    xbf = cfg["x_dtype"] == "bf16"
    layers = []
    for li, (N, K) in enumerate(cfg["layers"]):
        W = synth.layer_weight(workload, li)
        packed = [to_dev(torch, a) for a in qlin.qlin_w4_pack(W, G)]
        del W
        X = to_dev(torch, synth.activations(workload, li, M))
        ydt = torch.bfloat16 if cfg["y_dtype"] == "bf16" else torch.float16
        Y = torch.empty((M, N), dtype=ydt, device="cuda")
        wbytes = sum(t.numel() * t.element_size() for t in packed)
        layers.append(dict(N=N, K=K, M=M, G=G, packed=[packed], X=X, Y=Y, wbytes=wbytes,
                           xdt=qlin.QLIN_BF16 if xbf else qlin.QLIN_F16,
                           ydt=qlin.QLIN_BF16 if cfg["y_dtype"] == "bf16" else qlin.QLIN_F16,
                           io=X.numel() * X.element_size() + Y.numel() * Y.element_size()))
    need = max(qlin.qlin_w4_workspace_bytes(l["xdt"], M, l["K"], l["N"], G, l["ydt"]) for l in layers)
    ws = zeros_ws(torch, need)
    for l in layers:
        l["ws"] = ws
    rotate(torch, layers)
    return layers


def rotate(torch, layers):
    per_set = sum(l["wbytes"] for l in layers)
    R = copies_for(per_set)
    for l in layers:
        base = l["packed"][0]
        l["packed"] = [base] + [[t.clone() for t in base] for _ in range(R - 1)]
    return R


def w4_step_fns(qlin, layers):
    fns = []
    for l in layers:
        def f(i, l=l):
            qw, sc, qz = l["packed"][i % len(l["packed"])]
            qlin.qlin_w4_forward(l["X"], l["xdt"], l["M"], l["K"], qw, sc, qz, l["N"], l["G"], l["Y"], l["ydt"],
                                 workspace=l["ws"])
        fns.append(f)
    return fns


def spqr_layers(torch, qlin, synth, M):
    cfg = synth.WORKLOADS["spqr_33b"]
    layers = []
    for li, (N, K) in enumerate(cfg["layers"]):
        W = synth.layer_weight("spqr_33b", li)
        st = qlin.spqr_pack(W, cfg["outlier_frac"])
        del W
        packed = [to_dev(torch, st[k]) for k in ("codes", "stats1", "stats2", "row_ptr", "col_idx", "val")]
        X = to_dev(torch, synth.activations("spqr_33b", li, M))
        Y = torch.empty((M, N), dtype=torch.float16, device="cuda")
        wbytes = sum(t.numel() * t.element_size() for t in packed)
        layers.append(dict(N=N, K=K, M=M, nnz=len(st["val"]), packed=[packed], X=X, Y=Y, wbytes=wbytes,
                           io=X.numel() * 2 + Y.numel() * 2))
    rotate(torch, layers)
    return layers


def spqr_step_fns(qlin, layers):
    fns = []
    for l in layers:
        def f(i, l=l):
            c, s1, s2, rp, ci, v = l["packed"][i % len(l["packed"])]
            qlin.spqr_forward(l["X"], l["M"], l["K"], c, s1, s2, rp, ci, v, l["nnz"], l["N"], l["Y"], qlin.QLIN_F16)
        fns.append(f)
    return fns


def sq_layers(torch, qlin, synth, M):
    cfg = synth.WORKLOADS["sq_w8a8"]
    layers = []
    for li, (N, K) in enumerate(cfg["layers"]):
        W = synth.layer_weight("sq_w8a8", li)
        Xcal = synth.sq_calibration("sq_w8a8", li)
        s, inv = qlin.sq_compute_smoothing(qlin.sq_act_absmax(Xcal), W, cfg["alpha"])
        Wq, ws = qlin.sq_pack_weight(W, s)
        del W
        packed = [to_dev(torch, Wq), to_dev(torch, ws)]
        X = to_dev(torch, synth.activations("sq_w8a8", li, M))
        layers.append(dict(N=N, K=K, M=M, packed=[packed], X=X, inv=to_dev(torch, inv),
                           Xq=torch.empty((M, K), dtype=torch.int8, device="cuda"),
                           xs=torch.empty((M,), dtype=torch.float32, device="cuda"),
                           Y=torch.empty((M, N), dtype=torch.float16, device="cuda"),
                           wbytes=sum(t.numel() * t.element_size() for t in packed)))
    ws = zeros_ws(torch, max(qlin.sq_int8_gemm_workspace_bytes(M, l["N"], l["K"], qlin.QLIN_F16) for l in layers))
    for l in layers:
        l["ws"] = ws
    rotate(torch, layers)
    return layers


def sq_step_fns(qlin, layers):
    act, gemm = [], []
    for l in layers:
        def a(i, l=l):
            qlin.sq_smooth_quant_act(l["X"], l["inv"], l["M"], l["K"], l["Xq"], l["xs"])

        def g(i, l=l):
            Wq, ws = l["packed"][i % len(l["packed"])]
            qlin.sq_int8_gemm(l["Xq"], l["xs"], Wq, ws, l["M"], l["N"], l["K"], l["Y"], qlin.QLIN_F16, None,
                              workspace=l["ws"])
        act.append(a)
        gemm.append(g)
    return act, gemm


# ---------------------------------------------------------------------------
# sweeps (separate runs, not part of the headline line)

SWEEP_M = (1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024, 2048)
SWEEP_FRACS = (0.0, 0.0025, 0.005, 0.01, 0.02, 0.03, 0.04)


def graph_step_ms(torch, fns, copies, steps):
    """Average time of one step (every callable of ``fns`` with the step's copy
    index) over a HIP graph of one full weight rotation, replayed ``steps`` /
    ``copies`` times after a few eager warm-up steps."""
    for i in range(min(copies, 3)):
        for f in fns:
            f(i)
    torch.cuda.synchronize()
    g = _graph(torch, lambda: [f(i) for i in range(copies) for f in fns])
    ms = _replay_ms(torch, g, max(1, -(-steps // copies))) / copies
    del g
    return ms


def dense_f16_weights(torch, layers_w):
    """fp16 copies of the weights, rotated like the packed forms."""
    base = [torch.from_numpy(W.astype(np.float16)).cuda() for W in layers_w]
    per_set = sum(t.numel() * 2 for t in base)
    R = copies_for(per_set)
    return [base] + [[t.clone() for t in base] for _ in range(R - 1)]


def sweep_batch(torch, qlin, synth, steps):
    """W4A16 (GEMV up to M=16, MFMA GEMM above) vs SmoothQuant W8A8 (activation
    kernel + int8 GEMM) vs dense fp16 (torch.matmul, the vendor GEMM) on the
    Llama-7B-shaped layers, for M = 1 .. 2048.  Same fp16 activations for all
    three (N(0,1), 1% of channels x100, the SmoothQuant workload's recipe)."""
    shapes = synth.WORKLOADS["w4_llama7b"]["layers"]
    Mmax = max(SWEEP_M)
    Ws = [synth.layer_weight("w4_llama7b", li) for li in range(len(shapes))]
    Xs = []
    for li, (N, K) in enumerate(shapes):
        ch = synth.outlier_channels(K, 0.01, f"sweep/L{li}/channels")
        Xs.append(synth.x_f16(Mmax, K, f"sweep/L{li}/X", ch, 100.0))
    Xd = [to_dev(torch, x) for x in Xs]
    Yd = [torch.empty((Mmax, N), dtype=torch.float16, device="cuda") for N, _ in shapes]

    w4 = [[to_dev(torch, a) for a in qlin.qlin_w4_pack(W, 128)] for W in Ws]
    w4_bytes = sum(t.numel() * t.element_size() for l in w4 for t in l)
    w4 = [w4] + [[[t.clone() for t in l] for l in w4] for _ in range(copies_for(w4_bytes) - 1)]

    sq, inv = [], []
    for W, X in zip(Ws, Xs):
        s_, inv_ = qlin.sq_compute_smoothing(qlin.sq_act_absmax(X[:512]), W, 0.85)
        Wq, ws = qlin.sq_pack_weight(W, s_)
        sq.append([to_dev(torch, Wq), to_dev(torch, ws)])
        inv.append(to_dev(torch, inv_))
    sq_bytes = sum(t.numel() * t.element_size() for l in sq for t in l)
    sq = [sq] + [[[t.clone() for t in l] for l in sq] for _ in range(copies_for(sq_bytes) - 1)]
    Xq = [torch.empty((Mmax, K), dtype=torch.int8, device="cuda") for _, K in shapes]
    xs = [torch.empty((Mmax,), dtype=torch.float32, device="cuda") for _ in shapes]

    f16 = dense_f16_weights(torch, Ws)
    f16_bytes = sum(t.numel() * 2 for t in f16[0])
    del Ws
    wsp = zeros_ws(torch, max(max(qlin.qlin_w4_workspace_bytes(qlin.QLIN_F16, M, K, N, 128, qlin.QLIN_F16),
                                  qlin.sq_int8_gemm_workspace_bytes(M, N, K, qlin.QLIN_F16))
                              for M in SWEEP_M for N, K in shapes))

    rows = []
    for M in SWEEP_M:
        def w4_fns():
            out = []
            for li, (N, K) in enumerate(shapes):
                def f(i, li=li, N=N, K=K):
                    qw, sc, qz = w4[i % len(w4)][li]
                    qlin.qlin_w4_forward(Xd[li][:M], qlin.QLIN_F16, M, K, qw, sc, qz, N, 128, Yd[li][:M],
                                         qlin.QLIN_F16, workspace=wsp)
                out.append(f)
            return out

        def sq_fns():
            out = []
            for li, (N, K) in enumerate(shapes):
                def f(i, li=li, N=N, K=K):
                    Wq, ws = sq[i % len(sq)][li]
                    qlin.sq_smooth_quant_act(Xd[li][:M], inv[li], M, K, Xq[li][:M], xs[li][:M])
                    qlin.sq_int8_gemm(Xq[li][:M], xs[li][:M], Wq, ws, M, N, K, Yd[li][:M], qlin.QLIN_F16, None,
                                      workspace=wsp)
                out.append(f)
            return out

        def f16_fns():
            out = []
            for li in range(len(shapes)):
                def f(i, li=li):
                    torch.matmul(Xd[li][:M], f16[i % len(f16)][li].t(), out=Yd[li][:M])
                out.append(f)
            return out

        flops = sum(2.0 * M * N * K for N, K in shapes)
        io = sum(M * K * 2 + M * N * 2 for N, K in shapes)
        rec = {"M": M}
        for name, fns, copies, wb, peak in (("w4a16", w4_fns(), len(w4), w4_bytes, MFMA_PEAK_TFLOPS["f16"]),
                                            ("w8a8", sq_fns(), len(sq), sq_bytes, MFMA_PEAK_TFLOPS["i8"]),
                                            ("f16", f16_fns(), len(f16), f16_bytes, MFMA_PEAK_TFLOPS["f16"])):
            ms = graph_step_ms(torch, fns, copies, steps)
            floor_us = max((wb + io) / (HBM_PEAK_GBS * 1e9), flops / (peak * 1e12)) * 1e6
            rec[name] = {"us": round(ms * 1e3, 2), "TFLOP/s": round(flops / (ms * 1e-3) / 1e12, 1),
                         "GB/s": round((wb + io) / (ms * 1e-3) / 1e9, 1), "roofline_us": round(floor_us, 2)}
        rec["fastest"] = min(("w4a16", "w8a8", "f16"), key=lambda k: rec[k]["us"])
        print(json.dumps(rec), flush=True)
        rows.append(rec)
    return {"sweep": "batch", "layers": [f"{N}x{K}" for N, K in shapes], "weight_bytes":
            {"w4a16": w4_bytes, "w8a8": sq_bytes, "f16": f16_bytes}, "rows": rows}


def sweep_outliers(torch, qlin, synth, steps):
    """SpQR forward on the 33B-shaped layers at M = 1 and 4 for outlier fractions
    0 .. 4%, against the dense fp16 product of the same layers (torch.matmul).
    The share of time spent on the CSR part is (t(p) - t(0)) / t(p): the dense
    3-bit part costs the same whatever the fraction."""
    cfg = synth.WORKLOADS["spqr_33b"]
    shapes = cfg["layers"]
    Ms = (1, 4)
    Xd = {M: [to_dev(torch, synth.activations("spqr_33b", li, M)) for li in range(len(shapes))] for M in Ms}
    Yd = {M: [torch.empty((M, N), dtype=torch.float16, device="cuda") for N, _ in shapes] for M in Ms}
    Ws = []
    for li in range(len(shapes)):
        Ws.append(synth.layer_weight("spqr_33b", li))
        print(json.dumps({"generated_layer": li}), flush=True)
    f16 = dense_f16_weights(torch, Ws)
    base = {}
    for M in Ms:
        def f(i, M=M):
            for li in range(len(shapes)):
                torch.matmul(Xd[M][li], f16[i % len(f16)][li].t(), out=Yd[M][li])
        base[M] = graph_step_ms(torch, [f], len(f16), steps)
    del f16
    torch.cuda.empty_cache()

    rows = []
    t0 = {}
    for p in SWEEP_FRACS:
        packed, nnz, wb = [], [], 0
        for W in Ws:
            st = qlin.spqr_pack(W, p)
            packed.append([to_dev(torch, st[k]) for k in ("codes", "stats1", "stats2", "row_ptr", "col_idx", "val")])
            nnz.append(len(st["val"]))
            wb += sum(t.numel() * t.element_size() for t in packed[-1])
        R = copies_for(wb)
        sets = [packed] + [[[t.clone() for t in l] for l in packed] for _ in range(R - 1)]
        for M in Ms:
            def f(i, M=M):
                for li, (N, K) in enumerate(shapes):
                    c, s1, s2, rp, ci, v = sets[i % R][li]
                    qlin.spqr_forward(Xd[M][li], M, K, c, s1, s2, rp, ci, v, nnz[li], N, Yd[M][li], qlin.QLIN_F16)
            ms = graph_step_ms(torch, [f], R, steps)
            if p == 0.0:
                t0[M] = ms
            io = sum(M * K * 2 + M * N * 2 for N, K in shapes)
            rec = {"outlier_frac": p, "M": M, "nnz": sum(nnz), "bits_per_param": round(8.0 * wb / sum(N * K for N, K in shapes), 3),
                   "us": round(ms * 1e3, 2), "GB/s": round((wb + io) / (ms * 1e-3) / 1e9, 1),
                   "csr_time_share": round(max(0.0, (ms - t0[M]) / ms), 3),
                   "f16_us": round(base[M] * 1e3, 2), "speedup_vs_f16": round(base[M] / ms, 2)}
            print(json.dumps(rec), flush=True)
            rows.append(rec)
        del sets, packed
        torch.cuda.empty_cache()
    return {"sweep": "outliers", "layers": [f"{N}x{K}" for N, K in shapes], "rows": rows}


def sweep_actorder(torch, qlin, synth, steps):
    """Act-order storage without static groups needs the activations gathered
    through perm before the regular kernels (qlin_w4_forward_perm); with static
    groups the storage is natural (qlin_w4_forward).  Same Llama-7B-shaped
    layers and weight bytes; the timing does not depend on the values, so the
    weights are the round-to-nearest encode and perm a seeded permutation."""
    shapes = synth.WORKLOADS["w4_llama7b"]["layers"]
    Ms = (1, 8, 64)
    packed = [[to_dev(torch, a) for a in qlin.qlin_w4_pack(synth.layer_weight("w4_llama7b", li), 128)]
              for li in range(len(shapes))]
    wb = sum(t.numel() * t.element_size() for l in packed for t in l)
    sets = [packed] + [[[t.clone() for t in l] for l in packed] for _ in range(copies_for(wb) - 1)]
    perms = [to_dev(torch, synth.rng(f"actorder/perm{li}").permutation(K).astype(np.int32))
             for li, (_, K) in enumerate(shapes)]
    rows = []
    wsp = zeros_ws(torch, max(qlin.qlin_w4_workspace_bytes(qlin.QLIN_F16, M, K, N, 128, qlin.QLIN_F16)
                              for M in Ms for N, K in shapes))
    for M in Ms:
        Xd = [to_dev(torch, synth.x_f16(M, K, f"actorder/X{li}")) for li, (_, K) in enumerate(shapes)]
        Xp = [torch.empty_like(x) for x in Xd]
        Yd = [torch.empty((M, N), dtype=torch.float16, device="cuda") for N, _ in shapes]

        def natural(i):
            for li, (N, K) in enumerate(shapes):
                qw, sc, qz = sets[i % len(sets)][li]
                qlin.qlin_w4_forward(Xd[li], qlin.QLIN_F16, M, K, qw, sc, qz, N, 128, Yd[li], qlin.QLIN_F16,
                                     workspace=wsp)

        def gathered(i):
            for li, (N, K) in enumerate(shapes):
                qw, sc, qz = sets[i % len(sets)][li]
                qlin.qlin_w4_forward_perm(Xd[li], qlin.QLIN_F16, M, K, perms[li], Xp[li], qw, sc, qz, N, 128,
                                          Yd[li], qlin.QLIN_F16, workspace=wsp)
        t_nat = graph_step_ms(torch, [natural], len(sets), steps)
        t_gat = graph_step_ms(torch, [gathered], len(sets), steps)
        rec = {"M": M, "static_groups_us": round(t_nat * 1e3, 2), "act_order_gather_us": round(t_gat * 1e3, 2),
               "penalty_us": round((t_gat - t_nat) * 1e3, 2), "penalty_frac": round(t_gat / t_nat - 1.0, 3)}
        print(json.dumps(rec), flush=True)
        rows.append(rec)
    return {"sweep": "actorder", "layers": [f"{N}x{K}" for N, K in shapes], "rows": rows}


# ---------------------------------------------------------------------------

def cpu_baseline(synth):
    """The plain C++ oracle (oracle/qlin_oracle.cpp: fp64 decode + fp64 dot
    products, OpenMP over output rows), untouched, on full forward steps of the
    headline workload with one thread per core of the process affinity mask,
    plus the 1024x1024 4-bit layer at M=1 on one thread."""
    from oracle import cref
    from oracle import w4 as ow4
    cores = len(os.sched_getaffinity(0))
    cfg = synth.WORKLOADS["w4_llama7b"]
    packed = []
    total_bytes = 0
    for li, (N, K) in enumerate(cfg["layers"]):
        W = synth.layer_weight("w4_llama7b", li)
        st = ow4.encode(W, 128)
        X = synth.activations("w4_llama7b", li, 1)
        packed.append((X, st, K))
        total_bytes += sum(a.nbytes for a in st) + X.nbytes + N * 2
    cref.w4_forward(packed[0][0], *packed[0][1], packed[0][2], 128, threads=cores)     # load + warm
    t0 = time.perf_counter()
    reps = 0
    while True:
        for X, st, K in packed:
            cref.w4_forward(X, *st, K, 128, threads=cores)
        reps += 1
        if time.perf_counter() - t0 > 10.0 or reps >= 20:
            break
    dt = (time.perf_counter() - t0) / reps
    # small layer (1024 x 1024, M = 1) on one thread, median of 3
    c1 = synth.WORKLOADS["w4_1k"]
    N1, K1 = c1["layers"][0]
    st1 = ow4.encode(synth.layer_weight("w4_1k", 0), 128)
    X1 = synth.activations("w4_1k", 0, 1)
    b1 = sum(a.nbytes for a in st1) + X1.nbytes + N1 * 2
    ts = []
    for _ in range(3):
        t1 = time.perf_counter()
        cref.w4_forward(X1, *st1, K1, 128, threads=1)
        ts.append(time.perf_counter() - t1)
    t1 = sorted(ts)[1]
    return {"value": round(total_bytes / dt / 1e9, 3), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"{reps} full forward step(s) of the three 4-bit Llama-7B-shaped layers at M=1 through the "
                      f"plain C++ oracle (fp64 decode + fp64 dot, OpenMP over rows, {cores} threads = cores in "
                      f"the affinity mask), {dt * 1e3:.1f} ms per step",
            "one_thread_small_layer": {"layer": f"{N1}x{K1}, M=1", "GB/s": round(b1 / t1 / 1e9, 3),
                                       "ms": round(t1 * 1e3, 2), "threads": 1}}


# ---------------------------------------------------------------------------
# profile summaries (rocprofv3 csv -> text) and the counter-based traffic figure

GEMV_SOURCES = ("quantized_linear_layers_packed_amd/csrc/w4_gemv.hip",
                "quantized_linear_layers_packed_amd/csrc/device.hpp")
COUNTERS_FILE = os.path.join(ROOT, "profiles", "w4_gemv_w4_llama7b_m1_counters.txt")
COPY_BYTES = 256 << 20


def code_text(src):
    """C++ source with comments removed and whitespace runs collapsed: what the
    compiler sees, so that editing a comment does not invalidate a measurement."""
    import re
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def source_hash(paths=GEMV_SOURCES):
    import hashlib
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), encoding="utf-8") as f:
            h.update(code_text(f.read()).encode())
    return h.hexdigest()


def short_name(name):
    base = name.replace("(anonymous namespace)::", "").replace("qlin::", "")
    if base.startswith("void "):
        base = base[5:]
    return base.split("(")[0][:90]


def summarize(d):
    import csv
    from collections import defaultdict
    out = []
    tr = os.path.join(d, "trace", "run_kernel_trace.csv")
    if os.path.exists(tr):
        groups = defaultdict(list)
        with open(tr) as f:
            for r in csv.DictReader(f):
                key = (short_name(r["Kernel_Name"]), int(r["Grid_Size_X"]), int(r["LDS_Block_Size"]))
                groups[key].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
        out.append("kernel trace (rocprofv3 --kernel-trace --stats): per kernel and launch shape")
        out.append(f"{'kernel':92s} {'grid':>9s} {'lds':>6s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s}")
        for (k, g, l), v in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
            if "spin_kernel" in k or "FillFunctor" in k:
                continue
            out.append(f"{k:92s} {g:9d} {l:6d} {len(v):6d} {np.mean(v) / 1e3:9.3f} {np.min(v) / 1e3:9.3f}")
    cnt = {}
    for c in ("fetch", "write"):
        p = os.path.join(d, c, "run_counter_collection.csv")
        if not os.path.exists(p):
            continue
        groups = defaultdict(list)
        with open(p) as f:
            for r in csv.DictReader(f):
                key = (short_name(r["Kernel_Name"]), int(r["Grid_Size"]), int(r["LDS_Block_Size"]))
                groups[key].append(float(r["Counter_Value"]))
        cnt[c] = {k: float(np.mean(v)) for k, v in groups.items()}
    if cnt:
        out.append("")
        out.append("counters (rocprofv3 --pmc FETCH_SIZE / --pmc WRITE_SIZE, KiB per dispatch, mean)")
        scale = {}
        for c in cnt:
            copy = [v for k, v in cnt[c].items() if k[0].startswith("stream_copy_kernel")]
            scale[c] = (COPY_BYTES / 1024.0) / copy[0] if copy else None
            out.append(f"  {c}: plain copy of {COPY_BYTES >> 20} MiB reads {copy[0] if copy else float('nan'):.1f} KiB"
                       f" -> scale {scale[c]:.4f}")
        keys = sorted(set().union(*[set(v) for v in cnt.values()]))
        for k in keys:
            if "FillFunctor" in k[0]:
                continue
            f_ = cnt.get("fetch", {}).get(k, float("nan"))
            w_ = cnt.get("write", {}).get(k, float("nan"))
            out.append(f"  {k[0]:90s} grid {k[1]:9d} lds {k[2]:6d}  fetch {f_:12.1f}  write {w_:10.1f}")
        gemv = [k for k in keys if k[0].startswith("w4_gemv_kernel")]
        if gemv and scale.get("fetch") and scale.get("write"):
            fb = sum(cnt["fetch"][k] for k in gemv) * 1024 * scale["fetch"]
            wb = sum(cnt["write"][k] for k in gemv) * 1024 * scale["write"]
            rec = {"kernel": "w4_gemv_kernel", "launch_shapes": len(gemv), "fetch_bytes_per_step": round(fb),
                   "write_bytes_per_step": round(wb), "scale_fetch": scale["fetch"], "scale_write": scale["write"],
                   "source_sha256": source_hash()}
            out.append("COUNTERS_JSON: " + json.dumps(rec))
    return "\n".join(out)


def counter_traffic():
    """Calibrated HBM bytes per step of the W4 GEMV from the committed counter
    summary, or None when the summary is missing or the kernel source changed."""
    try:
        with open(COUNTERS_FILE) as f:
            line = [l for l in f if l.startswith("COUNTERS_JSON: ")][-1]
        rec = json.loads(line[len("COUNTERS_JSON: "):])
    except (OSError, IndexError, ValueError):
        return None
    if rec.get("source_sha256") != source_hash():
        return None
    return rec["fetch_bytes_per_step"] + rec["write_bytes_per_step"]


def main():
    args = parse()
    if args.summarize:
        print(summarize(args.summarize))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for {args.gpus}); this build has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import synth
    from quantized_linear_layers_packed_amd import qlin
    torch.cuda.set_device(0)

    if args.calibrate:
        nb = 256 << 20
        src = torch.ones(nb // 4, dtype=torch.int32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            qlin.qlin_stream_copy(dst, src, nb)
        torch.cuda.synchronize()
        del src, dst

    if args.sweep == "batch":
        print(json.dumps(sweep_batch(torch, qlin, synth, max(20, args.steps // 4))), flush=True)
        return
    if args.sweep == "actorder":
        print(json.dumps(sweep_actorder(torch, qlin, synth, max(20, args.steps // 4))), flush=True)
        return
    if args.sweep == "outliers":
        print(json.dumps(sweep_outliers(torch, qlin, synth, max(20, args.steps // 4))), flush=True)
        return

    # ---- headline: W4 GEMV, Llama-7B-shaped layers, M = 1
    layers = w4_layers(torch, qlin, synth, "w4_llama7b", 1)
    fns = w4_step_fns(qlin, layers)
    ms_step, per = time_steps(torch, fns, args.steps, args.warmup, len(layers[0]["packed"]))
    step_bytes = sum(l["wbytes"] + l["io"] for l in layers)
    value = step_bytes / (ms_step * 1e-3) / 1e9
    kern_ms = sum(per)
    achieved = step_bytes / (kern_ms * 1e-3) / 1e9
    per_layer = [{"shape": f"{l['N']}x{l['K']}", "bytes": l["wbytes"] + l["io"], "us": round(p * 1e3, 3),
                  "GB/s": round((l["wbytes"] + l["io"]) / (p * 1e-3) / 1e9, 1)} for l, p in zip(layers, per)]
    rot = len(layers[0]["packed"])
    del layers, fns
    torch.cuda.empty_cache()

    out = {
        "metric": "quantized-linear GB/s at M=1 (% HBM peak); TOPS at M=256 (% MFMA peak)",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u4 weights, f16 activations, f32 accumulate",
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) activations)",
        "config": {"workload": "w4_llama7b: 4-bit GEMV, layers 4096x4096 + 11008x4096 + 4096x11008, "
                               "group 128, M=1, fp16 in/out",
                   "global_batch": 1, "weight_copies_rotated": rot, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": counter_traffic(),
                     "kernel": "w4_gemv_kernel", "per": "step of three launches (bytes per step / kernel time per step)",
                     "algorithmic_bytes": step_bytes, "per_layer": per_layer},
    }

    if not args.no_paths:
        paths = {}
        steps = max(20, args.steps // 4)
        warm = max(5, args.warmup // 4)
        # SpQR M=1
        L = spqr_layers(torch, qlin, synth, 1)
        ms, per = time_steps(torch, spqr_step_fns(qlin, L), steps, warm, len(L[0]["packed"]))
        b = sum(l["wbytes"] + l["io"] for l in L)
        paths["spqr_33b_M1"] = {"value": round(b / (ms * 1e-3) / 1e9, 1), "unit": "GB/s",
                                "kernel_GB/s": round(b / (sum(per) * 1e-3) / 1e9, 1),
                                "frac_hbm": round(b / (sum(per) * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                "per_layer_us": [round(p * 1e3, 2) for p in per]}
        del L
        torch.cuda.empty_cache()
        # W4 GEMM M=256
        L = w4_layers(torch, qlin, synth, "w4_llama70b", 256)
        ms, per = time_steps(torch, w4_step_fns(qlin, L), steps, warm, len(L[0]["packed"]))
        fl = sum(2.0 * l["M"] * l["N"] * l["K"] for l in L)
        tf = fl / (sum(per) * 1e-3) / 1e12
        paths["w4_llama70b_M256"] = {"value": round(fl / (ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
                                     "kernel_TFLOP/s": round(tf, 2), "frac_mfma_f16": round(tf / 2500.0, 4),
                                     "per_layer_us": [round(p * 1e3, 2) for p in per]}
        del L
        torch.cuda.empty_cache()
        # SmoothQuant M=256
        L = sq_layers(torch, qlin, synth, 256)
        act, gemm = sq_step_fns(qlin, L)
        ms, per = time_steps(torch, [f for pair in zip(act, gemm) for f in pair], steps, warm, len(L[0]["packed"]))
        ops = sum(2.0 * l["M"] * l["N"] * l["K"] for l in L)
        gemm_ms = per[1] + per[3]
        tops = ops / (gemm_ms * 1e-3) / 1e12
        paths["sq_w8a8_M256"] = {"value": round(ops / (ms * 1e-3) / 1e12, 2), "unit": "TOPS (act+gemm)",
                                 "gemm_kernel_TOPS": round(tops, 2), "frac_mfma_i8": round(tops / 5000.0, 4),
                                 "act_us": [round(per[0] * 1e3, 2), round(per[2] * 1e3, 2)],
                                 "gemm_us": [round(per[1] * 1e3, 2), round(per[3] * 1e3, 2)]}
        del L
        torch.cuda.empty_cache()
        out["paths"] = paths

    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(synth)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
