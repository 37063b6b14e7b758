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
    p.add_argument("--profile", metavar="PATH",
                   help="run one workload point (e.g. w4_llama7b_M1, spqr_33b_M16, w4_llama70b_M256, "
                        "sq_w8a8_M256) --iters times, untimed, for a profiler, and exit")
    p.add_argument("--iters", type=int, default=5)
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
    bracket ``copies`` launches on the stream they run on).  Per-dispatch
    medians come from the rocprofv3 kernel trace (bench.py --summarize):
    events around single replays add the replay launch gap."""
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

def w4_layers(torch, qlin, synth, workload, Ms):
    """Packed, rotated weights of a W4 workload, with activations, outputs and a
    shared workspace for every batch size in Ms."""
    Ms = (Ms,) if isinstance(Ms, int) else tuple(Ms)
    cfg = synth.WORKLOADS[workload]
    G = cfg["G"]
    xbf = cfg["x_dtype"] == "bf16"
    xdt = qlin.QLIN_BF16 if xbf else qlin.QLIN_F16
    ydt = qlin.QLIN_BF16 if cfg["y_dtype"] == "bf16" else qlin.QLIN_F16
    ytd = torch.bfloat16 if cfg["y_dtype"] == "bf16" else torch.float16
    layers = []
    for li, (N, K) in enumerate(cfg["layers"]):
        W = synth.layer_weight(workload, li)
        packed = [to_dev(torch, a) for a in qlin.qlin_w4_pack(W, G)]
        del W
        X = {M: to_dev(torch, synth.activations(workload, li, M)) for M in Ms}
        Y = {M: torch.empty((M, N), dtype=ytd, device="cuda") for M in Ms}
        wbytes = sum(t.numel() * t.element_size() for t in packed)
        layers.append(dict(N=N, K=K, G=G, packed=[packed], Xs=X, Ys=Y, wbytes=wbytes, xdt=xdt, ydt=ydt,
                           ios={M: X[M].numel() * X[M].element_size() + Y[M].numel() * Y[M].element_size()
                                for M in Ms}))
    need = max(qlin.qlin_w4_workspace_bytes(xdt, M, l["K"], l["N"], G, ydt) for l in layers for M in Ms)
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


def w4_step_fns(qlin, layers, M):
    fns = []
    for l in layers:
        def f(i, l=l):
            qw, sc, qz = l["packed"][i % len(l["packed"])]
            qlin.qlin_w4_forward(l["Xs"][M], l["xdt"], M, l["K"], qw, sc, qz, l["N"], l["G"], l["Ys"][M], l["ydt"],
                                 workspace=l["ws"])
        fns.append(f)
    return fns


def spqr_layers(torch, qlin, synth, Ms):
    Ms = (Ms,) if isinstance(Ms, int) else tuple(Ms)
    cfg = synth.WORKLOADS["spqr_33b"]
    layers = []
    for li, (N, K) in enumerate(cfg["layers"]):
        W = synth.layer_weight("spqr_33b", li)
        st = qlin.spqr_pack(W, cfg["outlier_frac"])
        del W
        packed = [to_dev(torch, st[k]) for k in ("codes", "stats1", "stats2", "row_ptr", "col_idx", "val")]
        X = {M: to_dev(torch, synth.activations("spqr_33b", li, M)) for M in Ms}
        Y = {M: torch.empty((M, N), dtype=torch.float16, device="cuda") for M in Ms}
        wbytes = sum(t.numel() * t.element_size() for t in packed)
        layers.append(dict(N=N, K=K, nnz=len(st["val"]), packed=[packed], Xs=X, Ys=Y, wbytes=wbytes,
                           ios={M: M * K * 2 + M * N * 2 for M in Ms}))
    ws = zeros_ws(torch, max(qlin.spqr_workspace_bytes(M, l["K"], l["N"], qlin.QLIN_F16) for l in layers for M in Ms))
    for l in layers:
        l["ws"] = ws
    rotate(torch, layers)
    return layers


def spqr_step_fns(qlin, layers, M):
    fns = []
    for l in layers:
        def f(i, l=l):
            c, s1, s2, rp, ci, v = l["packed"][i % len(l["packed"])]
            qlin.spqr_forward(l["Xs"][M], M, l["K"], c, s1, s2, rp, ci, v, l["nnz"], l["N"], l["Ys"][M],
                              qlin.QLIN_F16, workspace=l["ws"])
        fns.append(f)
    return fns


def sq_layers(torch, qlin, synth, Ms):
    Ms = (Ms,) if isinstance(Ms, int) else tuple(Ms)
    cfg = synth.WORKLOADS["sq_w8a8"]
    layers = []
    for li, (N, K) in enumerate(cfg["layers"]):
        W = synth.layer_weight("sq_w8a8", li)
        Xcal = synth.sq_calibration("sq_w8a8", li)
        s, inv = qlin.sq_compute_smoothing(qlin.sq_act_absmax(Xcal), W, cfg["alpha"])
        Wq, ws = qlin.sq_pack_weight(W, s)
        del W
        packed = [to_dev(torch, Wq), to_dev(torch, ws)]
        layers.append(dict(N=N, K=K, packed=[packed], inv=to_dev(torch, inv),
                           Xs={M: to_dev(torch, synth.activations("sq_w8a8", li, M)) for M in Ms},
                           Xqs={M: torch.empty((M, K), dtype=torch.int8, device="cuda") for M in Ms},
                           xss={M: torch.empty((M,), dtype=torch.float32, device="cuda") for M in Ms},
                           Ys={M: torch.empty((M, N), dtype=torch.float16, device="cuda") for M in Ms},
                           wbytes=sum(t.numel() * t.element_size() for t in packed)))
    ws = zeros_ws(torch, max(qlin.sq_int8_gemm_workspace_bytes(M, l["N"], l["K"], qlin.QLIN_F16)
                             for l in layers for M in Ms))
    for l in layers:
        l["ws"] = ws
    rotate(torch, layers)
    return layers


def sq_step_fns(qlin, layers, M):
    act, gemm = [], []
    for l in layers:
        def a(i, l=l):
            qlin.sq_smooth_quant_act(l["Xs"][M], l["inv"], M, l["K"], l["Xqs"][M], l["xss"][M])

        def g(i, l=l):
            Wq, ws = l["packed"][i % len(l["packed"])]
            qlin.sq_int8_gemm(l["Xqs"][M], l["xss"][M], Wq, ws, M, l["N"], l["K"], l["Ys"][M], qlin.QLIN_F16, None,
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
    kernel + int8 GEMM) vs dense fp16 (this library's qlin_f16_gemm) on the
    Llama-7B-shaped layers, for M = 1 .. 2048, with the vendor fp16 GEMM
    (torch.matmul) as a context column.  Same fp16 activations for all (N(0,1),
    1% of channels x100, the SmoothQuant workload's recipe)."""
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
                                  qlin.sq_int8_gemm_workspace_bytes(M, N, K, qlin.QLIN_F16),
                                  qlin.qlin_f16_gemm_workspace_bytes(M, N, K, qlin.QLIN_F16))
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
            for li, (N, K) in enumerate(shapes):
                def f(i, li=li, N=N, K=K):
                    qlin.qlin_f16_gemm(Xd[li][:M], f16[i % len(f16)][li], M, N, K, Yd[li][:M], qlin.QLIN_F16,
                                       workspace=wsp)
                out.append(f)
            return out

        def vendor_fns():
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
                                            ("f16", f16_fns(), len(f16), f16_bytes, MFMA_PEAK_TFLOPS["f16"]),
                                            ("f16_vendor", vendor_fns(), len(f16), f16_bytes,
                                             MFMA_PEAK_TFLOPS["f16"])):
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
    wsp = zeros_ws(torch, max(qlin.spqr_workspace_bytes(M, K, N, qlin.QLIN_F16) for M in Ms for N, K in shapes))
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
                    qlin.spqr_forward(Xd[M][li], M, K, c, s1, s2, rp, ci, v, nnz[li], N, Yd[M][li], qlin.QLIN_F16,
                                      workspace=wsp)
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
        out.append(f"{'kernel':92s} {'grid':>9s} {'lds':>6s} {'calls':>6s} {'avg_us':>9s} {'med_us':>9s} {'min_us':>9s}")
        for (k, g, l), v in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
            if "spin_kernel" in k or "FillFunctor" in k:
                continue
            out.append(f"{k:92s} {g:9d} {l:6d} {len(v):6d} {np.mean(v) / 1e3:9.3f} {np.median(v) / 1e3:9.3f} "
                       f"{np.min(v) / 1e3:9.3f}")
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
            fmb = f_ * 1024 * scale["fetch"] / 1e6 if scale.get("fetch") else float("nan")
            wmb = w_ * 1024 * scale["write"] / 1e6 if scale.get("write") else float("nan")
            out.append(f"  {k[0]:90s} grid {k[1]:9d} lds {k[2]:6d}  fetch {f_:12.1f}  write {w_:10.1f}"
                       f"  -> {fmb:9.3f} MB read {wmb:8.3f} MB written")
        gemv = [k for k in keys if k[0].startswith("w4_gemv_kernel")]
        if gemv and scale.get("fetch") and scale.get("write"):
            fb = sum(cnt["fetch"][k] for k in gemv) * 1024 * scale["fetch"]
            wb = sum(cnt["write"][k] for k in gemv) * 1024 * scale["write"]
            rec = {"kernel": "w4_gemv_kernel", "launch_shapes": len(gemv), "fetch_bytes_per_step": round(fb),
                   "write_bytes_per_step": round(wb), "scale_fetch": scale["fetch"], "scale_write": scale["write"],
                   "source_sha256": source_hash()}
            out.append("COUNTERS_JSON: " + json.dumps(rec))
    # instruction / utilisation counters (passes "sq" and "tcc", several counters each)
    multi = defaultdict(dict)
    for c in ("sq", "tcc"):
        p = os.path.join(d, c, "run_counter_collection.csv")
        if not os.path.exists(p):
            continue
        groups = defaultdict(list)
        with open(p) as f:
            for r in csv.DictReader(f):
                key = (short_name(r["Kernel_Name"]), int(r["Grid_Size"]), int(r["LDS_Block_Size"]))
                groups[(key, r["Counter_Name"])].append(float(r["Counter_Value"]))
        for (key, name), v in groups.items():
            multi[key][name] = float(np.mean(v))
    if multi:
        out.append("")
        out.append("instruction and utilisation counters (rocprofv3 --pmc, mean per dispatch); per wave = / SQ_WAVES;")
        out.append("mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE * 4 * CUs), then divided by the same ratio")
        out.append("of the dense register-only MFMA loop (mfma_peak_kernel), so that loop reads 1.0;")
        out.append("l2_hit = TCC_HIT_sum / (TCC_HIT_sum + TCC_MISS_sum); lds_conflict = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE")
        raw = {k: (v.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / max(1.0, v.get("GRBM_GUI_ACTIVE", 0.0) * 4 * 256))
               for k, v in multi.items()}
        ref = [raw[k] for k in raw if k[0].startswith("mfma_peak_kernel")]
        norm = max(ref) if ref else None
        out.append(f"{'kernel':70s} {'grid':>8s} {'waves':>8s} {'VALU/w':>8s} {'SALU/w':>8s} {'MFMA/w':>8s} "
                   f"{'LDS/w':>7s} {'mfma_busy':>9s} {'l2_hit':>7s} {'lds_cfl':>7s}")
        for k, v in sorted(multi.items()):
            if "FillFunctor" in k[0] or "stream_copy" in k[0]:
                continue
            w = max(1.0, v.get("SQ_WAVES", 0.0))
            hit, miss = v.get("TCC_HIT_sum"), v.get("TCC_MISS_sum")
            l2 = f"{hit / (hit + miss):7.3f}" if hit is not None and miss is not None and hit + miss > 0 else f"{'-':>7s}"
            lc = v.get("SQ_LDS_BANK_CONFLICT"), v.get("SQ_LDS_IDX_ACTIVE")
            lcs = f"{lc[0] / lc[1]:7.3f}" if lc[0] is not None and lc[1] else f"{'-':>7s}"
            mb = f"{raw[k] / norm:9.3f}" if norm and "SQ_VALU_MFMA_BUSY_CYCLES" in v else f"{'-':>9s}"
            out.append(f"{k[0][:70]:70s} {k[1]:8d} {w:8.0f} {v.get('SQ_INSTS_VALU', 0) / w:8.1f} "
                       f"{v.get('SQ_INSTS_SALU', 0) / w:8.1f} {v.get('SQ_INSTS_MFMA', 0) / w:8.1f} "
                       f"{v.get('SQ_INSTS_LDS', 0) / w:7.1f} {mb} {l2} {lcs}")
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

    if args.profile:
        profile_path(torch, qlin, synth, args.profile, args.iters)
        return
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
    fns = w4_step_fns(qlin, layers, 1)
    ms_step, per = time_steps(torch, fns, args.steps, args.warmup, len(layers[0]["packed"]))
    step_bytes = sum(l["wbytes"] + l["ios"][1] for l in layers)
    value = step_bytes / (ms_step * 1e-3) / 1e9
    kern_ms = sum(per)
    achieved = step_bytes / (kern_ms * 1e-3) / 1e9
    layer_bytes = [l["wbytes"] + l["ios"][1] for l in layers]
    per_layer = [{"shape": f"{l['N']}x{l['K']}", "bytes": b, "us": round(p * 1e3, 3),
                  "GB/s": round(b / (p * 1e-3) / 1e9, 1)} for l, b, p in zip(layers, layer_bytes, per)]
    # the same steps all on the first weight copy: served from the 256 MB
    # last-level cache, not from HBM (a labelled cache-resident figure, never
    # the value); graphs of the same length as the rotation
    hot_ms, hot_per = time_steps(torch, [lambda i, f=f: f(0) for f in fns], args.steps, args.warmup,
                                 len(layers[0]["packed"]))
    hot = {"note": "one weight copy, cache-resident (256 MB last-level cache), not an HBM figure",
           "ms_per_step": round(hot_ms, 5), "GB/s_per_step": round(step_bytes / (hot_ms * 1e-3) / 1e9, 1),
           "per_layer_us": [round(p * 1e3, 3) for p in hot_per]}
    rot = len(layers[0]["packed"])
    del layers, fns
    torch.cuda.empty_cache()

    peaks = measured_peaks(torch, qlin, layer_bytes)
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
                     "algorithmic_bytes": step_bytes, "per_layer": per_layer,
                     "measured_peak": peaks["hbm_read_GB/s"],
                     "frac_measured_peak": round(achieved / peaks["hbm_read_GB/s"], 4),
                     "stream_read_floor_us": peaks["floor_us"],
                     "frac_of_floor": round(sum(peaks["floor_us"]) / (kern_ms * 1e3), 4)},
        "measured_peaks": {k: v for k, v in peaks.items() if k != "floor_us"},
        "hot_cache_resident": hot,
    }

    if not args.no_paths:
        out["paths"] = run_paths(torch, qlin, synth, max(20, args.steps // 4), max(5, args.warmup // 4), peaks)

    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(synth)
    print(json.dumps(out), flush=True)


def profile_path(torch, qlin, synth, names, iters):
    """Run workload points eagerly `iters` times each over their weight rotation
    (every launch reads its weights from HBM), for rocprofv3.  names: comma-
    separated, e.g. "spqr_33b_M1,spqr_33b_M16" (points of one workload share
    its packed weights) or "mfma_peak_f16"."""
    groups = {}
    for name in names.split(","):
        if name.startswith("mfma_peak_"):
            kind = {"f16": 0, "bf16": 1, "i8": 2}[name[len("mfma_peak_"):]]
            out = torch.empty(2048 * 4, dtype=torch.float32, device="cuda")
            for _ in range(iters):
                qlin.qlin_mfma_peak(kind, 2000, 2048, out)
            torch.cuda.synchronize()
            print(json.dumps({"profiled": name, "iters": iters}), flush=True)
            continue
        workload, M = name.rsplit("_M", 1)
        groups.setdefault(workload, []).append(int(M))
    for workload, Ms in groups.items():
        if workload == "sq_w8a8":
            L = sq_layers(torch, qlin, synth, Ms)
        elif workload == "spqr_33b":
            L = spqr_layers(torch, qlin, synth, Ms)
        else:
            L = w4_layers(torch, qlin, synth, workload, Ms)
        copies = len(L[0]["packed"])
        for M in Ms:
            if workload == "sq_w8a8":
                act, gemm = sq_step_fns(qlin, L, M)
                fns = [f for pair in zip(act, gemm) for f in pair]
            elif workload == "spqr_33b":
                fns = spqr_step_fns(qlin, L, M)
            else:
                fns = w4_step_fns(qlin, L, M)
            for i in range(iters):
                for f in fns:
                    f(i % copies)
            torch.cuda.synchronize()
            print(json.dumps({"profiled": f"{workload}_M{M}", "iters": iters, "launches": iters * len(fns)}),
                  flush=True)
        del L
        torch.cuda.empty_cache()


def measured_peaks(torch, qlin, floor_bytes):
    """Achievable rates measured on this GPU, next to the datasheet figures:
    a plain non-temporal streaming read of 2 GiB (16-byte loads, best of 5), the
    same read at each headline layer's byte count from a rotation of 1 GiB of
    buffers (the floor a single launch of that size can reach), and dense
    register-only MFMA loops per data type (best of 5)."""
    res = {}
    nb = 2 << 30
    buf = torch.empty(nb // 4, dtype=torch.int32, device="cuda")
    out = torch.empty(1 << 16, dtype=torch.int32, device="cuda")
    best = None
    for _ in range(5):
        ms = _event_ms(torch, lambda: qlin.qlin_stream_read(buf, nb, 8192, 8, 1, out))
        best = ms if best is None else min(best, ms)
    res["hbm_read_GB/s"] = round(nb / (best * 1e-3) / 1e9, 1)
    del buf
    floors = []
    for b in floor_bytes:
        b16 = (b + 15) // 16 * 16
        copies = copies_for(b16)
        bufs = [torch.empty(b16 // 4, dtype=torch.int32, device="cuda") for _ in range(copies)]
        grid = max(256, min(8192, b16 // (16 * 256 * 8) + 1))
        g = _graph(torch, lambda: [qlin.qlin_stream_read(x, b16, grid, 8, 1, out) for x in bufs])
        floors.append(round(_replay_ms(torch, g, 10) / copies * 1e3, 3))
        del g, bufs
    res["floor_us"] = floors
    flops = {0: 32768.0, 1: 32768.0, 2: 65536.0}
    grid, iters = 2048, 2000
    pk = torch.empty(grid * 4, dtype=torch.float32, device="cuda")
    res["mfma_TFLOP/s"] = {}
    for kind, name in ((0, "f16"), (1, "bf16"), (2, "i8")):
        best = None
        for _ in range(5):
            ms = _event_ms(torch, lambda: qlin.qlin_mfma_peak(kind, iters, grid, pk))
            best = ms if best is None else min(best, ms)
        res["mfma_TFLOP/s"][name] = round(grid * 4 * iters * 4 * flops[kind] / (best * 1e-3) / 1e12, 1)
    torch.cuda.empty_cache()
    return res


def _event_ms(torch, f):
    f()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    f()
    e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1)


def _rate_record(bytes_, ops, kern_us, mfma_kind, peaks, extra=None):
    """Rates of one timed kernel set against both rooflines: HBM (algorithmic
    bytes at 8 TB/s) and MFMA (algorithmic ops at the dtype's dense peak), with
    the binding one and the fraction of its ideal time reached; also against
    the measured peaks."""
    peak_tf = MFMA_PEAK_TFLOPS[mfma_kind] if mfma_kind else None
    t_hbm = bytes_ / (HBM_PEAK_GBS * 1e9) * 1e6
    t_mfma = ops / (peak_tf * 1e12) * 1e6 if peak_tf else 0.0
    mh = peaks["hbm_read_GB/s"]
    mt = peaks["mfma_TFLOP/s"][mfma_kind] if mfma_kind else None
    t_hbm_m = bytes_ / (mh * 1e9) * 1e6
    t_mfma_m = ops / (mt * 1e12) * 1e6 if mt else 0.0
    rec = {"kernel_us": round(kern_us, 2), "bytes": int(bytes_), "ops": int(ops),
           "GB/s": round(bytes_ / (kern_us * 1e-6) / 1e9, 1),
           "TOPS": round(ops / (kern_us * 1e-6) / 1e12, 2),
           "frac_hbm": round(bytes_ / (kern_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
           "bound": "hbm" if t_hbm >= t_mfma else "mfma",
           "roofline_us": round(max(t_hbm, t_mfma), 3),
           "frac_roofline": round(max(t_hbm, t_mfma) / kern_us, 4),
           "frac_measured_roofline": round(max(t_hbm_m, t_mfma_m) / kern_us, 4)}
    if peak_tf:
        rec["frac_mfma"] = round(ops / (kern_us * 1e-6) / 1e12 / peak_tf, 4)
    if extra:
        rec.update(extra)
    return rec


# batch sizes timed per workload besides the headline (the configurations'
# own M sets; 256 added for the int8 GEMM, where the metric is quoted)
PATH_POINTS = (("w4_1k", (1, 4)), ("spqr_33b", (1, 4, 8, 16)), ("w4_llama70b", (32, 64, 256)),
               ("sq_w8a8", (256, 512, 2048)))


def run_paths(torch, qlin, synth, steps, warm, peaks):
    paths = {}
    for workload, Ms in PATH_POINTS:
        if workload == "sq_w8a8":
            L = sq_layers(torch, qlin, synth, Ms)
        elif workload == "spqr_33b":
            L = spqr_layers(torch, qlin, synth, Ms)
        else:
            L = w4_layers(torch, qlin, synth, workload, Ms)
        copies = len(L[0]["packed"])
        for M in Ms:
            key = f"{workload}_M{M}"
            if workload == "sq_w8a8":
                act, gemm = sq_step_fns(qlin, L, M)
                ms, per = time_steps(torch, [f for pair in zip(act, gemm) for f in pair], steps, warm, copies)
                act_us = [per[2 * i] * 1e3 for i in range(len(L))]
                gemm_us = [per[2 * i + 1] * 1e3 for i in range(len(L))]
                ops = sum(2.0 * M * l["N"] * l["K"] for l in L)
                gb = sum(l["wbytes"] + M * l["K"] + 4 * M + 2 * M * l["N"] for l in L)
                ab = sum(2 * M * l["K"] + 4 * l["K"] + M * l["K"] + 4 * M for l in L)
                paths[key] = {"unit": "TOPS", "us_per_step": round(ms * 1e3, 2),
                              "gemm": _rate_record(gb, ops, sum(gemm_us), "i8", peaks,
                                                   {"per_layer_us": [round(x, 2) for x in gemm_us]}),
                              "act": _rate_record(ab, 0, sum(act_us), None, peaks,
                                                  {"per_layer_us": [round(x, 2) for x in act_us]}),
                              "TOPS_act_plus_gemm": round(ops / (ms * 1e-3) / 1e12, 2)}
            else:
                fns = spqr_step_fns(qlin, L, M) if workload == "spqr_33b" else w4_step_fns(qlin, L, M)
                ms, per = time_steps(torch, fns, steps, warm, copies)
                us = [p * 1e3 for p in per]
                bytes_ = sum(l["wbytes"] + l["ios"][M] for l in L)
                ops = sum(2.0 * M * l["N"] * l["K"] + 2.0 * M * l.get("nnz", 0) for l in L)
                kind = "bf16" if workload == "w4_llama70b" else "f16"
                paths[key] = _rate_record(bytes_, ops, sum(us), kind, peaks,
                                          {"us_per_step": round(ms * 1e3, 2),
                                           "per_layer_us": [round(x, 2) for x in us]})
            print(json.dumps({"path": key, **paths[key]}), file=sys.stderr, flush=True)
        del L
        torch.cuda.empty_cache()
    return paths


if __name__ == "__main__":
    main()
