"""The library's host encoders against the oracle's: byte-identical output.

Both sides implement the same written encode rules independently (fp32
arithmetic, round half to even), so every byte of codes, scales, zeros,
statistics, CSR arrays, smoothing vectors and int8 weights must agree."""
import numpy as np
import pytest

import synth
from oracle import smoothquant as osq
from oracle import spqr as ospqr
from oracle import w4 as ow4
from quantized_linear_layers_packed_amd import qlin


def _eq(a, b):
    a, b = np.asarray(a), np.asarray(b)
    assert a.shape == b.shape, (a.shape, b.shape)
    assert a.tobytes() == b.tobytes()


@pytest.mark.parametrize("N,K,G,sigma", [(64, 1024, 128, 0.02), (33, 11008, 128, 0.02),
                                         (16, 512, 32, 0.015), (8, 768, 256, 1e-3), (3, 128, 64, 3.0)])
def test_w4_pack_matches_oracle(N, K, G, sigma):
    W = synth.normal_f32((N, K), sigma, f"pack/w4/{N}x{K}")
    W[0, :G] = 0.0                                    # a constant-zero group
    if N > 1:
        W[1, :G] = np.abs(W[1, :G])                   # a one-signed group
    lib = qlin.qlin_w4_pack(W, G)
    ref = ow4.encode(W, G)
    for a, b in zip(lib, ref):
        _eq(a, b)


@pytest.mark.slow
def test_w4_pack_matches_oracle_full_layer():
    W = synth.layer_weight("w4_llama7b", 2)
    for a, b in zip(qlin.qlin_w4_pack(W, 128), ow4.encode(W, 128)):
        _eq(a, b)


@pytest.mark.parametrize("N,K,p,seed", [(16, 512, 0.01, 0), (40, 1024, 0.01, 1), (7, 2560, 0.03, 2),
                                        (5, 256, 0.0, 3), (64, 6656, 0.01, 4)])
def test_spqr_pack_matches_oracle(N, K, p, seed):
    W = synth.student_t3_f32((N, K), 0.02, f"pack/spqr/{seed}")
    W[0, 16:32] = 0.0                                 # a flat group
    if N > 2:
        W[2, 5] = W[2, 9] = np.float32(3.0)           # ties among the largest
    lib = qlin.spqr_pack(W, p)
    ref = ospqr.encode(W, p)
    for k in ("codes", "stats1", "stats2", "row_ptr", "col_idx", "val"):
        _eq(lib[k], ref[k])


@pytest.mark.slow
def test_spqr_pack_matches_oracle_full_layer():
    W = synth.layer_weight("spqr_33b", 0)
    lib = qlin.spqr_pack(W, 0.01)
    ref = ospqr.encode(W, 0.01)
    for k in ("codes", "stats1", "stats2", "row_ptr", "col_idx", "val"):
        _eq(lib[k], ref[k])


@pytest.mark.parametrize("N", [64, 4096])
def test_smoothquant_host_calls_match_oracle(N):
    X = synth.sq_calibration("sq_w8a8", 1)
    W = synth.normal_f32((N, 4096), 0.02, f"pack/sq/{N}")
    W[3] = 0.0                                         # a zero weight row
    amax = qlin.sq_act_absmax(X)
    _eq(amax, osq.act_absmax(X))
    amax[7] = 0.0                                      # a silent channel
    s, inv = qlin.sq_compute_smoothing(amax, W, 0.85)
    s_o, inv_o = osq.smoothing(amax, W, 0.85)
    _eq(s, s_o)
    _eq(inv, inv_o)
    Wq, ws = qlin.sq_pack_weight(W, s)
    Wq_o, ws_o = osq.quantize_weight(W, s_o)
    _eq(Wq, Wq_o)
    _eq(ws, ws_o)
