"""Pins of the SpQR oracle: hand-worked layout and second-level cases, grid points
that must round-trip exactly, outlier count and order, brute-force dense
reconstruction, a textbook CSR product, the RTN bound and the pages' range of
bits per parameter."""
import numpy as np
import pytest
import scipy.sparse

import synth
from oracle import spqr


def test_chunk_layout_hand_cases(golden):
    g = golden("spqr_layout.json")
    for case in g["code_cases"]:
        q = np.zeros((1, 32), np.uint8)
        q[0, case["code"]] = case["value"]
        assert spqr.pack_codes(q)[0, 0].tolist() == case["words"], case["why"]
    for case in g["stats1_cases"]:
        cs = np.zeros((1, 16), np.uint8)
        cz = np.zeros((1, 16), np.uint8)
        cs[0, case["group"]] = case["cs"]
        cz[0, case["group"]] = case["cz"]
        assert spqr.pack_stats1(cs, cz)[0, 0].tolist() == case["words"], case["why"]


def test_chunk_layout_uses_every_bit_once_and_keeps_groups_apart():
    seen = {}
    for c, bits in enumerate(spqr.CHUNK_POS):
        for wb in bits:
            assert wb not in seen
            seen[wb] = c
    assert len(seen) == 96
    for w in range(3):                       # field i of both halves: same group
        for i in range(5):
            lo, hi = seen[(w, 3 * i)], seen[(w, 16 + 3 * i)]
            assert (lo < 16) == (hi < 16)
    assert (seen[(0, 15)] >= 16) == (seen[(0, 31)] >= 16)


def test_round_trips():
    r = np.random.default_rng(3)
    q = r.integers(0, 8, size=(5, 512)).astype(np.uint8)
    assert np.array_equal(spqr.unpack_codes(spqr.pack_codes(q), 512), q)
    cs = r.integers(0, 8, size=(5, 64)).astype(np.uint8)
    cz = r.integers(0, 8, size=(5, 64)).astype(np.uint8)
    cs2, cz2 = spqr.unpack_stats1(spqr.pack_stats1(cs, cz))
    assert np.array_equal(cs2, cs) and np.array_equal(cz2, cz)


def test_second_level_hand_case(golden):
    g = golden("spqr_second_level.json")
    v = (3.0 + np.array(g["j"], np.float64)) * 2.0 ** -10
    SS, ZS, c, v_hat = spqr.second_level(v.astype(np.float32)[None, :])
    assert float(SS[0]) == g["SS"] and float(ZS[0]) == g["ZS"]
    assert c[0].tolist() == g["c"]
    assert np.array_equal(v_hat[0].astype(np.float64), g["SS"] * (np.array(g["c"]) - g["ZS"]))


def _grid_layer(N, K, seed):
    """Weights on the bi-level grid (no outliers): per block an fp16 scale step SS
    with ZS_s = -1 and codes 0..7 all present, zeros SS_z = 1, ZS_z = 0 with
    codes 0..7 all present, and weight codes 0 and 7 present in every group."""
    r = np.random.default_rng(seed)
    nb, ng = K // 256, K // 16
    SS = (2.0 ** r.integers(-12, -7, size=(N, nb)) * r.integers(1024, 2048, size=(N, nb)) / 1024)
    SS = SS.astype(np.float16)
    cs = np.stack([r.permutation(np.r_[np.arange(8), r.integers(0, 8, 8)]) for _ in range(N * nb)])
    cz = np.stack([r.permutation(np.r_[np.arange(8), r.integers(0, 8, 8)]) for _ in range(N * nb)])
    cs = cs.reshape(N, ng)
    cz = cz.reshape(N, ng)
    s_hat = np.repeat(SS.astype(np.float32), 16, axis=1) * (cs + 1).astype(np.float32)
    z_hat = cz.astype(np.float32)
    q = r.integers(0, 8, size=(N, ng, 16))
    q[:, :, 0] = 0
    q[:, :, 1] = 7
    for row in q.reshape(-1, 16):
        r.shuffle(row)
    W = s_hat[:, :, None] * (q.astype(np.float32) - z_hat[:, :, None])
    return W.reshape(N, K).astype(np.float32), q.reshape(N, K), cs, cz, SS


def test_grid_points_are_reproduced_exactly():
    W, q, cs, cz, SS = _grid_layer(6, 512, seed=4)
    d = spqr.quantize(W, p=0.0)
    assert np.array_equal(d["q"], q)
    assert np.array_equal(d["cs"], cs) and np.array_equal(d["cz"], cz)
    assert np.array_equal(d["SSs"].view(np.uint16), SS.view(np.uint16))
    assert np.all(d["ZSs"] == -1) and np.all(d["SSz"] == 1) and np.all(d["ZSz"] == 0)
    st = spqr.encode(W, p=0.0)
    assert len(st["val"]) == 0
    assert np.array_equal(spqr.dequantize_dense(st["codes"], st["stats1"], st["stats2"], 512),
                          W.astype(np.float64))


def test_outlier_count_order_and_ties():
    W = synth.student_t3_f32((40, 512), 0.02, "pin/spqr/out")
    W[3, 7] = W[5, 9] = W[1, 100] = np.float32(5.0)     # a three-way tie at the top ...
    W[0, 0] = np.float32(-5.0)                           # ... plus one of the other sign
    n_out = spqr.n_outliers(40, 512, 0.01)
    assert n_out == 204                                  # floor(0.01 * 20480)
    mask = spqr.select_outliers(W, n_out)
    assert mask.sum() == n_out
    assert np.array_equal(mask, spqr.select_outliers_by_sort(W, n_out))
    a = np.abs(W)
    assert a[mask].min() >= a[~mask].max()
    top2 = spqr.select_outliers(W, 2)                    # four equal |w|: lowest indices win
    assert set(zip(*np.nonzero(top2))) == {(0, 0), (1, 100)}
    for shape, expect in (((6656, 6656), 443023), ((17920, 6656), 1192755), ((6656, 17920), 1192755)):
        assert spqr.n_outliers(*shape, 0.01) == expect


def test_brute_force_dense_reconstruction():
    for (N, K, seed) in ((8, 256, 5), (32, 512, 6)):
        W = synth.student_t3_f32((N, K), 0.02, f"pin/spqr/bf{seed}")
        X = synth.x_f16(3, K, f"pin/spqr/bfx{seed}")
        st = spqr.encode(W, 0.01)
        assert len(st["val"]) == spqr.n_outliers(N, K, 0.01)
        dense = spqr.dequantize_dense(st["codes"], st["stats1"], st["stats2"], K)
        W_hat = dense + spqr.sparse_dense(st["row_ptr"], st["col_idx"], st["val"], N, K)
        Y = spqr.forward(X, st, K)
        Xd = X.astype(np.float64)
        for m in range(3):
            for n in range(N):
                ref = sum(Xd[m, k] * W_hat[n, k] for k in range(K))
                assert abs(ref - Y[m, n]) <= 1e-13 * max(1.0, np.abs(Xd[m]) @ np.abs(W_hat[n]))
        mask = np.zeros((N, K), bool)
        rp = st["row_ptr"]
        for n in range(N):
            cols = st["col_idx"][rp[n]:rp[n + 1]]
            assert np.all(np.diff(cols) > 0)
            mask[n, cols] = True
            assert np.array_equal(st["val"][rp[n]:rp[n + 1]], W[n, cols].astype(np.float16))
        s_hat, _ = spqr.decoded_stats(st["stats1"], st["stats2"])
        step = np.repeat(s_hat, 16, axis=1)
        assert np.all(np.abs(dense[mask]) <= step[mask])  # the dense part encodes 0 there
        assert np.array_equal(mask, spqr.select_outliers_by_sort(W, len(st["val"])))


def test_sparse_only_matches_textbook_csr_product():
    N, K = 16, 512
    W = synth.student_t3_f32((N, K), 0.02, "pin/spqr/sp")
    X = synth.x_f16(2, K, "pin/spqr/spx")
    st = spqr.encode(W, 0.05)
    st0 = dict(st)
    st0["codes"] = np.zeros_like(st["codes"])           # every code 0 ...
    s2 = st["stats2"].copy()
    s2[:, :, 2] = 0.0                                   # ... and z_hat = 0 -> dense part 0
    s2[:, :, 3] = 0.0
    st0["stats2"] = s2
    assert not np.any(spqr.dequantize_dense(st0["codes"], st0["stats1"], st0["stats2"], K))
    A = scipy.sparse.csr_matrix((st["val"].astype(np.float64), st["col_idx"], st["row_ptr"]), shape=(N, K))
    ref = (A @ X.astype(np.float64).T).T
    assert np.allclose(spqr.forward(X, st0, K), ref, rtol=1e-14, atol=1e-14)


def test_rtn_half_step_bound():
    N, K = 16, 1024
    W = synth.student_t3_f32((N, K), 0.02, "pin/spqr/rtn")
    d = spqr.quantize(W, 0.01)
    st = spqr.encode(W, 0.01)
    s_hat, z_hat = spqr.decoded_stats(st["stats1"], st["stats2"])
    R = np.where(d["mask"], 0.0, W.astype(np.float64)).reshape(N, K // 16, 16)
    w_hat = spqr.dequantize_dense(st["codes"], st["stats1"], st["stats2"], K).reshape(N, K // 16, 16)
    q = d["q"].reshape(N, K // 16, 16)
    inner = (q > 0) & (q < 7)
    err = np.abs(R - w_hat)
    step = np.broadcast_to(s_hat[:, :, None], err.shape)
    assert np.all(err[inner] <= step[inner] * (0.5 + 1e-5))
    print("clamped codes:", int((~inner).sum()), "of", q.size)


@pytest.mark.slow
def test_bits_per_parameter_in_the_pages_range():
    W = synth.layer_weight("spqr_33b", 0)
    st = spqr.encode(W, 0.01)
    bpp = spqr.bits_per_param(st, 6656, 6656)
    assert 3.36 <= bpp <= 4.75
    assert len(st["val"]) == 443023
    dense_bits = 8.0 * (st["codes"].nbytes + st["stats1"].nbytes + st["stats2"].nbytes) / 6656 ** 2
    assert dense_bits == 3.625


def test_row_subset_encode_equals_rows_of_full_encode():
    W = synth.student_t3_f32((48, 512), 0.02, "pin/spqr/rows")
    full = spqr.encode(W, 0.01)
    rows = np.array([0, 5, 17, 47])
    sub = spqr.encode_rows(W, 0.01, rows)
    for k in ("codes", "stats1", "stats2"):
        assert np.array_equal(sub[k], full[k][rows])
    rp = full["row_ptr"]
    for i, r in enumerate(rows):
        a, b = sub["row_ptr"][i], sub["row_ptr"][i + 1]
        assert np.array_equal(sub["col_idx"][a:b], full["col_idx"][rp[r]:rp[r + 1]])
        assert np.array_equal(sub["val"][a:b], full["val"][rp[r]:rp[r + 1]])
