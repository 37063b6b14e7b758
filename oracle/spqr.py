"""Oracle for the SpQR-style hybrid weight: dense 3-bit bi-level part + CSR fp16 outliers.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the SpQR bulletin fixes ("Makale Bülteni — SpQR", lead and "İddia ve
Gerçeklik"): the weight matrix is split into a dense low-precision matrix and
a sparse high-precision matrix; about 1% of the weights (the outliers) stay in
fp16 in the sparse matrix; the rest are quantized to 3 bits in groups of 16
with two-level quantization (the group statistics are themselves quantized);
the average cost lands between 3.36 and 4.75 bits per parameter; at inference
the dense 3-bit part is decompressed while the sparse fp16 product runs beside
it.  The page selects outliers by Hessian sensitivity; without calibration data
this oracle selects them by magnitude (a stated substitute, same storage).

Readings where the page is silent (each written out again in the library):

1. Outliers: n_out = floor(p * (N*K)) entries, the largest |w| of the whole
   layer; ties go to the lower row-major index.  They leave the dense part
   (which then holds 0 there) and enter a CSR matrix: rows = output rows n,
   int32 row_ptr [N+1], int32 col_idx ascending within a row, fp16 values.
2. First level, per row and group of 16 consecutive k of the remainder R:
   lo, hi = min, max; s = (hi - lo) / 7 and z = -lo / s in fp32
   (s = 1, z = -lo when hi == lo).  z stays real-valued.
3. Second level, per row and block of 16 consecutive groups (256 weights),
   separately for the 16 scales and the 16 zeros (values v):
   SS = fp16((max v - min v) / 7); ZS = fp16(-min v / SS) (SS = 1 if SS is 0 or
   that ZS is not finite); c = clamp(rint(v / SS + ZS), 0, 7);
   decoded v_hat = SS * (c - ZS).
4. Codes: q = clamp(rint(R / s_hat + z_hat), 0, 7) with the decoded fp32
   statistics (q = clamp(rint(z_hat), 0, 7) if s_hat == 0).
5. Dequantized dense weight: s_hat * (q - z_hat).

Storage (this library's layout; the page gives none):

* ``codes``  uint32 [N][K/32][3].  A 32-code chunk covers k = 32c .. 32c+31;
  its first 16 codes a0..a15 form group 2c, the next 16 b0..b15 group 2c+1.
  Each word has two 16-bit halves with five 3-bit fields each (field i of half
  h at bit 16h + 3i); bit 15 and bit 31 are spare.
  word 0: low fields a0..a4, high fields a5..a9;
  word 1: low fields a10 a11 a12 b0 b1, high fields a13 a14 a15 b2 b3;
  word 2: low fields b4..b8, high fields b9..b13;
  b14: bit j of the code at bit 15 of word j;  b15: bit j at bit 31 of word j.
  (Field i of the low half and field i of the high half always belong to the
  same group.)
* ``stats1`` uint32 [N][K/256][3]: 16 six-bit fields, field g (group g of the
  block) at bit 6g of the 96-bit little-endian stream, holding c_s | c_z << 3.
* ``stats2`` fp16 [N][K/256][4]: SS_s, ZS_s, SS_z, ZS_z.
"""
from __future__ import annotations

import math

import numpy as np

F32 = np.float32
BETA1 = 16          # group size (weights per first-level statistic)
BETA2 = 16          # groups per second-level statistic block
BLOCK = BETA1 * BETA2


def n_outliers(N: int, K: int, p: float) -> int:
    return int(math.floor(p * (N * K)))


# ---------------------------------------------------------------------------
# Step 1: outlier selection and CSR

def select_outliers(W, n_out: int) -> np.ndarray:
    """Boolean mask of the n_out entries that come first in the order
    (-|w|, row-major index): all entries above the n_out-th largest magnitude,
    then the lowest-index entries equal to it."""
    a = np.abs(np.asarray(W, dtype=F32)).ravel()
    mask = np.zeros(a.size, dtype=bool)
    if n_out <= 0:
        return mask.reshape(np.shape(W))
    if n_out >= a.size:
        mask[:] = True
        return mask.reshape(np.shape(W))
    t = np.partition(a, a.size - n_out)[a.size - n_out]
    mask = a > t
    need = n_out - int(mask.sum())
    mask[np.flatnonzero(a == t)[:need]] = True
    return mask.reshape(np.shape(W))


def select_outliers_by_sort(W, n_out: int) -> np.ndarray:
    """Same set as ``select_outliers`` by a full stable sort (used on small inputs)."""
    a = np.abs(np.asarray(W, dtype=F32)).ravel()
    order = np.argsort(-a, kind="stable")
    mask = np.zeros(a.size, dtype=bool)
    mask[order[:n_out]] = True
    return mask.reshape(np.shape(W))


def build_csr(W, mask):
    """CSR of the masked entries: (row_ptr int32 [N+1], col_idx int32, val fp16)."""
    W = np.asarray(W, dtype=F32)
    rows, cols = np.nonzero(mask)          # row-major order: rows, then cols ascending
    N = W.shape[0]
    row_ptr = np.zeros(N + 1, dtype=np.int64)
    np.add.at(row_ptr, rows + 1, 1)
    row_ptr = np.cumsum(row_ptr).astype(np.int32)
    return row_ptr, cols.astype(np.int32), W[rows, cols].astype(np.float16)


# ---------------------------------------------------------------------------
# Steps 2-4: bi-level 3-bit quantization

def first_level(R):
    """Per-group (s, z) in fp32 for R [N][K]: shape [N][K/16]."""
    N, K = R.shape
    Rg = R.reshape(N, K // BETA1, BETA1)
    lo = Rg.min(axis=2)
    hi = Rg.max(axis=2)
    flat = hi == lo
    with np.errstate(divide="ignore", invalid="ignore"):
        s = np.where(flat, F32(1.0), (hi - lo) / F32(7.0)).astype(F32)
        z = np.where(flat, -lo, -lo / s).astype(F32)
    return s, z


def second_level(v):
    """3-bit min/max quantizer over the last axis (16 values).

    Returns (SS fp16, ZS fp16, c uint8, v_hat fp32) with SS, ZS of shape v.shape[:-1]."""
    v = np.asarray(v, dtype=F32)
    lo2 = v.min(axis=-1)
    hi2 = v.max(axis=-1)
    SS = ((hi2 - lo2) / F32(7.0)).astype(np.float16)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        ZS = (-lo2 / SS.astype(F32)).astype(np.float16)
        bad = (SS == 0) | ~np.isfinite(ZS)
        SS = np.where(bad, np.float16(1.0), SS)
        ZS = np.where(bad, (-lo2 / F32(1.0)).astype(np.float16), ZS)
    ss = SS.astype(F32)[..., None]
    zs = ZS.astype(F32)[..., None]
    c = np.clip(np.rint(v / ss + zs), F32(0.0), F32(7.0))
    v_hat = ss * (c - zs)
    return SS, ZS, c.astype(np.uint8), v_hat.astype(F32)


def quantize(W, p: float = 0.01, mask=None):
    """Full encode.  Returns a dict of the unpacked quantities (codes, statistics, CSR).

    ``mask`` may carry an outlier selection made on a larger matrix (rows of a
    layer are encoded independently once the layer-wide selection is known)."""
    W = np.asarray(W, dtype=F32)
    N, K = W.shape
    if K % BLOCK:
        raise ValueError("K must be a multiple of 256")
    if mask is None:
        mask = select_outliers(W, n_outliers(N, K, p))
    row_ptr, col_idx, val = build_csr(W, mask)
    R = np.where(mask, F32(0.0), W)
    s, z = first_level(R)
    nb = K // BLOCK
    SSs, ZSs, cs, s_hat = second_level(s.reshape(N, nb, BETA2))
    SSz, ZSz, cz, z_hat = second_level(z.reshape(N, nb, BETA2))
    s_hat = s_hat.reshape(N, K // BETA1)
    z_hat = z_hat.reshape(N, K // BETA1)
    Rg = R.reshape(N, K // BETA1, BETA1)
    sh = s_hat[:, :, None]
    zh = z_hat[:, :, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.where(sh == 0, zh, Rg / sh + zh)
    q = np.clip(np.rint(t), F32(0.0), F32(7.0)).astype(np.uint8).reshape(N, K)
    return dict(q=q, cs=cs.reshape(N, K // BETA1), cz=cz.reshape(N, K // BETA1),
                SSs=SSs, ZSs=ZSs, SSz=SSz, ZSz=ZSz,
                row_ptr=row_ptr, col_idx=col_idx, val=val, mask=mask)


# ---------------------------------------------------------------------------
# Storage layout

def _chunk_bit_positions():
    """pos[c][b] = (word, bit) of bit b of code c in a 32-code chunk."""
    pos = [None] * 32

    def field(word, half, i):
        return [(word, 16 * half + 3 * i + b) for b in range(3)]

    for i in range(5):                      # word 0: a0..a4 | a5..a9
        pos[i] = field(0, 0, i)
        pos[5 + i] = field(0, 1, i)
    for i in range(3):                      # word 1: a10..a12 | a13..a15
        pos[10 + i] = field(1, 0, i)
        pos[13 + i] = field(1, 1, i)
    for i in range(2):                      # word 1: b0 b1 | b2 b3
        pos[16 + i] = field(1, 0, 3 + i)
        pos[18 + i] = field(1, 1, 3 + i)
    for i in range(5):                      # word 2: b4..b8 | b9..b13
        pos[20 + i] = field(2, 0, i)
        pos[25 + i] = field(2, 1, i)
    pos[30] = [(j, 15) for j in range(3)]   # b14 in the spare bits 15
    pos[31] = [(j, 31) for j in range(3)]   # b15 in the spare bits 31
    return pos


CHUNK_POS = _chunk_bit_positions()


def pack_codes(q):
    q = np.asarray(q, dtype=np.uint8)
    N, K = q.shape
    qc = q.reshape(N, K // 32, 32).astype(np.uint32)
    words = np.zeros((N, K // 32, 3), dtype=np.uint32)
    for c in range(32):
        for b, (w, bit) in enumerate(CHUNK_POS[c]):
            words[:, :, w] |= ((qc[:, :, c] >> np.uint32(b)) & np.uint32(1)) << np.uint32(bit)
    return words


def unpack_codes(words, K: int):
    words = np.asarray(words, dtype=np.uint32)
    N = words.shape[0]
    words = words.reshape(N, K // 32, 3)
    q = np.zeros((N, K // 32, 32), dtype=np.uint32)
    for c in range(32):
        for b, (w, bit) in enumerate(CHUNK_POS[c]):
            q[:, :, c] |= ((words[:, :, w] >> np.uint32(bit)) & np.uint32(1)) << np.uint32(b)
    return q.reshape(N, K).astype(np.uint8)


def pack_stats1(cs, cz):
    """cs, cz uint8 [N][K/16] -> uint32 [N][K/256][3]."""
    N, ng = cs.shape
    f = (np.asarray(cs, np.uint64) | (np.asarray(cz, np.uint64) << np.uint64(3)))
    f = f.reshape(N, ng // BETA2, BETA2)
    out = np.zeros((N, ng // BETA2, 3), dtype=np.uint64)
    for g in range(BETA2):
        bit = 6 * g
        for b in range(6):
            w, o = divmod(bit + b, 32)
            out[:, :, w] |= ((f[:, :, g] >> np.uint64(b)) & np.uint64(1)) << np.uint64(o)
    return out.astype(np.uint32)


def unpack_stats1(stats1):
    """uint32 [N][nb][3] -> (cs, cz) uint8 [N][nb*16]."""
    s = np.asarray(stats1, dtype=np.uint32)
    N, nb, _ = s.shape
    f = np.zeros((N, nb, BETA2), dtype=np.uint32)
    for g in range(BETA2):
        for b in range(6):
            w, o = divmod(6 * g + b, 32)
            f[:, :, g] |= ((s[:, :, w] >> np.uint32(o)) & np.uint32(1)) << np.uint32(b)
    f = f.reshape(N, nb * BETA2)
    return (f & 7).astype(np.uint8), (f >> 3).astype(np.uint8)


def pack_stats2(SSs, ZSs, SSz, ZSz):
    return np.stack([SSs, ZSs, SSz, ZSz], axis=-1).astype(np.float16)


def encode(W, p: float = 0.01, mask=None):
    """fp32 W -> storage dict: codes, stats1, stats2, row_ptr, col_idx, val."""
    d = quantize(W, p, mask)
    return dict(codes=pack_codes(d["q"]),
                stats1=pack_stats1(d["cs"], d["cz"]),
                stats2=pack_stats2(d["SSs"], d["ZSs"], d["SSz"], d["ZSz"]),
                row_ptr=d["row_ptr"], col_idx=d["col_idx"], val=d["val"])


def encode_rows(W, p: float, rows):
    """Storage of the given rows of a layer, with the outliers selected over the
    whole layer (the same bytes the full encode holds for those rows)."""
    W = np.asarray(W, dtype=F32)
    N, K = W.shape
    mask = select_outliers(W, n_outliers(N, K, p))
    rows = np.asarray(rows)
    return encode(W[rows], p, mask[rows])


# ---------------------------------------------------------------------------
# Decode and forward (fp64)

def decoded_stats(stats1, stats2):
    """(s_hat, z_hat) fp64 [N][K/16] from the stored statistics."""
    cs, cz = unpack_stats1(stats1)
    st = np.asarray(stats2, dtype=np.float16).astype(np.float64)
    N, nb, _ = st.shape
    SSs, ZSs, SSz, ZSz = (np.repeat(st[:, :, i], BETA2, axis=1) for i in range(4))
    s_hat = SSs * (cs.astype(np.float64) - ZSs)
    z_hat = SSz * (cz.astype(np.float64) - ZSz)
    return s_hat, z_hat


def dequantize_dense(codes, stats1, stats2, K: int):
    q = unpack_codes(codes, K).astype(np.float64)
    s_hat, z_hat = decoded_stats(stats1, stats2)
    N = q.shape[0]
    w = s_hat[:, :, None] * (q.reshape(N, K // BETA1, BETA1) - z_hat[:, :, None])
    return w.reshape(N, K)


def sparse_dense(row_ptr, col_idx, val, N: int, K: int):
    """The CSR matrix written out densely (fp64)."""
    out = np.zeros((N, K), dtype=np.float64)
    rp = np.asarray(row_ptr, dtype=np.int64)
    rows = np.repeat(np.arange(N), np.diff(rp))
    out[rows, np.asarray(col_idx, dtype=np.int64)] = np.asarray(val, dtype=np.float16).astype(np.float64)
    return out


def forward(X, st, K: int):
    """Y = X . W_dense^T + X . W_sparse^T in fp64; the sparse term walks the CSR
    rows (X fp16 [M][K])."""
    Xd = np.asarray(X).astype(np.float64)
    codes = st["codes"]
    N = codes.shape[0]
    Y = Xd @ dequantize_dense(codes, st["stats1"], st["stats2"], K).T
    rp = np.asarray(st["row_ptr"], dtype=np.int64)
    rows = np.repeat(np.arange(N), np.diff(rp))
    cols = np.asarray(st["col_idx"], dtype=np.int64)
    vals = np.asarray(st["val"], dtype=np.float16).astype(np.float64)
    for m in range(Xd.shape[0]):
        Y[m] += np.bincount(rows, weights=Xd[m, cols] * vals, minlength=N)
    return Y


def stored_bytes(st) -> int:
    return sum(int(np.asarray(st[k]).nbytes) for k in
               ("codes", "stats1", "stats2", "row_ptr", "col_idx", "val"))


def bits_per_param(st, N: int, K: int) -> float:
    """Average storage cost: 8 * (all stored bytes) / (N*K)."""
    return 8.0 * stored_bytes(st) / (N * K)
