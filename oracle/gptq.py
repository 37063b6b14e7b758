"""Oracle for the second-order encoders: GPTQ error feedback into the 4-bit
storage, and Hessian-sensitivity outlier selection for the SpQR storage.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix:

* GPTQ bulletin ("Makale Bülteni — GPTQ", "İddia ve Gerçeklik"): a
  second-order (Taylor) treatment of the layer's quantization error in the
  spirit of Optimal Brain Surgeon; the inverse Hessian is approximated from
  the covariance of the layer inputs and a Cholesky decomposition keeps the
  diagonal of the inverse numerically stable; weights are handled in blocks
  (groups such as 128); the deviation each quantized column causes is spread
  at once over the columns not yet quantized.
* SpQR bulletin ("Makale Bülteni — SpQR", "İddia ve Gerçeklik"): the outlier
  weights are the ones a Hessian-based sensitivity analysis marks.

Readings where the pages are silent (each written out again in the library):

G1. H = (2 / n) * X^T X over the n calibration rows, in fp64 (the quadratic
    form of the layer's squared output error, one row of W at a time).
G2. Damping: H + lam * I with lam = damp * mean(diag H) (the diagonal summed
    left to right in fp64, then divided by K), damp = 0.01 by default; when
    mean(diag H) is 0 (no calibration signal) H = I.
G3. U is the upper-triangular Cholesky factor of H^-1 (H^-1 = U^T U), fp64.
G4. Columns are quantized in natural order.  When column j starts a group of
    G, the group's scale and zero come from the round-to-nearest rule of the
    4-bit storage applied (in fp32) to the group's current weights rounded to
    fp32; column j's code is the same rule's code of its current weight
    rounded to fp32.  Then, in fp64, e_j = (w_j - w_hat_j) / U[j, j] and every
    later column k of the row moves by -e_j * U[j, k].  Rows are independent.
G5. H proportional to I makes U diagonal: no feedback, and the codes, scales
    and zeros equal round-to-nearest's bit for bit.
A1. Act-order: columns are quantized in decreasing order of diag(H) (ties to
    the lower index).  With static groups, every group keeps its natural columns
    k .. k+G-1 and its round-to-nearest statistics are taken from the original
    weights before any error feedback; the storage stays in natural order.
    Without static groups, groups are G consecutive columns of the quantization
    order, i.e. plain G4 applied to W[:, order] with H[order][:, order]; the
    storage holds the columns in that order and the forward reads the
    activations through it: Y = X[:, order] . W_stored^T.
S1. SpQR sensitivity of weight (n, k): how much the row's output error on the
    calibration inputs falls when that weight leaves the dense part.  The
    error of a group of 16 weights (one row, 16 consecutive k) is
    sum_k c_k (w_k - w_hat_k)^2 with c_k the k-th diagonal entry of the
    damped H (G2) and w_hat the group's 3-bit min/max quantization with
    real-valued statistics (s = (hi - lo) / 7, z = -lo / s; s = 1, z = -lo when
    hi == lo; w_hat = s * (clamp(rint(w / s + z), 0, 7) - z)), all in fp64 and
    summed in index order.  Sensitivity = error of the whole group minus error
    of the other 15 with statistics recomputed without the weight (the weight
    itself is then stored exactly).  Second-level quantization of the
    statistics is left out of this estimate.
S2. Outliers: the floor(p * N * K) entries first in the order
    (-sensitivity, row-major index); the rest of the encoding is unchanged.
    With H = 0 (no calibration) c_k = 1 and the criterion is the plain
    leave-one-out gain.
"""
from __future__ import annotations

import numpy as np

from . import spqr as ospqr

F32 = np.float32


def hessian(X) -> np.ndarray:
    """G1: H = (2/n) X^T X in fp64 for calibration rows X [n][K] (any float dtype)."""
    Xd = np.asarray(X).astype(np.float64)
    n = Xd.shape[0]
    return (2.0 / n) * (Xd.T @ Xd)


def damped(H, damp: float = 0.01) -> np.ndarray:
    """G2."""
    H = np.array(H, dtype=np.float64, copy=True)
    total = 0.0
    for v in np.diag(H).tolist():          # left to right
        total += v
    mean_diag = total / H.shape[0]
    if mean_diag == 0.0:
        return np.eye(H.shape[0])
    H[np.diag_indices_from(H)] += damp * mean_diag
    return H


def inverse_cholesky_upper(H, damp: float = 0.01) -> np.ndarray:
    """G3: upper-triangular U with (H + lam I)^-1 = U^T U."""
    Hinv = np.linalg.inv(damped(H, damp))
    Hinv = 0.5 * (Hinv + Hinv.T)
    return np.linalg.cholesky(Hinv).T


def _group_rule(wg32):
    """Round-to-nearest scale / zero of one group (fp32 values of one row), as
    in the 4-bit storage: lo = min(0, min), hi = max(0, max), S = fp16((hi-lo)/15)
    (1 if 0), z = clamp(rint(-lo/S), 0, 15).  Returns (S fp16, s fp32, z fp32)."""
    lo = min(F32(0.0), wg32.min())
    hi = max(F32(0.0), wg32.max())
    S = np.float16((hi - lo) / F32(15.0))
    if S == 0:
        S = np.float16(1.0)
    s = F32(S)
    z = F32(np.clip(np.rint(-lo / s), F32(0.0), F32(15.0)))
    return S, s, z


def quantize_w4(W, H, G: int = 128, damp: float = 0.01):
    """G4: GPTQ encode of fp32 W [N][K] given the (undamped) Hessian H [K][K].

    Returns (q uint8 [N][K], S fp16 [N][K/G], z uint8 [N][K/G]), the same
    quantities the round-to-nearest encoder returns, ready for ``w4.pack``."""
    W = np.asarray(W, dtype=F32)
    N, K = W.shape
    if K % G:
        raise ValueError("K must be a multiple of the group size")
    U = inverse_cholesky_upper(H, damp)
    Wc = W.astype(np.float64)                    # current (updated) weights
    q = np.zeros((N, K), dtype=np.uint8)
    S = np.zeros((N, K // G), dtype=np.float16)
    z = np.zeros((N, K // G), dtype=np.uint8)
    s_row = np.zeros(N, dtype=F32)
    z_row = np.zeros(N, dtype=F32)
    for j in range(K):
        g = j // G
        if j % G == 0:
            for n in range(N):
                S[n, g], s_row[n], z_row[n] = _group_rule(Wc[n, j:j + G].astype(F32))
            z[:, g] = z_row.astype(np.uint8)
        w32 = Wc[:, j].astype(F32)
        qj = np.clip(np.rint(w32 / s_row) + z_row, F32(0.0), F32(15.0))
        q[:, j] = qj.astype(np.uint8)
        w_hat = s_row.astype(np.float64) * (qj.astype(np.float64) - z_row.astype(np.float64))
        e = (Wc[:, j] - w_hat) / U[j, j]
        Wc[:, j + 1:] -= np.outer(e, U[j, j + 1:])
    return q, S, z


def encode_w4(W, H, G: int = 128, damp: float = 0.01):
    """GPTQ encode into the (qweight, scales, qzeros) storage of the 4-bit form."""
    from . import w4 as ow4
    return ow4.pack(*quantize_w4(W, H, G, damp))


def _group_error(w, c):
    """Weighted 3-bit min/max quantization error of one group (1-D fp64 arrays
    of the member weights and their column weights), summed in index order."""
    lo = float(np.min(w))
    hi = float(np.max(w))
    if hi == lo:
        s, z = 1.0, -lo
    else:
        s = (hi - lo) / 7.0
        z = -lo / s
    err = 0.0
    for wk, ck in zip(w.tolist(), c.tolist()):
        q = min(max(float(np.rint(wk / s + z)), 0.0), 7.0)
        d = wk - s * (q - z)
        err += ck * (d * d)
    return err


def act_order(H) -> np.ndarray:
    """A1: column order by decreasing diag(H), ties to the lower index (int64 [K])."""
    return np.argsort(-np.diag(np.asarray(H, dtype=np.float64)), kind="stable")


def quantize_w4_actorder(W, H, G: int = 128, damp: float = 0.01, static_groups: bool = True):
    """A1.  Returns (q, S, z, perm): with static groups q/S/z are in natural
    column order and perm is the identity; otherwise they are in the stored
    (quantization) order and perm[t] is the original column of stored column t."""
    W = np.asarray(W, dtype=F32)
    N, K = W.shape
    H = np.asarray(H, dtype=np.float64)
    order = act_order(H)
    if not static_groups:
        q, S, z = quantize_w4(W[:, order], H[np.ix_(order, order)], G, damp)
        return q, S, z, order.astype(np.int32)
    if K % G:
        raise ValueError("K must be a multiple of the group size")
    S = np.zeros((N, K // G), dtype=np.float16)
    s = np.zeros((N, K // G), dtype=F32)
    z = np.zeros((N, K // G), dtype=F32)
    for n in range(N):
        for g in range(K // G):
            S[n, g], s[n, g], z[n, g] = _group_rule(W[n, g * G:(g + 1) * G])
    U = inverse_cholesky_upper(H[np.ix_(order, order)], damp)
    Wc = W[:, order].astype(np.float64)
    q = np.zeros((N, K), dtype=np.uint8)
    for t in range(K):
        j = int(order[t])
        g = j // G
        w32 = Wc[:, t].astype(F32)
        qj = np.clip(np.rint(w32 / s[:, g]) + z[:, g], F32(0.0), F32(15.0))
        q[:, j] = qj.astype(np.uint8)
        w_hat = s[:, g].astype(np.float64) * (qj.astype(np.float64) - z[:, g].astype(np.float64))
        e = (Wc[:, t] - w_hat) / U[t, t]
        Wc[:, t + 1:] -= np.outer(e, U[t, t + 1:])
    return q, S, z.astype(np.uint8), np.arange(K, dtype=np.int32)


def encode_w4_actorder(W, H, G: int = 128, damp: float = 0.01, static_groups: bool = True):
    """(qweight, scales, qzeros, perm) storage of the act-order encode."""
    from . import w4 as ow4
    q, S, z, perm = quantize_w4_actorder(W, H, G, damp, static_groups)
    return (*ow4.pack(q, S, z), perm)


def forward_perm(X, qweight, scales, qzeros, perm, K: int, G: int = 128):
    """Y = X[:, perm] . W_stored^T in fp64 (the stored columns in quantization order)."""
    from . import w4 as ow4
    from .metrics import x_to_f64
    Xd = x_to_f64(X)
    return Xd[:, np.asarray(perm, dtype=np.int64)] @ ow4.dequantize(qweight, scales, qzeros, K, G).T


def spqr_sensitivity(W, H, damp: float = 0.01) -> np.ndarray:
    """S1: leave-one-out sensitivities [N][K] in fp64 (a plain loop: use on
    small layers)."""
    W = np.asarray(W, dtype=F32)
    N, K = W.shape
    c = np.diag(damped(H, damp)).copy()
    sens = np.zeros((N, K), dtype=np.float64)
    others = [np.array([j for j in range(16) if j != i]) for i in range(16)]
    for n in range(N):
        for g in range(K // 16):
            w = W[n, 16 * g:16 * g + 16].astype(np.float64)
            cg = c[16 * g:16 * g + 16]
            full = _group_error(w, cg)
            for i in range(16):
                sens[n, 16 * g + i] = full - _group_error(w[others[i]], cg[others[i]])
    return sens


def spqr_select_outliers(W, H, p: float, damp: float = 0.01) -> np.ndarray:
    """S2: boolean outlier mask (stable order by decreasing sensitivity)."""
    W = np.asarray(W, dtype=F32)
    N, K = W.shape
    n_out = ospqr.n_outliers(N, K, p)
    sig = spqr_sensitivity(W, H, damp).ravel()
    order = np.argsort(-sig, kind="stable")
    mask = np.zeros(sig.size, dtype=bool)
    mask[order[:n_out]] = True
    return mask.reshape(N, K)


def encode_spqr(W, H, p: float = 0.01, damp: float = 0.01):
    """SpQR storage with sensitivity-chosen outliers."""
    return ospqr.encode(W, p, spqr_select_outliers(W, H, p, damp))
