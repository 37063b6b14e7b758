"""Oracle for 4-bit group-quantized weights (GPTQ-style storage, RTN encoder).

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the GPTQ bulletin fixes ("Makale Bülteni — GPTQ", lead and "İddia ve
Gerçeklik"): weights go to 4 bits, quantized in blocks (groups of 128 weights
along the input dimension); naive round-to-nearest (RTN) is the baseline the
second-order method improves on.  The encoder here is that RTN baseline; it
fills the same storage that a second-order encoder would.

Readings where the page is silent:

* asymmetric min/max quantizer per (row n, group g): the range always contains
  0, lo = min(0, min w), hi = max(0, max w);
* the fp16 scale S = fp16((hi - lo) / 15) is rounded first and the codes are
  computed against it; S = 1 when that rounds to zero (a constant-zero group);
* zero point z = clamp(rint(-lo / S), 0, 15); code q = clamp(rint(w / S) + z, 0, 15);
  rint is round-half-to-even; the dequantized weight is w_hat = S * (q - z);
* storage: ``qweight`` uint32 [N][K/8] with code k in bits 4*(k%8) of word k/8;
  ``scales`` fp16 [N][K/G]; ``qzeros`` uint32 [N][ceil(K/G/8)] with the zero of
  group g in bits 4*(g%8) of word g/8, padding nibbles 0.
"""
from __future__ import annotations

import numpy as np

F32 = np.float32


def quantize_rtn(W, G: int = 128):
    """Per-group RTN encode of fp32 W [N][K].  Returns (q uint8 [N][K],
    S fp16 [N][K/G], z uint8 [N][K/G]).  All arithmetic in fp32."""
    W = np.asarray(W, dtype=F32)
    N, K = W.shape
    if K % G:
        raise ValueError("K must be a multiple of the group size")
    Wg = W.reshape(N, K // G, G)
    lo = np.minimum(Wg.min(axis=2), F32(0.0))
    hi = np.maximum(Wg.max(axis=2), F32(0.0))
    S = ((hi - lo) / F32(15.0)).astype(np.float16)
    S = np.where(S == 0, np.float16(1.0), S)
    s = S.astype(F32)
    z = np.clip(np.rint(-lo / s), F32(0.0), F32(15.0))
    q = np.clip(np.rint(Wg / s[:, :, None]) + z[:, :, None], F32(0.0), F32(15.0))
    return q.reshape(N, K).astype(np.uint8), S, z.astype(np.uint8)


def pack(q, S, z):
    """Pack codes and zeros into the uint32 storage described in the module docstring."""
    q = np.asarray(q, dtype=np.uint8)
    z = np.asarray(z, dtype=np.uint8)
    N, K = q.shape
    ng = z.shape[1]
    qw = np.zeros((N, K // 8), dtype=np.uint32)
    q8 = q.reshape(N, K // 8, 8).astype(np.uint32)
    for j in range(8):
        qw |= q8[:, :, j] << np.uint32(4 * j)
    nzw = (ng + 7) // 8
    zp = np.zeros((N, nzw * 8), dtype=np.uint32)
    zp[:, :ng] = z
    zp = zp.reshape(N, nzw, 8)
    qz = np.zeros((N, nzw), dtype=np.uint32)
    for j in range(8):
        qz |= zp[:, :, j] << np.uint32(4 * j)
    return qw, np.asarray(S, dtype=np.float16).copy(), qz


def unpack(qweight, qzeros, K: int, G: int = 128):
    """Inverse of ``pack`` for codes and zeros: (q uint8 [N][K], z uint8 [N][K/G])."""
    qweight = np.asarray(qweight, dtype=np.uint32)
    N = qweight.shape[0]
    q = np.empty((N, K // 8, 8), dtype=np.uint8)
    for j in range(8):
        q[:, :, j] = (qweight >> np.uint32(4 * j)) & np.uint32(15)
    qzeros = np.asarray(qzeros, dtype=np.uint32)
    z = np.empty((N, qzeros.shape[1], 8), dtype=np.uint8)
    for j in range(8):
        z[:, :, j] = (qzeros >> np.uint32(4 * j)) & np.uint32(15)
    return q.reshape(N, K), z.reshape(N, -1)[:, : K // G]


def encode(W, G: int = 128):
    """fp32 W -> (qweight, scales, qzeros) storage."""
    return pack(*quantize_rtn(W, G))


def dequantize(qweight, scales, qzeros, K: int, G: int = 128):
    """W_hat [N][K] in fp64: S * (q - z), exact in fp64."""
    q, z = unpack(qweight, qzeros, K, G)
    N = q.shape[0]
    S = np.asarray(scales, dtype=np.float16).astype(np.float64)
    qd = q.reshape(N, K // G, G).astype(np.float64)
    w = S[:, :, None] * (qd - z[:, :, None].astype(np.float64))
    return w.reshape(N, K)


def forward(X, qweight, scales, qzeros, K: int, G: int = 128):
    """Y = X . W_hat^T in fp64 (X fp16, or uint16 bf16 bit patterns)."""
    from .metrics import x_to_f64
    return x_to_f64(X) @ dequantize(qweight, scales, qzeros, K, G).T
