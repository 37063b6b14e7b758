"""Seeded synthetic inputs for the quantized linear-layer workloads.

This module only draws random numbers and rounds them once to a storage dtype.
It holds none of the quantization arithmetic: both the library path and the
oracle receive the arrays produced here, and nothing here depends on either.

Workloads (layer shapes are N x K, i.e. out x in, and Y = X . W^T):

* ``w4_1k``          1024x1024, M in {1, 4}, W ~ N(0, 0.02), X fp16 ~ N(0, 1).
* ``w4_llama7b``     4096x4096, 11008x4096, 4096x11008, M = 1, same laws.
* ``spqr_33b``       6656x6656, 17920x6656, 6656x17920, M in {1, 4, 16},
                     W = 0.02 * t(nu=3), X fp16 ~ N(0, 1).
* ``w4_llama70b``    8192x8192, 28672x8192, 8192x28672, M in {32, 64, 256},
                     W ~ N(0, 0.015), X bf16 ~ N(0, 1).
* ``sq_w8a8``        11008x4096, 4096x4096, M in {512, 2048} (+256 for the
                     TOPS figure), W ~ N(0, 0.02), X fp16 ~ N(0, 1) with 1% of
                     the K channels (41 of 4096) multiplied by 100.

Every stream is a PCG64 generator seeded from (seed, a text tag naming the
workload, layer and tensor), so any tensor can be regenerated on its own.
"""
from __future__ import annotations

import hashlib

import numpy as np

SEED = 0

WORKLOADS = {
    "w4_1k": dict(kind="w4", layers=[(1024, 1024)], M=(1, 4), G=128,
                  w_sigma=0.02, x_dtype="f16", y_dtype="f16"),
    "w4_llama7b": dict(kind="w4", layers=[(4096, 4096), (11008, 4096), (4096, 11008)],
                       M=(1,), G=128, w_sigma=0.02, x_dtype="f16", y_dtype="f16"),
    "spqr_33b": dict(kind="spqr", layers=[(6656, 6656), (17920, 6656), (6656, 17920)],
                     M=(1, 4, 16), w_scale=0.02, outlier_frac=0.01,
                     x_dtype="f16", y_dtype="f16"),
    "w4_llama70b": dict(kind="w4", layers=[(8192, 8192), (28672, 8192), (8192, 28672)],
                        M=(32, 64, 256), G=128, w_sigma=0.015, x_dtype="bf16", y_dtype="bf16"),
    "sq_w8a8": dict(kind="sq", layers=[(11008, 4096), (4096, 4096)], M=(256, 512, 2048),
                    w_sigma=0.02, alpha=0.85, outlier_channel_frac=0.01,
                    outlier_channel_gain=100.0, calib_rows=512,
                    x_dtype="f16", y_dtype="f16"),
}


def rng(tag: str, seed: int = SEED) -> np.random.Generator:
    """Independent PCG64 stream for one named tensor, seeded from a hash of the tag."""
    digest = hashlib.sha256(f"{seed}/{tag}".encode()).digest()
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(
        int.from_bytes(digest[:16], "little"))))


def normal_f32(shape, sigma: float, tag: str) -> np.ndarray:
    """fp32 array with entries sigma * N(0, 1)."""
    g = rng(tag)
    out = g.standard_normal(size=shape, dtype=np.float32)
    out *= np.float32(sigma)
    return out


def student_t3_f32(shape, scale: float, tag: str, rows_per_block: int = 1024) -> np.ndarray:
    """fp32 array with entries scale * T, T ~ Student-t with 3 degrees of freedom.

    T is built from four standard normals by its textbook definition,
    T = Z0 / sqrt((Z1^2 + Z2^2 + Z3^2) / 3), evaluated in fp32.
    """
    n, k = shape
    g = rng(tag)
    out = np.empty((n, k), dtype=np.float32)
    for r0 in range(0, n, rows_per_block):
        r1 = min(n, r0 + rows_per_block)
        z = g.standard_normal(size=(4, r1 - r0, k), dtype=np.float32)
        chi = (z[1] * z[1] + z[2] * z[2] + z[3] * z[3]) / np.float32(3.0)
        out[r0:r1] = np.float32(scale) * z[0] / np.sqrt(chi)
    return out


def outlier_channels(K: int, frac: float, tag: str) -> np.ndarray:
    """Sorted indices of round(frac*K) distinct channels."""
    n = int(round(frac * K))
    g = rng(tag)
    return np.sort(g.choice(K, size=n, replace=False)).astype(np.int64)


def x_f16(M: int, K: int, tag: str, channels=None, gain: float = 1.0) -> np.ndarray:
    """fp16 activations ~ N(0, 1); optional channels scaled by ``gain`` before rounding."""
    g = rng(tag)
    x = g.standard_normal(size=(M, K))
    if channels is not None and len(channels):
        x[:, channels] *= gain
    return x.astype(np.float16)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bfloat16 (nearest, ties to even); return the uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def x_bf16_bits(M: int, K: int, tag: str) -> np.ndarray:
    """bf16 activations ~ N(0, 1), as uint16 bit patterns."""
    g = rng(tag)
    return f32_to_bf16_bits(g.standard_normal(size=(M, K), dtype=np.float32))


# ---------------------------------------------------------------------------
# Per-workload tensors.  Tags name workload, layer and tensor.

def layer_weight(workload: str, layer: int) -> np.ndarray:
    cfg = WORKLOADS[workload]
    N, K = cfg["layers"][layer]
    tag = f"{workload}/L{layer}/W"
    if cfg["kind"] == "spqr":
        return student_t3_f32((N, K), cfg["w_scale"], tag)
    return normal_f32((N, K), cfg["w_sigma"], tag)


def layer_weight_rows(workload: str, layer: int, rows) -> np.ndarray:
    """Rows of ``layer_weight`` (regenerates the full tensor; use for small checks)."""
    return layer_weight(workload, layer)[np.asarray(rows)]


def activations(workload: str, layer: int, M: int) -> np.ndarray:
    """X for one layer and batch size M: fp16 array, or uint16 bf16 bit patterns.

    X(M) is the first M rows of one master batch per layer (as many rows as the
    largest M of the workload), so batches of different sizes are prefixes of
    each other.
    """
    cfg = WORKLOADS[workload]
    N, K = cfg["layers"][layer]
    rows = max(max(cfg["M"]), cfg.get("calib_rows", 0))
    if M > rows:
        raise ValueError(f"M={M} exceeds the {rows} rows drawn for {workload}")
    tag = f"{workload}/L{layer}/X"
    if cfg["x_dtype"] == "bf16":
        return x_bf16_bits(rows, K, tag)[:M].copy()
    if cfg["kind"] == "sq":
        ch = outlier_channels(K, cfg["outlier_channel_frac"], f"{workload}/L{layer}/channels")
        return x_f16(rows, K, tag, ch, cfg["outlier_channel_gain"])[:M].copy()
    return x_f16(rows, K, tag)[:M].copy()


def sq_calibration(workload: str, layer: int) -> np.ndarray:
    """Calibration rows for the smoothing vector: the first ``calib_rows`` rows of
    the layer's master batch (the same for every M)."""
    cfg = WORKLOADS[workload]
    return activations(workload, layer, cfg["calib_rows"])
