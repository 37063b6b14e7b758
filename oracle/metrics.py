"""Comparison metrics and storage-dtype decoders used by the oracle checks.

Pinned by hand-worked values in tests/golden/metrics.json (tests/test_oracle_metrics.py).

TEST INFRASTRUCTURE ONLY (see the package docstring).
"""
from __future__ import annotations

import numpy as np

# Float tolerance for every floating-point output of the path: the largest
# absolute error may not exceed 2e-3 of the largest reference magnitude, and the
# relative Frobenius error may not exceed 5e-4.
MAX_ABS_RATIO = 2e-3
REL_FROB = 5e-4


def max_abs_ratio(y, y_ref) -> float:
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    den = np.max(np.abs(y_ref))
    return float(np.max(np.abs(y - y_ref)) / den) if den > 0 else float(np.max(np.abs(y)))


def rel_frob(y, y_ref) -> float:
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    den = np.linalg.norm(y_ref)
    return float(np.linalg.norm(y - y_ref) / den) if den > 0 else float(np.linalg.norm(y))


def within_tolerance(y, y_ref) -> tuple[bool, float, float]:
    a, f = max_abs_ratio(y, y_ref), rel_frob(y, y_ref)
    return (a <= MAX_ABS_RATIO and f <= REL_FROB), a, f


def bf16_bits_to_f64(bits) -> np.ndarray:
    """bfloat16 bit patterns (uint16) to fp64: a bf16 is the top half of an fp32."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def x_to_f64(x) -> np.ndarray:
    """Activations as fp64: fp16 arrays directly, uint16 arrays as bf16 patterns."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return bf16_bits_to_f64(x)
    return x.astype(np.float64)
