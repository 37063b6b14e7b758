"""Pins of the comparison metrics and storage-dtype decoders in oracle.metrics.

Every float parity verdict goes through these functions, so each is checked
against hand-worked values (tests/golden/metrics.json) chosen so that a
plausible slip fails: dividing by max|y| instead of max|y_ref|, dropping the
abs in the denominator, a mean instead of a max, a Frobenius ratio over the
wrong norm, a tolerance gate that tests only one bar, a bf16 decode with the
wrong shift, or fp16 data decoded as bf16.
"""
import math

import numpy as np
import pytest

from oracle import metrics


def test_tolerance_constants():
    # the stated bars of the path
    assert metrics.MAX_ABS_RATIO == 2e-3
    assert metrics.REL_FROB == 5e-4


def test_max_abs_ratio(golden):
    for c in golden("metrics.json")["max_abs_ratio"]:
        got = metrics.max_abs_ratio(np.array(c["y"], float), np.array(c["y_ref"], float))
        assert got == pytest.approx(c["value"], rel=1e-15, abs=0), c["derivation"]


def test_rel_frob(golden):
    for c in golden("metrics.json")["rel_frob"]:
        got = metrics.rel_frob(np.array(c["y"], float), np.array(c["y_ref"], float))
        assert got == pytest.approx(c["value"], rel=1e-14, abs=0), c["derivation"]


def _tolerance_case(c):
    if "delta" in c:
        y_ref = np.full(100, 1000.0)
        y = y_ref.copy()
        y[37] += c["delta"]
    else:
        y_ref = np.concatenate([[100.0], np.ones(10000)])
        y = y_ref.copy()
        y[1:] += c["eps"]
    return y, y_ref


def test_within_tolerance_gates_each_bar(golden):
    for c in golden("metrics.json")["within_tolerance"]:
        y, y_ref = _tolerance_case(c)
        ok, a, f = metrics.within_tolerance(y, y_ref)
        assert bool(ok) == c["ok"], c["derivation"]
        assert a == pytest.approx(c["max_abs_ratio"], rel=1e-6)
        assert f == pytest.approx(c["rel_frob"], rel=1e-6)


def test_rel_frob_is_not_vacuous():
    # a nonzero error must give a nonzero ratio (guards identity checks that
    # would pass if rel_frob returned 0)
    y_ref = np.arange(1.0, 7.0)
    assert metrics.rel_frob(y_ref + 1e-9, y_ref) > 0
    assert metrics.rel_frob(y_ref, y_ref) == 0.0


def test_bf16_decode(golden):
    cases = golden("metrics.json")["bf16"]
    bits = np.array([c["bits"] for c in cases], dtype=np.uint16)
    got = metrics.bf16_bits_to_f64(bits)
    assert got.dtype == np.float64
    for c, v in zip(cases, got):
        want = math.inf if c["value"] == "inf" else c["value"]
        assert v == want, c["derivation"]
        assert math.copysign(1.0, v) == math.copysign(1.0, want), c["derivation"]


def test_x_to_f64(golden):
    a, b = golden("metrics.json")["x_to_f64"]
    got = metrics.x_to_f64(np.array(a["fp16"], dtype=np.float16))
    assert got.dtype == np.float64 and list(got) == a["value"], a["derivation"]
    got = metrics.x_to_f64(np.array(b["uint16_bits"], dtype=np.uint16))
    assert got.dtype == np.float64 and list(got) == b["value"], b["derivation"]
