"""CPU-only checks of the C-ABI library: it loads, exports every entry point the
header declares, and rejects bad arguments on the host before any launch."""
import os
import re

import numpy as np
import pytest

from quantized_linear_layers_packed_amd import qlin

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "qlin.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", src, flags=re.M)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) == len(qlin.EXPORTS)
    assert set(names) == set(qlin.EXPORTS)
    for name in names:
        assert hasattr(qlin._lib, name), name


def test_status_strings_and_version():
    assert qlin.qlin_version() >= 100
    assert qlin.status_str(0) == "QLIN_OK"
    assert qlin.status_str(2) == "QLIN_EALIGN"
    assert qlin.status_str(99) == "QLIN_UNKNOWN"


FAKE = 0x10000          # aligned non-NULL address, never dereferenced by host-side validation


def _raises(status, fn, *args, **kw):
    with pytest.raises(qlin.QlinError) as e:
        fn(*args, **kw)
    assert e.value.status == status, str(e.value)
    return str(e.value)


def test_w4_forward_rejects_bad_arguments():
    F, B, F32 = qlin.QLIN_F16, qlin.QLIN_BF16, qlin.QLIN_F32
    fw = qlin.qlin_w4_forward
    _raises(qlin.QLIN_EINVAL, fw, FAKE, F, 0, 1024, FAKE, FAKE, FAKE, 64, 128, FAKE, F, stream=0)
    _raises(qlin.QLIN_EINVAL, fw, FAKE, F, 1, 1000, FAKE, FAKE, FAKE, 64, 128, FAKE, F, stream=0)     # K % G
    _raises(qlin.QLIN_EUNSUPPORTED, fw, FAKE, F, 1, 960, FAKE, FAKE, FAKE, 64, 96, FAKE, F, stream=0)
    _raises(qlin.QLIN_EUNSUPPORTED, fw, FAKE, F, 1, 1024, FAKE, FAKE, FAKE, 64, 16, FAKE, F, stream=0)
    _raises(qlin.QLIN_EINVAL, fw, FAKE, 7, 1, 1024, FAKE, FAKE, FAKE, 64, 128, FAKE, F, stream=0)      # x dtype
    _raises(qlin.QLIN_EINVAL, fw, FAKE, F32, 1, 1024, FAKE, FAKE, FAKE, 64, 128, FAKE, F, stream=0)
    _raises(qlin.QLIN_EINVAL, fw, FAKE, B, 1, 1024, FAKE, FAKE, FAKE, 64, 128, FAKE, 9, stream=0)      # y dtype
    _raises(qlin.QLIN_EINVAL, fw, 0, F, 1, 1024, FAKE, FAKE, FAKE, 64, 128, FAKE, F, stream=0)         # NULL
    msg = _raises(qlin.QLIN_EALIGN, fw, FAKE + 2, F, 1, 1024, FAKE, FAKE, FAKE, 64, 128, FAKE, F, stream=0)
    assert "X" in msg
    msg = _raises(qlin.QLIN_EALIGN, fw, FAKE, F, 1, 1024, FAKE, FAKE + 8, FAKE, 64, 128, FAKE, F, stream=0)
    assert "scales" in msg


def test_spqr_forward_rejects_bad_arguments():
    fw = qlin.spqr_forward
    _raises(qlin.QLIN_EINVAL, fw, FAKE, 1, 1000, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 10, 64, FAKE, 1, stream=0)
    _raises(qlin.QLIN_EUNSUPPORTED, fw, FAKE, 17, 1024, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 10, 64, FAKE, 1, stream=0)
    _raises(qlin.QLIN_EINVAL, fw, FAKE, 1, 1024, FAKE, FAKE, FAKE, FAKE, 0, 0, 10, 64, FAKE, 1, stream=0)
    _raises(qlin.QLIN_EINVAL, fw, FAKE, 1, 1024, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, -1, 64, FAKE, 1, stream=0)
    _raises(qlin.QLIN_EINVAL, fw, FAKE, 1, 1024, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 10, 64, FAKE, 2, stream=0)
    _raises(qlin.QLIN_EALIGN, fw, FAKE, 1, 1024, FAKE + 4, FAKE, FAKE, FAKE, FAKE, FAKE, 10, 64, FAKE, 1, stream=0)
    # batches that take the matrix-core path need the prepass workspace (K * 68
    # bytes), placed after the 16 KiB of split-K counters it leaves untouched
    need = qlin.spqr_workspace_bytes(8, 1024, 64)
    assert need == 16384 + 1024 * 32 + 1024 * 4 + 1024 * 32 and qlin.spqr_workspace_bytes(1, 1024, 64) == 0
    msg = _raises(qlin.QLIN_EINVAL, fw, FAKE, 8, 1024, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 10, 64, FAKE, 1, stream=0)
    assert str(need) in msg
    _raises(qlin.QLIN_EINVAL, fw, FAKE, 8, 1024, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 10, 64, FAKE, 1, FAKE, need - 1,
            stream=0)


def test_dense_gemm_rejects_bad_arguments():
    fw = qlin.qlin_f16_gemm
    need = qlin.qlin_f16_gemm_workspace_bytes(256, 1024, 4096, qlin.QLIN_F16)
    assert need > 16384                                  # every shape runs split-K: counters + partials
    _raises(qlin.QLIN_EINVAL, fw, FAKE, FAKE, 4, 64, 100, FAKE, 1, FAKE, need, 0)       # K % 64
    _raises(qlin.QLIN_EINVAL, fw, FAKE, FAKE, 0, 64, 128, FAKE, 1, FAKE, need, 0)       # M
    _raises(qlin.QLIN_EINVAL, fw, FAKE, FAKE, 4, 64, 128, FAKE, 7, FAKE, need, 0)       # y_dtype
    _raises(qlin.QLIN_EINVAL, fw, 0, FAKE, 4, 64, 128, FAKE, 1, FAKE, need, 0)          # NULL X
    _raises(qlin.QLIN_EALIGN, fw, FAKE, FAKE + 2, 4, 64, 128, FAKE, 1, FAKE, need, 0)   # W misaligned
    msg = _raises(qlin.QLIN_EINVAL, fw, FAKE, FAKE, 256, 1024, 4096, FAKE, 1, None, None, 0)
    assert str(need) in msg
    _raises(qlin.QLIN_EINVAL, fw, FAKE, FAKE, 256, 1024, 4096, FAKE, 1, FAKE, need - 1, 0)
    with pytest.raises(qlin.QlinError):
        qlin.qlin_f16_gemm_workspace_bytes(4, 64, 96)


def test_sq_calls_reject_bad_arguments():
    _raises(qlin.QLIN_EINVAL, qlin.sq_smooth_quant_act, FAKE, FAKE, 4, 100, FAKE, FAKE, 0)
    _raises(qlin.QLIN_EALIGN, qlin.sq_smooth_quant_act, FAKE + 2, FAKE, 4, 128, FAKE, FAKE, 0)
    _raises(qlin.QLIN_EINVAL, qlin.sq_int8_gemm, FAKE, FAKE, FAKE, FAKE, 4, 4, 100, FAKE, 1, None, stream=0)
    _raises(qlin.QLIN_EUNSUPPORTED, qlin.sq_int8_gemm, FAKE, FAKE, FAKE, FAKE, 4, 4, 131136, FAKE, 1, None, stream=0)
    _raises(qlin.QLIN_EINVAL, qlin.sq_int8_gemm, FAKE, FAKE, FAKE, FAKE, 4, 4, 128, FAKE, 2, None, stream=0)
    _raises(qlin.QLIN_EALIGN, qlin.sq_int8_gemm, FAKE, FAKE, FAKE, FAKE, 4, 4, 128, FAKE, 1, FAKE + 4, stream=0)
    with pytest.raises(qlin.QlinError):
        qlin.sq_compute_smoothing(np.ones(8, np.float32), np.ones((2, 8), np.float32), 1.5)


def test_workspace_sizes_and_checks():
    F, B, F32 = qlin.QLIN_F16, qlin.QLIN_BF16, qlin.QLIN_F32
    counters = 16384
    # the GEMV and the small-batch kernel on fp16 activations need none
    assert qlin.qlin_w4_workspace_bytes(F, 1, 4096, 4096, 128, F) == 0
    assert qlin.qlin_w4_workspace_bytes(F, 16, 4096, 4096, 128, F) == 0
    # bf16 activations on the small-batch kernel: counters + the fp16 copy + row exponents
    assert qlin.qlin_w4_workspace_bytes(B, 8, 4096, 4096, 128, F) == counters + 8 * 4096 * 2 + 256
    assert qlin.qlin_w4_workspace_bytes(B, 1, 4096, 4096, 128, F) == 0          # the GEMV takes bf16
    # the split-K GEMM: counters + partial tiles (two per workgroup)
    sk = qlin.qlin_w4_workspace_bytes(F, 256, 8192, 8192, 128, F32)
    assert sk > counters and (sk - counters) % (2 * 128 * 256 * 4) == 0
    skb = qlin.qlin_w4_workspace_bytes(B, 256, 8192, 8192, 128, F32)
    assert skb == sk + 256 * 8192 * 2 + 1024
    assert qlin.sq_int8_gemm_workspace_bytes(2, 4096, 4096) == 0
    assert qlin.sq_int8_gemm_workspace_bytes(32, 4096, 4096) == 0
    assert qlin.sq_int8_gemm_workspace_bytes(256, 11008, 4096) > counters
    with pytest.raises(qlin.QlinError):
        qlin.qlin_w4_workspace_bytes(F, 1, 1000, 64, 128, F)
    with pytest.raises(qlin.QlinError):
        qlin.sq_int8_gemm_workspace_bytes(4, 4, 100)
    # a forward that needs a workspace refuses NULL, a short one, or a misaligned one
    fw = qlin.qlin_w4_forward
    msg = _raises(qlin.QLIN_EINVAL, fw, FAKE, F, 256, 8192, FAKE, FAKE, FAKE, 8192, 128, FAKE, F32, None, None, 0)
    assert str(sk) in msg
    _raises(qlin.QLIN_EINVAL, fw, FAKE, F, 256, 8192, FAKE, FAKE, FAKE, 8192, 128, FAKE, F32, FAKE, sk - 16, 0)
    _raises(qlin.QLIN_EALIGN, fw, FAKE, F, 256, 8192, FAKE, FAKE, FAKE, 8192, 128, FAKE, F32, FAKE + 8, sk, 0)
    need = qlin.sq_int8_gemm_workspace_bytes(256, 1024, 4096)
    _raises(qlin.QLIN_EINVAL, qlin.sq_int8_gemm, FAKE, FAKE, FAKE, FAKE, 256, 1024, 4096, FAKE, 1, None, None, None, 0)
    _raises(qlin.QLIN_EINVAL, qlin.sq_int8_gemm, FAKE, FAKE, FAKE, FAKE, 256, 1024, 4096, FAKE, 1, None, FAKE,
            need - 1, 0)


def test_sizes():
    assert qlin.qlin_w4_sizes(4096, 11008, 128) == (4096 * 11008 // 2, 4096 * 86 * 2, 4096 * 11 * 4)
    c, s1, s2, nnz = qlin.spqr_sizes(6656, 6656, 0.01)
    assert (c, s1, s2, nnz) == (6656 * 6656 * 3 // 8, 6656 * 26 * 12, 6656 * 26 * 8, 443023)
    with pytest.raises(qlin.QlinError):
        qlin.spqr_sizes(64, 1000, 0.01)
    with pytest.raises(qlin.QlinError):
        qlin.spqr_sizes(64, 1024, 1.0)
