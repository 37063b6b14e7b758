"""Sanitizer build of the host encoders (CPU only).

tests/sanitize/host_encoders.cpp calls every host encoder of the C ABI (W4
round-to-nearest, SpQR, SmoothQuant smoothing and weights, Hessian, GPTQ-style
and act-order encodes, sensitivity SpQR) on small inputs with edge cases, plus
the argument checks that must refuse a call.  It is compiled here with the host
compiler under AddressSanitizer and UndefinedBehaviorSanitizer (every report
fatal, leak check at exit) together with the library's host sources, run, and
its outputs are compared byte for byte with the regular library's on the same
inputs."""
import os
import shutil
import subprocess

import numpy as np
import pytest

from quantized_linear_layers_packed_amd import qlin

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "quantized_linear_layers_packed_amd", "csrc")
ROCM = "/opt/rocm"


@pytest.fixture(scope="module")
def outputs(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.exists(os.path.join(ROCM, "lib", "libamdhip64.so")):
        pytest.skip("host compiler or HIP runtime library not available")
    d = tmp_path_factory.mktemp("sanitize")
    exe = str(d / "host_encoders")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-pthread", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include",
           f"-I{os.path.join(ROOT, 'include')}", os.path.join(ROOT, "tests", "sanitize", "host_encoders.cpp"),
           os.path.join(CSRC, "host_pack.cpp"), os.path.join(CSRC, "host_gptq.cpp"), os.path.join(CSRC, "status.cpp"),
           f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    out = d / "out"
    out.mkdir()
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe, str(out)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, f"sanitized run failed:\n{r.stdout[-2000:]}\n{r.stderr[-6000:]}"
    assert "host encoders OK" in r.stdout

    def load(name, dtype, shape=None):
        a = np.fromfile(str(out / name), dtype=dtype)
        return a.reshape(shape) if shape is not None else a
    return load


def test_w4_round_to_nearest(outputs):
    for tag, (N, K, G) in (("w4a", (5, 256, 128)), ("w4b", (3, 64, 32))):
        W = outputs(f"{tag}_W", np.float32, (N, K))
        qw, sc, qz = qlin.qlin_w4_pack(W, G)
        assert np.array_equal(outputs(f"{tag}_qweight", np.uint32), qw.ravel())
        assert np.array_equal(outputs(f"{tag}_scales", np.uint16), sc.view(np.uint16).ravel())
        assert np.array_equal(outputs(f"{tag}_qzeros", np.uint32), qz.ravel())


@pytest.mark.parametrize("tag,N,K,p", [("spqra", 7, 256, 0.0), ("spqrb", 4, 512, 0.05)])
def test_spqr(outputs, tag, N, K, p):
    st = qlin.spqr_pack(outputs(f"{tag}_W", np.float32, (N, K)), p)
    for k, dt in (("codes", np.uint32), ("stats1", np.uint32), ("stats2", np.uint16), ("row_ptr", np.int32),
                  ("col_idx", np.int32), ("val", np.uint16)):
        assert np.array_equal(outputs(f"{tag}_{k}", dt), np.ascontiguousarray(st[k]).view(dt).ravel()), k


def test_smoothquant(outputs):
    X = outputs("sq_X", np.uint16, (9, 128)).view(np.float16)
    W = outputs("sq_W", np.float32, (6, 128))
    amax = qlin.sq_act_absmax(X)
    assert np.array_equal(outputs("sq_amax", np.float32), amax)
    s, inv = qlin.sq_compute_smoothing(amax, W, 0.85)
    assert np.array_equal(outputs("sq_s", np.float32), s) and np.array_equal(outputs("sq_inv", np.float32), inv)
    Wq, ws = qlin.sq_pack_weight(W, s)
    assert np.array_equal(outputs("sq_Wq", np.int8), Wq.ravel()) and np.array_equal(outputs("sq_wscale", np.float32), ws)


def test_second_order(outputs):
    X = outputs("so_X", np.float32, (16, 128))
    H = qlin.qlin_hessian(X)
    assert np.array_equal(outputs("so_H", np.float64), H.ravel())
    qw, sc, qz = qlin.qlin_w4_pack_gptq(outputs("gq_W", np.float32, (6, 128)), 64, H)
    assert np.array_equal(outputs("gq_qweight", np.uint32), qw.ravel())
    assert np.array_equal(outputs("gq_scales", np.uint16), sc.view(np.uint16).ravel())
    assert np.array_equal(outputs("gq_qzeros", np.uint32), qz.ravel())
    for tag, static in (("ao_dynamic", False), ("ao_static", True)):
        qw, sc, qz, perm = qlin.qlin_w4_pack_gptq_actorder(outputs(f"{tag}_W", np.float32, (5, 128)), 32, H,
                                                           static_groups=static)
        assert np.array_equal(outputs(f"{tag}_qweight", np.uint32), qw.ravel())
        assert np.array_equal(outputs(f"{tag}_scales", np.uint16), sc.view(np.uint16).ravel())
        assert np.array_equal(outputs(f"{tag}_qzeros", np.uint32), qz.ravel())
        assert np.array_equal(outputs(f"{tag}_perm", np.int32), perm)
    H2 = qlin.qlin_hessian(outputs("sh_X", np.float32, (16, 256)))
    st = qlin.spqr_pack_hessian(outputs("sh_W", np.float32, (5, 256)), 0.02, H2)
    for k, dt in (("codes", np.uint32), ("stats1", np.uint32), ("stats2", np.uint16), ("row_ptr", np.int32),
                  ("col_idx", np.int32), ("val", np.uint16)):
        assert np.array_equal(outputs(f"sh_{k}", dt), np.ascontiguousarray(st[k]).view(dt).ravel()), k
