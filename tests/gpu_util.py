"""Helpers for the GPU parity tests (device copies, tolerance checks)."""
import sys

import numpy as np

from oracle import metrics


def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        import pytest
        pytest.skip("no GPU")
    return torch


def dev(a: np.ndarray):
    """Host array -> contiguous device tensor with the same bytes."""
    torch = torch_cuda()
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        t = torch.from_numpy(a.view(np.int16)).view(torch.float16)
    elif a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16))
    elif a.dtype == np.uint32:
        t = torch.from_numpy(a.view(np.int32))
    else:
        t = torch.from_numpy(a)
    return t.to("cuda")


def empty(shape, dtype):
    torch = torch_cuda()
    return torch.empty(shape, dtype=dtype, device="cuda")


def host(t, np_dtype=None):
    torch = torch_cuda()
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    a = t.cpu().numpy()
    return a.view(np_dtype) if np_dtype is not None else a


_WORKSPACES = []


def workspace(nbytes):
    """A zero-filled device workspace of at least ``nbytes`` (None when 0).

    Buffers are shared by the calls of a test process (which run one after the
    other on one stream) and are never freed: a captured graph may still refer
    to one."""
    if nbytes == 0:
        return None
    torch = torch_cuda()
    for t in _WORKSPACES:
        if t.numel() >= nbytes:
            return t
    t = torch.zeros(max(int(nbytes), 1 << 20), dtype=torch.uint8, device="cuda")
    _WORKSPACES.append(t)
    return t


def w4_ws(x_dtype, M, K, N, G, y_dtype):
    from quantized_linear_layers_packed_amd import qlin
    return workspace(qlin.qlin_w4_workspace_bytes(x_dtype, M, K, N, G, y_dtype))


def spqr_ws(M, K, N, y_dtype):
    from quantized_linear_layers_packed_amd import qlin
    return workspace(qlin.spqr_workspace_bytes(M, K, N, y_dtype))


def sq_ws(M, N, K, y_dtype):
    from quantized_linear_layers_packed_amd import qlin
    return workspace(qlin.sq_int8_gemm_workspace_bytes(M, N, K, y_dtype))


def bf16_bits_to_f64(bits):
    return metrics.bf16_bits_to_f64(bits)


def check_close(y, y_ref, what=""):
    ok, a, f = metrics.within_tolerance(y, y_ref)
    print(f"  {what}: max_abs_ratio={a:.3e} rel_frob={f:.3e}", flush=True)
    assert ok, f"{what}: max_abs_ratio {a:.3e} (<= {metrics.MAX_ABS_RATIO}), rel_frob {f:.3e} (<= {metrics.REL_FROB})"


def say(*args):
    print(*args, flush=True)
    sys.stdout.flush()
