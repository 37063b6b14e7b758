"""Build the HIP library libqlin.so in-tree for gfx950.

Every source under csrc/ is compiled to an object under _build/ (git-ignored)
and linked into quantized_linear_layers_packed_amd/libqlin.so.  Device code is
compiled with packed-fp32 instructions disabled and without floating-point
contraction, so every multiply-add in the kernels is the one written in the
source (fmaf where fused, separate operations elsewhere).

The compiler's per-kernel resource report (registers, occupancy, scratch) is
collected into _build/kernel_resources.txt, and the build fails if any kernel
uses scratch memory: a register array the compiler could not keep in
registers turns every access to it into a memory round trip.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libqlin.so")
BUILD = os.path.join(ROOT, "_build")
ARCH = os.environ.get("QLIN_OFFLOAD_ARCH", "gfx950")

COMMON = ["-O3", "-fPIC", "-std=c++17", "-ffp-contract=off", "-Wall", "-Wno-unused-function",
          f"-I{os.path.join(ROOT, 'include')}"]
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-munsafe-fp-atomics"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


_REMARK = re.compile(r"remark: +(Function Name|VGPRs|AGPRs|ScratchSize \[bytes/lane\]|Occupancy \[waves/SIMD\]"
                     r"|VGPRs Spill|LDS Size \[bytes/block\]): (\S+) \[-Rpass-analysis")


def _resources(stderr: str):
    """Per-kernel fields of the compiler's kernel-resource-usage remarks."""
    out, cur = [], None
    for m in _REMARK.finditer(stderr):
        key, val = m.group(1), m.group(2)
        if key == "Function Name":
            cur = {"kernel": val}
            out.append(cur)
        elif cur is not None:
            cur[key.split(" [")[0]] = val
    return out


def _compile(src: str):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    if src.endswith(".hip"):
        cmd = [hipcc(), "-x", "hip", *DEVICE, *COMMON, "-Rpass-analysis=kernel-resource-usage", "-c", src, "-o", obj]
    else:
        cmd = [hipcc(), *COMMON, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    res = _resources(r.stderr)
    warn = "\n".join(l for l in r.stderr.splitlines()
                     if "packed-fp32-ops" not in l and "kernel-resource-usage" not in l and l.strip()
                     and not l.startswith("In file included from")
                     and not l.lstrip().startswith(("|", "^")) and not re.match(r"^\s*\d+ \|", l))
    if warn:
        print(warn, file=sys.stderr)
    return obj, res


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))
    jobs = min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        done = list(ex.map(_compile, srcs))
    objs = [o for o, _ in done]
    res = [k for _, r in done for k in r]
    with open(os.path.join(BUILD, "kernel_resources.txt"), "w") as f:
        for k in res:
            f.write(" ".join(f"{a}={b}" for a, b in k.items()) + "\n")
    bad = [k["kernel"] for k in res if k.get("ScratchSize", "0") != "0"]
    if bad:
        raise RuntimeError("kernels using scratch memory (a register array spilled to memory): " + ", ".join(bad))
    tmp = OUT + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT} from {len(srcs)} sources")
    return OUT


if __name__ == "__main__":
    build()
