"""Build libbitlinear.so, the gfx950 HIP library behind include/bitlinear.h.

Every source is compiled with hipcc for gfx950 only.  Floating-point flags
pin the arithmetic the quantizers and the epilogue rely on: no fast-math
(fp32 division stays correctly rounded), no FMA contraction, and packed fp32
instructions disabled.  The build fails if any kernel uses scratch memory:
every kernel is written to fit its registers, and a spill (for instance a
shared body the inliner outlined into a call) silently costs a large share
of its bandwidth.
"""
import concurrent.futures
import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libbitlinear.so")
SOURCES = ["api.hip", "weight_quant.hip", "pack.hip", "pack5.hip", "act_quant.hip",
           "gemv_stream.hip", "gemm_tile.hip", "gemv5.hip", "probes.hip"]
ARCH = "gfx950"

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.isabs(c) and os.path.exists(c) or not os.path.isabs(c)):
            return c
    raise RuntimeError("hipcc not found")


RESOURCE_REMARKS = "-Rpass-analysis=kernel-resource-usage"


def spilling_kernels(remarks):
    """(kernel, bytes per lane) for every function whose resource-usage
    remark reports scratch memory."""
    out, name = [], None
    for ln in remarks.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", ln)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"remark:\s+ScratchSize \[bytes/lane\]: (\d+)", ln)
        if m and name is not None and int(m.group(1)) > 0:
            out.append((name, int(m.group(1))))
    return out


def _compile(src, verbose):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *CFLAGS, RESOURCE_REMARKS, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(ln for ln in r.stderr.splitlines()
                     if "packed-fp32-ops" not in ln and "kernel-resource-usage" not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{errs}")
    spills = spilling_kernels(r.stderr)
    if spills:
        raise RuntimeError(f"{src}: kernels use scratch memory (bytes per lane): "
                           + ", ".join(f"{k} {b}" for k, b in spills))
    if verbose and errs.strip():
        print(errs)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", LIB + ".tmp", *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
