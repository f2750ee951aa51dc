"""Compile libssm.so (HIP kernels for gfx950 + host layer) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libssm.so")
SOURCES = [os.path.join(CSRC, f) for f in
           ("ssm_api.hip", "scan_fast.hip", "scan_fast_zoh.hip", "scan_fast_bilinear.hip",
            "scan_generic.hip", "scan_generic_zoh.hip", "scan_generic_bilinear.hip", "decode.hip",
            "scan_bwd.hip", "conv1d.hip", "ssd.hip", "probe.hip", "ssm_host.cpp")]

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-shared",
    # no packed-FP32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    return subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)


def _finish(proc, what):
    _, err = proc.communicate()
    err = "\n".join(l for l in err.splitlines() if "packed-fp32-ops" not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed on {what} ({proc.returncode}):\n{err}")
    return err


def build(verbose: bool = False) -> str:
    """Compile every source to an object in parallel, then link libssm.so."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    compile_flags = [f for f in HIPCC_FLAGS if f != "-shared"]
    procs, objs = [], []
    for src in SOURCES:
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        objs.append(obj)
        procs.append((src, _run([hipcc, *compile_flags, "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj], verbose)))
    warnings = [_finish(p, src) for src, p in procs]
    tmp = LIB + ".tmp"
    link = _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    warnings.append(_finish(link, "link"))
    if verbose and any(w.strip() for w in warnings):
        print("\n".join(w for w in warnings if w.strip()), file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
