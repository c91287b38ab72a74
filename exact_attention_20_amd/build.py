"""Build libfa.so (the C-ABI library) in-tree with hipcc for gfx950, and the
MFMA throughput probe libfa_probe.so that bench.py reports beside the roofline.

    python -m exact_attention_20_amd.build

Every HIP source is compiled with packed-FP32 instructions disabled
(``-Xclang -target-feature -Xclang -packed-fp32-ops``); the host pass prints
a harmless warning about the unknown feature.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfa.so")
ARCH = os.environ.get("FA_OFFLOAD_ARCH", "gfx950")

SOURCES = ["fa_api.cpp", "fa_fwd.hip", "fa_bwd.hip", "fa_noalloc.hip"]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libfa.so")


def flags(extra=()):
    return [
        "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-command-line-argument",
        f"-I{INCLUDE}", f"-I{CSRC}", *extra,
    ]


def build(verbose: bool = False, extra=()) -> str:
    """Compile every source into an object and link libfa.so; returns its path."""
    cc = hipcc()
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src.replace(".", "_") + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [cc, *flags(extra), *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    # the MFMA throughput probe bench.py reports beside the roofline
    probe = os.path.join(PKG, "libfa_probe.so")
    cmd = [cc, *flags(extra), "-x", "hip", "-shared", os.path.join(CSRC, "probe_mfma.hip"), "-o", probe + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(probe + ".tmp", probe)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
