"""Build libfa.so (the C-ABI library) in-tree with hipcc for gfx950, and the
MFMA throughput probe libfa_probe.so that bench.py reports beside the roofline.

    python -m exact_attention_20_amd.build
    python -m exact_attention_20_amd.build --resource-usage [out.md]

The second form compiles the kernel sources for the device only with the
compiler's kernel-resource-usage remarks and prints, per instantiated kernel,
its VGPRs, AGPRs, spills, scratch, LDS and occupancy as a markdown table.

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

SOURCES = ["fa_api.cpp", "fa_fwd.hip", "fa_bwd.hip", "fa_bwd_f32.hip", "fa_noalloc.hip"]


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


_FIELDS = (
    ("VGPRs", "VGPRs"),
    ("AGPRs", "AGPRs"),
    ("VGPRs Spill", "VGPR spill"),
    ("SGPRs Spill", "SGPR spill"),
    ("ScratchSize [bytes/lane]", "scratch B/lane"),
    ("LDS Size [bytes/block]", "LDS B/block"),
    ("Occupancy [waves/SIMD]", "waves/SIMD"),
)


def _demangle(names):
    tool = shutil.which("llvm-cxxfilt") or shutil.which("c++filt")
    if tool is None:
        return list(names)
    out = subprocess.run([tool], input="\n".join(names), capture_output=True, text=True, check=True)
    return out.stdout.splitlines()


def parse_remarks(text: str):
    """Split the compiler's kernel-resource-usage remarks into one dict per
    kernel: ``_name`` (mangled) plus each ``key: value`` remark after it."""
    rows, cur = [], None
    for line in text.splitlines():
        if "remark:" not in line:
            continue
        body = line.split("remark:", 1)[1].split("[-Rpass-analysis", 1)[0].strip()
        if body.startswith("Function Name:"):
            cur = {"_name": body.split(":", 1)[1].strip()}
            rows.append(cur)
        elif cur is not None and ":" in body:
            key, val = body.rsplit(":", 1)
            cur[key.strip()] = val.strip()
    return rows


def resource_usage(sources=("fa_fwd.hip", "fa_bwd.hip", "fa_bwd_f32.hip")):
    """Per-kernel register, spill, LDS and occupancy figures from the compiler.

    Returns a list of ``(source, kernel, {field: value})`` in the order the
    compiler reports them.
    """
    cc = hipcc()
    rows = []
    for src in sources:
        cmd = [cc, *flags(), "-x", "hip", "--cuda-device-only", "-c", os.path.join(CSRC, src),
               "-o", os.devnull, "-Rpass-analysis=kernel-resource-usage"]
        res = subprocess.run(cmd, capture_output=True, text=True, check=True)
        rows += [(src, r) for r in parse_remarks(res.stderr)]
    names = _demangle([r["_name"] for _, r in rows])
    return [(src, name, r) for (src, r), name in zip(rows, names)]


def resource_table(rows) -> str:
    head = "| source | kernel | " + " | ".join(h for _, h in _FIELDS) + " |"
    sep = "|" + "---|" * (2 + len(_FIELDS))
    out = [head, sep]
    for src, name, r in rows:
        name = name.replace("void ", "", 1).split("(", 1)[0].replace("fa::", "")
        out.append(f"| {src} | `{name}` | " + " | ".join(r.get(k, "") for k, _ in _FIELDS) + " |")
    return "\n".join(out)


if __name__ == "__main__":
    if "--resource-usage" in sys.argv:
        table = resource_table(resource_usage())
        rest = [a for a in sys.argv[1:] if a != "--resource-usage"]
        if rest:
            with open(rest[0], "w") as f:
                f.write(table + "\n")
        print(table)
    else:
        print(build(verbose="-v" in sys.argv))
