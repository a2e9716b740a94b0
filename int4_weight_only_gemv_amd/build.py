"""Build the W4A16 HIP library (libw4a16.so) in-tree for gfx950 with hipcc.

    python -m int4_weight_only_gemv_amd.build

Every HIP source is compiled with packed-FP32 instructions disabled.  The
packing kernel is additionally compiled without FMA contraction, with
correctly rounded division and without fast-math, because its float32 steps
must match IEEE single operations bit for bit.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libw4a16.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
ARCH = "gfx950"

COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-I", INCLUDE, "-I", CSRC,
]
EXACT = ["-ffp-contract=off", "-fno-fast-math", "-fno-gpu-flush-denormals-to-zero"]

SOURCES = {
    "api.cpp": [],
    "pack.hip": EXACT,
    "gemv.hip": [],
    "gemm.hip": [],
    "awq.hip": EXACT,
    "dense.hip": EXACT,
    "probe.hip": [],
    "chain.hip": [],
}


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compile every source and link libw4a16.so next to this file."""
    cc = hipcc()
    tmp = tempfile.mkdtemp(prefix="w4a16_build_")
    try:
        procs = []
        objs = []
        for src, extra in SOURCES.items():
            obj = os.path.join(tmp, src.replace(".", "_") + ".o")
            objs.append(obj)
            lang = ["-x", "hip"] if src.endswith(".hip") else []
            cmd = [cc, *COMMON, *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
            if len(procs) >= jobs:
                _wait(procs.pop(0))
        while procs:
            _wait(procs.pop(0))
        out_tmp = LIB_PATH + ".tmp"
        cmd = [cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-Wl,-z,defs", *objs, "-o", out_tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        _wait(("link", subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        os.replace(out_tmp, LIB_PATH)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return LIB_PATH


def _wait(item):
    name, p = item
    out, _ = p.communicate()
    text = out.decode(errors="replace")
    if p.returncode != 0:
        raise RuntimeError(f"hipcc failed on {name}:\n{text}")
    noise = [ln for ln in text.splitlines() if ln.strip() and "packed-fp32-ops" not in ln]
    if noise:
        sys.stderr.write(f"[{name}]\n" + "\n".join(noise) + "\n")


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
