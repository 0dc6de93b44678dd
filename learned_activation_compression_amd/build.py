"""Build libmapl.so (hand-written HIP for gfx950) in-tree.

Usage:  python -m learned_activation_compression_amd.build [-v]

Each HIP source is compiled to an object under _build/ in parallel, then
linked into learned_activation_compression_amd/libmapl.so.  Every call
recompiles (the build is a few seconds per file and the driver uses it as a
"does it build" check).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmapl.so")
ARCH = "gfx950"

SOURCES = ["abi.hip", "pack.hip", "codec_bf16.hip", "codec_gemm.hip", "codec_f32.hip", "rvq.hip", "spel.hip", "anchor_grad.hip"]

# -packed-fp32-ops: keep the compiler from forming packed fp32 VALU ops.
COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmapl.so)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass does not know the packed-fp32 feature flag; that note is expected
    out = "\n".join(l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    objs = []
    jobs = []
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        for src in SOURCES:
            obj = os.path.join(BUILD, src.replace(".hip", ".o"))
            objs.append(obj)
            cmd = [cc, *COMMON_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
            jobs.append(ex.submit(_run, cmd, verbose))
        for j in jobs:
            j.result()
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv[1:]))
