"""Build the gfx950 HIP library (libfa_mi355x.so) in-tree with hipcc.

Usage:  python -m exact_tiled_attention_37_amd.build [-v]

Each source is compiled in parallel, then linked into one shared library
next to this file. Packed fp32 VALU instructions are disabled for all device
code (-packed-fp32-ops).
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libfa_mi355x.so")
SOURCES = ["fa_api.hip", "fa_fwd.hip", "fa_bwd.hip", "fa_merge.hip", "fa_fp8.hip"]
# Per-source compiler flags (none at present).
EXTRA_FLAGS = {}
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def common_flags():
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-fvisibility=hidden",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"),
        "-I", CSRC,
    ]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so.
    err = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    objs = []
    jobs = []
    for src in SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        objs.append(obj)
        jobs.append([cc, *common_flags(), *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj])
    workers = min(len(jobs), max(1, (os.cpu_count() or 1)))
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        for f in [ex.submit(_run, j, verbose) for j in jobs]:
            f.result()
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
