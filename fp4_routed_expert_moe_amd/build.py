"""Compile the HIP sources under csrc/ into the in-tree C-ABI library libmoe_fp4.so (gfx950 only)."""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(HERE, "libmoe_fp4.so")
SOURCES = ("route.hip", "gemv.hip", "gemm.hip", "pack.hip", "chain.hip", "api.hip", "bank.hip")

# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU ops.
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", CSRC,
             "-Wall", "-Wno-unused-result", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm required to build the MoE library)")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = r.stdout + r.stderr
    # the host pass does not know the gfx950 feature flag; that warning is harmless
    out = "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, extra_flags=(), out: str = LIB_PATH, build_dir: str = BUILD_DIR) -> str:
    """Compile every source (always) and link the shared library; returns its path.

    ``extra_flags`` (e.g. ``-DMOE_GEMV_TILES=2``) and ``out`` build a variant elsewhere."""
    cc = hipcc()
    os.makedirs(build_dir, exist_ok=True)
    objs = []
    jobs = []
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        for src in SOURCES:
            obj = os.path.join(build_dir, src.replace(".hip", ".o"))
            objs.append(obj)
            cmd = [cc, *HIP_FLAGS, *extra_flags, "-c", os.path.join(CSRC, src), "-o", obj]
            jobs.append(ex.submit(_run, cmd))
        for j in jobs:
            log = j.result()
            if verbose and log.strip():
                print(log, file=sys.stderr)
    tmp = out + ".tmp"
    _run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
