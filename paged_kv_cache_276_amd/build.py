"""Build libpagedkv.so for gfx950 with hipcc (in-tree; run ``python -m paged_kv_cache_276_amd.build``)."""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(PKG, "_build")
LIBRARY = os.path.join(PKG, "libpagedkv.so")
# The benchmark's streaming-read probe (achievable HBM read rate); not part of the library.
PROBE_SOURCE = os.path.join(PKG, "probe", "stream_read.hip")
PROBE_LIBRARY = os.path.join(PKG, "libpkvprobe.so")

SOURCES = ["kv_write.hip", "attn_generic.hip", "attn_fast.hip", "attn_combine.hip", "api.hip", "block_manager.cpp"]
ARCH = "gfx950"

# Packed-fp32 instructions are kept out of the generated code on purpose.
COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False, jobs: int = 8) -> str:
    hipcc = _hipcc()
    os.makedirs(OBJDIR, exist_ok=True)

    def compile_one(src: str) -> str:
        obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
        cmd = [hipcc, *COMMON_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        p = subprocess.run(cmd, capture_output=True, text=True)
        errs = "\n".join(l for l in p.stderr.splitlines() if "packed-fp32-ops" not in l)
        if p.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{errs}")
        if errs.strip() and verbose:
            print(errs, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIBRARY + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIBRARY)
    build_probe(verbose)
    return LIBRARY


def build_probe(verbose: bool = False) -> str:
    tmp = PROBE_LIBRARY + ".tmp"
    cmd = [_hipcc(), *COMMON_FLAGS, "-shared", "-o", tmp, PROBE_SOURCE]
    if verbose:
        print(" ".join(cmd), flush=True)
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"hipcc failed on {PROBE_SOURCE}:\n{p.stderr}")
    os.replace(tmp, PROBE_LIBRARY)
    return PROBE_LIBRARY


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
