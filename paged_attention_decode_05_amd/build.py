"""Build libpa_decode.so for gfx950 with hipcc (in-tree, no JIT cache).

    python -m paged_attention_decode_05_amd.build [--resource-usage]

All HIP sources are compiled with packed-fp32 instructions disabled
(``-target-feature -packed-fp32-ops``): the kernels are written as scalar
fp32 code and must not be turned into v_pk_* forms.
"""
from __future__ import annotations

import argparse
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libpa_decode.so")

SOURCES = ["pa_api.hip", "pa_gqa.hip", "pa_mla.hip", "pa_cache.hip", "pa_validate.cpp"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++20", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-fvisibility=hidden",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.sep not in c or os.path.exists(c)):
            return c
    raise RuntimeError("hipcc not found")


def build(resource_usage: bool = False, verbose: bool = False, out: str = LIB) -> str:
    """Compile every source to an object in parallel (no relocatable device
    code: each source holds its own kernels), then link the shared library."""
    from concurrent.futures import ThreadPoolExecutor

    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    compile_flags = [f for f in HIPCC_FLAGS if f != "-shared"]

    def compile_one(src: str) -> str:
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        cmd = [hipcc(), *compile_flags, "-c", os.path.join(CSRC, src), "-o", obj]
        if resource_usage:
            cmd.insert(1, "-Rpass-analysis=kernel-resource-usage")
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        return obj

    jobs = max(1, min(len(SOURCES), int(os.environ.get("MAX_JOBS", "8") or 8)))
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--resource-usage", action="store_true")
    a = ap.parse_args()
    print(build(resource_usage=a.resource_usage, verbose=True))
    return 0


if __name__ == "__main__":
    sys.exit(main())
