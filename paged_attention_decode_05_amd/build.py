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
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if resource_usage:
        cmd.insert(1, "-Rpass-analysis=kernel-resource-usage")
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
