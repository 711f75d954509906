"""Build the CPU oracle (test infrastructure only) with gcc.

``build()`` compiles ``pa_oracle.c`` into ``oracle/libpa_oracle.so``.
``build(mutation=k, out=path)`` compiles a copy with planted mistake ``k``
for the tests that show the pins can fail.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
DEFAULT_LIB = os.path.join(HERE, "libpa_oracle.so")

# -ffp-contract=off: no fused multiply-add, so each product and sum rounds
# once at the instantiation's precision.  No -ffast-math.
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
          "-Wall", "-Wextra", "-Wno-unused-parameter"]


def build(mutation: int = 0, out: str | None = None, verbose: bool = False) -> str:
    out = out or DEFAULT_LIB
    tmp = out + ".tmp"
    cmd = ["gcc", *CFLAGS, f"-DORACLE_MUTATION={int(mutation)}",
           os.path.join(HERE, "pa_oracle.c"), "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
