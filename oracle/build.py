"""Build the CPU oracle library (``oracle/liboracle.so``) with gcc.

Test infrastructure: the oracle is compiled with ``-O2 -ffp-contract=off`` so
that every float operation in ``oracle.c`` is one IEEE rounding (no FMA
contraction, no fast-math), and with OpenMP so that full-size checks finish in
seconds.  Run ``python oracle/build.py`` or call :func:`build_oracle`.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC",
          "-Wall", "-Wextra", "-Werror"]


def build_oracle(src: str = SRC, out: str = LIB, extra_flags: list[str] | None = None) -> str:
    """Compile ``src`` into the shared library ``out`` and return its path."""
    tmp = out + ".tmp"
    cmd = ["gcc", *CFLAGS, *(extra_flags or []), "-shared", "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_oracle())
    sys.exit(0)
