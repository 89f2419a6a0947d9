"""Compile the fp64 C oracle into a shared library with the host C compiler.

Test infrastructure only.  Plain ``-O2``: no fast-math, no contraction of
``a*b+c`` into fused multiply-adds, so each sum is the sequence of
IEEE double operations written in ``dsc_oracle.c``.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "dsc_oracle.c")
LIB = os.path.join(HERE, "liboracle_dsc.so")

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
          "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra"]


def build(src=SRC, out=LIB, extra_flags=()):
    """Compile ``src`` into ``out``; returns the output path."""
    cmd = ["gcc", *CFLAGS, *extra_flags, src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build())
    sys.exit(0)
