"""Build the CPU oracle (test infrastructure only) into oracle/liboracle.so.

gcc, -O2, no contraction of a*b+c into fused multiply-adds, no fast-math,
SSE scalar floating point: every binary32 operation in the C source rounds
once, to nearest-even.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")
SRC = os.path.join(HERE, "zf_oracle.c")

CFLAGS = [
    "-O2", "-std=c99", "-Wall", "-Wextra", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-fast-math", "-fexcess-precision=standard",
    "-msse2", "-mfpmath=sse",
]


def build(extra_flags=()):
    """Compile the oracle; returns the path of the shared library."""
    tmp = LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, *extra_flags, "-o", tmp, SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
