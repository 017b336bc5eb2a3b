"""Build the fp64 CPU oracle (fwa_oracle.c) into oracle/liboracle_fwa.so with gcc.

TEST INFRASTRUCTURE ONLY: the oracle is the checker for the HIP path, never part of it.
Plain C99 + OpenMP, IEEE double, no -ffast-math, no FTZ: rounding and denormals are the
platform's defaults.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "fwa_oracle.c")
LIB = os.path.join(HERE, "liboracle_fwa.so")


def build(src=SRC, out=LIB, extra_flags=()):
    """Compile `src` into the shared library `out`; returns `out`."""
    cmd = ["gcc", "-std=c99", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
           "-fPIC", "-shared", "-Wall", "-Wextra", *extra_flags, src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(*sys.argv[1:2]) if len(sys.argv) > 1 else build())
