"""Build the fp64 CPU oracle (liboracle.so) with gcc.

Test infrastructure only: the oracle is the checker, never part of the
product path.  Compiling it is not using it.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ssd_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(src=SRC, out=LIB, extra_flags=()):
    """Compile `src` into the shared library `out`; returns `out`."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall",
           "-Werror", *extra_flags, src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(*sys.argv[1:2]))
