"""Build the fp64 CPU oracle (plain C, gcc, OpenMP) into oracle/libfa_oracle.so.

Test infrastructure: only the tests, the smoke check and the benchmark's CPU
baseline use the library this produces.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "fa_oracle.c")
LIB = os.path.join(HERE, "libfa_oracle.so")


def build(src: str = SRC, out: str = LIB, extra_flags=()) -> str:
    """Compile `src` to the shared library `out` and return its path."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           *extra_flags, src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(*sys.argv[1:2]))
