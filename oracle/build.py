"""Build the fp64 CPU oracle (test infrastructure only) with gcc.

The oracle is a plain C shared library; it shares nothing with the HIP path.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "pda_oracle.c")
LIB = os.path.join(HERE, "libpda_oracle.so")


def build(verbose: bool = False, src: str = SRC, lib: str = LIB) -> str:
    """Compile oracle/pda_oracle.c into oracle/libpda_oracle.so and return its path.

    -O2 without fast-math keeps IEEE fp64 semantics; OpenMP spreads rows over cores.
    ``src``/``lib`` let the mutation tests build planted-mistake copies elsewhere.
    """
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-Wall", "-Wextra",
           "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
