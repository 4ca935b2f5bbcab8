"""Compile the CPU oracle into oracle/liboracle.so (gcc, no fast-math).

Test infrastructure: only the tests, the smoke check and the benchmark's
CPU-baseline leg use liboracle.so.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

# -ffp-contract=off: every float operation in the oracle is rounded on its
# own; -fno-fast-math is gcc's default and is spelled out for the reader.
# -fopenmp: the *_threads entry points hand whole destination rows to threads.
CFLAGS = ["-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off",
          "-fno-fast-math", "-fopenmp", "-Wall", "-Wextra"]


def build(verbose: bool = False, src: str = SRC, out: str = LIB) -> str:
    """Compile `src` (oracle.c, or a copy of it) into the shared library `out`."""
    cmd = ["gcc", *CFLAGS, src, "-o", out + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
