"""Build the CPU oracle shared library (test infrastructure; plain g++ with OpenMP).

``python oracle/build.py`` writes ``oracle/liboracle.so``.  Strict IEEE fp64: no
fast-math and no contraction of multiply-add, so the oracle's sums are the textbook
left-to-right ones.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.cpp")
OUT = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False, out: str = OUT, extra=()) -> str:
    """Compile oracle.cpp into ``out``; ``extra`` flags go after the standard ones (the
    sanitizer test builds an instrumented copy elsewhere this way)."""
    cmd = ["g++", "-std=c++17", "-O2", "-fPIC", "-shared", "-fopenmp",
           "-ffp-contract=off", "-fno-fast-math", *extra, SRC, "-o", out + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
