"""Compile the CPU oracle (plain C, double precision) into oracle/liboracle.so.

Test infrastructure: the oracle is what the GPU library is checked against.
Built with gcc -O2 (no fast-math, so every sum is evaluated as written) and
OpenMP over the outer (batch, query) loops.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "sa_oracle.c")
OUT = os.path.join(HERE, "liboracle.so")
OUT_SAN = os.path.join(HERE, "liboracle_san.so")


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """sanitize=True: liboracle_san.so with AddressSanitizer and
    UndefinedBehaviorSanitizer (gcc runtimes, to be preloaded by the caller)."""
    out = OUT_SAN if sanitize else OUT
    san = (["-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
            "-fno-omit-frame-pointer"] if sanitize else [])
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-fno-fast-math", "-Wall", "-Wextra", "-Wno-unused-parameter", *san,
           SRC, "-o", out + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv)
