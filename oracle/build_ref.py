"""Builds the plain C oracle (oracle/ref_decode.c -> oracle/libbref.so) with
gcc: -O2, OpenMP, no floating-point contraction.  Test infrastructure: the
tests and the benchmark's CPU baseline load the result; nothing in the HIP
library does."""
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ref_decode.c")
OUT = os.path.join(HERE, "libbref.so")


def build(verbose: bool = False) -> str:
    cc = os.environ.get("CC") or shutil.which("gcc") or "cc"
    cmd = [cc, "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", SRC, "-o", OUT + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(OUT + ".tmp", OUT)
    return OUT


if __name__ == "__main__":
    build(verbose=True)
