"""Build the NVFP4 reference oracle (test infrastructure) into oracle/liboracle.so.

Plain gcc, no FMA contraction, no fast-math, generic x86-64 code so the
library built here also runs on another host.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "nvfp4_oracle.c")
OUT = os.path.join(HERE, "liboracle.so")
FLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fexcess-precision=standard",
         "-fopenmp", "-fPIC", "-shared"]


def build(verbose: bool = False) -> str:
    tmp = OUT + ".tmp"
    cmd = ["gcc"] + FLAGS + [SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
