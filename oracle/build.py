"""Builds liboracle.so with the host compiler: IEEE binary32, no contraction, no fast-math."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
FLAGS = ["-O2", "-std=c++17", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-pthread"]


def build(src: str = os.path.join(HERE, "oracle.cpp"), out: str = os.path.join(HERE, "liboracle.so"),
          verbose: bool = False) -> str:
    cmd = ["g++", *FLAGS, src, "-o", out]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return out


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
