"""Builds the synthetic-input generators: host (gcc, OpenMP) and device (hipcc, gfx950)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-shared", "-std=c++17",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(verbose: bool = False) -> None:
    cmds = [
        ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", os.path.join(HERE, "synth_host.c"),
         "-o", os.path.join(HERE, "libsynth_host.so")],
        ["hipcc", *HIP_FLAGS, os.path.join(HERE, "synth_dev.hip"), "-o", os.path.join(HERE, "libsynth_dev.so")],
    ]
    for cmd in cmds:
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True, stderr=subprocess.PIPE if not verbose else None)


if __name__ == "__main__":
    build(verbose=True)
