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
    noise = "is not a recognized feature for this target"
    for cmd in cmds:
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        msgs = [l for l in r.stdout.splitlines() if noise not in l]
        if r.returncode != 0:
            raise RuntimeError("build failed:\n" + "\n".join(msgs))


if __name__ == "__main__":
    build(verbose=True)
