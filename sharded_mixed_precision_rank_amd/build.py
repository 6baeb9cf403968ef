"""Builds libzshard.so (gfx950) in place with hipcc."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libzshard.so")
SOURCES = [os.path.join(CSRC, "zs_kernels.hip"), os.path.join(CSRC, "zs_twopass.hip"), os.path.join(CSRC, "zs_api.cpp")]
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-fvisibility=hidden",
    # one rounding per operation, correctly rounded divide and sqrt
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    # no packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def build(verbose: bool = False, out: str = LIB, extra=()) -> str:
    cmd = ["hipcc", *FLAGS, *extra]
    for src in SOURCES:
        cmd += ["-x", "hip", src]
    cmd += ["-o", out]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [l for l in r.stdout.splitlines() if noise not in l]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    return out


if __name__ == "__main__":
    build(verbose=True)
