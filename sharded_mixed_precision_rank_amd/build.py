"""Builds libzshard.so (gfx950) in place with hipcc."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libzshard.so")
# Device code and HIP-runtime host code compile as HIP in one hipcc command.
SOURCES = [os.path.join(CSRC, f) for f in ("zs_kernels.hip", "zs_twopass.hip", "zs_api.cpp", "zs_offload.cpp")]
# The host AdamW is plain C++ built by the host compiler into an object that
# the hipcc link takes as is (its AVX2 path is chosen at run time).  Compiling
# it as a C++ input inside the hipcc command produced a library that crashed
# when loaded, so it stays a separate object.
HOST_SOURCES = [os.path.join(CSRC, "zs_cpu_adam.cpp")]
HOST_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-ffp-contract=off", "-fno-fast-math", "-Wall"]
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-fvisibility=hidden",
    # one rounding per operation, correctly rounded divide and sqrt
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    # no packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def _hipcc(sources, objs, out, extra, verbose):
    cmd = ["hipcc", *FLAGS, *extra]
    for src in sources:
        cmd += ["-x", "hip", src]
    if objs:
        cmd += ["-x", "none", *objs]
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


def build(verbose: bool = False, out: str = LIB, extra=()) -> str:
    objs = []
    for src in HOST_SOURCES:
        obj = os.path.join(HERE, os.path.splitext(os.path.basename(src))[0] + ".o")
        hcmd = ["g++", *HOST_FLAGS, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(hcmd), flush=True)
        subprocess.run(hcmd, check=True)
        objs.append(obj)
    _hipcc(SOURCES, objs, out, extra, verbose)
    return out


if __name__ == "__main__":
    build(verbose=True)
