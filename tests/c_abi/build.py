"""Builds the plain C client of libzshard (zs_c_client) with the host C compiler.

It links libzshard, the CPU oracle (the reference it compares with) and the
HIP runtime; run paths are relative to the binary, so the tree can move.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SRC = os.path.join(HERE, "zs_c_client.c")
OUT = os.path.join(HERE, "zs_c_client")


def build(verbose: bool = False) -> str:
    pkg = os.path.join(ROOT, "sharded_mixed_precision_rank_amd")
    orc = os.path.join(ROOT, "oracle")
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"), SRC, "-o", OUT,
           "-L", pkg, "-lzshard", "-L", orc, "-loracle", "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
           "-Wl,-rpath,$ORIGIN/../../sharded_mixed_precision_rank_amd:$ORIGIN/../../oracle:" + os.path.join(ROCM, "lib")]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
