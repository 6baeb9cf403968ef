"""Builds tests/devmath/libzs_devmath.so with libzshard's own hipcc flags."""
import importlib.util
import os

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
LIB = os.path.join(HERE, "libzs_devmath.so")


def build(verbose: bool = False) -> str:
    path = os.path.join(ROOT, "sharded_mixed_precision_rank_amd", "build.py")
    spec = importlib.util.spec_from_file_location("_zshard_build", path)
    lb = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(lb)
    lb._hipcc([os.path.join(HERE, "zs_devmath.hip")], [], LIB, [], verbose)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
