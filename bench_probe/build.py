"""Builds the benchmark's measurement probe, libzshard_probe.so (gfx950), with
the library's own compiler flags and device helpers."""
import importlib.util
import os

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libzshard_probe.so")
SOURCES = [os.path.join(HERE, "zs_probe.hip")]


def _library_build():
    path = os.path.join(ROOT, "sharded_mixed_precision_rank_amd", "build.py")
    spec = importlib.util.spec_from_file_location("_zshard_build", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def build(verbose: bool = False) -> str:
    lb = _library_build()
    lb._hipcc(SOURCES, [], LIB, ["-I", lb.CSRC], verbose)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
