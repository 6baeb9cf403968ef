"""ctypes loader of the benchmark's measurement probe (libzshard_probe.so): the
fused step's access pattern without its arithmetic, and a copy kernel built
like the step's kernels.  Instrumentation for bench.py and its tests; not part
of the library."""
import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libzshard_probe.so")
_lib = None


def load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        # the HIP runtime torch brought in must be the one the probe binds to
        import torch  # noqa: F401

        lib = ctypes.CDLL(LIB_PATH)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        lib.zs_probe_pattern.restype = ctypes.c_int
        lib.zs_probe_pattern.argtypes = [ctypes.POINTER(vp), i32, i64, vp, vp, vp, vp, i32, vp]
        lib.zs_probe_pattern_windowed.restype = ctypes.c_int
        lib.zs_probe_pattern_windowed.argtypes = [ctypes.POINTER(vp), i32, i64, vp, vp, vp, vp, i32, i32, vp]
        lib.zs_probe_pattern_phased.restype = ctypes.c_int
        lib.zs_probe_pattern_phased.argtypes = [ctypes.POINTER(vp), i32, i64, vp, vp, vp, vp, vp, vp]
        lib.zs_probe_copy.restype = ctypes.c_int
        lib.zs_probe_copy.argtypes = [vp, vp, i64, vp]
        _lib = lib
    return _lib
