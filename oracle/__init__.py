"""ctypes face of the CPU oracle (``oracle.cpp``).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``, never by the library package.  The
oracle shares no code with the GPU library.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(_HERE, "liboracle.so")

FOLD_NAMES = ("b1", "c1", "b2", "c2", "e", "ss", "rb", "dk")


class OracleHP(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("beta1", ctypes.c_double), ("beta2", ctypes.c_double),
                ("eps", ctypes.c_double), ("weight_decay", ctypes.c_double)]


def _hp(hp: dict) -> OracleHP:
    return OracleHP(hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp.get("weight_decay", 0.0))


def _ptr_table(G):
    """G: 2-D uint16 array (N, n) or a sequence of 1-D uint16 arrays -> (c_void_p * N, keepalive)."""
    rows = [np.ascontiguousarray(g, dtype=np.uint16) for g in G]
    tab = (ctypes.c_void_p * len(rows))(*[r.ctypes.data for r in rows])
    return tab, rows


class Oracle:
    def __init__(self, path: str = LIB):
        if not os.path.exists(path):
            raise ImportError(f"{path} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(path)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        lib.oracle_fold.argtypes = [ctypes.POINTER(OracleHP), i64, vp]
        lib.oracle_f32_to_bf16.restype = ctypes.c_uint16
        lib.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
        lib.oracle_f32_to_bf16_array.argtypes = [vp, vp, i64]
        lib.oracle_reduce_mean.restype = ctypes.c_int
        lib.oracle_reduce_mean.argtypes = [vp, i32, i64, vp, i32]
        lib.oracle_reduce_adam.restype = ctypes.c_int
        lib.oracle_reduce_adam.argtypes = [vp, i32, i64, vp, vp, vp, vp, ctypes.POINTER(OracleHP), i64, i32]
        lib.oracle_state_bytes_per_param.restype = i64
        lib.oracle_sharded_state_bytes.restype = ctypes.c_double
        lib.oracle_sharded_state_bytes.argtypes = [ctypes.c_double, i32]
        lib.oracle_step_traffic_bytes.restype = i64
        lib.oracle_step_traffic_bytes.argtypes = [i32, i64]
        self.lib = lib
        self.path = path

    def fold(self, hp: dict, t: int) -> np.ndarray:
        out = np.empty(8, dtype=np.float32)
        h = _hp(hp)
        self.lib.oracle_fold(ctypes.byref(h), t, out.ctypes.data)
        return out

    def bf16(self, x) -> np.ndarray:
        x = np.ascontiguousarray(x, dtype=np.float32)
        out = np.empty(x.shape, dtype=np.uint16)
        self.lib.oracle_f32_to_bf16_array(x.ctypes.data, out.ctypes.data, x.size)
        return out

    def reduce_mean(self, G, threads: int = 0) -> np.ndarray:
        tab, rows = _ptr_table(G)
        n = rows[0].size
        out = np.empty(n, dtype=np.float32)
        rc = self.lib.oracle_reduce_mean(tab, len(rows), n, out.ctypes.data, threads)
        if rc:
            raise ValueError("oracle_reduce_mean: bad arguments")
        return out

    def step_inplace(self, G, P, M, V, B, hp: dict, t: int, threads: int = 0) -> None:
        """Run the step in place on contiguous numpy arrays P, M, V (float32) and B (uint16)."""
        tab, rows = _ptr_table(G)
        n = P.size
        for a, dt in ((P, np.float32), (M, np.float32), (V, np.float32), (B, np.uint16)):
            assert a.dtype == dt and a.flags.c_contiguous and a.size == n
        assert all(r.size == n for r in rows)
        h = _hp(hp)
        rc = self.lib.oracle_reduce_adam(tab, len(rows), n, P.ctypes.data, M.ctypes.data, V.ctypes.data,
                                         B.ctypes.data, ctypes.byref(h), t, threads)
        if rc:
            raise ValueError("oracle_reduce_adam: bad arguments")

    def step(self, G, P, M, V, hp: dict, t: int, threads: int = 0):
        """Functional form: returns (P1, M1, V1, B1) and leaves the inputs alone."""
        P1 = np.array(P, dtype=np.float32, copy=True)
        M1 = np.array(M, dtype=np.float32, copy=True)
        V1 = np.array(V, dtype=np.float32, copy=True)
        B1 = np.empty(P1.size, dtype=np.uint16)
        self.step_inplace(G, P1, M1, V1, B1, hp, t, threads)
        return P1, M1, V1, B1

    def state_bytes_per_param(self) -> int:
        return int(self.lib.oracle_state_bytes_per_param())

    def sharded_state_bytes(self, psi: float, ndp: int) -> float:
        return float(self.lib.oracle_sharded_state_bytes(psi, ndp))

    def step_traffic_bytes(self, N: int, n: int) -> int:
        return int(self.lib.oracle_step_traffic_bytes(N, n))


_default = None


def load() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default
