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


class OracleScaler(ctypes.Structure):
    _fields_ = [("scale", ctypes.c_double), ("min_scale", ctypes.c_double), ("window", ctypes.c_int64),
                ("hysteresis", ctypes.c_int64), ("overflows", ctypes.c_int64), ("clean", ctypes.c_int64)]


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
        lib.oracle_f32_to_f16_array.argtypes = [vp, vp, i64]
        lib.oracle_f16_to_f32.restype = ctypes.c_float
        lib.oracle_f16_to_f32.argtypes = [ctypes.c_uint16]
        lib.oracle_reduce_unscale.restype = ctypes.c_int
        lib.oracle_reduce_unscale.argtypes = [vp, i32, i64, i32, ctypes.c_double, vp, i32]
        lib.oracle_sqnorm.restype = ctypes.c_double
        lib.oracle_sqnorm.argtypes = [vp, i64]
        lib.oracle_clip_coef.restype = ctypes.c_float
        lib.oracle_clip_coef.argtypes = [ctypes.c_double, ctypes.c_double]
        lib.oracle_adam_from_gbar.restype = ctypes.c_int
        lib.oracle_adam_from_gbar.argtypes = [vp, i64, vp, vp, vp, vp, i32, ctypes.POINTER(OracleHP), i64,
                                              ctypes.c_double, ctypes.c_double, i32, i32]
        lib.oracle_scaler_update.restype = ctypes.c_int
        lib.oracle_scaler_update.argtypes = [ctypes.POINTER(OracleScaler), i32]
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

    # ---- two-pass form (clipping, fp16 loss scaling)
    def f16(self, x) -> np.ndarray:
        x = np.ascontiguousarray(x, dtype=np.float32)
        out = np.empty(x.shape, dtype=np.uint16)
        self.lib.oracle_f32_to_f16_array(x.ctypes.data, out.ctypes.data, x.size)
        return out

    def f16_to_f32(self, h) -> np.ndarray:
        return np.array([self.lib.oracle_f16_to_f32(int(v)) for v in np.asarray(h).ravel()], dtype=np.float32)

    def reduce_unscale(self, G, fmt: int = 0, loss_scale: float = 1.0, threads: int = 0) -> np.ndarray:
        tab, rows = _ptr_table(G)
        n = rows[0].size
        out = np.empty(n, dtype=np.float32)
        rc = self.lib.oracle_reduce_unscale(tab, len(rows), n, fmt, loss_scale, out.ctypes.data, threads)
        if rc:
            raise ValueError("oracle_reduce_unscale: bad arguments")
        return out

    def sqnorm(self, gbar) -> float:
        g = np.ascontiguousarray(gbar, dtype=np.float32)
        return float(self.lib.oracle_sqnorm(g.ctypes.data, g.size))

    def clip_coef(self, total_sq: float, max_norm: float) -> float:
        return float(self.lib.oracle_clip_coef(total_sq, max_norm))

    def adam_from_gbar(self, gbar, P, M, V, hp: dict, t: int, total_sq: float, max_norm: float = 0.0,
                       out_fmt: int = 0, skip_nonfinite: bool = True, threads: int = 0):
        """Functional pass 2: returns (P1, M1, V1, B1, taken)."""
        g = np.ascontiguousarray(gbar, dtype=np.float32)
        P1 = np.array(P, dtype=np.float32, copy=True)
        M1 = np.array(M, dtype=np.float32, copy=True)
        V1 = np.array(V, dtype=np.float32, copy=True)
        B1 = np.zeros(P1.size, dtype=np.uint16)
        h = _hp(hp)
        rc = self.lib.oracle_adam_from_gbar(g.ctypes.data, g.size, P1.ctypes.data, M1.ctypes.data, V1.ctypes.data,
                                            B1.ctypes.data, out_fmt, ctypes.byref(h), t, total_sq, max_norm,
                                            int(skip_nonfinite), threads)
        if rc == 1:
            raise ValueError("oracle_adam_from_gbar: bad arguments")
        return P1, M1, V1, B1, rc == 0

    def scaler(self, scale: float = 2.0 ** 16, min_scale: float = 1.0, window: int = 1000, hysteresis: int = 2):
        return OracleScaler(scale, min_scale, window, hysteresis, 0, 0)

    def scaler_update(self, st: "OracleScaler", overflow: bool) -> bool:
        return bool(self.lib.oracle_scaler_update(ctypes.byref(st), int(overflow)))

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
