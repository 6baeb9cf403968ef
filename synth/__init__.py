"""Seeded synthetic inputs shared by the CPU oracle side and the GPU side.

This package draws numbers; it holds none of the optimizer's arithmetic.  The
host generator (``synth_host.c``) and the device generator
(``synth_dev.hip``) implement one counter-based definition (stated at the top
of ``synth_host.c``) and produce identical bits, so an element of a 140 GB
device-resident input can be redrawn on the host on its own.

Streams: every array of a workload has its own stream id (``stream_id``), and
every element is addressed by its position in that array (for ragged lists,
its position in the per-array arena).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
HOST_LIB = os.path.join(_HERE, "libsynth_host.so")
DEV_LIB = os.path.join(_HERE, "libsynth_dev.so")

# Array kinds (upper 32 bits of a stream id); the low 32 bits carry the replica rank.
KIND_P, KIND_M, KIND_V, KIND_MASK, KIND_SIZES, KIND_GRAD = 1, 2, 3, 4, 5, 16

_u64 = ctypes.c_uint64
_i64 = ctypes.c_int64
_dbl = ctypes.c_double
_int = ctypes.c_int
_vp = ctypes.c_void_p

_host = None
_dev = None


def _host_lib():
    global _host
    if _host is None:
        if not os.path.exists(HOST_LIB):
            raise ImportError(f"{HOST_LIB} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(HOST_LIB)
        lib.synth_key.restype = _u64
        lib.synth_key.argtypes = [_u64, _u64]
        lib.synth_word.restype = _u64
        lib.synth_word.argtypes = [_u64, _u64, _int]
        lib.synth_normal_f32.argtypes = [_u64, _u64, _i64, _dbl, _int, _vp]
        lib.synth_normal_f32_at.argtypes = [_u64, _vp, _i64, _dbl, _int, _vp]
        lib.synth_normal_bf16.argtypes = [_u64, _u64, _i64, _dbl, _u64, _u64, _vp]
        lib.synth_normal_bf16_at.argtypes = [_u64, _vp, _i64, _dbl, _u64, _u64, _vp]
        lib.synth_uniform_f64.argtypes = [_u64, _u64, _i64, _vp]
        _host = lib
    return _host


def _dev_lib():
    global _dev
    if _dev is None:
        import torch  # noqa: F401  (torch's HIP runtime must be the one in the process)

        if not os.path.exists(DEV_LIB):
            raise ImportError(f"{DEV_LIB} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(DEV_LIB)
        lib.synth_dev_fill_normal_f32.restype = _int
        lib.synth_dev_fill_normal_f32.argtypes = [_u64, _u64, _i64, _dbl, _int, _vp, _vp]
        lib.synth_dev_fill_normal_bf16.restype = _int
        lib.synth_dev_fill_normal_bf16.argtypes = [_u64, _u64, _i64, _dbl, _u64, _u64, _vp, _vp]
        _dev = lib
    return _dev


def stream_id(kind: int, rank: int = 0) -> int:
    return (kind << 32) | rank


def key(seed: int, kind: int, rank: int = 0) -> int:
    return int(_host_lib().synth_key(seed, stream_id(kind, rank)))


def mask_threshold(p: float) -> int:
    """Threshold t with P(word < t) = p for a uniform 64-bit word."""
    return int(p * 2.0**64) if p > 0 else 0


# ---------------------------------------------------------------- host draws
def normal_f32(k: int, offset: int, n: int, sigma: float, absval: bool = False) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    if n:
        _host_lib().synth_normal_f32(k, offset, n, sigma, int(absval), out.ctypes.data)
    return out


def normal_f32_at(k: int, idx: np.ndarray, sigma: float, absval: bool = False) -> np.ndarray:
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    out = np.empty(idx.size, dtype=np.float32)
    if idx.size:
        _host_lib().synth_normal_f32_at(k, idx.ctypes.data, idx.size, sigma, int(absval), out.ctypes.data)
    return out


def normal_bf16(k: int, offset: int, n: int, sigma: float, mask_key: int = 0, mask_thresh: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint16)
    if n:
        _host_lib().synth_normal_bf16(k, offset, n, sigma, mask_key, mask_thresh, out.ctypes.data)
    return out


def normal_bf16_at(k: int, idx: np.ndarray, sigma: float, mask_key: int = 0, mask_thresh: int = 0) -> np.ndarray:
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    out = np.empty(idx.size, dtype=np.uint16)
    if idx.size:
        _host_lib().synth_normal_bf16_at(k, idx.ctypes.data, idx.size, sigma, mask_key, mask_thresh,
                                         out.ctypes.data)
    return out


def uniform_f64(k: int, offset: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.float64)
    if n:
        _host_lib().synth_uniform_f64(k, offset, n, out.ctypes.data)
    return out


# -------------------------------------------------------------- device fills
def _stream_ptr(stream):
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def dev_fill_normal_f32(t, k: int, offset: int, sigma: float, absval: bool = False, stream=None) -> None:
    import torch

    assert t.dtype == torch.float32 and t.is_cuda and t.is_contiguous()
    rc = _dev_lib().synth_dev_fill_normal_f32(k, offset, t.numel(), sigma, int(absval), t.data_ptr(),
                                              _stream_ptr(stream))
    if rc:
        raise RuntimeError(f"synth_dev_fill_normal_f32 failed: hip error {rc}")


def dev_fill_normal_bf16(t, k: int, offset: int, sigma: float, mask_key: int = 0, mask_thresh: int = 0,
                         stream=None) -> None:
    import torch

    assert t.dtype in (torch.bfloat16, torch.int16, torch.uint16) and t.is_cuda and t.is_contiguous()
    rc = _dev_lib().synth_dev_fill_normal_bf16(k, offset, t.numel(), sigma, mask_key, mask_thresh, t.data_ptr(),
                                               _stream_ptr(stream))
    if rc:
        raise RuntimeError(f"synth_dev_fill_normal_bf16 failed: hip error {rc}")
