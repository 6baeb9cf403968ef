"""Python binding of libzshard (see include/zshard.h for the contract).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libzshard.so``.  PyTorch supplies device memory and streams.
Importing this module fails if the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libzshard.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                      "(there is no fallback implementation)")

# PyTorch-ROCm ships its own HIP runtime (same soname).  Load it first so the
# library binds to the runtime that owns torch's devices, streams and memory;
# loading the library first would bring in a second runtime.
import numpy as np  # noqa: E402
import torch  # noqa: E402

_lib = ctypes.CDLL(LIB_PATH)

ZS_MAX_REPLICAS = 256
STATUS = {0: "ZS_OK", 1: "ZS_ERR_NULL", 2: "ZS_ERR_RANGE", 3: "ZS_ERR_ALIAS", 4: "ZS_ERR_ALIGN", 5: "ZS_ERR_HIP",
          6: "ZS_ERR_NOMEM"}


class AdamHPStruct(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("beta1", ctypes.c_double), ("beta2", ctypes.c_double),
                ("eps", ctypes.c_double), ("weight_decay", ctypes.c_double)]


class FoldedStruct(ctypes.Structure):
    _fields_ = [(k, ctypes.c_float) for k in ("b1", "c1", "b2", "c2", "eps", "ss", "rb", "dk")]


class TensorStruct(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int64), ("master", ctypes.c_void_p), ("m", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("param_bf16", ctypes.c_void_p), ("grad_chunks", ctypes.POINTER(ctypes.c_void_p))]


_vp, _i32, _i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64


class StepSourceStruct(ctypes.Structure):
    _fields_ = [("table", ctypes.c_void_p), ("t0", ctypes.c_int64), ("count", ctypes.c_int64),
                ("step", ctypes.c_void_p), ("status", ctypes.c_void_p)]


_lib.zs_abi_version.restype = ctypes.c_int
_lib.zs_status_string.restype = ctypes.c_char_p
_lib.zs_status_string.argtypes = [ctypes.c_int]
_lib.zs_last_error.restype = ctypes.c_char_p
_lib.zs_fold.restype = ctypes.c_int
_lib.zs_fold.argtypes = [ctypes.POINTER(AdamHPStruct), _i64, ctypes.POINTER(FoldedStruct)]
_lib.zs_reduce_adam_flat.restype = ctypes.c_int
_lib.zs_reduce_adam_flat.argtypes = [ctypes.POINTER(_vp), _i32, _i64, _vp, _vp, _vp, _vp,
                                     ctypes.POINTER(AdamHPStruct), _i64, _vp]
_lib.zs_list_plan_create.restype = ctypes.c_int
_lib.zs_list_plan_create.argtypes = [ctypes.POINTER(TensorStruct), _i32, _i32, _vp, ctypes.POINTER(_vp)]
_lib.zs_reduce_adam_list_plan.restype = ctypes.c_int
_lib.zs_reduce_adam_list_plan.argtypes = [_vp, ctypes.POINTER(AdamHPStruct), _i64, _vp]
_lib.zs_reduce_adam_list.restype = ctypes.c_int
_lib.zs_reduce_adam_list.argtypes = [ctypes.POINTER(TensorStruct), _i32, _i32, ctypes.POINTER(AdamHPStruct), _i64,
                                     _vp]
_lib.zs_reduce_adam_list_static.restype = ctypes.c_int
_lib.zs_reduce_adam_list_static.argtypes = [ctypes.POINTER(TensorStruct), _i32, _i32, ctypes.POINTER(AdamHPStruct),
                                            _i64, _vp]
_lib.zs_list_plan_destroy.restype = None
_lib.zs_list_plan_destroy.argtypes = [_vp]
_lib.zs_list_plan_set_groups.restype = ctypes.c_int
_lib.zs_list_plan_set_groups.argtypes = [_vp, ctypes.POINTER(_i32), _i32, _vp]
_lib.zs_reduce_adam_list_plan_groups.restype = ctypes.c_int
_lib.zs_reduce_adam_list_plan_groups.argtypes = [_vp, ctypes.POINTER(AdamHPStruct), _i32, _i64, _vp]
_lib.zs_list_plan_info.restype = ctypes.c_int
_lib.zs_list_plan_info.argtypes = [_vp, ctypes.POINTER(_i64), ctypes.POINTER(_i32), ctypes.POINTER(_i32)]
_lib.zs_fold_table.restype = ctypes.c_int
_lib.zs_fold_table.argtypes = [ctypes.POINTER(AdamHPStruct), _i64, _i64, _vp]
_lib.zs_reduce_adam_flat_devstep.restype = ctypes.c_int
_lib.zs_reduce_adam_flat_devstep.argtypes = [ctypes.POINTER(_vp), _i32, _i64, _vp, _vp, _vp, _vp,
                                             ctypes.POINTER(StepSourceStruct), _vp]
_lib.zs_reduce_adam_list_plan_devstep.restype = ctypes.c_int
_lib.zs_reduce_adam_list_plan_devstep.argtypes = [_vp, ctypes.POINTER(StepSourceStruct), _vp]
_lib.zs_step_advance.restype = ctypes.c_int
_lib.zs_step_advance.argtypes = [_vp, _vp]
_lib.zs_set_grid_blocks.restype = ctypes.c_int
_lib.zs_set_grid_blocks.argtypes = [_i32]
_lib.zs_set_launch_bytes.restype = ctypes.c_int
_lib.zs_set_launch_bytes.argtypes = [ctypes.c_int64]
_lib.zs_launch_bytes.restype = ctypes.c_int64
_lib.zs_launch_bytes.argtypes = []
_lib.zs_set_write_window.restype = ctypes.c_int
_lib.zs_set_write_window.argtypes = [_i32, _i32]
_lib.zs_write_window.restype = ctypes.c_int
_lib.zs_write_window.argtypes = [_i32, _i32, _i64, ctypes.POINTER(_i32), ctypes.POINTER(_i32)]
WINDOW_KERNELS = {"flat": 0, "reduce": 1, "list": 2}
_lib.zs_set_flat_schedule.restype = ctypes.c_int
_lib.zs_set_flat_schedule.argtypes = [_i32]
_lib.zs_flat_schedule.restype = ctypes.c_int
_lib.zs_flat_schedule.argtypes = [_i32, _i64, ctypes.POINTER(_i32)]
_lib.zs_reduce_schedule.restype = ctypes.c_int
_lib.zs_reduce_schedule.argtypes = [_i32, _i64, ctypes.POINTER(_i32)]
_lib.zs_list_schedule.restype = ctypes.c_int
_lib.zs_list_schedule.argtypes = [ctypes.POINTER(TensorStruct), _i32, _i32, ctypes.POINTER(_i32)]
_lib.zs_set_phased_max_polls.restype = ctypes.c_int
_lib.zs_set_phased_max_polls.argtypes = [_i32]
SCHEDULES = {"auto": 0, "stream": 1, "windowed": 2, "phased": 3}
_lib.zs_two_pass_workspace_bytes.restype = ctypes.c_size_t
_lib.zs_two_pass_workspace_bytes.argtypes = [_i64]
_lib.zs_reduce_grads_flat.restype = ctypes.c_int
_lib.zs_reduce_grads_flat.argtypes = [ctypes.POINTER(_vp), _i32, _i64, _i32, ctypes.c_double, _vp, ctypes.c_size_t,
                                      _vp, _vp]
_lib.zs_adam_from_grads_flat_devstep.restype = ctypes.c_int
_lib.zs_adam_from_grads_flat_devstep.argtypes = [_vp, ctypes.c_size_t, _i64, _vp, _vp, _vp, _vp, _i32,
                                                 ctypes.POINTER(StepSourceStruct), _vp, ctypes.c_double, _i32, _vp]
_lib.zs_adam_from_grads_flat.restype = ctypes.c_int
_lib.zs_adam_from_grads_flat.argtypes = [_vp, ctypes.c_size_t, _i64, _vp, _vp, _vp, _vp, _i32,
                                         ctypes.POINTER(AdamHPStruct), _i64, _vp, ctypes.c_double, _i32, _vp]


class LossScalerStruct(ctypes.Structure):
    _fields_ = [("scale", ctypes.c_double), ("min_scale", ctypes.c_double), ("window", ctypes.c_int64),
                ("hysteresis", ctypes.c_int64), ("overflows", ctypes.c_int64), ("clean", ctypes.c_int64)]


_lib.zs_loss_scaler_init.restype = ctypes.c_int
_lib.zs_loss_scaler_init.argtypes = [ctypes.POINTER(LossScalerStruct), ctypes.c_double, ctypes.c_double, _i64, _i64]
_lib.zs_loss_scaler_update.restype = _i32
_lib.zs_loss_scaler_update.argtypes = [ctypes.POINTER(LossScalerStruct), _i32]
_lib.zs_loss_scaler_update_device.restype = ctypes.c_int
_lib.zs_loss_scaler_update_device.argtypes = [_vp, _vp, _vp, _vp]
_lib.zs_reduce_grads_flat_device_scale.restype = ctypes.c_int
_lib.zs_reduce_grads_flat_device_scale.argtypes = [ctypes.POINTER(_vp), _i32, _i64, _i32, _vp, _vp, ctypes.c_size_t,
                                                   _vp, _vp]

_lib.zs_offload_create.restype = ctypes.c_int
_lib.zs_offload_create.argtypes = [_i64, _i32, ctypes.POINTER(_vp)]
_lib.zs_offload_step_flat.restype = ctypes.c_int
_lib.zs_offload_step_flat.argtypes = [_vp, ctypes.POINTER(_vp), _i32, _i64, _vp, _vp, _vp, _vp,
                                      ctypes.POINTER(AdamHPStruct), _i64, _vp]
_lib.zs_offload_destroy.restype = None
_lib.zs_offload_destroy.argtypes = [_vp]
_lib.zs_cpu_adam.restype = ctypes.c_int
_lib.zs_cpu_adam.argtypes = [_vp, _i64, _vp, _vp, _vp, _vp, ctypes.POINTER(AdamHPStruct), _i64, _i32]

FORMATS = {"bf16": 0, "fp16": 1}


class ZShardError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        self.name = STATUS.get(status, f"status {status}")
        detail = _lib.zs_last_error().decode(errors="replace")
        super().__init__(f"{where}: {self.name}: {detail}")


def _check(status: int, where: str) -> None:
    if status != 0:
        raise ZShardError(status, where)


@dataclass(frozen=True)
class AdamHP:
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.0

    def _c(self) -> AdamHPStruct:
        return AdamHPStruct(self.lr, self.beta1, self.beta2, self.eps, self.weight_decay)


def _hp(hp) -> AdamHPStruct:
    if isinstance(hp, AdamHP):
        return hp._c()
    if isinstance(hp, dict):
        return AdamHP(**hp)._c()
    raise TypeError("hp must be an AdamHP or a dict of lr, beta1, beta2, eps, weight_decay")


def abi_version() -> int:
    return int(_lib.zs_abi_version())


def fold(hp, step: int) -> dict:
    """The fp32 scalars the step uses (computed on the host, no GPU needed)."""
    out = FoldedStruct()
    h = _hp(hp)
    _check(_lib.zs_fold(ctypes.byref(h), step, ctypes.byref(out)), "zs_fold")
    return {k: getattr(out, k) for k, _ in FoldedStruct._fields_}


def set_grid_blocks(blocks: int) -> None:
    _check(_lib.zs_set_grid_blocks(blocks), "zs_set_grid_blocks")


def set_launch_bytes(nbytes: int) -> None:
    """Most algorithmic bytes per launch of the one-tile-per-workgroup kernels (0 = library default);
    see zs_set_launch_bytes."""
    _check(_lib.zs_set_launch_bytes(nbytes), "zs_set_launch_bytes")


def launch_bytes() -> int:
    """The per-launch byte limit in force."""
    return int(_lib.zs_launch_bytes())


def set_write_window(period_ticks: int, open_ticks: int = 0) -> None:
    """Write windows of the flat step (0 = library default, 1 = off); see zs_set_write_window."""
    _check(_lib.zs_set_write_window(period_ticks, open_ticks), "zs_set_write_window")


def write_window(kernel: str, N: int, n: int):
    """(period_ticks, open_ticks) that the flat step (kernel="flat"), pass 1 of the two-pass form
    (kernel="reduce") or a list plan (kernel="list", n parameters in all) takes for N replicas on n
    parameters; (0, 0) = no windows."""
    p, o = _i32(), _i32()
    _check(_lib.zs_write_window(WINDOW_KERNELS[kernel], N, n, ctypes.byref(p), ctypes.byref(o)), "zs_write_window")
    return p.value, o.value


def set_flat_schedule(schedule) -> None:
    """How the flat step schedules its reads and writes: "auto" (the default), "stream", "windowed" or
    "phased" (or the ZS_SCHEDULE_* value); see zs_set_flat_schedule.  Results do not depend on it."""
    _check(_lib.zs_set_flat_schedule(SCHEDULES[schedule] if isinstance(schedule, str) else int(schedule)),
           "zs_set_flat_schedule")


def flat_schedule(N: int, n: int) -> str:
    """The schedule ("stream", "windowed" or "phased") a flat step for N replicas on n parameters takes."""
    out = _i32()
    _check(_lib.zs_flat_schedule(N, n, ctypes.byref(out)), "zs_flat_schedule")
    return {v: k for k, v in SCHEDULES.items()}[out.value]


def reduce_schedule(N: int, n: int) -> str:
    """The schedule ("stream", "windowed" or "phased") pass 1 of the two-pass form takes for N replicas
    on n parameters."""
    out = _i32()
    _check(_lib.zs_reduce_schedule(N, n, ctypes.byref(out)), "zs_reduce_schedule")
    return {v: k for k, v in SCHEDULES.items()}[out.value]


def list_schedule(sizes, N: int, offsets=None) -> str:
    """The schedule ("stream", "windowed" or "phased") a list plan over tensors of these sizes takes with N
    replicas: the tensors in per-array arenas at ``offsets`` (by default back to back on 8-element
    boundaries), each arena on a 2 MiB boundary, as the caching allocator places large blocks.  No GPU
    call: the addresses only stand for their alignment."""
    sizes = np.asarray(sizes, dtype=np.int64)
    if offsets is None:
        padded = (sizes + 7) // 8 * 8
        offsets = np.concatenate([[0], np.cumsum(padded)[:-1]]) if sizes.size else sizes
    offsets = np.asarray(offsets, dtype=np.int64)
    L = int((offsets + sizes).max()) if sizes.size else 0
    step2 = -(-max(L, 1) * 4 // (1 << 21)) * (1 << 21)   # every arena's span, 2 MiB-rounded
    base = 1 << 40
    rec, gtab = _arena_records(sizes, offsets, [base + step2 * (4 + r) for r in range(N)], base, base + step2,
                               base + 2 * step2, base + 3 * step2)
    out = _i32()
    _check(_lib.zs_list_schedule(ctypes.cast(rec.ctypes.data, ctypes.POINTER(TensorStruct)), sizes.size, N,
                                 ctypes.byref(out)), "zs_list_schedule")
    del gtab
    return {v: k for k, v in SCHEDULES.items()}[out.value]


def set_phased_max_polls(polls: int) -> None:
    """The longest wait at a grid barrier of the phased schedule, in polls of about 50 ns (0 = default)."""
    _check(_lib.zs_set_phased_max_polls(polls), "zs_set_phased_max_polls")


def _stream_handle(stream, device=None):
    """The raw stream handle: torch's current stream of ``device`` by default."""
    if stream is None:
        return torch.cuda.current_stream(device).cuda_stream
    if isinstance(stream, int):
        return stream
    if device is not None and getattr(stream, "device", device) != device:
        raise ValueError(f"stream is on {stream.device}, the tensors on {device}")
    return stream.cuda_stream


def _one_device(*tensors):
    """The device every tensor lives on (the current device if there are none).
    The library launches on the current device, so each call runs with this
    device made current; tensors spread over devices are rejected."""
    devs = {t.device for t in tensors}
    if len(devs) > 1:
        raise ValueError(f"tensors live on several devices: {sorted(str(d) for d in devs)}")
    return devs.pop() if devs else torch.device("cuda", torch.cuda.current_device())


def _dev_check(t, dtypes, name):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


# Accepted dtypes: 16-bit arrays are passed as raw bits, so integer views of them are accepted too.
_BF16 = (torch.bfloat16, torch.int16, torch.uint16)
_HALF = (torch.bfloat16, torch.float16, torch.int16, torch.uint16)
_F32 = (torch.float32,)


def _tensor_args(grads, master, m, v, param):
    n = master.numel()
    _dev_check(master, _F32, "master")
    _dev_check(m, _F32, "m")
    _dev_check(v, _F32, "v")
    _dev_check(param, _BF16, "param")
    for name, t in (("m", m), ("v", v), ("param", param)):
        if t.numel() != n:
            raise ValueError(f"{name} has {t.numel()} elements, master has {n}")
    for r, g in enumerate(grads):
        _dev_check(g, _BF16, f"grads[{r}]")
        if g.numel() != n:
            raise ValueError(f"grads[{r}] has {g.numel()} elements, master has {n}")
    return n


def reduce_adam_flat(grads: Sequence, master, m, v, param, hp, step: int, stream=None) -> None:
    """One shard step: average ``grads`` (N bf16 device tensors, rank order) and
    apply AdamW to ``master``/``m``/``v`` in place, writing the bf16 copy to
    ``param``.  Enqueued on ``stream`` (default: torch's current stream)."""
    N = len(grads)
    n = _tensor_args(grads, master, m, v, param)
    dev = _one_device(master, m, v, param, *grads)
    tab = (_vp * max(N, 1))(*[g.data_ptr() for g in grads])
    h = _hp(hp)
    with torch.cuda.device(dev):
        _check(_lib.zs_reduce_adam_flat(tab, N, n, master.data_ptr(), m.data_ptr(), v.data_ptr(), param.data_ptr(),
                                        ctypes.byref(h), step, _stream_handle(stream, dev)), "zs_reduce_adam_flat")


def reduce_adam_flat_ptrs(grad_ptrs: Sequence[int], n: int, master: int, m: int, v: int, param: int, hp,
                          step: int, stream) -> None:
    """Raw-pointer form of :func:`reduce_adam_flat` (device addresses as ints,
    all on the current device)."""
    N = len(grad_ptrs)
    tab = (_vp * max(N, 1))(*grad_ptrs)
    h = _hp(hp)
    _check(_lib.zs_reduce_adam_flat(tab, N, n, master, m, v, param, ctypes.byref(h), step, _stream_handle(stream)),
           "zs_reduce_adam_flat")


class FlatStep:
    """:func:`reduce_adam_flat` on fixed tensors, prepared once: the argument
    checks, the device and the replica pointer table are done at construction,
    so a call only packs the hyperparameters (kept while the same frozen
    :class:`AdamHP` comes back; a dict is packed on every call, since it may
    have changed) and enqueues the step.  For small shards, where the per-call
    checks cost more than the device time.  The object holds references to the
    tensors; it reads their addresses once, so re-pointing a tensor at new
    storage (``Tensor.set_``) after construction is not seen.  ``stream`` fixed
    here (a torch stream or a raw handle) saves looking up torch's current
    stream on every call."""

    def __init__(self, grads: Sequence, master, m, v, param, stream=None):
        self._tensors = (tuple(grads), master, m, v, param)
        self._N = len(grads)
        self._n = _tensor_args(grads, master, m, v, param)
        self._dev = _one_device(master, m, v, param, *grads)
        self._dev_index = self._dev.index if self._dev.index is not None else torch.cuda.current_device()
        self._tab = (_vp * max(self._N, 1))(*[g.data_ptr() for g in grads])
        self._ptrs = (master.data_ptr(), m.data_ptr(), v.data_ptr(), param.data_ptr())
        self._stream = None if stream is None else _stream_handle(stream, self._dev)
        self._hp_obj = None
        self._hp = None

    def __call__(self, hp, step: int, stream=None) -> None:
        if hp is not self._hp_obj:
            self._hp = _hp(hp)
            self._hp_obj = hp if isinstance(hp, AdamHP) else None
        if stream is not None:
            s = _stream_handle(stream, self._dev)
        elif self._stream is not None:
            s = self._stream
        else:
            s = torch.cuda.current_stream(self._dev).cuda_stream
        args = (self._tab, self._N, self._n, *self._ptrs, ctypes.byref(self._hp), step, s)
        if torch.cuda.current_device() == self._dev_index:
            st = _lib.zs_reduce_adam_flat(*args)
        else:
            with torch.cuda.device(self._dev):
                st = _lib.zs_reduce_adam_flat(*args)
        _check(st, "zs_reduce_adam_flat")


# ------------------------------------------------------------ device-resident step index
def fold_table(hp, t0: int, count: int):
    """The folded scalars of steps t0 .. t0+count-1: a (count, 8) float32 array, rows as :func:`fold`."""
    out = np.empty((count, 8), dtype=np.float32)
    h = _hp(hp)
    _check(_lib.zs_fold_table(ctypes.byref(h), t0, count, out.ctypes.data), "zs_fold_table")
    return out


class StepSource:
    """A device-resident step index with the folded scalars of steps
    t0 .. t0+count-1, for steps captured in a HIP graph: the *_devstep calls
    read the current step on the device and :meth:`advance` increments it
    there, so each replay takes the next step."""

    def __init__(self, hp, t0: int, count: int, device="cuda", start: Optional[int] = None):
        self.table = torch.from_numpy(fold_table(hp, t0, count)).to(device)
        self.step_t = torch.tensor([t0 if start is None else start], dtype=torch.int64, device=device)
        self.status_t = torch.zeros(1, dtype=torch.int32, device=device)
        self.device = self.table.device
        self._s = StepSourceStruct(self.table.data_ptr(), t0, count, self.step_t.data_ptr(),
                                   self.status_t.data_ptr())

    def advance(self, stream=None) -> None:
        with torch.cuda.device(self.device):
            _check(_lib.zs_step_advance(self.step_t.data_ptr(), _stream_handle(stream, self.device)),
                   "zs_step_advance")

    @property
    def step(self) -> int:
        return int(self.step_t.item())

    @property
    def status(self) -> int:
        return int(self.status_t.item())


def reduce_adam_flat_devstep(grads: Sequence, master, m, v, param, src: StepSource, stream=None) -> None:
    """:func:`reduce_adam_flat` with the step (and its folded scalars) read from ``src`` on the device."""
    N = len(grads)
    n = _tensor_args(grads, master, m, v, param)
    dev = _one_device(master, m, v, param, src.table, *grads)
    tab = (_vp * max(N, 1))(*[g.data_ptr() for g in grads])
    with torch.cuda.device(dev):
        _check(_lib.zs_reduce_adam_flat_devstep(tab, N, n, master.data_ptr(), m.data_ptr(), v.data_ptr(),
                                                param.data_ptr(), ctypes.byref(src._s), _stream_handle(stream, dev)),
               "zs_reduce_adam_flat_devstep")


@dataclass
class ShardTensor:
    """One tensor of a ragged list: its replicas' grads and its state."""
    grads: Sequence
    master: object
    m: object
    v: object
    param: object


def _tensor_table(tensors: Sequence[ShardTensor], N: int):
    _one_device(*[x for t in tensors for x in (t.master, t.m, t.v, t.param, *t.grads)])
    keep = []
    tab = (TensorStruct * max(len(tensors), 1))()
    for i, t in enumerate(tensors):
        if len(t.grads) != N:
            raise ValueError(f"tensor {i} has {len(t.grads)} grads, expected N={N}")
        n = _tensor_args(t.grads, t.master, t.m, t.v, t.param)
        g = (_vp * N)(*[x.data_ptr() for x in t.grads])
        keep.append(g)
        tab[i] = TensorStruct(n, t.master.data_ptr(), t.m.data_ptr(), t.v.data_ptr(), t.param.data_ptr(),
                              ctypes.cast(g, ctypes.POINTER(_vp)))
    return tab, keep


def _arena_records(sizes, offsets, gbases, pbase, mbase, vbase, bbase):
    """zs_tensor records (and the replica-pointer table they point into, which the caller keeps alive) for
    tensors at ``offsets`` of arenas starting at the given addresses."""
    T, N = sizes.size, len(gbases)
    gtab = np.empty((max(T, 1), N), dtype=np.uint64)
    for r, gb in enumerate(gbases):
        gtab[:T, r] = np.uint64(gb) + (offsets * 2).astype(np.uint64)
    rec = np.zeros((max(T, 1), 6), dtype=np.uint64)
    rec[:T, 0] = sizes.astype(np.uint64)
    rec[:T, 1] = np.uint64(pbase) + (offsets * 4).astype(np.uint64)
    rec[:T, 2] = np.uint64(mbase) + (offsets * 4).astype(np.uint64)
    rec[:T, 3] = np.uint64(vbase) + (offsets * 4).astype(np.uint64)
    rec[:T, 4] = np.uint64(bbase) + (offsets * 2).astype(np.uint64)
    rec[:T, 5] = np.uint64(gtab.ctypes.data) + np.arange(max(T, 1), dtype=np.uint64) * np.uint64(8 * N)
    assert ctypes.sizeof(TensorStruct) == 48
    return rec, gtab


class ListPlan:
    """A device-resident chunk table for a fixed ragged list of tensors; each
    :meth:`step` is one kernel covering every tensor (in consecutive launches of a few GB each on long
    lists; see zs_set_launch_bytes)."""

    def __init__(self, tensors: Sequence[ShardTensor], N: int, stream=None):
        tab, keep = _tensor_table(tensors, N)
        dev = _one_device(*[t.master for t in tensors])
        h = _vp()
        with torch.cuda.device(dev):
            _check(_lib.zs_list_plan_create(tab, len(tensors), N, _stream_handle(stream, dev), ctypes.byref(h)),
                   "zs_list_plan_create")
        self._h = h
        self._dev = dev
        self.N = N
        self._tensors = list(tensors)   # the plan holds their addresses: keep them alive

    @classmethod
    def from_arenas(cls, sizes, offsets, grads: Sequence, master, m, v, param, stream=None) -> "ListPlan":
        """Plan over tensors laid out in per-array arenas: tensor t is elements
        [offsets[t], offsets[t] + sizes[t]) of ``master``, ``m``, ``v``, ``param``
        and of every replica's gradient arena in ``grads``."""
        N = len(grads)
        L = master.numel()
        _tensor_args(grads, master, m, v, param)
        dev = _one_device(master, m, v, param, *grads)
        sizes = np.asarray(sizes, dtype=np.int64)
        offsets = np.asarray(offsets, dtype=np.int64)
        if sizes.shape != offsets.shape or (sizes.size and (offsets.min() < 0 or (offsets + sizes).max() > L)):
            raise ValueError("tensor ranges must lie inside the arenas")
        T = sizes.size
        rec, gtab = _arena_records(sizes, offsets, [g.data_ptr() for g in grads], master.data_ptr(), m.data_ptr(),
                                   v.data_ptr(), param.data_ptr())
        self = cls.__new__(cls)
        h = _vp()
        with torch.cuda.device(dev):
            _check(_lib.zs_list_plan_create(ctypes.cast(rec.ctypes.data, ctypes.POINTER(TensorStruct)), T, N,
                                            _stream_handle(stream, dev), ctypes.byref(h)), "zs_list_plan_create")
        self._h = h
        self._dev = dev
        self.N = N
        self._tensors = [grads, master, m, v, param]
        return self

    def step(self, hp, step: int, stream=None) -> None:
        if not self._h:
            raise ValueError("plan is closed")
        h = _hp(hp)
        with torch.cuda.device(self._dev):
            _check(_lib.zs_reduce_adam_list_plan(self._h, ctypes.byref(h), step, _stream_handle(stream, self._dev)),
                   "zs_reduce_adam_list_plan")

    def set_groups(self, groups: Sequence[int], n_groups: int, stream=None) -> None:
        """Assign tensor t to hyperparameter group groups[t] (0 <= groups[t] < n_groups <= 8)."""
        if not self._h:
            raise ValueError("plan is closed")
        arr = (_i32 * max(len(groups), 1))(*groups)
        with torch.cuda.device(self._dev):
            _check(_lib.zs_list_plan_set_groups(self._h, arr, n_groups, _stream_handle(stream, self._dev)),
                   "zs_list_plan_set_groups")

    def step_devstep(self, src: "StepSource", stream=None) -> None:
        """The step with the step index read from ``src`` on the device."""
        if not self._h:
            raise ValueError("plan is closed")
        if src.device != self._dev:
            raise ValueError(f"the step source is on {src.device}, the plan on {self._dev}")
        with torch.cuda.device(self._dev):
            _check(_lib.zs_reduce_adam_list_plan_devstep(self._h, ctypes.byref(src._s),
                                                         _stream_handle(stream, self._dev)),
                   "zs_reduce_adam_list_plan_devstep")

    def step_groups(self, hps: Sequence, step: int, stream=None) -> None:
        """The step with hps[g] for the tensors of group g."""
        if not self._h:
            raise ValueError("plan is closed")
        arr = (AdamHPStruct * max(len(hps), 1))(*[_hp(h) for h in hps])
        with torch.cuda.device(self._dev):
            _check(_lib.zs_reduce_adam_list_plan_groups(self._h, arr, len(hps), step,
                                                        _stream_handle(stream, self._dev)),
                   "zs_reduce_adam_list_plan_groups")

    def info(self) -> dict:
        n, t, c = _i64(), _i32(), _i32()
        _check(_lib.zs_list_plan_info(self._h, ctypes.byref(n), ctypes.byref(t), ctypes.byref(c)),
               "zs_list_plan_info")
        return dict(n_params=n.value, n_tensors=t.value, n_items=c.value)

    def close(self) -> None:
        if self._h:
            _lib.zs_list_plan_destroy(self._h)
            self._h = _vp()
            self._tensors = []

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def reduce_adam_list(tensors: Sequence[ShardTensor], N: int, hp, step: int, stream=None) -> None:
    """One-shot list step (builds a plan, runs it, waits, frees it)."""
    tab, keep = _tensor_table(tensors, N)
    dev = _one_device(*[t.master for t in tensors])
    h = _hp(hp)
    with torch.cuda.device(dev):
        _check(_lib.zs_reduce_adam_list(tab, len(tensors), N, ctypes.byref(h), step, _stream_handle(stream, dev)),
               "zs_reduce_adam_list")


def reduce_adam_list_static(tensors: Sequence[ShardTensor], N: int, hp, step: int, stream=None) -> None:
    """:func:`reduce_adam_list` with its table in the library's fixed device array (no device
    allocation; see zs_reduce_adam_list_static for the size limit and the sharing rule)."""
    tab, keep = _tensor_table(tensors, N)
    dev = _one_device(*[t.master for t in tensors])
    h = _hp(hp)
    with torch.cuda.device(dev):
        _check(_lib.zs_reduce_adam_list_static(tab, len(tensors), N, ctypes.byref(h), step,
                                               _stream_handle(stream, dev)), "zs_reduce_adam_list_static")


# ------------------------------------------------------------ two-pass form
def two_pass_workspace_bytes(n: int) -> int:
    return int(_lib.zs_two_pass_workspace_bytes(n))


def _fmt(name) -> int:
    if isinstance(name, int):
        return name
    return FORMATS[name]


_WORKSPACE_TYPES = (torch.uint8, torch.int8, torch.float32, torch.float64)


def _pass1_args(grads, workspace, sqnorm) -> int:
    n = grads[0].numel() if grads else 0
    for r, g in enumerate(grads):
        _dev_check(g, _HALF, f"grads[{r}]")
        if g.numel() != n:
            raise ValueError(f"grads[{r}] has {g.numel()} elements, grads[0] has {n}")
    _dev_check(workspace, _WORKSPACE_TYPES, "workspace")
    _dev_check(sqnorm, (torch.float64,), "sqnorm")
    return n


def _pass2_args(workspace, n, master, m, v, param, total_sq) -> None:
    _dev_check(master, _F32, "master")
    _dev_check(m, _F32, "m")
    _dev_check(v, _F32, "v")
    _dev_check(param, _HALF, "param")
    _dev_check(total_sq, (torch.float64,), "total_sq")
    _dev_check(workspace, _WORKSPACE_TYPES, "workspace")
    for name, t in (("master", master), ("m", m), ("v", v), ("param", param)):
        if t.numel() != n:
            raise ValueError(f"{name} has {t.numel()} elements, expected {n}")


def reduce_grads_flat(grads: Sequence, workspace, sqnorm, loss_scale: float = 1.0, grad_format="bf16",
                      stream=None) -> None:
    """Pass 1: average (and unscale) the replicas into ``workspace`` and write the
    shard's squared gradient norm to ``sqnorm`` (a 1-element float64 device tensor)."""
    N = len(grads)
    n = _pass1_args(grads, workspace, sqnorm)
    dev = _one_device(workspace, sqnorm, *grads)
    tab = (_vp * max(N, 1))(*[g.data_ptr() for g in grads])
    with torch.cuda.device(dev):
        _check(_lib.zs_reduce_grads_flat(tab, N, n, _fmt(grad_format), loss_scale, workspace.data_ptr(),
                                         workspace.numel() * workspace.element_size(), sqnorm.data_ptr(),
                                         _stream_handle(stream, dev)), "zs_reduce_grads_flat")


def adam_from_grads_flat(workspace, n: int, master, m, v, param, hp, step: int, total_sq, max_norm: float = 0.0,
                         param_format="bf16", skip_nonfinite: bool = True, stream=None) -> None:
    """Pass 2: AdamW from the reduced gradient in ``workspace``, clipped to
    ``max_norm`` by the global squared norm ``total_sq`` (device float64), and
    skipped entirely when that norm is not finite."""
    _pass2_args(workspace, n, master, m, v, param, total_sq)
    dev = _one_device(workspace, master, m, v, param, total_sq)
    h = _hp(hp)
    with torch.cuda.device(dev):
        _check(_lib.zs_adam_from_grads_flat(workspace.data_ptr(), workspace.numel() * workspace.element_size(), n,
                                            master.data_ptr(), m.data_ptr(), v.data_ptr(), param.data_ptr(),
                                            _fmt(param_format), ctypes.byref(h), step, total_sq.data_ptr(), max_norm,
                                            int(skip_nonfinite), _stream_handle(stream, dev)),
               "zs_adam_from_grads_flat")


def adam_from_grads_flat_devstep(workspace, n: int, master, m, v, param, src: StepSource, total_sq,
                                 max_norm: float = 0.0, param_format="bf16", skip_nonfinite: bool = True,
                                 stream=None) -> None:
    """:func:`adam_from_grads_flat` with the step read from ``src`` on the device."""
    _pass2_args(workspace, n, master, m, v, param, total_sq)
    dev = _one_device(workspace, master, m, v, param, total_sq, src.table)
    with torch.cuda.device(dev):
        _check(_lib.zs_adam_from_grads_flat_devstep(workspace.data_ptr(),
                                                    workspace.numel() * workspace.element_size(), n,
                                                    master.data_ptr(), m.data_ptr(), v.data_ptr(), param.data_ptr(),
                                                    _fmt(param_format), ctypes.byref(src._s), total_sq.data_ptr(),
                                                    max_norm, int(skip_nonfinite), _stream_handle(stream, dev)),
               "zs_adam_from_grads_flat_devstep")


def clipped_step_flat(grads: Sequence, master, m, v, param, hp, step: int, max_norm: float = 0.0,
                      loss_scale: float = 1.0, grad_format="bf16", param_format="bf16", workspace=None,
                      sqnorm=None, stream=None):
    """Both passes on one shard, the shard's own norm standing for the global
    one (one GPU).  Returns the device tensor holding the squared norm: a
    non-finite value means the step was skipped (an fp16 overflow)."""
    n = master.numel()
    own = []  # buffers allocated here: torch's allocator must not hand them out before `stream` is done
    if workspace is None:
        workspace = torch.empty(two_pass_workspace_bytes(n), dtype=torch.uint8, device=master.device)
        own.append(workspace)
    if sqnorm is None:
        sqnorm = torch.empty(1, dtype=torch.float64, device=master.device)
        own.append(sqnorm)
    reduce_grads_flat(grads, workspace, sqnorm, loss_scale, grad_format, stream)
    adam_from_grads_flat(workspace, n, master, m, v, param, hp, step, sqnorm, max_norm, param_format, True, stream)
    if stream is not None and own:
        # the allocations were made on torch's current stream, the work runs on `stream`: tie their reuse
        # to `stream` so a later allocation cannot take them while either pass is still queued there
        ts = stream if isinstance(stream, torch.cuda.Stream) else \
            torch.cuda.ExternalStream(stream, device=master.device)
        for t in own:
            t.record_stream(ts)
    return sqnorm


class LossScaler:
    """Dynamic loss scale for fp16 training: doubles after `window` clean steps;
    an overflow halves it (not below `min_scale`) once `hysteresis` overflows
    have been counted since the last growth (see zs_loss_scaler_update)."""

    def __init__(self, initial_scale: float = 2.0 ** 16, min_scale: float = 1.0, window: int = 1000,
                 hysteresis: int = 2):
        self._s = LossScalerStruct()
        _check(_lib.zs_loss_scaler_init(ctypes.byref(self._s), initial_scale, min_scale, window, hysteresis),
               "zs_loss_scaler_init")

    @property
    def scale(self) -> float:
        return self._s.scale

    def update(self, overflow: bool) -> bool:
        """Record a step; returns True if the step was taken."""
        return bool(_lib.zs_loss_scaler_update(ctypes.byref(self._s), int(overflow)))

    def state(self) -> dict:
        return {k: getattr(self._s, k) for k, _ in LossScalerStruct._fields_}

    def to_device(self, device="cuda") -> "DeviceLossScaler":
        """A copy of this state in device memory, updated there by the device forms."""
        return DeviceLossScaler(self, device)


class DeviceLossScaler:
    """Loss-scaler state in device memory: pass 1 reads the scale there
    (:func:`reduce_grads_flat_device_scale`) and :meth:`update` applies the
    scaler's rule on the device from the global squared norm, so an fp16 step
    never waits on the host."""

    def __init__(self, host: LossScaler, device="cuda"):
        raw = bytes(memoryview(host._s))
        self.tensor = torch.frombuffer(bytearray(raw), dtype=torch.uint8).to(device)
        self.device = self.tensor.device

    def update(self, total_sq, taken=None, stream=None) -> None:
        """Record the step whose global squared norm is ``total_sq`` (device float64); ``taken``
        (optional device int32) receives 1 if the step was taken, 0 if it was skipped."""
        _dev_check(total_sq, (torch.float64,), "total_sq")
        tensors = [self.tensor, total_sq] + ([taken] if taken is not None else [])
        if taken is not None:
            _dev_check(taken, (torch.int32,), "taken")
        dev = _one_device(*tensors)
        with torch.cuda.device(dev):
            _check(_lib.zs_loss_scaler_update_device(self.tensor.data_ptr(), total_sq.data_ptr(),
                                                     taken.data_ptr() if taken is not None else None,
                                                     _stream_handle(stream, dev)), "zs_loss_scaler_update_device")

    def state(self) -> dict:
        """The state, copied to the host (synchronises)."""
        s = LossScalerStruct.from_buffer_copy(bytes(self.tensor.cpu().numpy()))
        return {k: getattr(s, k) for k, _ in LossScalerStruct._fields_}


def reduce_grads_flat_device_scale(grads: Sequence, workspace, sqnorm, scaler: DeviceLossScaler,
                                   grad_format="fp16", stream=None) -> None:
    """Pass 1 with the loss scale read on the device from ``scaler``."""
    N = len(grads)
    n = _pass1_args(grads, workspace, sqnorm)
    dev = _one_device(workspace, sqnorm, scaler.tensor, *grads)
    tab = (_vp * max(N, 1))(*[g.data_ptr() for g in grads])
    with torch.cuda.device(dev):
        _check(_lib.zs_reduce_grads_flat_device_scale(tab, N, n, _fmt(grad_format), scaler.tensor.data_ptr(),
                                                      workspace.data_ptr(),
                                                      workspace.numel() * workspace.element_size(),
                                                      sqnorm.data_ptr(), _stream_handle(stream, dev)),
               "zs_reduce_grads_flat_device_scale")


# ------------------------------------------------------------ optimizer offload
def _host_ptr(a, dtype_name: str):
    """Address of a contiguous host array (numpy array or CPU torch tensor)."""
    if isinstance(a, np.ndarray):
        if not a.flags.c_contiguous or a.dtype.name != dtype_name:
            raise TypeError(f"expected a contiguous {dtype_name} numpy array")
        return a.ctypes.data, a.size
    want = {"float32": (torch.float32,), "uint16": (torch.int16, torch.uint16, torch.bfloat16)}[dtype_name]
    if not isinstance(a, torch.Tensor) or a.is_cuda or not a.is_contiguous() or a.dtype not in want:
        raise TypeError(f"expected a contiguous host {dtype_name} array")
    return a.data_ptr(), a.numel()


def cpu_adam(gbar, master, m, v, param, hp, step: int, threads: int = 1) -> None:
    """Host AdamW (no GPU): master/m/v updated from gbar, bf16 copy into param."""
    g, n = _host_ptr(gbar, "float32")
    ptrs = [_host_ptr(x, "float32") for x in (master, m, v)]
    b, nb = _host_ptr(param, "uint16")
    if any(k != n for _, k in ptrs) or nb != n:
        raise ValueError("all arrays must have the same length")
    h = _hp(hp)
    _check(_lib.zs_cpu_adam(g, n, ptrs[0][0], ptrs[1][0], ptrs[2][0], b, ctypes.byref(h), step, threads),
           "zs_cpu_adam")


class Offload:
    """Optimizer offload: fp32 master/m/v in host memory, AdamW on the CPU,
    replica reduction on the GPU, chunks pipelined over PCIe."""

    def __init__(self, chunk_elems: int = 1 << 26, threads: int = 16):
        h = _vp()
        _check(_lib.zs_offload_create(chunk_elems, threads, ctypes.byref(h)), "zs_offload_create")
        self._h = h

    def step(self, grads: Sequence, master, m, v, param, hp, step: int, stream=None) -> None:
        if not self._h:
            raise ValueError("offload context is closed")
        N = len(grads)
        n = param.numel()
        _dev_check(param, _BF16, "param")
        for r, g in enumerate(grads):
            _dev_check(g, _BF16, f"grads[{r}]")
            if g.numel() != n:
                raise ValueError(f"grads[{r}] has {g.numel()} elements, param has {n}")
        ptrs = [_host_ptr(x, "float32") for x in (master, m, v)]
        if any(k != n for _, k in ptrs):
            raise ValueError("host master/m/v must have the parameter count")
        dev = _one_device(param, *grads)
        tab = (_vp * max(N, 1))(*[g.data_ptr() for g in grads])
        h = _hp(hp)
        with torch.cuda.device(dev):
            _check(_lib.zs_offload_step_flat(self._h, tab, N, n, ptrs[0][0], ptrs[1][0], ptrs[2][0],
                                             param.data_ptr(), ctypes.byref(h), step, _stream_handle(stream, dev)),
                   "zs_offload_step_flat")

    def close(self) -> None:
        if self._h:
            _lib.zs_offload_destroy(self._h)
            self._h = _vp()

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def library():
    """The loaded ctypes library (for tests of the raw ABI)."""
    return _lib
