"""The C-ABI library without a GPU: it loads, exports what the header
declares, folds scalars exactly as specified, and rejects bad arguments before
touching the HIP runtime."""
import ctypes
import math
import os
import re

import numpy as np
import pytest

import sharded_mixed_precision_rank_amd as zs
from tests import pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "zshard.h")


def declared_functions():
    src = open(HEADER, encoding="utf-8").read()
    return sorted(set(re.findall(r"ZS_API\s+[\w\s\*]+?\b(zs_\w+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ("zs_reduce_adam_flat", "zs_reduce_adam_list", "zs_list_plan_create", "zs_reduce_adam_list_plan",
                 "zs_list_plan_destroy", "zs_fold", "zs_last_error", "zs_status_string", "zs_abi_version"):
        assert must in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(zs.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), f"libzshard.so does not export {name}"


def test_only_the_abi_is_exported():
    import subprocess

    out = subprocess.run(["nm", "-D", "--defined-only", zs.LIB_PATH], stdout=subprocess.PIPE, text=True).stdout
    text_syms = [l.split()[-1] for l in out.splitlines() if " T " in l]
    assert sorted(text_syms) == declared_functions()


def test_abi_version():
    assert zs.abi_version() == 1


@pytest.mark.parametrize("wd", [0.0, 0.1])
@pytest.mark.parametrize("t", [1, 2, 100, 1000, 5000, 10000])
def test_fold_matches_definition_and_oracle(orc, wd, t):
    hp = dict(pins.HP, weight_decay=wd)
    got = zs.fold(hp, t)
    b1, b2 = hp["beta1"], hp["beta2"]
    want = dict(b1=b1, c1=1.0 - b1, b2=b2, c2=1.0 - b2, eps=hp["eps"], ss=hp["lr"] / (1.0 - b1 ** t),
                rb=1.0 / math.sqrt(1.0 - b2 ** t), dk=1.0 - hp["lr"] * wd)
    for k, x in want.items():
        assert got[k] == pins.f32(x), k
    assert [got[k] for k in ("b1", "c1", "b2", "c2", "eps", "ss", "rb", "dk")] == [float(x) for x in orc.fold(hp, t)]


def _flat(lib, ptrs, N, n, p, m, v, b, hp, step):
    tab = (ctypes.c_void_p * max(len(ptrs), 1))(*ptrs)
    h = zs.AdamHPStruct(*[hp[k] for k in ("lr", "beta1", "beta2", "eps", "weight_decay")])
    return lib.zs_reduce_adam_flat(tab, N, n, p, m, v, b, ctypes.byref(h), step, None)


HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0)
# fake, never dereferenced: every call below fails validation before any HIP call
A = 0x7F0000000000


@pytest.mark.parametrize("case,status", [
    (dict(N=0), "ZS_ERR_RANGE"),
    (dict(N=257), "ZS_ERR_RANGE"),
    (dict(n=-1), "ZS_ERR_RANGE"),
    (dict(step=0), "ZS_ERR_RANGE"),
    (dict(hp=dict(HP, beta1=1.0)), "ZS_ERR_RANGE"),
    (dict(hp=dict(HP, beta2=-0.1)), "ZS_ERR_RANGE"),
    (dict(hp=dict(HP, eps=0.0)), "ZS_ERR_RANGE"),
    (dict(hp=dict(HP, lr=float("nan"))), "ZS_ERR_RANGE"),
    (dict(hp=dict(HP, weight_decay=-1.0)), "ZS_ERR_RANGE"),
    (dict(p=0), "ZS_ERR_NULL"),
    (dict(ptrs=[A + 0x100000, 0]), "ZS_ERR_NULL"),
    (dict(p=A + 2), "ZS_ERR_ALIGN"),
    (dict(b=A + 0x300001), "ZS_ERR_ALIGN"),
    (dict(ptrs=[A + 0x100001, A + 0x200000]), "ZS_ERR_ALIGN"),
    (dict(m=A + 0x10), "ZS_ERR_ALIAS"),                       # m overlaps master
    (dict(b=A + 0x100000 + 64), "ZS_ERR_ALIAS"),              # copy overlaps grad 0
    (dict(v=A + 0x200000 - 16), "ZS_ERR_ALIAS"),              # v runs into grad 1
])
def test_flat_rejects_bad_arguments_without_gpu(case, status):
    lib = zs.library()
    n = 1024
    args = dict(ptrs=[A + 0x100000, A + 0x200000], N=2, n=n, p=A, m=A + 0x10000, v=A + 0x20000, b=A + 0x30000,
                hp=HP, step=1)
    args.update(case)
    if "ptrs" in case and "N" not in case:
        args["N"] = len(case["ptrs"])
    st = _flat(lib, args["ptrs"], args["N"], args["n"], args["p"], args["m"], args["v"], args["b"], args["hp"],
               args["step"])
    assert zs.STATUS[st] == status, zs.library().zs_last_error()
    assert zs.library().zs_last_error()


def test_n_zero_is_a_noop():
    lib = zs.library()
    assert _flat(lib, [0, 0], 2, 0, 0, 0, 0, 0, HP, 1) == 0


def test_list_plan_rejects_overlaps_without_gpu():
    lib = zs.library()
    N = 2
    g0 = (ctypes.c_void_p * 2)(A + 0x1000000, A + 0x2000000)
    g1 = (ctypes.c_void_p * 2)(A + 0x1100000, A + 0x2100000)
    T = (zs.TensorStruct * 2)()
    T[0] = zs.TensorStruct(100, A, A + 0x1000, A + 0x2000, A + 0x3000, ctypes.cast(g0, ctypes.POINTER(ctypes.c_void_p)))
    # tensor 1's master overlaps tensor 0's m
    T[1] = zs.TensorStruct(100, A + 0x1000 + 8, A + 0x5000, A + 0x6000, A + 0x7000,
                           ctypes.cast(g1, ctypes.POINTER(ctypes.c_void_p)))
    plan = ctypes.c_void_p()
    st = lib.zs_list_plan_create(T, 2, N, None, ctypes.byref(plan))
    assert zs.STATUS[st] == "ZS_ERR_ALIAS" and not plan
    # a gradient chunk of tensor 1 lying inside tensor 0's copy
    T[1] = zs.TensorStruct(100, A + 0x8000, A + 0x9000, A + 0xA000, A + 0xB000,
                           ctypes.cast((ctypes.c_void_p * 2)(A + 0x3000 + 20, A + 0x2100000),
                                       ctypes.POINTER(ctypes.c_void_p)))
    st = lib.zs_list_plan_create(T, 2, N, None, ctypes.byref(plan))
    assert zs.STATUS[st] == "ZS_ERR_ALIAS"
    st = lib.zs_list_plan_create(T, -1, N, None, ctypes.byref(plan))
    assert zs.STATUS[st] == "ZS_ERR_RANGE"
    st = lib.zs_list_plan_create(T, 2, 0, None, ctypes.byref(plan))
    assert zs.STATUS[st] == "ZS_ERR_RANGE"


def test_status_strings():
    for k, v in zs.STATUS.items():
        assert zs.library().zs_status_string(k).decode() == v


def test_python_binding_refuses_host_tensors():
    import torch

    g = torch.zeros(8, dtype=torch.bfloat16)
    p = torch.zeros(8)
    with pytest.raises(ValueError):
        zs.reduce_adam_flat([g], p, p.clone(), p.clone(), g.clone(), HP, 1)


# ------------------------------------------------------------ two-pass form
def test_loss_scaler_matches_the_oracle(orc):
    rng = np.random.default_rng(3)
    for window, hyst, init, mn in ((1000, 2, 2.0 ** 16, 1.0), (3, 1, 8.0, 2.0), (7, 3, 2.0 ** 10, 1.0)):
        lib_s = zs.LossScaler(init, mn, window, hyst)
        o_s = orc.scaler(init, mn, window, hyst)
        for k in range(5000):
            ov = bool(rng.random() < (0.3 if k % 500 < 50 else 0.002))
            assert lib_s.update(ov) == orc.scaler_update(o_s, ov)
            st = lib_s.state()
            assert (st["scale"], st["overflows"], st["clean"]) == (o_s.scale, o_s.overflows, o_s.clean)


def test_loss_scaler_rejects_bad_settings():
    with pytest.raises(zs.ZShardError):
        zs.LossScaler(1.0, 2.0, 10, 1)
    with pytest.raises(zs.ZShardError):
        zs.LossScaler(2.0, 1.0, 0, 1)


def test_workspace_size_covers_gradient_and_tiles():
    """fp32 gradient + one norm slot per 2048-parameter tile (plus the head
    slot) + one first-stage sum per 4096 of those, plus alignment slack."""
    for n in (0, 1, 2047, 2048, 10 ** 6, 1093750000):
        need = zs.two_pass_workspace_bytes(n)
        slots = n // 2048 + 2
        core = 4 * n + 8 * (slots + slots // 4096 + 1)
        assert core <= need < core + 600


def test_two_pass_rejects_bad_arguments_without_gpu():
    lib = zs.library()
    n = 4096
    g = (ctypes.c_void_p * 2)(A + 0x100000, A + 0x200000)
    ws_bytes = zs.two_pass_workspace_bytes(n)
    ws = A + 0x400000
    sq = A + 0x800000
    ok = dict(N=2, n=n, fmt=0, scale=1.0, ws=ws, wsb=ws_bytes, sq=sq)
    def call(**kw):
        a = dict(ok, **kw)
        return zs.STATUS[lib.zs_reduce_grads_flat(g, a["N"], a["n"], a["fmt"], a["scale"], a["ws"], a["wsb"],
                                                  a["sq"], None)]
    assert call(fmt=2) == "ZS_ERR_RANGE"
    assert call(scale=0.0) == "ZS_ERR_RANGE"
    assert call(scale=float("inf")) == "ZS_ERR_RANGE"
    assert call(wsb=ws_bytes - 300) == "ZS_ERR_RANGE"
    assert call(sq=0) == "ZS_ERR_NULL"
    assert call(sq=sq + 4) == "ZS_ERR_ALIGN"
    assert call(ws=A + 0x100000 + 64) == "ZS_ERR_ALIAS"          # workspace over a gradient
    assert call(sq=A + 0x200000 + 8) == "ZS_ERR_ALIAS"            # norm slot inside a gradient
    h = zs.AdamHPStruct(1e-3, 0.9, 0.999, 1e-8, 0.0)
    def call2(**kw):
        a = dict(ws=ws, wsb=ws_bytes, n=n, p=A + 0x1000000, m=A + 0x1100000, v=A + 0x1200000, b=A + 0x1300000,
                 fmt=0, step=1, tsq=sq, max_norm=1.0)
        a.update(kw)
        return zs.STATUS[lib.zs_adam_from_grads_flat(a["ws"], a["wsb"], a["n"], a["p"], a["m"], a["v"], a["b"],
                                                     a["fmt"], ctypes.byref(h), a["step"], a["tsq"], a["max_norm"],
                                                     1, None)]
    assert call2(fmt=3) == "ZS_ERR_RANGE"
    assert call2(max_norm=float("nan")) == "ZS_ERR_RANGE"
    assert call2(step=0) == "ZS_ERR_RANGE"
    assert call2(tsq=0) == "ZS_ERR_NULL"
    assert call2(m=A + 0x1000000 + 16) == "ZS_ERR_ALIAS"           # m over master
    assert call2(p=ws + 256) == "ZS_ERR_ALIAS"                      # master over the workspace
    assert call2(tsq=A + 0x1100000 + 8) == "ZS_ERR_ALIAS"           # norm inside m
    assert call2(wsb=100) == "ZS_ERR_RANGE"


# ------------------------------------------------------------ optimizer offload (host AdamW)
@pytest.mark.parametrize("n,threads", [(1, 1), (7, 1), (8, 1), (1000, 3), (300_001, 8)])
def test_cpu_adam_matches_oracle(orc, n, threads):
    rng = np.random.default_rng(n)
    g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    P = (rng.standard_normal(n) * 0.02).astype(np.float32)
    M = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    V = np.abs(rng.standard_normal(n) * 1e-6).astype(np.float32)
    if n >= 16:
        g[:6] = [0.0, -0.0, np.inf, -np.inf, np.nan, 1e-40]
        P[6:9] = [1e-40, -0.0, 3e38]
    hp = dict(pins.HP, weight_decay=0.1)
    rP, rM, rV, rB, _ = orc.adam_from_gbar(g, P, M, V, hp, 42, 1.0, 0.0)
    Pc, Mc, Vc = P.copy(), M.copy(), V.copy()
    for shift in (0, 1):  # the bf16 output 16-byte aligned (streamed stores) and not
        Pc, Mc, Vc = P.copy(), M.copy(), V.copy()
        Bc = np.zeros(n + 8, dtype=np.uint16)[8 - shift:8 - shift + n]
        zs.cpu_adam(g, Pc, Mc, Vc, Bc, hp, 42, threads)
        if shift == 0:
            B0 = Bc.copy()
        else:
            assert np.array_equal(Bc, B0)
    for got, ref in ((Pc, rP), (Mc, rM), (Vc, rV)):
        both_nan = np.isnan(got) & np.isnan(ref)
        assert np.array_equal(got.view(np.uint32)[~both_nan], ref.view(np.uint32)[~both_nan])
    nan = lambda b: ((b & 0x7F80) == 0x7F80) & ((b & 0x7F) != 0)
    assert np.array_equal(nan(Bc), nan(rB)) and np.array_equal(Bc[~nan(Bc)], rB[~nan(rB)])


def test_offload_rejects_bad_arguments_without_gpu():
    lib = zs.library()
    h = ctypes.c_void_p()
    assert zs.STATUS[lib.zs_offload_create(100, 4, ctypes.byref(h))] == "ZS_ERR_RANGE"
    assert zs.STATUS[lib.zs_offload_create(1 << 20, 0, ctypes.byref(h))] == "ZS_ERR_RANGE"
    assert zs.STATUS[lib.zs_offload_create(1 << 20, 4, ctypes.byref(h))] == "ZS_OK" and h
    g = (ctypes.c_void_p * 2)(A + 0x100000, A + 0x200000)
    hp = zs.AdamHPStruct(1e-3, 0.9, 0.999, 1e-8, 0.0)
    P = np.zeros(1024, np.float32)
    # host arrays overlapping, before any device work
    st = lib.zs_offload_step_flat(h, g, 2, 1024, P.ctypes.data, P.ctypes.data + 64, A, A + 0x300000,
                                  ctypes.byref(hp), 1, None)
    assert zs.STATUS[st] == "ZS_ERR_ALIAS"
    st = lib.zs_offload_step_flat(h, g, 0, 1024, P.ctypes.data, P.ctypes.data, P.ctypes.data, A, ctypes.byref(hp), 1,
                                  None)
    assert zs.STATUS[st] == "ZS_ERR_RANGE"
    lib.zs_offload_destroy(h)   # never allocated device buffers: nothing to wait for


def test_binding_rejects_tensors_on_several_devices():
    """The library launches on the current device, so the binding makes the
    tensors' device current and refuses a call whose tensors are spread over
    several devices (checked here with host and meta tensors, no GPU)."""
    import torch

    import sharded_mixed_precision_rank_amd as zs

    a = torch.zeros(4)
    b = torch.zeros(4, device="meta")
    assert zs._one_device(a, torch.ones(2)) == torch.device("cpu")
    with pytest.raises(ValueError, match="several devices"):
        zs._one_device(a, b)


def test_probe_library_rejects_unsupported_arguments_without_gpu():
    """The benchmark's measurement probe (bench_probe/libzshard_probe.so) checks its arguments before any
    launch."""
    import bench_probe

    lib = bench_probe.load()
    f = lib.zs_probe_pattern
    g = (ctypes.c_void_p * 3)(A + 0x100000, A + 0x200000, A + 0x300000)
    arr = [A + 0x400000, A + 0x500000, A + 0x600000, A + 0x700000]
    assert f(g, 3, 1 << 20, *arr, 0, None) == 1            # N = 3 is not covered
    assert f(g, 2, 500, *arr, 0, None) == 1                # less than one 512-parameter tile
    assert f(g, 2, 1 << 20, A + 0x400004, *arr[1:], 0, None) == 1   # not on a 128-byte boundary
    fw = lib.zs_probe_pattern_windowed
    assert fw(g, 3, 1 << 20, *arr, 4096, 512, None) == 1   # N = 3 is not covered
    assert fw(g, 2, 500, *arr, 4096, 512, None) == 1       # less than one tile
    assert fw(g, 2, 1 << 20, *arr, 4000, 512, None) == 1   # period not a power of two
    fc = lib.zs_probe_copy
    assert fc(A + 0x100000, A + 0x200004, 1024, None) == 1  # not 16-byte aligned
    assert fc(A + 0x100000, A + 0x100800, 1024, None) == 1  # overlapping arrays
    assert fc(0, A + 0x200000, 1024, None) == 1             # NULL
    assert fc(A + 0x100000, A + 0x200000, -1, None) == 1    # negative length
    assert fc(0, 0, 0, None) == 0                           # nothing to copy
    assert fw(g, 2, 1 << 20, *arr, 32, 8, None) == 1       # period below 64 ticks
    assert fw(g, 2, 1 << 20, *arr, 4096, 4096, None) == 1  # window not shorter than the period
    assert fw(g, 2, 1 << 20, A + 0x400004, *arr[1:], 4096, 512, None) == 1


def test_write_window_query():
    """The query reports the window each kernel takes.  The flat step and pass 1 take windows only on
    the windowed schedule (explicit, or an explicit window setting under the automatic one): their
    automatic default is the phased schedule, and the windowed one's default window is 4096 / 512
    (flat, N = 64) and 4096 / 256 (pass 1), on shards of at least 2^25 parameters."""
    assert zs.write_window("flat", 64, 1_093_750_000) == (0, 0)
    assert zs.write_window("reduce", 64, 1_093_750_000) == (0, 0)
    assert zs.write_window("list", 64, 1_093_750_000) == (0, 0)   # list plans: the flat step's schedule
    assert zs.write_window("list", 64, (1 << 25) - 1) == (0, 0)
    assert zs.write_window("list", 8, 1 << 30) == (0, 0)
    try:
        zs.set_flat_schedule("windowed")
        for kernel, default in (("reduce", (4096, 256)), ("flat", (4096, 512))):
            assert zs.write_window(kernel, 64, 1_093_750_000) == default
            assert zs.write_window(kernel, 64, 1 << 25) == default
            assert zs.write_window(kernel, 64, (1 << 25) - 1) == (0, 0)
            assert zs.write_window(kernel, 100, 1 << 30) == default     # runtime replica counts too
            if kernel == "reduce":
                assert zs.write_window(kernel, 8, 124_000_000) == default   # windowed on request, any N
                assert zs.write_window(kernel, 47, 1 << 30) == default
            zs.set_write_window(1)
            assert zs.write_window(kernel, 64, 1 << 30) == (0, 0)
            zs.set_write_window(1024, 128)
            assert zs.write_window(kernel, 16, 1 << 30) == (1024, 128)
            assert zs.write_window(kernel, 5, 1 << 30) == (1024, 128)
            zs.set_write_window(0)
        assert zs.write_window("list", 64, 1 << 30) == (4096, 512)   # a list plan as a flat shard of its size
        assert zs.write_window("list", 64, (1 << 25) - 1) == (0, 0)
        # the flat step's open length follows the writes' share of the bytes
        assert zs.write_window("flat", 48, 1 << 30) == (4096, 640)
        assert zs.write_window("flat", 128, 1 << 30) == (4096, 512)
        assert zs.write_window("flat", 129, 1 << 30) == (4096, 384)
        assert zs.write_window("flat", 256, 1 << 30) == (4096, 384)
        assert zs.write_window("flat", 8, 1 << 30) == (4096, 640)      # windowed on request, any N
    finally:
        zs.set_flat_schedule("auto")
        zs.set_write_window(0)
    # an explicit window under the automatic schedule still takes the windowed kernel
    zs.set_write_window(2048, 256)
    try:
        assert zs.write_window("flat", 64, 1 << 30) == (2048, 256)
        assert zs.flat_schedule(64, 1 << 30) == "windowed"
    finally:
        zs.set_write_window(0)
    with pytest.raises(zs.ZShardError):
        zs.write_window("flat", 0, 1 << 20)
    lib = ctypes.CDLL(zs.LIB_PATH)
    lib.zs_write_window.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
                                    ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32)]
    p, o = ctypes.c_int32(), ctypes.c_int32()
    assert lib.zs_write_window(3, 64, 1 << 30, ctypes.byref(p), ctypes.byref(o)) == 2   # unknown kernel
    assert lib.zs_write_window(0, 64, 1 << 30, None, ctypes.byref(o)) == 1


def test_device_scaler_entry_points_reject_bad_arguments_without_gpu():
    lib = zs.library()
    st, sq, tk = A + 0x100000, A + 0x200000, A + 0x300000
    assert zs.STATUS[lib.zs_loss_scaler_update_device(None, sq, tk, None)] == "ZS_ERR_NULL"
    assert zs.STATUS[lib.zs_loss_scaler_update_device(st, None, tk, None)] == "ZS_ERR_NULL"
    assert zs.STATUS[lib.zs_loss_scaler_update_device(st + 4, sq, tk, None)] == "ZS_ERR_ALIGN"
    assert zs.STATUS[lib.zs_loss_scaler_update_device(st, sq, tk + 2, None)] == "ZS_ERR_ALIGN"
    assert zs.STATUS[lib.zs_loss_scaler_update_device(st, st + 8, tk, None)] == "ZS_ERR_ALIAS"
    assert zs.STATUS[lib.zs_loss_scaler_update_device(st, sq, st + 40, None)] == "ZS_ERR_ALIAS"
    n = 4096
    g = (ctypes.c_void_p * 2)(A + 0x1000000, A + 0x2000000)
    ws, wsb = A + 0x4000000, zs.two_pass_workspace_bytes(n)
    f = lib.zs_reduce_grads_flat_device_scale
    assert zs.STATUS[f(g, 2, n, 1, None, ws, wsb, sq, None)] == "ZS_ERR_NULL"
    assert zs.STATUS[f(g, 2, n, 1, st + 4, ws, wsb, sq, None)] == "ZS_ERR_ALIGN"
    assert zs.STATUS[f(g, 2, n, 1, ws + 1024, ws, wsb, sq, None)] == "ZS_ERR_ALIAS"   # state inside the workspace
    assert zs.STATUS[f(g, 2, n, 1, sq, ws, wsb, sq, None)] == "ZS_ERR_ALIAS"          # state over the norm slot


def test_list_plan_groups_reject_bad_arguments_without_gpu():
    """An empty plan needs no device table, so the group calls' checks run without a GPU."""
    lib = zs.library()
    h = ctypes.c_void_p()
    assert zs.STATUS[lib.zs_list_plan_create(None, 0, 2, None, ctypes.byref(h))] == "ZS_OK"
    try:
        g = (ctypes.c_int32 * 1)(0)
        assert zs.STATUS[lib.zs_list_plan_set_groups(None, g, 2, None)] == "ZS_ERR_NULL"
        assert zs.STATUS[lib.zs_list_plan_set_groups(h, g, 0, None)] == "ZS_ERR_RANGE"
        assert zs.STATUS[lib.zs_list_plan_set_groups(h, g, 9, None)] == "ZS_ERR_RANGE"
        assert zs.STATUS[lib.zs_list_plan_set_groups(h, None, 3, None)] == "ZS_OK"     # no tensors to assign
        hps = (zs.AdamHPStruct * 3)(*[zs.AdamHPStruct(1e-3, 0.9, 0.999, 1e-8, wd) for wd in (0.1, 0.0, 0.01)])
        assert zs.STATUS[lib.zs_reduce_adam_list_plan_groups(h, hps, 2, 1, None)] == "ZS_ERR_RANGE"  # plan has 3
        assert zs.STATUS[lib.zs_reduce_adam_list_plan_groups(h, None, 3, 1, None)] == "ZS_ERR_NULL"
        bad = (zs.AdamHPStruct * 3)(*[zs.AdamHPStruct(1e-3, 0.9, 1.5, 1e-8, 0.0)] * 3)
        assert zs.STATUS[lib.zs_reduce_adam_list_plan_groups(h, bad, 3, 1, None)] == "ZS_ERR_RANGE"
        assert zs.STATUS[lib.zs_reduce_adam_list_plan_groups(h, hps, 3, 1, None)] == "ZS_OK"         # nothing to do
    finally:
        lib.zs_list_plan_destroy(h)


@pytest.mark.parametrize("t0,count", [(1, 40), (4990, 25)])
def test_fold_table_rows_are_the_oracle_fold(orc, t0, count):
    hp = dict(pins.HP, weight_decay=0.1)
    table = zs.fold_table(hp, t0, count)
    for k in range(count):
        ref = np.array(orc.fold(hp, t0 + k), dtype=np.float32)
        assert np.array_equal(table[k].view(np.uint32), ref.view(np.uint32)), t0 + k


def test_devstep_entry_points_reject_bad_arguments_without_gpu():
    lib = zs.library()
    hp = zs.AdamHPStruct(1e-3, 0.9, 0.999, 1e-8, 0.0)
    out = (ctypes.c_float * 8)()
    assert zs.STATUS[lib.zs_fold_table(ctypes.byref(hp), 1, 0, out)] == "ZS_ERR_RANGE"
    assert zs.STATUS[lib.zs_fold_table(ctypes.byref(hp), 0, 1, out)] == "ZS_ERR_RANGE"
    assert zs.STATUS[lib.zs_fold_table(ctypes.byref(hp), 1, 1, None)] == "ZS_ERR_NULL"
    assert zs.STATUS[lib.zs_step_advance(None, None)] == "ZS_ERR_NULL"
    assert zs.STATUS[lib.zs_step_advance(A + 4, None)] == "ZS_ERR_ALIGN"
    n = 4096
    g = (ctypes.c_void_p * 2)(A + 0x1000000, A + 0x2000000)
    P, M, V, B = A + 0x3000000, A + 0x4000000, A + 0x5000000, A + 0x6000000
    tab, step, status = A + 0x7000000, A + 0x7100000, A + 0x7200000
    def src(**kw):
        d = dict(table=tab, t0=1, count=100, step=step, status=status)
        d.update(kw)
        return zs.StepSourceStruct(d["table"], d["t0"], d["count"], d["step"], d["status"])
    f = lambda s: zs.STATUS[lib.zs_reduce_adam_flat_devstep(g, 2, n, P, M, V, B, ctypes.byref(s) if s else None,
                                                             None)]
    assert f(None) == "ZS_ERR_NULL"
    assert f(src(table=None)) == "ZS_ERR_NULL"
    assert f(src(step=None)) == "ZS_ERR_NULL"
    assert f(src(t0=0)) == "ZS_ERR_RANGE"
    assert f(src(count=0)) == "ZS_ERR_RANGE"
    assert f(src(step=step + 4)) == "ZS_ERR_ALIGN"
    assert f(src(status=status + 2)) == "ZS_ERR_ALIGN"
    assert f(src(status=tab + 64)) == "ZS_ERR_ALIAS"        # status inside the table
    assert f(src(table=P + 1024)) == "ZS_ERR_ALIAS"         # table inside the master array (written)
    assert f(src(status=A + 0x1000000 + 8)) == "ZS_ERR_ALIAS"  # status inside a gradient chunk


def test_tuning_knobs_check_their_ranges():
    lib = ctypes.CDLL(zs.LIB_PATH)
    lib.zs_set_write_window.argtypes = [ctypes.c_int32, ctypes.c_int32]
    lib.zs_set_grid_blocks.argtypes = [ctypes.c_int32]
    ok, rng = 0, 2
    for period, open_ticks, want in [(0, 0, ok), (1, 0, ok), (0, 999, ok), (64, 1, ok), (64, 63, ok),
                                     (4096, 512, ok), (1 << 20, 1 << 14, ok), (2, 1, rng), (32, 1, rng),
                                     (96, 1, rng), (4096, 0, rng), (4096, 4096, rng), (1 << 20, (1 << 14) + 1, rng),
                                     (1 << 21, 1, rng), (-4, 1, rng), (256, -1, rng)]:
        assert lib.zs_set_write_window(period, open_ticks) == want, (period, open_ticks)
    assert lib.zs_set_write_window(0, 0) == ok
    assert lib.zs_set_grid_blocks(-1) == rng and lib.zs_set_grid_blocks(0) == ok
    with pytest.raises(zs.ZShardError):
        zs.set_write_window(100, 10)
    zs.set_write_window(0)
    # the per-launch byte limit: 0 restores the 3e9 default, any positive value is taken as is
    lib.zs_set_launch_bytes.argtypes = [ctypes.c_int64]
    assert lib.zs_set_launch_bytes(-1) == rng
    assert zs.launch_bytes() == 3_000_000_000
    for b in (1, 4096, 10 ** 12, 2 ** 63 - 1):
        zs.set_launch_bytes(b)
        assert zs.launch_bytes() == b
    zs.set_launch_bytes(0)
    assert zs.launch_bytes() == 3_000_000_000
    with pytest.raises(zs.ZShardError):
        zs.set_launch_bytes(-5)


def test_reduce_schedule_query():
    """Pass 1 of the two-pass form follows the same setting: phased for N >= 12 on shards of at least
    2^25 parameters, one tile per workgroup otherwise; windowed only on request."""
    assert zs.reduce_schedule(64, 1_093_750_000) == "phased"
    assert zs.reduce_schedule(12, 1 << 25) == "phased"
    assert zs.reduce_schedule(16, 1 << 30) == "phased"
    assert zs.reduce_schedule(11, 1 << 30) == "stream"
    assert zs.reduce_schedule(8, 124_000_000) == "stream"
    assert zs.reduce_schedule(64, (1 << 25) - 1) == "stream"
    try:
        zs.set_write_window(1)
        assert zs.reduce_schedule(64, 1 << 30) == "stream"
        zs.set_write_window(2048, 256)
        assert zs.reduce_schedule(8, 1 << 30) == "windowed"
        assert zs.reduce_schedule(8, 1 << 20) == "stream"   # below the windowed kernel's size
        zs.set_write_window(0)
        zs.set_flat_schedule("phased")
        assert zs.reduce_schedule(8, 512) == "phased"       # one whole wave tile is enough
        assert zs.reduce_schedule(8, 511) == "stream"
        zs.set_flat_schedule("stream")
        assert zs.reduce_schedule(64, 1 << 30) == "stream"
        with pytest.raises(zs.ZShardError):
            zs.reduce_schedule(0, 1 << 20)
        with pytest.raises(zs.ZShardError):
            zs.reduce_schedule(8, -1)
    finally:
        zs.set_flat_schedule("auto")
        zs.set_write_window(0)


def test_list_schedule_query():
    """List plans: phased for N >= 64 from 3 * 2^24 parameters in all, N >= 40 from 3 * 2^25 and N >= 32
    from 3 * 2^26, when at most 1 in 20 wave tiles lies outside whole spans; an explicit schedule or window
    wins as for flat shards."""
    big = [1 << 22] * 64                                    # 2^28 in tensors of 8,192 tiles
    assert zs.list_schedule(big, 32) == "phased"
    assert zs.list_schedule(big, 31) == "stream"
    assert zs.list_schedule(big[:32], 40) == "phased"       # 2^27
    assert zs.list_schedule(big[:32], 39) == "stream"
    assert zs.list_schedule(big[:32], 32) == "stream"
    assert zs.list_schedule(big[:16], 64) == "phased"       # 2^26
    assert zs.list_schedule(big[:16], 63) == "stream"
    assert zs.list_schedule(big[:8], 64) == "stream"        # 2^25
    three = [3 << 21] * 64                                  # 3 * 2^27, in tensors of 12,288 tiles
    assert zs.list_schedule(three[:8], 64) == "phased"      # 3 * 2^24
    assert zs.list_schedule(three[:7] + [(3 << 21) - 8], 64) == "stream"
    assert zs.list_schedule(three[:16], 40) == "phased"     # 3 * 2^25
    assert zs.list_schedule(three[:15] + [(3 << 21) - 8], 40) == "stream"
    assert zs.list_schedule(three[:32], 32) == "phased"     # 3 * 2^26
    assert zs.list_schedule(three[:31] + [(3 << 21) - 8], 32) == "stream"
    assert zs.list_schedule(big[:16], 24) == "stream"
    assert zs.list_schedule(big * 4, 24) == "stream"        # 2^30 at N = 24: per-tile stores on lists
    assert zs.flat_schedule(24, 1 << 30) == "phased"        # the flat step takes it from 24 on 2^27 and more
    # 20,000 tensors of 32 tiles: spans of 10 tiles from a multiple of 10 leave 2-12 of each tensor's 32
    # tiles outside whole spans, far above 1 in 20
    small = [1 << 14] * 20000
    assert sum(small) > 1 << 28
    assert zs.list_schedule(small, 64) == "stream"
    # 2,000 tensors of 320 tiles, each starting on a multiple of 10 tiles: every tile in a whole span
    assert zs.list_schedule([320 * 512] * 2000, 64) == "phased"
    # the same with a 1-element tensor before each: the large tensors move off the tile grid (a partial
    # first and last tile, 321 in all) and 31 whole spans fit in each, so 11 of its tiles and the scalar
    # tensor's one are loose: 12 in 322, under 1 in 20
    mixed = [x for _ in range(2000) for x in (1, 320 * 512)]
    assert zs.list_schedule(mixed, 64) == "phased"
    try:
        zs.set_flat_schedule("phased")
        assert zs.list_schedule(small, 8) == "phased"
        zs.set_flat_schedule("auto")
        zs.set_write_window(2048, 256)
        assert zs.list_schedule(big, 8) == "windowed"
        assert zs.list_schedule([1 << 20], 8) == "stream"   # below the windowed kernel's size
    finally:
        zs.set_flat_schedule("auto")
        zs.set_write_window(0)
    with pytest.raises(zs.ZShardError):
        zs.list_schedule(big, 0)
    with pytest.raises(zs.ZShardError):
        zs.list_schedule([-1], 8)


def test_flat_schedule_query_and_setting():
    """The automatic schedule: phased for N >= 40 on shards of at least 2^25 parameters and for N >= 24
    on at least 2^27, per-tile stores otherwise; an explicit schedule wins (each kernel's own size
    conditions aside)."""
    assert zs.flat_schedule(64, 1_093_750_000) == "phased"
    assert zs.flat_schedule(40, 1 << 25) == "phased"
    assert zs.flat_schedule(39, 1 << 25) == "stream"
    assert zs.flat_schedule(24, 1 << 27) == "phased"
    assert zs.flat_schedule(24, (1 << 27) - 1) == "stream"
    assert zs.flat_schedule(256, 1 << 30) == "phased"
    assert zs.flat_schedule(23, 1 << 30) == "stream"
    assert zs.flat_schedule(16, 1 << 30) == "stream"
    assert zs.flat_schedule(8, 124_000_000) == "stream"
    assert zs.flat_schedule(64, (1 << 25) - 1) == "stream"
    zs.set_write_window(1)   # an explicit "no windows" keeps per-tile stores
    try:
        assert zs.flat_schedule(64, 1 << 30) == "stream"
    finally:
        zs.set_write_window(0)
    try:
        zs.set_flat_schedule("phased")
        assert zs.flat_schedule(8, 512) == "phased"       # one whole tile is enough
        assert zs.flat_schedule(8, 511) == "stream"       # no whole tile
        zs.set_flat_schedule("windowed")
        assert zs.flat_schedule(64, 1 << 30) == "windowed"
        assert zs.flat_schedule(64, 1 << 20) == "stream"  # below the windowed kernel's size
        zs.set_flat_schedule("stream")
        assert zs.flat_schedule(64, 1 << 30) == "stream"
        with pytest.raises(zs.ZShardError):
            zs.set_flat_schedule(4)
        with pytest.raises(zs.ZShardError):
            zs.set_flat_schedule(-1)
        with pytest.raises(zs.ZShardError):
            zs.flat_schedule(0, 1 << 20)
        with pytest.raises(zs.ZShardError):
            zs.set_phased_max_polls(-1)
        zs.set_phased_max_polls(1)
        zs.set_phased_max_polls(0)
    finally:
        zs.set_flat_schedule("auto")


def test_static_list_step_refuses_a_table_beyond_its_array_without_gpu():
    """zs_reduce_adam_list_static checks the table's size against its fixed array before any GPU work:
    one tensor of 5e9 parameters needs about 9.8M work items of 4 bytes, 39 MB of table, beyond 32 MiB."""
    lib = zs.library()
    n = 5_000_000_000
    span = 1 << 40
    g = (ctypes.c_void_p * 1)(A + 1 * span)
    t = (zs.TensorStruct * 1)()
    t[0] = zs.TensorStruct(n, A + 2 * span, A + 3 * span, A + 4 * span, A + 5 * span,
                           ctypes.cast(g, ctypes.POINTER(ctypes.c_void_p)))
    h = zs.AdamHPStruct(1e-3, 0.9, 0.999, 1e-8, 0.0)
    assert zs.STATUS[lib.zs_reduce_adam_list_static(t, 1, 1, ctypes.byref(h), 1, None)] == "ZS_ERR_RANGE"
    assert b"zs_reduce_adam_list_static holds at most" in lib.zs_last_error()
    assert zs.STATUS[lib.zs_reduce_adam_list_static(t, 1, 1, None, 1, None)] == "ZS_ERR_NULL"
    assert zs.STATUS[lib.zs_reduce_adam_list_static(t, 1, 0, ctypes.byref(h), 1, None)] == "ZS_ERR_RANGE"
    assert zs.STATUS[lib.zs_reduce_adam_list_static(t, 0, 1, ctypes.byref(h), 1, None)] == "ZS_OK"  # no tensors
