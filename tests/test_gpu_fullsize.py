"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (the library's default grid), on sampled outputs.

Inputs are drawn in device memory by the seeded counter-based generator; the
oracle recomputes each sampled position from the host's draws of the same
counters, so no expected value comes from the device.  The tiny workload is
compared at every position.  Ragged lists also check every gap position
between tensors (the step must leave it untouched).  The two-pass global
norm, which no sample covers, is the oracle's own: its mean gradient over the
whole shard (from the generator's replica values) and its sum of squares over
that, in index order; the GPU's norm is only compared with it.
"""
import os

import numpy as np
import pytest

from tests import parity

pytestmark = pytest.mark.gpu

SAMPLES = 200_000
SENTINEL = 0x7FBF


def workload(name):
    from synth import workloads as W

    return {"flat-1m": lambda: W.FLAT_1M_N2, "flat-124m": lambda: W.FLAT_124M_N8,
            "list-llama7b": W.list_llama7b_dp8_n8, "flat-70b": lambda: W.FLAT_70B_DP64_N64,
            "list-llama70b": W.list_llama70b_dp64_n64,
            "list-ragged": lambda: W.list_ragged_20000_n16(1),
            "list-ragged-warm": lambda: W.list_ragged_20000_n16(10_000)}[name]()


def positions(w, L, seed=1234):
    """Sampled arena positions inside tensors (plus both ends), and every gap position."""
    if L <= 1 << 21:
        idx = np.arange(L, dtype=np.int64)
    else:
        rng = np.random.default_rng(seed)
        idx = np.unique(np.concatenate([rng.integers(0, L, SAMPLES), np.arange(4096), np.arange(L - 4096, L)]))
    gaps = np.zeros(0, dtype=np.int64)
    if w.is_list:
        offs, _ = w.layout()
        sizes = np.asarray(w.sizes, dtype=np.int64)
        inside = np.zeros(L, dtype=bool)
        for o, n in zip(offs.tolist(), sizes.tolist()):
            inside[o:o + n] = True
        idx = idx[inside[idx]]
        gaps = np.flatnonzero(~inside)
    return idx, gaps


def host_threads() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def oracle_full_mean_and_norm(orc, torch, G, fmt, loss_scale, slice_elems=1 << 23):
    """The oracle's pass 1 over the whole shard and its squared norm of the
    result (one sum over every position, in index order, as the oracle defines
    it).  The replica values are the generator's draws: they are copied from
    the device buffers the library only reads, slice by slice, through pinned
    memory."""
    import torch as _t

    N, n = len(G), G[0].numel()
    gbar = np.empty(n, dtype=np.float32)
    buf = _t.empty((N, min(n, slice_elems)), dtype=_t.int16).pin_memory()
    for lo in range(0, n, slice_elems):
        hi = min(n, lo + slice_elems)
        for r in range(N):
            buf[r, :hi - lo].copy_(G[r][lo:hi].view(_t.int16), non_blocking=True)
        torch.cuda.synchronize()
        rows = [buf[r, :hi - lo].numpy().view(np.uint16) for r in range(N)]
        gbar[lo:hi] = orc.reduce_unscale(rows, fmt, loss_scale, threads=host_threads())
    del buf
    return gbar, orc.sqnorm(gbar)


def assert_norm(orc, sqv, ref_sq, n, max_norm):
    """The GPU's squared norm against the oracle's: both sum the same n
    non-negative doubles, in different orders, so they differ by at most
    2(n-1)u of the sum (u = 2^-53); and the fp32 clip coefficient, which is
    what the update uses, must be the same."""
    assert abs(sqv - ref_sq) <= 2 * max(n - 1, 1) * 2.0 ** -53 * ref_sq, (sqv, ref_sq)
    assert orc.clip_coef(sqv, max_norm) == orc.clip_coef(ref_sq, max_norm), (sqv, ref_sq)


def gather(torch, d, idx):
    it = torch.from_numpy(idx).to(d["P"].device)
    return dict(P=d["P"][it].cpu().numpy(), M=d["M"][it].cpu().numpy(), V=d["V"][it].cpu().numpy(),
                B=d["B"].view(torch.int16)[it].cpu().numpy().view(np.uint16))


@pytest.mark.parametrize("name", ["flat-1m", "flat-124m", "list-llama7b", "flat-70b", "list-llama70b",
                                  "list-ragged", "list-ragged-warm"])
def test_fused_step_full_size(orc, name):
    import torch

    import sharded_mixed_precision_rank_amd as zs
    from synth import workloads as W

    w = workload(name)
    zs.set_grid_blocks(0)
    d = W.device_inputs(w, b_fill=SENTINEL)
    L = d["arena_len"]
    plan = None
    if w.is_list:
        offs, _ = w.layout()
        plan = zs.ListPlan.from_arenas(w.sizes, offs, d["G"], d["P"], d["M"], d["V"], d["B"])
        plan.step(w.hp(), w.step)
    else:
        zs.reduce_adam_flat(d["G"], d["P"], d["M"], d["V"], d["B"], w.hp(), w.step)
    torch.cuda.synchronize()
    idx, gaps = positions(w, L)
    got = gather(torch, d, idx)
    h = W.host_inputs_at(w, idx)
    P, M, V, B = orc.step(h["G"], h["P"], h["M"], h["V"], w.hp(), w.step)
    ref = dict(P=P, M=M, V=V, B=B)
    parity.assert_step(got, ref, f"{w.name} ({idx.size} positions)")
    assert parity.bit_identical(got, ref), w.name
    if gaps.size:
        g = gather(torch, d, gaps)
        hg = W.host_inputs_at(w, gaps)
        for k in "PMV":
            assert np.array_equal(g[k].view(np.uint32), hg[k].view(np.uint32)), f"{w.name}: gap {k} was written"
        assert np.all(g["B"] == SENTINEL), f"{w.name}: gap of the working copy was written"
    if plan is not None:
        plan.close()
    del d, plan
    torch.cuda.empty_cache()


@pytest.mark.parametrize("path", ["clip", "fp16"])
def test_two_pass_full_size(orc, path):
    """The 70B/64 shard through both passes: global-norm clipping at 1.0, with
    bf16 replicas, or fp16 replicas at loss scale 2^16 with an fp16 working copy."""
    import torch

    import sharded_mixed_precision_rank_amd as zs
    import synth
    from synth import workloads as W

    w = W.FLAT_70B_DP64_N64
    zs.set_grid_blocks(0)
    d = W.device_inputs(w)
    n = d["arena_len"]
    loss_scale = 2.0 ** 16 if path == "fp16" else 1.0
    fmt = "fp16" if path == "fp16" else "bf16"
    k = w.keys()
    if path == "fp16":
        tmp = torch.empty(n, dtype=torch.float32, device="cuda")
        for r in range(w.N):
            synth.dev_fill_normal_f32(tmp, k["G"][r], 0, w.g_sigma * loss_scale)
            d["G"][r] = tmp.half()
        del tmp
        d["B"] = torch.zeros(n, dtype=torch.float16, device="cuda")
    ws = torch.empty(zs.two_pass_workspace_bytes(n), dtype=torch.uint8, device="cuda")
    sq = torch.empty(1, dtype=torch.float64, device="cuda")
    zs.reduce_grads_flat(d["G"], ws, sq, loss_scale, fmt)
    torch.cuda.synchronize()
    start = (256 - ws.data_ptr() % 256) % 256
    gbar = ws[start:start + 4 * n].view(torch.float32)
    sqv = float(sq.item())
    gfmt = 1 if path == "fp16" else 0
    # the oracle's own norm over the whole shard; the GPU's is only compared with it
    print(f"two-pass {path}: oracle pass 1 over {n} positions x {w.N} replicas", flush=True)
    ref_gbar, ref_sq = oracle_full_mean_and_norm(orc, torch, d["G"], gfmt, loss_scale)
    assert_norm(orc, sqv, ref_sq, n, 1.0)
    assert orc.clip_coef(ref_sq, 1.0) < 1.0  # clipping is active
    idx, _ = positions(w, n)
    it = torch.from_numpy(idx).to("cuda")
    gbar_s = gbar[it].cpu().numpy()
    zs.adam_from_grads_flat(ws, n, d["P"], d["M"], d["V"], d["B"], w.hp(), w.step, sq, 1.0, fmt)
    torch.cuda.synchronize()
    got = gather(torch, d, idx)
    h = W.host_inputs_at(w, idx)
    if path == "fp16":
        G = np.stack([orc.f16(synth.normal_f32_at(k["G"][r], idx, w.g_sigma * loss_scale)) for r in range(w.N)])
    else:
        G = h["G"]
    g = orc.reduce_unscale(G, gfmt, loss_scale)
    # the replica values the whole-shard pass read are the host generator's at the sampled positions
    assert np.array_equal(ref_gbar[idx].view(np.uint32), g.view(np.uint32)), "replica values"
    assert np.array_equal(gbar_s.view(np.uint32), g.view(np.uint32)), "pass 1 mean gradient"
    del ref_gbar
    P, M, V, B, taken = orc.adam_from_gbar(g, h["P"], h["M"], h["V"], w.hp(), w.step, ref_sq, 1.0, out_fmt=gfmt)
    assert taken
    ref = dict(P=P, M=M, V=V, B=B)
    for key in "PMV":
        parity.assert_f32(got[key], ref[key], f"{path} {key}")
    assert parity.bit_identical(got, ref), path
    del d, ws, sq, gbar
    torch.cuda.empty_cache()


def test_clipped_step_every_position_124m(orc):
    """The 124M-parameter shard (N=8) through both passes with global-norm
    clipping at 1.0, compared at every position: the oracle's mean gradient
    over the whole shard, its norm, and its update from the pristine state."""
    import torch

    import sharded_mixed_precision_rank_amd as zs
    from synth import workloads as W

    w = W.FLAT_124M_N8
    zs.set_grid_blocks(0)
    d = W.device_inputs(w)
    n = d["arena_len"]
    host = {k: d[k].cpu().numpy().copy() for k in "PMV"}  # the generator's draws, before the step
    ref_gbar, ref_sq = oracle_full_mean_and_norm(orc, torch, d["G"], 0, 1.0)
    assert orc.clip_coef(ref_sq, 1.0) < 1.0  # clipping is active
    ws = torch.empty(zs.two_pass_workspace_bytes(n), dtype=torch.uint8, device="cuda")
    sq = torch.empty(1, dtype=torch.float64, device="cuda")
    zs.reduce_grads_flat(d["G"], ws, sq)
    torch.cuda.synchronize()
    start = (256 - ws.data_ptr() % 256) % 256
    gbar = ws[start:start + 4 * n].view(torch.float32).cpu().numpy()
    assert np.array_equal(gbar.view(np.uint32), ref_gbar.view(np.uint32)), "pass 1 mean gradient"
    assert_norm(orc, float(sq.item()), ref_sq, n, 1.0)
    zs.adam_from_grads_flat(ws, n, d["P"], d["M"], d["V"], d["B"], w.hp(), w.step, sq, 1.0)
    torch.cuda.synchronize()
    got = dict(P=d["P"].cpu().numpy(), M=d["M"].cpu().numpy(), V=d["V"].cpu().numpy(),
               B=d["B"].view(torch.int16).cpu().numpy().view(np.uint16))
    P, M, V, B, taken = orc.adam_from_gbar(ref_gbar, host["P"], host["M"], host["V"], w.hp(), w.step, ref_sq, 1.0,
                                           threads=host_threads())
    assert taken
    ref = dict(P=P, M=M, V=V, B=B)
    parity.assert_step(got, ref, "clipped 124M, every position")
    assert parity.bit_identical(got, ref)
    del d, ws, sq
    torch.cuda.empty_cache()


def test_offload_full_size(orc):
    """The 124M-parameter shard (N=8) with its fp32 state in pinned host memory."""
    import torch

    import sharded_mixed_precision_rank_amd as zs
    from synth import workloads as W

    w = W.FLAT_124M_N8
    d = W.device_inputs(w)
    for key in "PMV":
        d[key] = d[key].cpu().pin_memory()
    torch.cuda.empty_cache()
    with zs.Offload() as off:
        off.step(d["G"], d["P"], d["M"], d["V"], d["B"], w.hp(), w.step)
    torch.cuda.synchronize()
    idx, _ = positions(w, d["arena_len"])
    got = dict(P=d["P"].numpy()[idx], M=d["M"].numpy()[idx], V=d["V"].numpy()[idx],
               B=d["B"].view(torch.int16)[torch.from_numpy(idx).cuda()].cpu().numpy().view(np.uint16))
    h = W.host_inputs_at(w, idx)
    P, M, V, B = orc.step(h["G"], h["P"], h["M"], h["V"], w.hp(), w.step)
    ref = dict(P=P, M=M, V=V, B=B)
    parity.assert_step(got, ref, "offload 124M")
    assert parity.bit_identical(got, ref)
    del d
    torch.cuda.empty_cache()


def test_flat_shard_beyond_2_31_elements(orc):
    """A flat shard of 2^31 + 12,345 parameters (N=2): element indices pass the
    32-bit range, so positions around 2^31 and at the tail are checked, through
    the fused step and the two-pass form, each with the write windows off and
    forced on (the windowed kernels' tile indices pass 2^31 too)."""
    import torch

    import sharded_mixed_precision_rank_amd as zs
    from synth import workloads as W

    n = (1 << 31) + 12_345
    w = W.FLAT_124M_N8.with_(name="flat-2^31+12345-N2", n_flat=n, N=2, step=3)
    zs.set_grid_blocks(0)
    d = W.device_inputs(w)
    rng = np.random.default_rng(31)
    edge = np.arange((1 << 31) - 4096, (1 << 31) + 4096, dtype=np.int64)
    idx = np.unique(np.concatenate([rng.integers(0, n, 50_000), edge, np.arange(n - 4096, n), np.arange(4096)]))
    h = W.host_inputs_at(w, idx)
    P, M, V, B = orc.step(h["G"], h["P"], h["M"], h["V"], w.hp(), w.step)
    ref = dict(P=P, M=M, V=V, B=B)
    pristine = {k: d[k].clone() for k in ("P", "M", "V")}
    ws = torch.empty(zs.two_pass_workspace_bytes(n), dtype=torch.uint8, device="cuda")
    sq = torch.empty(1, dtype=torch.float64, device="cuda")
    try:
        for window in ((1, 0), (256, 32)):
            zs.set_write_window(*window)
            assert (zs.write_window("flat", 2, n)[0] != 0) == (window[0] > 1)
            for path in ("two-pass", "fused"):
                print(f"beyond 2^31: {path}, window {window}", flush=True)
                for k in ("P", "M", "V"):
                    d[k].copy_(pristine[k])
                d["B"].zero_()
                if path == "two-pass":  # unclipped: the same result as the fused step
                    zs.reduce_grads_flat(d["G"], ws, sq)
                    zs.adam_from_grads_flat(ws, n, d["P"], d["M"], d["V"], d["B"], w.hp(), w.step, sq)
                else:
                    zs.reduce_adam_flat(d["G"], d["P"], d["M"], d["V"], d["B"], w.hp(), w.step)
                torch.cuda.synchronize()
                got = gather(torch, d, idx)
                parity.assert_step(got, ref, f"{w.name} {path} {window}")
                assert parity.bit_identical(got, ref), f"{path} beyond 2^31, window {window}"
    finally:
        zs.set_write_window(0)
    del d, pristine, ws, sq
    torch.cuda.empty_cache()
