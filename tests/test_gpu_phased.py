"""GPU parity of the phased schedule of the flat step (flat_phased_kernel)
against the oracle, and against the other two schedules.

The phased kernel cuts a shard into super-chunks of (workgroups x 12 waves x 12
tiles) whole tiles, then a part super-chunk of 6 to 11 tiles per wave when at
least half a super-chunk's tiles are left, then the whole tiles after those
one per wave, then the one partial tile and the head and tail elements.  A
forced small grid (1 to 3 workgroups: super-chunks of 73,728 to 221,184
parameters) puts every one of those parts in shards the oracle checks in full;
the library's own grid is checked on a shard of 2^25 + 3,707 parameters (one
super-chunk, a part super-chunk of 9 tiles per wave and a remainder).  The
grid barrier only shapes timing: the same results must come out when a
workgroup gives up waiting after a single poll."""
import numpy as np
import pytest

from tests import parity
from tests.test_gpu_flat import HP, download, rand_host, upload

pytestmark = pytest.mark.gpu

HP_WD = dict(HP, weight_decay=0.1)
SUPER = 12 * 12 * 512  # parameters per super-chunk per workgroup
ROW = 12 * 512  # parameters of one tile per wave of one workgroup


@pytest.fixture
def env():
    import torch

    import sharded_mixed_precision_rank_amd as zs

    zs.set_flat_schedule("phased")
    zs.set_grid_blocks(0)
    yield dict(torch=torch, zs=zs, dev=torch.device("cuda:0"))
    zs.set_flat_schedule("auto")
    zs.set_grid_blocks(0)
    zs.set_phased_max_polls(0)


def run(env, host, hp, t, offset=0):
    """One step on device copies of `host`, the arrays starting `offset` elements into their buffers."""
    torch, zs, dev = env["torch"], env["zs"], env["dev"]
    n = host["P"].size
    pad = lambda a: np.concatenate([np.zeros(offset, a.dtype), a])  # noqa: E731
    G = [torch.from_numpy(pad(g).view(np.int16)).to(dev)[offset:] for g in host["G"]]
    d = dict(G=G, P=torch.from_numpy(pad(host["P"])).to(dev)[offset:],
             M=torch.from_numpy(pad(host["M"])).to(dev)[offset:], V=torch.from_numpy(pad(host["V"])).to(dev)[offset:],
             B=torch.full((n + offset,), 0x7FBF, dtype=torch.int16, device=dev)[offset:])
    zs.reduce_adam_flat(d["G"], d["P"], d["M"], d["V"], d["B"], hp, t)
    torch.cuda.synchronize()
    return download(d)


def check(env, orc, host, hp, t, what, offset=0):
    got = run(env, host, hp, t, offset)
    P, M, V, B = orc.step(host["G"], host["P"], host["M"], host["V"], hp, t)
    ref = dict(P=P, M=M, V=V, B=B)
    parity.assert_step(got, ref, what)
    assert parity.bit_identical(got, ref), what
    return got


@pytest.mark.parametrize("grid,N,n,offset", [
    (1, 64, 2 * SUPER + 777, 0),            # two super-chunks, remainder tiles, partial tile, tail
    (1, 64, 2 * SUPER + 777, 5),            # the same behind a 5-element head peel
    (2, 64, 3 * 2 * SUPER, 0),              # whole super-chunks only
    (3, 50, 2 * 3 * SUPER + 512 * 40 + 9, 0),   # run-time replica count
    (2, 8, 4 * 2 * SUPER + 3, 61),          # few replicas, a 61-element offset
    (2, 3, 2 * SUPER - 1, 0),               # less than one super-chunk: a part super-chunk of 11 tiles per wave
    (1, 64, 2 * SUPER + 7 * ROW + 777, 0),  # a part super-chunk of 7 tiles per wave, remainder, partial tile
    (2, 64, 2 * SUPER + 22 * ROW + 515, 3), # a part of 11 tiles per wave behind a 3-element peel
    (3, 50, 3 * SUPER + 18 * ROW + 5, 0),   # a part of 6 tiles per wave at a run-time replica count
    (1, 64, 2 * SUPER + 5 * ROW + 9, 0),    # 5 tiles per wave left: below a part, one tile per wave
    (2, 3, 10 * ROW + 7, 0),                # less than half a super-chunk: remainder tiles only
    (1, 64, 512, 0),                        # one tile
    (1, 65, 1300, 3),                       # one tile, a partial one, head and tail
])
def test_phased_matches_oracle(env, orc, grid, N, n, offset):
    env["zs"].set_grid_blocks(grid)
    rng = np.random.default_rng(grid * 100_000 + N * 100 + offset)
    host = rand_host(rng, N, n)
    check(env, orc, host, HP_WD, 1234, f"phased grid={grid} N={N} n={n} offset={offset}", offset)


def test_phased_bounded_barrier_wait(env, orc):
    """One poll per barrier: every workgroup goes on at once, the results are the same bits."""
    zs = env["zs"]
    zs.set_grid_blocks(3)
    zs.set_phased_max_polls(1)
    rng = np.random.default_rng(77)
    host = rand_host(rng, 64, 4 * 3 * SUPER + 1000)
    check(env, orc, host, HP_WD, 9, "phased, one poll per barrier")


def drawn(n, N=64):
    """A flat workload of n parameters and N replicas (the 70B/64 shard's draws, warm state, step 5000,
    weight decay 0.1), and its inputs drawn in device memory by the counter-based generator."""
    from synth import workloads as W

    w = W.FLAT_70B_DP64_N64.with_(name=f"flat-{n}-N{N}", n_flat=n, N=N)
    d = W.device_inputs(w)
    d["B"] = d["B"].view(env_torch().int16)   # bf16 bits, downloadable as int16
    return w, d


def env_torch():
    import torch

    return torch


def test_phased_library_grid_multi_super_chunk(env, orc):
    """The library's own grid (one workgroup per compute unit) on 2^25 + 3,707 parameters at N = 64 (a
    super-chunk and a part super-chunk), every position against the oracle (the host redraws the same
    inputs)."""
    from synth import workloads as W

    torch = env["torch"]
    n = (1 << 25) + 3_707
    w, d = drawn(n)
    env["zs"].reduce_adam_flat(d["G"], d["P"], d["M"], d["V"], d["B"], w.hp(), w.step)
    torch.cuda.synchronize()
    got = download(d)
    del d
    torch.cuda.empty_cache()
    h = W.host_inputs(w, 0, n)
    P, M, V, B = orc.step(h["G"], h["P"], h["M"], h["V"], w.hp(), w.step)
    ref = dict(P=P, M=M, V=V, B=B)
    parity.assert_step(got, ref, "phased, library grid")
    assert parity.bit_identical(got, ref)


def test_schedules_agree(env):
    """The same inputs through the phased, windowed and per-tile schedules give the same bits."""
    torch, zs = env["torch"], env["zs"]
    w, d = drawn((1 << 25) + 12_345)
    pristine = {k: d[k].clone() for k in "PMV"}
    outs = {}
    try:
        for sched in ("phased", "windowed", "stream"):
            zs.set_flat_schedule(sched)
            for k in "PMV":
                d[k].copy_(pristine[k])
            zs.reduce_adam_flat(d["G"], d["P"], d["M"], d["V"], d["B"], w.hp(), w.step)
            torch.cuda.synchronize()
            outs[sched] = download(d)
    finally:
        zs.set_flat_schedule("phased")
    for sched in ("windowed", "stream"):
        assert parity.bit_identical(outs[sched], outs["phased"]), sched
    del d, pristine
    torch.cuda.empty_cache()


def test_phased_device_step(env, orc):
    """The device-step form on the phased schedule: the step index and folded scalars come from a
    device table; a step outside the table leaves everything untouched."""
    torch, zs, dev = env["torch"], env["zs"], env["dev"]
    zs.set_grid_blocks(2)
    rng = np.random.default_rng(31)
    n = 2 * 2 * SUPER + 4_321
    host = rand_host(rng, 64, n)
    d = upload(torch, dev, host)
    d["B"] = torch.zeros(n, dtype=torch.int16, device=dev)
    src = zs.StepSource(HP_WD, 100, 3, device=dev, start=101)
    zs.reduce_adam_flat_devstep(d["G"], d["P"], d["M"], d["V"], d["B"], src)
    torch.cuda.synchronize()
    got = download(d)
    P, M, V, B = orc.step(host["G"], host["P"], host["M"], host["V"], HP_WD, 101)
    assert parity.bit_identical(got, dict(P=P, M=M, V=V, B=B))
    src.advance()
    src.advance()  # step 103: outside [100, 103)
    zs.reduce_adam_flat_devstep(d["G"], d["P"], d["M"], d["V"], d["B"], src)
    torch.cuda.synchronize()
    assert src.status == 1
    assert parity.bit_identical(download(d), got)


def test_phased_in_a_graph(env, orc):
    """Captured once in a HIP graph (the barrier counter's clear is a kernel node), replayed four times
    with eager work and synchronisation between replays; every replay equals the eager step.  The shard
    has three super-chunks, a part super-chunk of 7 tiles per wave and a partial tile."""
    torch, zs, dev = env["torch"], env["zs"], env["dev"]
    zs.set_grid_blocks(2)
    rng = np.random.default_rng(41)
    n = 3 * 2 * SUPER + 2 * 7 * ROW + 100
    host = rand_host(rng, 64, n)
    P, M, V, B = orc.step(host["G"], host["P"], host["M"], host["V"], HP_WD, 7)
    ref = dict(P=P, M=M, V=V, B=B)
    d = upload(torch, dev, host)
    d["B"] = torch.zeros(n, dtype=torch.int16, device=dev)
    pristine = {k: d[k].clone() for k in "PMV"}
    s = torch.cuda.Stream(device=dev)
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        zs.reduce_adam_flat(d["G"], d["P"], d["M"], d["V"], d["B"], HP_WD, 7)
    torch.cuda.synchronize()
    for rep in range(4):
        for k in "PMV":
            d[k].copy_(pristine[k])
        d["B"].zero_()
        torch.cuda.synchronize()
        junk = torch.randn(1 << 20, device=dev).sum()  # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert parity.bit_identical(download(d), ref), f"replay {rep}"
        del junk


def test_two_phased_steps_at_once(env, orc):
    """Two phased steps on two streams at the same time (two barrier slots); each gives its own
    oracle's bits."""
    torch, zs, dev = env["torch"], env["zs"], env["dev"]
    zs.set_grid_blocks(2)
    zs.set_phased_max_polls(2000)   # bounded waits if the two grids share the device
    rng = np.random.default_rng(51)
    hosts = [rand_host(rng, 64, 2 * 2 * SUPER + 999), rand_host(rng, 64, 3 * 2 * SUPER + 5)]
    ds = []
    for h in hosts:
        d = upload(torch, dev, h)
        d["B"] = torch.zeros(h["P"].size, dtype=torch.int16, device=dev)
        ds.append(d)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(device=dev) for _ in ds]
    for d, st in zip(ds, streams):
        zs.reduce_adam_flat(d["G"], d["P"], d["M"], d["V"], d["B"], HP_WD, 3, stream=st)
    torch.cuda.synchronize()
    for h, d in zip(hosts, ds):
        P, M, V, B = orc.step(h["G"], h["P"], h["M"], h["V"], HP_WD, 3)
        assert parity.bit_identical(download(d), dict(P=P, M=M, V=V, B=B))
