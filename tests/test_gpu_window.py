"""GPU parity of the windowed flat step (persistent workgroups that hold
finished tiles and store them in device-clock windows) against the CPU oracle.

The shards are just above the size at which the library takes the windowed
kernel (65,536 whole 512-parameter tiles), start off a line boundary (a head
of peeled elements) and end in a partial tile and a tail.  Replica counts
cover templated (2, 64) and run-time (5, 100) kernel instances.  Each window
setting, including the extremes (a window open 63 ticks of a 64-tick period;
one open 1 tick of 2^20, which makes every wave store its older tile as soon
as both slots are full), and a forced small grid (many tiles per wave) must
give every output bit-identical to the oracle: the schedule of the stores
cannot change what is stored.
"""
import math

import numpy as np
import pytest

from tests import parity

pytestmark = pytest.mark.gpu

# 2^25 + 7 tiles + 123 parameters: 65,543 whole tiles after the head (plus a
# partial tile and a tail), past the 65,536-tile threshold
N_PARAMS = (1 << 25) + 7 * 512 + 123
OFFSET = 8  # elements: every array starts 32 or 16 bytes past a line boundary

WINDOWS = [(0, 0), (1, 0), (256, 32), (64, 63), (1 << 20, 1), (4096, 512)]
HP_WD = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1)


@pytest.fixture(scope="module")
def env():
    import torch

    import sharded_mixed_precision_rank_amd as zs

    yield dict(torch=torch, zs=zs, dev=torch.device("cuda:0"))
    zs.set_write_window(0)
    zs.set_grid_blocks(0)


def _inputs(N, step, wd):
    from synth import workloads as W

    w = W.FLAT_1M_N2.with_(n_flat=N_PARAMS, N=N, step=step, warm=True, weight_decay=wd)
    return w, W.host_inputs(w, 0, w.n_flat)


def _upload(torch, dev, host):
    def put(a, dtype):
        t = torch.empty(a.size + OFFSET, dtype=dtype, device=dev)
        view = t[OFFSET:]
        view.copy_(torch.from_numpy(a))
        return view

    G = [put(g.view(np.int16), torch.int16) for g in host["G"]]
    return dict(G=G, P=put(host["P"], torch.float32), M=put(host["M"], torch.float32),
                V=put(host["V"], torch.float32),
                B=put(np.full(host["P"].size, 0x7FBF, dtype=np.uint16).view(np.int16), torch.int16))


@pytest.mark.parametrize("N", [2, 5, 64, 100])
def test_windowed_step_matches_oracle(env, orc, N):
    torch, zs, dev = env["torch"], env["zs"], env["dev"]
    w, host = _inputs(N, 5000 if N == 64 else 100, 0.1 if N == 64 else 0.0)
    P, M, V, B = orc.step(host["G"], host["P"], host["M"], host["V"], w.hp(), w.step)
    ref = dict(P=P, M=M, V=V, B=B)
    for blocks in (0, 37):
        zs.set_grid_blocks(blocks)
        for period, open_ticks in WINDOWS:
            zs.set_write_window(period, open_ticks)
            print(f"windowed step: N={N} n={N_PARAMS} blocks={blocks} window={period}/{open_ticks}", flush=True)
            d = _upload(torch, dev, host)
            zs.reduce_adam_flat(d["G"], d["P"], d["M"], d["V"], d["B"], w.hp(), w.step)
            torch.cuda.synchronize()
            got = dict(P=d["P"].cpu().numpy(), M=d["M"].cpu().numpy(), V=d["V"].cpu().numpy(),
                       B=d["B"].cpu().numpy().view(np.uint16))
            what = f"N={N} blocks={blocks} window={period}/{open_ticks}"
            rep = parity.assert_step(got, ref, what)
            assert parity.bit_identical(got, ref), f"{what}: not bit-identical: {rep}"
            del d
    zs.set_grid_blocks(0)
    zs.set_write_window(0)


def test_windowed_device_step(env, orc):
    """The device-step form takes the same windowed kernel: equal to the host step."""
    torch, zs, dev = env["torch"], env["zs"], env["dev"]
    w, host = _inputs(8, 3, 0.0)
    zs.set_write_window(256, 64)
    a, b = _upload(torch, dev, host), _upload(torch, dev, host)
    src = zs.StepSource(w.hp(), 1, 10, dev, start=3)
    zs.reduce_adam_flat_devstep(a["G"], a["P"], a["M"], a["V"], a["B"], src)
    zs.set_write_window(1)
    zs.reduce_adam_flat(b["G"], b["P"], b["M"], b["V"], b["B"], w.hp(), 3)
    torch.cuda.synchronize()
    zs.set_write_window(0)
    for k in ("P", "M", "V", "B"):
        assert torch.equal(a[k], b[k]), k
    assert src.status == 0
    P, M, V, B = orc.step(host["G"], host["P"], host["M"], host["V"], w.hp(), 3)
    got = dict(P=a["P"].cpu().numpy(), M=a["M"].cpu().numpy(), V=a["V"].cpu().numpy(),
               B=a["B"].cpu().numpy().view(np.uint16))
    assert parity.bit_identical(got, dict(P=P, M=M, V=V, B=B))


@pytest.mark.parametrize("N,fmt,scale", [(64, "bf16", 1.0), (8, "fp16", 256.0), (100, "bf16", 1.0)])
def test_windowed_pass1_matches_unwindowed_and_oracle(env, orc, N, fmt, scale):
    """Pass 1 of the two-pass form under write windows: the mean gradients bit-identical to the
    oracle's and the squared norm bit-identical to the unwindowed pass (the same fixed-order tile
    partials), for every window setting and grid; then pass 2 from it against the oracle.  The shard
    has 16,385 whole 2048-parameter tiles after the head, past the 16,384-tile threshold."""
    torch, zs, dev = env["torch"], env["zs"], env["dev"]
    w, host = _inputs(N, 40, 0.0)
    n = N_PARAMS
    d = _upload(torch, dev, host)
    ws = torch.empty(zs.two_pass_workspace_bytes(n), dtype=torch.uint8, device=dev)
    start = (256 - ws.data_ptr() % 256) % 256
    fmt_id = 1 if fmt == "fp16" else 0
    ref_g = orc.reduce_unscale(host["G"], fmt_id, scale)
    # the norm's definition, summed exactly: over 2^25 terms a plain sequential double sum (the
    # oracle's) drifts by up to n*u, more than the GPU's fixed-order tree (a chain of about 50 adds
    # of exact squares, so within 50u); 1e-13 is far below what one dropped or doubled tile moves
    ref_sq = math.fsum((ref_g.astype(np.float64) ** 2).tolist())
    results = []
    for blocks in (0, 37):
        zs.set_grid_blocks(blocks)
        for period, open_ticks in [(1, 0), (0, 0), (256, 32), (64, 63), (1 << 20, 1), (4096, 256)]:
            zs.set_write_window(period, open_ticks)
            print(f"windowed pass 1: N={N} {fmt} n={n} blocks={blocks} window={period}/{open_ticks} "
                  f"(takes {zs.write_window('reduce', N, n)})", flush=True)
            ws.fill_(0xFF)   # NaN everywhere the pass does not write
            sq = torch.full((1,), float("nan"), dtype=torch.float64, device=dev)
            zs.reduce_grads_flat(d["G"], ws, sq, scale, fmt)
            torch.cuda.synchronize()
            g = ws[start:start + 4 * n].cpu().numpy().view(np.float32)
            assert np.array_equal(g.view(np.uint32), ref_g.view(np.uint32)), f"{period}/{open_ticks}: means"
            results.append(sq.item())
    zs.set_grid_blocks(0)
    zs.set_write_window(0)
    assert len(set(results)) == 1, results
    assert abs(results[0] - ref_sq) <= 1e-13 * ref_sq, (results[0], ref_sq)
    zs.adam_from_grads_flat(ws, n, d["P"], d["M"], d["V"], d["B"], w.hp(), w.step, sq, 1.0, "bf16")
    torch.cuda.synchronize()
    P1, M1, V1, B1, taken = orc.adam_from_gbar(ref_g, host["P"], host["M"], host["V"], w.hp(), w.step,
                                               results[0], 1.0)
    assert taken
    got = dict(P=d["P"].cpu().numpy(), M=d["M"].cpu().numpy(), V=d["V"].cpu().numpy(),
               B=d["B"].cpu().numpy().view(np.uint16))
    assert parity.bit_identical(got, dict(P=P1, M=M1, V=V1, B=B1))


def test_windowed_kernels_in_a_graph(env, orc):
    """The windowed flat step and the windowed pass 1, captured in HIP graphs and replayed: every
    replay equals the same call run eagerly (with eager work and synchronisation between replays)."""
    torch, zs, dev = env["torch"], env["zs"], env["dev"]
    w, host = _inputs(2, 9, 0.0)
    zs.set_write_window(256, 32)
    try:
        a, b = _upload(torch, dev, host), _upload(torch, dev, host)
        ws_a = torch.empty(zs.two_pass_workspace_bytes(N_PARAMS), dtype=torch.uint8, device=dev)
        ws_b = torch.empty_like(ws_a)
        sq_a = torch.empty(1, dtype=torch.float64, device=dev)
        sq_b = torch.empty_like(sq_a)
        assert zs.write_window("flat", 2, N_PARAMS) == (256, 32)
        assert zs.write_window("reduce", 2, N_PARAMS) == (256, 32)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):  # first calls outside capture settle the one-time occupancy queries
            zs.reduce_adam_flat(a["G"], a["P"], a["M"], a["V"], a["B"], w.hp(), w.step)
            zs.reduce_grads_flat(a["G"], ws_a, sq_a)
        torch.cuda.current_stream().wait_stream(side)
        zs.reduce_adam_flat(b["G"], b["P"], b["M"], b["V"], b["B"], w.hp(), w.step)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            zs.reduce_adam_flat(a["G"], a["P"], a["M"], a["V"], a["B"], w.hp(), w.step)
            zs.reduce_grads_flat(a["G"], ws_a, sq_a)
        for replay in range(3):
            print(f"windowed kernels in a graph: replay {replay}", flush=True)
            ws_a.fill_(0)
            ws_b.fill_(0xFF)
            sq_a.fill_(-1.0)
            graph.replay()
            zs.reduce_adam_flat(b["G"], b["P"], b["M"], b["V"], b["B"], w.hp(), w.step)
            zs.reduce_grads_flat(b["G"], ws_b, sq_b)
            torch.cuda.synchronize()
            for k in ("P", "M", "V", "B"):
                assert torch.equal(a[k], b[k]), f"replay {replay}: {k}"
            sa = (256 - ws_a.data_ptr() % 256) % 256
            sb = (256 - ws_b.data_ptr() % 256) % 256
            assert torch.equal(ws_a[sa:sa + 4 * N_PARAMS], ws_b[sb:sb + 4 * N_PARAMS]), f"replay {replay}: means"
            assert sq_a.item() == sq_b.item(), f"replay {replay}: norm"
    finally:
        zs.set_write_window(0)


# a ragged list of about 2^25 parameters: empty, 1- and 9-element (scalar-only) tensors, tensors that end in
# partial wave tiles, and tensors of many wave tiles
LIST_SIZES = (1, 9, 0, 5_000, 4_097, 70_001, (1 << 20) + 3, 3_000_001, 10_000_003, 20_000_017)


@pytest.mark.parametrize("N,window", [(64, (0, 0)), (50, (0, 0)), (8, (256, 32))])
def test_windowed_list_plan_matches_oracle(env, orc, N, window):
    """List plans under write windows (the windowed schedule's default window at N = 64 and at the
    run-time count 50, a forced window at N = 8): one set for every tensor, then hyperparameter groups, then
    the device step, each bit-identical to the oracle applied tensor by tensor (the gaps between tensors
    untouched)."""
    from synth import workloads as W
    from tests.test_gpu_list import arena_case, oracle_list, oracle_list_groups

    torch, zs, dev = env["torch"], env["zs"], env["dev"]
    w = W.Workload(f"window-list-N{N}", N=N, step=7, weight_decay=0.1, warm=True, sizes=LIST_SIZES, seed=N)
    assert w.n_params >= 1 << 25
    host, d, offsets, L = arena_case(env, w)

    def got():
        return dict(P=d["P"].cpu().numpy(), M=d["M"].cpu().numpy(), V=d["V"].cpu().numpy(),
                    B=d["B"].cpu().numpy().view(np.uint16))

    zs.set_write_window(*window)
    zs.set_flat_schedule("windowed")
    try:
        with zs.ListPlan.from_arenas(w.sizes, offsets, d["G"], d["P"], d["M"], d["V"], d["B"]) as plan:
            print(f"windowed list: N={N} window={window} (takes {zs.write_window('list', N, w.n_params)})",
                  flush=True)
            assert zs.write_window("list", N, w.n_params) != (0, 0)
            plan.step(w.hp(), w.step)
            torch.cuda.synchronize()
            ref = oracle_list(orc, w, host, offsets, w.step, w.hp())
            assert parity.bit_identical(got(), ref), "one set"
            groups = [k % 3 for k in range(len(w.sizes))]
            hps = [dict(lr=1e-3 * (1 + g), beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1 * (g % 2))
                   for g in range(3)]
            plan.set_groups(groups, 3)
            plan.step_groups(hps, 8)
            torch.cuda.synchronize()
            state = dict(G=host["G"], P=ref["P"], M=ref["M"], V=ref["V"])
            ref = oracle_list_groups(orc, w, state, offsets, 8, hps, groups)
            assert parity.bit_identical(got(), ref), "groups"
            src = zs.StepSource(w.hp(), 1, 20, dev, start=9)
            plan.step_devstep(src)
            torch.cuda.synchronize()
            state = dict(G=host["G"], P=ref["P"], M=ref["M"], V=ref["V"])
            ref = oracle_list(orc, w, state, offsets, 9, w.hp())
            assert parity.bit_identical(got(), ref), "device step"
            assert src.status == 0
    finally:
        zs.set_write_window(0)
        zs.set_flat_schedule("auto")


@pytest.mark.parametrize("N,window,schedule", [(64, (0, 0), "windowed"), (8, (256, 32), "windowed"),
                                               (64, (0, 0), "phased"), (50, (0, 0), "phased")])
def test_windowed_list_plan_with_peels_and_scalar_tensors(env, orc, N, window, schedule):
    """List plans under write windows (and on the phased schedule) on tensors in buffers of their own:
    2^25 + 1,003 parameters whose
    arrays all start 3 elements past a 16-byte boundary (a 5-element head peel, whole tiles, a partial
    tile and tail elements), 100 parameters with that phase, and 10,000 parameters whose arrays share no
    16-byte phase (stepped element by element).  Bit-identical to the oracle per tensor, over two steps."""
    torch, zs, dev = env["torch"], env["zs"], env["dev"]
    rng = np.random.default_rng(N + 11)
    n_of = [(1 << 25) + 1003, 100, 10_000]
    # element offsets of each tensor's arrays in their buffers: G_0..G_{N-1}, P, M, V, B
    shifts = [[3] * (N + 4), [3] * (N + 4), [(1 + r) % 4 for r in range(N)] + [3, 0, 1, 2]]
    host, tensors, views = [], [], []
    for n, sh in zip(n_of, shifts):
        base = ((rng.standard_normal(n) * 1e-3).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        G = [np.roll(base, 977 * r) for r in range(N)]  # distinct replicas, cheaply
        P = (rng.standard_normal(n) * 0.02).astype(np.float32)
        M = (rng.standard_normal(n) * 1e-2).astype(np.float32)
        V = np.abs(rng.standard_normal(n) * 1e-4).astype(np.float32)
        host.append(dict(G=G, P=P, M=M, V=V))

        def place(a, k, dtype):
            buf = torch.zeros(n + 8, dtype=dtype, device=dev)
            view = buf[k:k + n]
            view.copy_(torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a))
            return view

        g = [place(G[r], sh[r], torch.int16) for r in range(N)]
        p, m, v = (place(a, sh[N + j], torch.float32) for j, a in enumerate((P, M, V)))
        b = place(np.zeros(n, np.uint16), sh[N + 3], torch.int16)
        views.append((p, m, v, b))
        tensors.append(zs.ShardTensor(g, p, m, v, b))
    assert sum(n_of) >= 1 << 25
    zs.set_write_window(*window)
    zs.set_flat_schedule(schedule)
    try:
        if schedule == "windowed":
            assert zs.write_window("list", N, sum(n_of))[0] > 0, "the plan takes write windows"
        else:
            assert zs.flat_schedule(N, sum(n_of)) == "phased"
        with zs.ListPlan(tensors, N) as plan:
            print(f"list, peels and scalar tensors: N={N} window={window} schedule={schedule}", flush=True)
            for t in (3, 4):
                plan.step(HP_WD, t)
                torch.cuda.synchronize()
                for k, (h, (p, m, v, b)) in enumerate(zip(host, views)):
                    rP, rM, rV, rB = orc.step(h["G"], h["P"], h["M"], h["V"], HP_WD, t)
                    got = dict(P=p.cpu().numpy(), M=m.cpu().numpy(), V=v.cpu().numpy(),
                               B=b.cpu().numpy().view(np.uint16))
                    assert parity.bit_identical(got, dict(P=rP, M=rM, V=rV, B=rB)), f"tensor {k}, step {t}"
                    h.update(P=rP, M=rM, V=rV)
    finally:
        zs.set_write_window(0)
        zs.set_flat_schedule("auto")
