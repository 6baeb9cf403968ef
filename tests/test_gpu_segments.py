"""Shards covered in consecutive launches (zs_set_launch_bytes): with the limit forced down to a few
tiles per launch, every one-tile-per-workgroup path still gives the oracle's bits.  The flat step
(aligned, with a common head peel, and element by element; templated and run-time replica counts; the
device-step form), list plans (one set and hyperparameter groups) and both passes of the two-pass form
(whose norm must also keep its bits, the per-tile partials being the same whichever launch forms them)."""
import numpy as np
import pytest

from tests import parity
from tests.test_gpu_flat import HP, download, rand_host, upload

pytestmark = pytest.mark.gpu

HP_WD = dict(HP, weight_decay=0.1)


@pytest.fixture(scope="module")
def env():
    import torch

    import sharded_mixed_precision_rank_amd as zs

    zs.set_grid_blocks(0)
    yield dict(torch=torch, zs=zs, dev=torch.device("cuda:0"))
    zs.set_launch_bytes(0)
    zs.set_grid_blocks(0)


def _place(torch, dev, a, k):
    """a (host) copied to device memory k elements past the start of a buffer of its own."""
    dt = torch.int16 if a.dtype == np.uint16 else torch.float32
    buf = torch.zeros(a.size + 8, dtype=dt, device=dev)
    view = buf[k:k + a.size]
    view.copy_(torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a))
    return view


@pytest.mark.parametrize("N", [3, 5, 8, 64])
@pytest.mark.parametrize("layout", ["aligned", "peel", "elementwise"])
@pytest.mark.parametrize("tiles", [1, 3, 10**9])
def test_flat_step_in_consecutive_launches(env, orc, N, layout, tiles):
    torch, zs, dev = env["torch"], env["zs"], env["dev"]
    n = 100_003
    rng = np.random.default_rng(N * 7 + len(layout))
    host = rand_host(rng, N, n)
    shift = {"aligned": [0] * (N + 4), "peel": [3] * (N + 4),
             "elementwise": [(1 + r) % 4 for r in range(N)] + [3, 0, 1, 2]}[layout]
    G = [_place(torch, dev, host["G"][r], shift[r]) for r in range(N)]
    P, M, V = (_place(torch, dev, host[k], shift[N + j]) for j, k in enumerate("PMV"))
    B = _place(torch, dev, np.full(n, 0x7FBF, np.uint16), shift[N + 3])
    zs.set_launch_bytes(tiles * 512 * (2 * N + 26) if tiles < 10**9 else 0)
    try:
        print(f"flat in launches: N={N} layout={layout} tiles per launch={tiles}", flush=True)
        zs.reduce_adam_flat(G, P, M, V, B, HP_WD, 11)
        torch.cuda.synchronize()
    finally:
        zs.set_launch_bytes(0)
    got = dict(P=P.cpu().numpy(), M=M.cpu().numpy(), V=V.cpu().numpy(), B=B.cpu().numpy().view(np.uint16))
    rP, rM, rV, rB = orc.step(host["G"], host["P"], host["M"], host["V"], HP_WD, 11)
    assert parity.bit_identical(got, dict(P=rP, M=rM, V=rV, B=rB)), (N, layout, tiles)


@pytest.mark.parametrize("n", [0, 5, 511, 512, 513, 4097])
def test_short_shards_in_one_tile_launches(env, orc, n):
    """Shards of no whole tile, exactly one, and a few: one launch per tile, the edges in the last."""
    torch, zs, dev = env["torch"], env["zs"], env["dev"]
    N = 4
    host = rand_host(np.random.default_rng(n + 1), N, n)
    d = upload(torch, dev, host)
    d["B"] = torch.full((n,), 0x7FBF, dtype=torch.int16, device=dev)
    zs.set_launch_bytes(1)
    try:
        zs.reduce_adam_flat(d["G"], d["P"], d["M"], d["V"], d["B"], HP, 3)
        torch.cuda.synchronize()
    finally:
        zs.set_launch_bytes(0)
    P, M, V, B = orc.step(host["G"], host["P"], host["M"], host["V"], HP, 3)
    assert parity.bit_identical(download(d), dict(P=P, M=M, V=V, B=B)), n


def test_device_step_in_consecutive_launches(env, orc):
    """The device-step form reads the step once per launch: every launch takes the same row."""
    torch, zs, dev = env["torch"], env["zs"], env["dev"]
    N, n = 8, 50_001
    host = rand_host(np.random.default_rng(3), N, n)
    d = upload(torch, dev, host)
    d["B"] = torch.zeros(n, dtype=torch.int16, device=dev)
    src = zs.StepSource(HP_WD, 1, 10, dev, start=6)
    zs.set_launch_bytes(2 * 512 * (2 * N + 26))
    try:
        zs.reduce_adam_flat_devstep(d["G"], d["P"], d["M"], d["V"], d["B"], src)
        torch.cuda.synchronize()
    finally:
        zs.set_launch_bytes(0)
    P, M, V, B = orc.step(host["G"], host["P"], host["M"], host["V"], HP_WD, 6)
    assert parity.bit_identical(download(d), dict(P=P, M=M, V=V, B=B))
    assert src.status == 0


@pytest.mark.parametrize("N", [3, 16])
def test_list_plan_in_consecutive_launches(env, orc, N):
    from tests.test_gpu_list import arena_case, oracle_list, oracle_list_groups, small_ragged

    torch, zs = env["torch"], env["zs"]
    w = small_ragged(N, 60, seed=N + 40)
    host, d, offsets, L = arena_case(env, w)
    zs.set_launch_bytes(3 * 512 * (2 * N + 26))  # three work items per launch
    try:
        with zs.ListPlan.from_arenas(w.sizes, offsets, d["G"], d["P"], d["M"], d["V"], d["B"]) as plan:
            assert plan.info()["n_items"] > 240
            plan.step(w.hp(), w.step)
            torch.cuda.synchronize()
            got = dict(P=d["P"].cpu().numpy(), M=d["M"].cpu().numpy(), V=d["V"].cpu().numpy(),
                       B=d["B"].cpu().numpy().view(np.uint16))
            ref = oracle_list(orc, w, host, offsets, w.step, w.hp())
            assert parity.bit_identical(got, ref), "one set"
            groups = [k % 2 for k in range(len(w.sizes))]
            hps = [HP, HP_WD]
            plan.set_groups(groups, 2)
            plan.step_groups(hps, w.step + 1)
            torch.cuda.synchronize()
            got = dict(P=d["P"].cpu().numpy(), M=d["M"].cpu().numpy(), V=d["V"].cpu().numpy(),
                       B=d["B"].cpu().numpy().view(np.uint16))
            state = dict(G=host["G"], P=ref["P"], M=ref["M"], V=ref["V"])
            ref = oracle_list_groups(orc, w, state, offsets, w.step + 1, hps, groups)
            assert parity.bit_identical(got, ref), "groups"
    finally:
        zs.set_launch_bytes(0)


@pytest.mark.parametrize("fmt,offset", [("bf16", 0), ("bf16", 3), ("fp16", 40)])
def test_two_pass_in_consecutive_launches(env, orc, fmt, offset):
    from tests.test_gpu_twopass import rand_case, run

    zs = env["zs"]
    N, n = 8, 123_457
    scale = 256.0 if fmt == "fp16" else 1.0
    host = rand_case(np.random.default_rng(17 + offset), N, n, fmt=fmt, scale=scale, orc=orc)
    base = run(env, host, HP_WD, 4, max_norm=0.05, loss_scale=scale, gfmt=fmt, offset=offset)
    zs.set_launch_bytes(2 * 2048 * 30)  # N = 8: three pass-1 tiles (2048 params) or eight pass-2 tiles (512) per launch
    try:
        gbar, sqv, got = run(env, host, HP_WD, 4, max_norm=0.05, loss_scale=scale, gfmt=fmt, offset=offset)
    finally:
        zs.set_launch_bytes(0)
    ref_g = orc.reduce_unscale(host["G"], 1 if fmt == "fp16" else 0, scale)
    assert np.array_equal(gbar.view(np.uint32), ref_g.view(np.uint32))
    assert sqv == base[1], "the norm keeps its bits"
    P1, M1, V1, B1, taken = orc.adam_from_gbar(ref_g, host["P"], host["M"], host["V"], HP_WD, 4, sqv, 0.05)
    assert taken
    assert parity.bit_identical(got, dict(P=P1, M=M1, V=V1, B=B1))
    assert parity.bit_identical(got, base[2])
