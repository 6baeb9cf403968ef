"""Seeded random shapes through every schedule of the flat step and of pass 1,
against the oracle bit for bit: replica counts 1-70 (templated and run-time
instances), shards of 0-400,000 parameters at head offsets 0-63 elements, and
forced grids of 1-5 workgroups, so that whole super-chunks, part
super-chunks, remainder tiles, partial tiles and head and tail elements come
in every combination.  The draws are fixed: 60 for the step (seed 2024), 30
for pass 1 (seed 2025); each case prints its parameters before it runs."""
import numpy as np
import pytest

from tests import parity
from tests.test_gpu_flat import HP, download, rand_host

pytestmark = pytest.mark.gpu

SCHEDULES = ("stream", "windowed", "phased")


def draws(count=60, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        N = int(rng.choice([1, 2, 3, 8, 16, 17, 32, 50, 64, 70]))
        n = int(rng.integers(0, 400_001)) if i % 6 else int(rng.integers(0, 2_000))
        off = int(rng.integers(0, 64))
        sched = SCHEDULES[i % 3]
        grid = int(rng.integers(1, 6))
        t = int(rng.integers(1, 20_000))
        out.append((i, N, n, off, sched, grid, t))
    return out


@pytest.fixture
def env():
    import torch

    import sharded_mixed_precision_rank_amd as zs

    yield dict(torch=torch, zs=zs, dev=torch.device("cuda:0"))
    zs.set_flat_schedule("auto")
    zs.set_grid_blocks(0)


@pytest.mark.parametrize("case", draws(), ids=lambda c: f"{c[0]}-N{c[1]}-n{c[2]}-off{c[3]}-{c[4]}-g{c[5]}")
def test_random_flat_step(env, orc, case):
    i, N, n, off, sched, grid, t = case
    torch, zs, dev = env["torch"], env["zs"], env["dev"]
    print(f"case {i}: N={N} n={n} offset={off} schedule={sched} grid={grid} t={t}", flush=True)
    host = rand_host(np.random.default_rng(1000 + i), N, n)
    pad = lambda a: np.concatenate([np.zeros(off, a.dtype), a])  # noqa: E731
    G = [torch.from_numpy(pad(g).view(np.int16)).to(dev)[off:] for g in host["G"]]
    d = dict(G=G, P=torch.from_numpy(pad(host["P"])).to(dev)[off:], M=torch.from_numpy(pad(host["M"])).to(dev)[off:],
             V=torch.from_numpy(pad(host["V"])).to(dev)[off:],
             B=torch.zeros(n + off, dtype=torch.int16, device=dev)[off:])
    zs.set_flat_schedule(sched)
    zs.set_grid_blocks(grid)
    hp = dict(HP, weight_decay=0.05)
    zs.reduce_adam_flat(d["G"], d["P"], d["M"], d["V"], d["B"], hp, t)
    torch.cuda.synchronize()
    P, M, V, B = orc.step(host["G"], host["P"], host["M"], host["V"], hp, t)
    assert parity.bit_identical(download(d), dict(P=P, M=M, V=V, B=B)), f"case {i}"


@pytest.mark.parametrize("case", draws(30, seed=2025), ids=lambda c: f"{c[0]}-N{c[1]}-n{c[2]}-off{c[3]}-{c[4]}-g{c[5]}")
def test_random_pass1(env, orc, case):
    """Pass 1's mean gradient bit for bit against the oracle, and its norm the same bits on every
    schedule."""
    i, N, n, off, sched, grid, _ = case
    torch, zs, dev = env["torch"], env["zs"], env["dev"]
    print(f"pass-1 case {i}: N={N} n={n} offset={off} schedule={sched} grid={grid}", flush=True)
    host = rand_host(np.random.default_rng(2000 + i), N, n)
    pad = lambda a: np.concatenate([np.zeros(off, a.dtype), a])  # noqa: E731
    G = [torch.from_numpy(pad(g).view(np.int16)).to(dev)[off:] for g in host["G"]]
    ws = torch.empty(zs.two_pass_workspace_bytes(n), dtype=torch.uint8, device=dev)
    sq = torch.empty(1, dtype=torch.float64, device=dev)
    norms = {}
    for s in (sched, "stream"):
        zs.set_flat_schedule(s)
        zs.set_grid_blocks(grid if s == sched else 0)
        zs.reduce_grads_flat(G, ws, sq, 1.0, "bf16")
        torch.cuda.synchronize()
        start = (256 - ws.data_ptr() % 256) % 256
        gbar = ws[start:start + 4 * n].view(torch.int32).cpu().numpy().view(np.uint32).copy()
        norms[s] = float(sq.cpu().item())
        ref = orc.reduce_unscale(host["G"], 0, 1.0)
        assert np.array_equal(gbar, ref.view(np.uint32)), f"pass-1 case {i}, schedule {s}"
    assert norms[sched] == norms["stream"], norms
