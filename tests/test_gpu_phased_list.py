"""GPU parity of list plans on the phased schedule (list_phased_kernel) against the oracle, tensor by
tensor.

A wave takes 10 consecutive work items per super-chunk: whole tiles of one tensor go through phase A and
B, any other span (near a tensor's ends, scalar-only tensors) goes one item at a time after the
super-chunks, and the items after the last whole super-chunk go one per wave.  Forced grids of 1 to 3
workgroups (super-chunks of 120 to 360 items) put every case in lists the oracle checks in full."""
import numpy as np
import pytest

from tests import parity

pytestmark = pytest.mark.gpu

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1)


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


def got_of(d):
    return dict(P=d["P"].cpu().numpy(), M=d["M"].cpu().numpy(), V=d["V"].cpu().numpy(),
                B=d["B"].cpu().numpy().view(np.uint16))


@pytest.mark.parametrize("grid,N,count,hi", [
    (1, 64, 60, 70_000),     # tensors of a few to ~140 tiles, every span kind, many super-chunks
    (2, 50, 60, 70_000),     # the run-time replica count
    (3, 8, 200, 200_000),    # few replicas (phased only on request)
    (2, 64, 12, 2_000_000),  # long tensors: almost every span whole
])
def test_phased_list_matches_oracle(env, orc, grid, N, count, hi):
    """One set for every tensor, then three hyperparameter groups, then the device step."""
    from tests.test_gpu_list import arena_case, oracle_list, oracle_list_groups, small_ragged

    torch, zs, dev = env["torch"], env["zs"], env["dev"]
    zs.set_grid_blocks(grid)
    w = small_ragged(N, count, seed=grid * 100 + N, hi=hi, zero_frac=0.01, wd=0.1)
    host, d, offsets, L = arena_case(env, w)
    with zs.ListPlan.from_arenas(w.sizes, offsets, d["G"], d["P"], d["M"], d["V"], d["B"]) as plan:
        print(f"phased list: grid={grid} N={N} {len(w.sizes)} tensors, {w.n_params} params, "
              f"{plan.info()['n_items']} items", flush=True)
        plan.step(w.hp(), w.step)
        torch.cuda.synchronize()
        ref = oracle_list(orc, w, host, offsets, w.step, w.hp())
        parity.assert_step(got_of(d), ref, f"phased list N={N}")
        assert parity.bit_identical(got_of(d), ref), "one set"
        groups = [k % 3 for k in range(len(w.sizes))]
        hps = [dict(lr=1e-3 * (1 + g), beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1 * (g % 2))
               for g in range(3)]
        plan.set_groups(groups, 3)
        plan.step_groups(hps, w.step + 1)
        torch.cuda.synchronize()
        state = dict(G=host["G"], P=ref["P"], M=ref["M"], V=ref["V"])
        ref = oracle_list_groups(orc, w, state, offsets, w.step + 1, hps, groups)
        assert parity.bit_identical(got_of(d), ref), "groups"
        src = zs.StepSource(w.hp(), 1, 50, dev, start=w.step + 2)
        plan.step_devstep(src)
        torch.cuda.synchronize()
        state = dict(G=host["G"], P=ref["P"], M=ref["M"], V=ref["V"])
        ref = oracle_list(orc, w, state, offsets, w.step + 2, w.hp())
        assert parity.bit_identical(got_of(d), ref), "device step"
        assert src.status == 0


def test_phased_list_one_poll_per_barrier(env, orc):
    """A workgroup that stops waiting after one poll changes nothing in the results."""
    from tests.test_gpu_list import arena_case, oracle_list, small_ragged

    torch, zs = env["torch"], env["zs"]
    zs.set_grid_blocks(3)
    zs.set_phased_max_polls(1)
    w = small_ragged(64, 40, seed=5, hi=300_000, wd=0.1)
    host, d, offsets, L = arena_case(env, w)
    with zs.ListPlan.from_arenas(w.sizes, offsets, d["G"], d["P"], d["M"], d["V"], d["B"]) as plan:
        plan.step(w.hp(), w.step)
        torch.cuda.synchronize()
    assert parity.bit_identical(got_of(d), oracle_list(orc, w, host, offsets, w.step, w.hp()))


def test_phased_list_library_grid_and_schedules_agree(env):
    """The library's grid on the 70B/64 shard's first 96 per-layer tensors (about 140M parameters, N = 64):
    the phased, windowed and one-tile schedules give the same bits."""
    from synth import workloads as W

    torch, zs = env["torch"], env["zs"]
    w0 = W.list_llama70b_dp64_n64()
    w = w0.with_(name="llama70b-96", sizes=w0.sizes[:96])
    assert w.n_params >= 1 << 25
    d = W.device_inputs(w)
    offs, L = w.layout()
    pristine = {k: d[k].clone() for k in "PMV"}
    outs = {}
    for sched in ("phased", "windowed", "stream"):
        zs.set_flat_schedule(sched)
        for k in "PMV":
            d[k].copy_(pristine[k])
        with zs.ListPlan.from_arenas(w.sizes, offs, d["G"], d["P"], d["M"], d["V"], d["B"]) as plan:
            plan.step(w.hp(), w.step)
            torch.cuda.synchronize()
        outs[sched] = {k: d[k].view(torch.int32 if d[k].element_size() == 4 else torch.int16).cpu().numpy()
                       for k in ("P", "M", "V", "B")}
    for sched in ("windowed", "stream"):
        for k in ("P", "M", "V", "B"):
            assert np.array_equal(outs[sched][k], outs["phased"][k]), (sched, k)


def test_phased_list_in_a_graph(env, orc):
    """Captured once in a HIP graph and replayed three times with eager work between replays; every replay
    equals the oracle's step."""
    from tests.test_gpu_list import arena_case, oracle_list, small_ragged

    torch, zs, dev = env["torch"], env["zs"], env["dev"]
    zs.set_grid_blocks(2)
    w = small_ragged(64, 30, seed=9, hi=200_000, wd=0.1)
    host, d, offsets, L = arena_case(env, w)
    ref = oracle_list(orc, w, host, offsets, w.step, w.hp())
    pristine = {k: d[k].clone() for k in ("P", "M", "V", "B")}
    with zs.ListPlan.from_arenas(w.sizes, offsets, d["G"], d["P"], d["M"], d["V"], d["B"]) as plan:
        s = torch.cuda.Stream(device=dev)
        s.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            plan.step(w.hp(), w.step)
        torch.cuda.synchronize()
        for rep in range(3):
            for k in pristine:
                d[k].copy_(pristine[k])
            torch.cuda.synchronize()
            junk = torch.randn(1 << 20, device=dev).sum()
            g.replay()
            torch.cuda.synchronize()
            assert parity.bit_identical(got_of(d), ref), f"replay {rep}"
            del junk
