"""GPU parity of pass 1 of the two-pass form on the phased schedule
(reduce_phased_kernel): the mean gradient bit for bit and the squared norm
against the oracle, and both the same bits as on the one-tile schedule.

Pass 1 takes super-chunks of (workgroups x 12 waves x 14 tiles: 10 in
registers, 4 in LDS) whole wave tiles, then a part super-chunk of 7 to 13
tiles per wave when at least half a super-chunk's tiles are left.  Forced
small grids (1 to 3 workgroups: super-chunks of 86,016 to 258,048
parameters) put whole super-chunks, part super-chunks, the norm tiles after
them, the partial tile and the head elements in shards the oracle checks in
full; the library's own grid is checked on 56,626,811 parameters at N = 64
(two super-chunks and a part of 8 tiles per wave)."""
import numpy as np
import pytest

from tests.test_gpu_twopass import HP, rand_case

pytestmark = pytest.mark.gpu

SUPER = 12 * 14 * 512  # parameters per super-chunk per workgroup
ROW = 12 * 512  # parameters of one tile per wave of one workgroup


@pytest.fixture
def env():
    import torch

    import sharded_mixed_precision_rank_amd as zs

    zs.set_grid_blocks(0)
    yield dict(torch=torch, zs=zs, dev=torch.device("cuda:0"))
    zs.set_flat_schedule("auto")
    zs.set_grid_blocks(0)
    zs.set_phased_max_polls(0)


def pass1(env, G, n, schedule, loss_scale=1.0, gfmt="bf16"):
    """Pass 1 on device replicas G under `schedule`: (mean gradient as uint32 bits, squared norm)."""
    torch, zs, dev = env["torch"], env["zs"], env["dev"]
    zs.set_flat_schedule(schedule)
    ws = torch.empty(zs.two_pass_workspace_bytes(n), dtype=torch.uint8, device=dev)
    sq = torch.empty(1, dtype=torch.float64, device=dev)
    zs.reduce_grads_flat(G, ws, sq, loss_scale, gfmt)
    torch.cuda.synchronize()
    start = (256 - ws.data_ptr() % 256) % 256
    return ws[start:start + 4 * n].view(torch.int32).cpu().numpy().view(np.uint32).copy(), float(sq.cpu().item())


def assert_norm(sq, ref_sq, n):
    """The norm against the oracle's: the two add the same n doubles in different orders, so they may
    differ by the bound on the rounding of a sum of n non-negative terms, n * 2^-53 of the sum each."""
    assert abs(sq - ref_sq) <= 2.0 * n * 2.0 ** -53 * ref_sq, (sq, ref_sq)


def device_replicas(env, host, offset):
    torch, dev = env["torch"], env["dev"]
    pad = np.zeros(offset, np.uint16)
    return [torch.from_numpy(np.concatenate([pad, g]).view(np.int16)).to(dev)[offset:] for g in host["G"]]


@pytest.mark.parametrize("grid,N,n,offset,gfmt,scale", [
    (1, 64, 2 * SUPER + 2048 * 3 + 777, 0, "bf16", 1.0),   # two super-chunks, norm tiles after, a partial one
    (2, 50, 3 * 2 * SUPER + 100, 5, "bf16", 1.0),         # run-time replica count behind a head peel
    (3, 32, 2 * 3 * SUPER, 0, "fp16", 256.0),             # whole super-chunks only; fp16, loss-scaled
    (2, 64, 2 * 2 * SUPER + 9, 61, "fp16", 65536.0),      # a 61-element offset, fp16
    (1, 8, SUPER - 1, 0, "bf16", 1.0),                    # less than one super-chunk: a part of 13 tiles per wave
    (1, 8, 5 * ROW + 7, 0, "bf16", 1.0),                  # less than half a super-chunk: the one-tile kernel
    (1, 64, 2 * SUPER + 7 * ROW + 2048 + 5, 0, "bf16", 1.0),   # a part super-chunk of 7 tiles per wave
    (2, 64, 2 * SUPER + 18 * ROW + 777, 3, "fp16", 1024.0),    # a part of 9 tiles per wave behind a peel
    (3, 50, 3 * SUPER + 21 * ROW + 11, 0, "bf16", 1.0),        # a part of 7 tiles per wave, run-time N
    (3, 50, 3 * SUPER + 18 * ROW + 11, 0, "bf16", 1.0),        # 6 tiles per wave left: no part
    (1, 64, 2 * SUPER + 4 * ROW + 100, 0, "bf16", 1.0),        # 4 tiles per wave left: no part
])
def test_phased_pass1_matches_oracle_and_stream(env, orc, grid, N, n, offset, gfmt, scale):
    zs = env["zs"]
    rng = np.random.default_rng(grid * 10_000 + N * 10 + offset)
    host = rand_case(rng, N, n, gfmt, scale, orc=orc)
    G = device_replicas(env, host, offset)
    zs.set_grid_blocks(grid)
    g_ph, sq_ph = pass1(env, G, n, "phased", scale, gfmt)
    zs.set_grid_blocks(0)
    g_st, sq_st = pass1(env, G, n, "stream", scale, gfmt)
    assert np.array_equal(g_ph, g_st), "mean gradient differs between schedules"
    assert sq_ph == sq_st, (sq_ph, sq_st)
    ref_g = orc.reduce_unscale(host["G"], 1 if gfmt == "fp16" else 0, scale)
    assert np.array_equal(g_ph, ref_g.view(np.uint32))
    assert_norm(sq_ph, orc.sqnorm(ref_g), n)


def test_phased_pass1_one_poll_per_barrier(env, orc):
    """A workgroup that stops waiting after one poll changes nothing in the results."""
    zs = env["zs"]
    rng = np.random.default_rng(5)
    n = 4 * 3 * SUPER + 1000
    host = rand_case(rng, 64, n)
    G = device_replicas(env, host, 0)
    zs.set_grid_blocks(3)
    zs.set_phased_max_polls(1)
    g_ph, sq_ph = pass1(env, G, n, "phased")
    zs.set_grid_blocks(0)
    g_st, sq_st = pass1(env, G, n, "stream")
    assert np.array_equal(g_ph, g_st) and sq_ph == sq_st
    ref_g = orc.reduce_unscale(host["G"], 0, 1.0)
    assert np.array_equal(g_ph, ref_g.view(np.uint32))
    assert_norm(sq_ph, orc.sqnorm(ref_g), n)


def test_phased_pass1_library_grid(env, orc):
    """The library's own grid at N = 64 on 56,626,811 parameters (the automatic schedule: two
    super-chunks and a part super-chunk of 8 tiles per wave on 256 compute units): the mean gradient and
    the norm are the bits of the one-tile schedule, and the mean gradient is the oracle's at 100,000
    sampled positions (the host redraws the same inputs there)."""
    from synth import workloads as W

    torch, zs = env["torch"], env["zs"]
    n = 2 * 256 * SUPER + 8 * 256 * ROW + 3_707
    assert zs.reduce_schedule(64, n) == "phased"
    w = W.FLAT_70B_DP64_N64.with_(name="pass1", n_flat=n)
    d = W.device_inputs(w)
    G = [g.view(torch.int16) for g in d["G"]]
    g_ph, sq_ph = pass1(env, G, n, "auto")
    g_st, sq_st = pass1(env, G, n, "stream")
    del d, G
    torch.cuda.empty_cache()
    assert np.array_equal(g_ph, g_st)
    assert sq_ph == sq_st
    idx = np.sort(np.random.default_rng(9).choice(n, 100_000, replace=False))
    h = W.host_inputs_at(w, idx)
    ref_g = orc.reduce_unscale(h["G"], 0, 1.0)
    assert np.array_equal(g_ph[idx], ref_g.view(np.uint32))


def test_phased_clipped_step_in_a_graph(env, orc):
    """The clipped step (phased pass 1, finalize, pass 2) captured once in a HIP graph and replayed three
    times with eager work between replays; every replay equals the oracle's step."""
    torch, zs, dev = env["torch"], env["zs"], env["dev"]
    zs.set_flat_schedule("phased")
    zs.set_grid_blocks(2)
    rng = np.random.default_rng(61)
    n, N = 3 * 2 * SUPER + 4_097, 64
    host = rand_case(rng, N, n, gscale=3e-3)
    ref_g = orc.reduce_unscale(host["G"], 0, 1.0)
    ref_sq = orc.sqnorm(ref_g)
    max_norm = 0.5 * float(np.sqrt(ref_sq))   # the step clips
    P, M, V, B, _ = orc.adam_from_gbar(ref_g, host["P"], host["M"], host["V"], HP, 4, ref_sq, max_norm)
    G = device_replicas(env, host, 0)
    d = {k: torch.from_numpy(host[k]).to(dev) for k in ("P", "M", "V")}
    pristine = {k: d[k].clone() for k in d}
    Bd = torch.zeros(n, dtype=torch.int16, device=dev)
    ws = torch.empty(zs.two_pass_workspace_bytes(n), dtype=torch.uint8, device=dev)
    sq = torch.empty(1, dtype=torch.float64, device=dev)
    s = torch.cuda.Stream(device=dev)
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        zs.clipped_step_flat(G, d["P"], d["M"], d["V"], Bd, HP, 4, max_norm=max_norm, workspace=ws, sqnorm=sq)
    torch.cuda.synchronize()
    for rep in range(3):
        for k in d:
            d[k].copy_(pristine[k])
        Bd.zero_()
        torch.cuda.synchronize()
        junk = torch.randn(1 << 20, device=dev).sum()
        g.replay()
        torch.cuda.synchronize()
        got = dict(P=d["P"].cpu().numpy(), M=d["M"].cpu().numpy(), V=d["V"].cpu().numpy(),
                   B=Bd.cpu().numpy().view(np.uint16))
        for k, ref in (("P", P), ("M", M), ("V", V), ("B", B)):
            assert np.array_equal(got[k].view(np.uint32 if k != "B" else np.uint16),
                                  ref.view(np.uint32 if k != "B" else np.uint16)), f"replay {rep}: {k}"
        del junk
