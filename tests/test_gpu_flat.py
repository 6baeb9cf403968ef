"""GPU parity of the flat shard step against the CPU oracle (through the C ABI)."""
import numpy as np
import pytest

from tests import parity

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch

    import sharded_mixed_precision_rank_amd as zs

    zs.set_grid_blocks(0)
    return dict(torch=torch, zs=zs, dev=torch.device("cuda:0"))


def upload(torch, dev, host):
    G = [torch.from_numpy(np.ascontiguousarray(g).view(np.int16)).to(dev) for g in host["G"]]
    return dict(G=G, P=torch.from_numpy(host["P"]).to(dev), M=torch.from_numpy(host["M"]).to(dev),
                V=torch.from_numpy(host["V"]).to(dev))


def download(d):
    return dict(P=d["P"].cpu().numpy(), M=d["M"].cpu().numpy(), V=d["V"].cpu().numpy(),
                B=d["B"].cpu().numpy().view(np.uint16))


def run_and_compare(env, orc, host, hp, t, what, bit_exact=True):
    torch, zs, dev = env["torch"], env["zs"], env["dev"]
    n = host["P"].size
    d = upload(torch, dev, host)
    d["B"] = torch.full((n,), 0x7FBF, dtype=torch.int16, device=dev)
    zs.reduce_adam_flat(d["G"], d["P"], d["M"], d["V"], d["B"], hp, t)
    torch.cuda.synchronize()
    got = download(d)
    P, M, V, B = orc.step(host["G"], host["P"], host["M"], host["V"], hp, t)
    ref = dict(P=P, M=M, V=V, B=B)
    rep = parity.assert_step(got, ref, what)
    if bit_exact:
        assert parity.bit_identical(got, ref), f"{what}: within tolerance but not bit-identical: {rep}"
    return got, ref


def rand_host(rng, N, n, warm=True, gscale=1e-3):
    G = np.stack([(((rng.standard_normal(n) * gscale).astype(np.float32).view(np.uint32)) >> 16).astype(np.uint16)
                  for _ in range(N)]) if n else np.zeros((N, 0), dtype=np.uint16)
    P = (rng.standard_normal(n) * 0.02).astype(np.float32)
    M = (rng.standard_normal(n) * 1e-4).astype(np.float32) if warm else np.zeros(n, dtype=np.float32)
    V = np.abs(rng.standard_normal(n) * 1e-6).astype(np.float32) if warm else np.zeros(n, dtype=np.float32)
    return dict(G=G, P=P, M=M, V=V)


HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0)


def test_c1_flat_1M_N2_first_step(env, orc):
    """Flat shard of 2^20 params, 2 replicas, cold state, step 1 (the small workload)."""
    from synth import workloads as W

    w = W.FLAT_1M_N2
    host = W.host_inputs(w, 0, w.n_flat)
    run_and_compare(env, orc, host, w.hp(), w.step, "flat-1M-N2")


@pytest.mark.parametrize("N", [1, 2, 3, 4, 5, 7, 8, 9, 16, 17, 31, 32, 33, 63, 64, 65, 100, 256])
def test_replica_counts(env, orc, N):
    rng = np.random.default_rng(1000 + N)
    n = 2048 * 3 + 5 if N <= 64 else 4099
    host = rand_host(rng, N, n)
    run_and_compare(env, orc, host, dict(HP, weight_decay=0.1), 37, f"N={N}")


@pytest.mark.parametrize("n", [0, 1, 7, 8, 9, 15, 16, 17, 255, 511, 512, 513, 2047, 2048, 2049, 4095, 100_003])
def test_lengths(env, orc, n):
    rng = np.random.default_rng(2000 + n)
    host = rand_host(rng, 8, n)
    if n == 0:
        torch, zs, dev = env["torch"], env["zs"], env["dev"]
        e = torch.empty(0, device=dev)
        zs.reduce_adam_flat([torch.empty(0, dtype=torch.bfloat16, device=dev)] * 8, e, e.clone(), e.clone(),
                            torch.empty(0, dtype=torch.bfloat16, device=dev), HP, 1)
        torch.cuda.synchronize()
        return
    run_and_compare(env, orc, host, HP, 100, f"n={n}")


@pytest.mark.parametrize("shift,n", [(1, 10_000), (2, 10_000), (3, 10_000), (5, 10_000), (7, 10_000),
                                     (8, 10_000), (24, 10_000), (32, 10_000), (40, 10_000), (56, 10_000),
                                     (63, 10_000), (72, 10_000), (8, 9), (8, 63), (8, 64), (8, 70), (8, 71),
                                     (40, 33), (1, 70), (1, 10_007), (1, 1_000_007)])
def test_common_misalignment_peels_a_head(env, orc, shift, n):
    """Every array starts `shift` elements past a 256-byte boundary: the kernel
    peels a head up to the next common line boundary (up to 63 elements; a
    16-byte one when no line boundary is common) and runs the vector path on
    the rest; shards too short for one group after the head run element by
    element.  shift=1 with n=10,007 leaves 63 head and 7 tail elements, more
    than one per thread of the last workgroup."""
    torch, zs, dev = env["torch"], env["zs"], env["dev"]
    rng = np.random.default_rng(3000 + shift + n)
    N = 4
    host = rand_host(rng, N, n)
    d = upload(torch, dev, host)
    B = torch.zeros(n, dtype=torch.int16, device=dev)
    zs.reduce_adam_flat([g[shift:] for g in d["G"]], d["P"][shift:], d["M"][shift:], d["V"][shift:], B[shift:],
                        HP, 3)
    torch.cuda.synchronize()
    rP, rM, rV, rB = orc.step([g[shift:] for g in host["G"]], host["P"][shift:], host["M"][shift:],
                              host["V"][shift:], HP, 3)
    got = download(dict(d, B=B))
    ref = dict(P=rP, M=rM, V=rV, B=rB)
    got_s = {k: v[shift:] for k, v in got.items()}
    parity.assert_step(got_s, ref, f"shift={shift} n={n}")
    assert parity.bit_identical(got_s, ref)
    # the elements before the view are untouched
    assert np.array_equal(got["P"][:shift], host["P"][:shift]) and np.all(got["B"][:shift] == 0)


@pytest.mark.parametrize("shift", [64, 128, 200, 256, 448, 504, 511])
def test_tile_anchor_splits_the_shard(env, orc, shift):
    """Every array starts `shift` elements past a boundary of 512 of its own
    elements: the elements up to the next such boundary run as a shard of
    their own, the rest as a shard whose tiles start on those boundaries.
    The split changes no result."""
    torch, zs, dev = env["torch"], env["zs"], env["dev"]
    rng = np.random.default_rng(3500 + shift)
    N, n = 8, 512 * 12 + 37
    host = rand_host(rng, N, n + shift)
    d = upload(torch, dev, host)
    B = torch.zeros(n + shift, dtype=torch.int16, device=dev)
    zs.reduce_adam_flat([g[shift:] for g in d["G"]], d["P"][shift:], d["M"][shift:], d["V"][shift:], B[shift:],
                        HP, 9)
    torch.cuda.synchronize()
    rP, rM, rV, rB = orc.step([g[shift:] for g in host["G"]], host["P"][shift:], host["M"][shift:],
                              host["V"][shift:], HP, 9)
    got = download(dict(d, B=B))
    ref = dict(P=rP, M=rM, V=rV, B=rB)
    got_s = {k: v[shift:] for k, v in got.items()}
    parity.assert_step(got_s, ref, f"anchor shift={shift}")
    assert parity.bit_identical(got_s, ref)
    assert np.array_equal(got["P"][:shift], host["P"][:shift]) and np.all(got["B"][:shift] == 0)


def test_mixed_alignment_takes_the_element_path(env, orc):
    """Arrays whose 16-byte phases differ cannot share a head peel: every
    element goes through the per-element path, with the same results."""
    torch, zs, dev = env["torch"], env["zs"], env["dev"]
    rng = np.random.default_rng(4000)
    n, N = 5000, 3
    host = rand_host(rng, N, n)
    d = upload(torch, dev, dict(G=[np.concatenate([np.zeros(r + 1, np.uint16), g]) for r, g in enumerate(host["G"])],
                                P=np.concatenate([np.zeros(1, np.float32), host["P"]]),
                                M=np.concatenate([np.zeros(2, np.float32), host["M"]]),
                                V=host["V"]))
    G = [g[r + 1:] for r, g in enumerate(d["G"])]
    P, M, V = d["P"][1:], d["M"][2:], d["V"]
    B = torch.zeros(n + 3, dtype=torch.int16, device=dev)[3:]
    zs.reduce_adam_flat(G, P, M, V, B, HP, 2)
    torch.cuda.synchronize()
    rP, rM, rV, rB = orc.step(host["G"], host["P"], host["M"], host["V"], HP, 2)
    got = dict(P=P.cpu().numpy(), M=M.cpu().numpy(), V=V.cpu().numpy(), B=B.cpu().numpy().view(np.uint16))
    ref = dict(P=rP, M=rM, V=rV, B=rB)
    parity.assert_step(got, ref, "mixed alignment")
    assert parity.bit_identical(got, ref)


def test_same_pointer_N_times_is_the_replica(env, orc):
    """Averaging N identical replicas gives that replica exactly (the
    averaging equation with equal terms), so the step equals the 1-replica step."""
    torch, zs, dev = env["torch"], env["zs"], env["dev"]
    rng = np.random.default_rng(5000)
    n = 20_000
    host = rand_host(rng, 1, n)
    outs = []
    for N in (1, 7, 64):
        d = upload(torch, dev, host)
        B = torch.zeros(n, dtype=torch.int16, device=dev)
        zs.reduce_adam_flat([d["G"][0]] * N, d["P"], d["M"], d["V"], B, HP, 5)
        torch.cuda.synchronize()
        outs.append(download(dict(d, B=B)))
    assert parity.bit_identical(outs[0], outs[1]) and parity.bit_identical(outs[0], outs[2])


def test_special_values(env, orc):
    """NaN, +-Inf, -0 and subnormal gradients, zero gradients, subnormal moments."""
    rng = np.random.default_rng(6000)
    n, N = 4096, 4
    host = rand_host(rng, N, n)
    G = host["G"]
    G[0, :16] = [0x7F80, 0xFF80, 0x7FC0, 0xFFC1, 0x8000, 0x0000, 0x0001, 0x8001, 0x007F, 0x807F, 0x7F7F, 0xFF7F,
                 0x3F80, 0xBF80, 0x0080, 0x8080]
    G[:, 100:200] = 0
    G[:, 200:300] = 0x8000
    host["M"][300:310] = np.array([1e-40, -1e-40, 1e-45, -1e-45, 0, -0.0, 1e-38, 3e-39, 5e-44, 1e-41],
                                  dtype=np.float32)
    host["V"][300:310] = np.array([1e-40, 1e-40, 1e-45, 1e-45, 0, 0, 1e-38, 3e-39, 5e-44, 1e-41], dtype=np.float32)
    host["P"][310:320] = np.array([1e-40, -1e-40, 0, -0.0, 3e38, -3e38, 1e-45, np.inf, -np.inf, np.nan],
                                  dtype=np.float32)
    run_and_compare(env, orc, host, dict(HP, weight_decay=0.1), 1, "special values")
    run_and_compare(env, orc, host, HP, 1000, "special values t=1000")


def test_deterministic_across_runs_and_grids(env, orc):
    torch, zs, dev = env["torch"], env["zs"], env["dev"]
    rng = np.random.default_rng(7000)
    n, N = 300_001, 8
    host = rand_host(rng, N, n)
    outs = []
    try:
        for blocks in (0, 0, 0, 1, 7, 4096):
            zs.set_grid_blocks(blocks)
            d = upload(torch, dev, host)
            d["B"] = torch.zeros(n, dtype=torch.int16, device=dev)
            zs.reduce_adam_flat(d["G"], d["P"], d["M"], d["V"], d["B"], HP, 9)
            torch.cuda.synchronize()
            outs.append(download(d))
    finally:
        zs.set_grid_blocks(0)
    for o in outs[1:]:
        assert parity.bit_identical(outs[0], o)


def test_consecutive_steps_track_the_oracle(env, orc):
    """State carried across 5 steps on the GPU equals 5 oracle steps."""
    torch, zs, dev = env["torch"], env["zs"], env["dev"]
    rng = np.random.default_rng(8000)
    n, N = 50_000, 4
    host = rand_host(rng, N, n, warm=False)
    d = upload(torch, dev, host)
    d["B"] = torch.zeros(n, dtype=torch.int16, device=dev)
    P, M, V = host["P"].copy(), host["M"].copy(), host["V"].copy()
    B = np.zeros(n, dtype=np.uint16)
    hp = dict(HP, weight_decay=0.01)
    for t in range(1, 6):
        zs.reduce_adam_flat(d["G"], d["P"], d["M"], d["V"], d["B"], hp, t)
        orc.step_inplace(host["G"], P, M, V, B, hp, t)
    torch.cuda.synchronize()
    assert parity.bit_identical(download(d), dict(P=P, M=M, V=V, B=B))


def test_rejects_overlapping_outputs_on_gpu(env):
    torch, zs, dev = env["torch"], env["zs"], env["dev"]
    buf = torch.zeros(4096, device=dev)
    g = torch.zeros(1024, dtype=torch.bfloat16, device=dev)
    with pytest.raises(zs.ZShardError) as ei:
        zs.reduce_adam_flat([g], buf[:1024], buf[512:1536], buf[2048:3072], torch.zeros(1024, dtype=torch.int16,
                                                                                           device=dev), HP, 1)
    assert ei.value.name == "ZS_ERR_ALIAS"
