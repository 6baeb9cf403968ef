"""GPU parity of the ragged-list step (work-table plan) against the oracle."""
import numpy as np
import pytest

from tests import parity

pytestmark = pytest.mark.gpu

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0)


@pytest.fixture(scope="module")
def env():
    import torch

    import sharded_mixed_precision_rank_amd as zs

    zs.set_grid_blocks(0)
    return dict(torch=torch, zs=zs, dev=torch.device("cuda:0"))


def arena_case(env, w, sentinel=0x7FBF):
    """Upload a workload's full arenas (host-drawn) and return host + device copies."""
    from synth import workloads as W

    torch, dev = env["torch"], env["dev"]
    offsets, L = w.layout()
    host = W.host_inputs(w, 0, L)
    d = dict(G=[torch.from_numpy(g.view(np.int16)).to(dev) for g in host["G"]],
             P=torch.from_numpy(host["P"]).to(dev), M=torch.from_numpy(host["M"]).to(dev),
             V=torch.from_numpy(host["V"]).to(dev),
             B=torch.full((L,), sentinel, dtype=torch.int16, device=dev))
    return host, d, offsets, L


def oracle_list(orc, w, host, offsets, t, hp):
    """The oracle applied tensor by tensor; gaps between tensors keep their inputs."""
    L = host["P"].size
    P, M, V = host["P"].copy(), host["M"].copy(), host["V"].copy()
    B = np.full(L, 0x7FBF, dtype=np.uint16)
    for o, n in zip(offsets, w.sizes):
        sl = slice(int(o), int(o) + int(n))
        p, m, v, b = P[sl].copy(), M[sl].copy(), V[sl].copy(), B[sl].copy()
        orc.step_inplace([g[sl] for g in host["G"]], p, m, v, b, hp, t)
        P[sl], M[sl], V[sl], B[sl] = p, m, v, b
    return dict(P=P, M=M, V=V, B=B)


def small_ragged(N, count, seed, lo=1, hi=70_000, step=3, warm=True, zero_frac=0.0, wd=0.0):
    from synth import workloads as W

    rng = np.random.default_rng(seed)
    sizes = tuple(int(x) for x in np.exp(rng.uniform(np.log(lo), np.log(hi), count)).astype(np.int64))
    sizes = sizes[:-3] + (1, 9, 0)  # a 1-element, a 9-element and an empty tensor
    return W.Workload(f"ragged-{count}", N=N, step=step, weight_decay=wd, warm=warm, sizes=sizes, seed=seed,
                      zero_frac=zero_frac)


@pytest.mark.parametrize("N", [1, 2, 3, 8, 16, 64, 70])
def test_ragged_list_matches_oracle(env, orc, N):
    torch, zs = env["torch"], env["zs"]
    w = small_ragged(N, 60 if N > 16 else 200, seed=N, zero_frac=0.01, wd=0.1 if N % 2 else 0.0)
    host, d, offsets, L = arena_case(env, w)
    with zs.ListPlan.from_arenas(w.sizes, offsets, d["G"], d["P"], d["M"], d["V"], d["B"]) as plan:
        info = plan.info()
        assert info["n_params"] == w.n_params and info["n_tensors"] == len(w.sizes)
        plan.step(w.hp(), w.step)
        torch.cuda.synchronize()
    got = dict(P=d["P"].cpu().numpy(), M=d["M"].cpu().numpy(), V=d["V"].cpu().numpy(),
               B=d["B"].cpu().numpy().view(np.uint16))
    ref = oracle_list(orc, w, host, offsets, w.step, w.hp())
    parity.assert_step(got, ref, f"list N={N}")
    assert parity.bit_identical(got, ref)   # includes the untouched gaps


def test_list_plan_reused_over_steps(env, orc):
    torch, zs = env["torch"], env["zs"]
    w = small_ragged(8, 100, seed=77, warm=False)
    host, d, offsets, L = arena_case(env, w)
    ref_state = dict(P=host["P"].copy(), M=host["M"].copy(), V=host["V"].copy())
    with zs.ListPlan.from_arenas(w.sizes, offsets, d["G"], d["P"], d["M"], d["V"], d["B"]) as plan:
        for t in range(1, 5):
            plan.step(w.hp(), t)
            h = dict(G=host["G"], **ref_state)
            ref = oracle_list(orc, w, h, offsets, t, w.hp())
            ref_state = dict(P=ref["P"], M=ref["M"], V=ref["V"])
        torch.cuda.synchronize()
    got = dict(P=d["P"].cpu().numpy(), M=d["M"].cpu().numpy(), V=d["V"].cpu().numpy(),
               B=d["B"].cpu().numpy().view(np.uint16))
    assert parity.bit_identical(got, ref)


def test_list_equals_flat_calls(env, orc):
    """One list launch gives the same bits as one flat call per tensor."""
    torch, zs = env["torch"], env["zs"]
    w = small_ragged(4, 50, seed=91)
    host, d1, offsets, L = arena_case(env, w)
    _, d2, _, _ = arena_case(env, w)
    zs.reduce_adam_list([zs.ShardTensor([g[o:o + n] for g in d1["G"]], d1["P"][o:o + n], d1["M"][o:o + n],
                                        d1["V"][o:o + n], d1["B"][o:o + n])
                         for o, n in zip(offsets.tolist(), w.sizes)], 4, w.hp(), w.step)
    for o, n in zip(offsets.tolist(), w.sizes):
        if n:
            zs.reduce_adam_flat([g[o:o + n] for g in d2["G"]], d2["P"][o:o + n], d2["M"][o:o + n],
                                d2["V"][o:o + n], d2["B"][o:o + n], w.hp(), w.step)
    torch.cuda.synchronize()
    for k in "PMV":
        assert torch.equal(d1[k], d2[k])
    assert torch.equal(d1["B"], d2["B"])


def test_misaligned_tensor_in_list(env, orc):
    """A tensor whose arrays share no 16-byte phase runs element by element."""
    torch, zs, dev = env["torch"], env["zs"], env["dev"]
    rng = np.random.default_rng(5)
    n, N = 3000, 2
    G = [torch.from_numpy(((rng.standard_normal(n + 4) * 1e-3).astype(np.float32).view(np.uint32) >> 16)
                          .astype(np.uint16).view(np.int16)).to(dev) for _ in range(N)]
    P = torch.from_numpy((rng.standard_normal(n + 4) * 0.02).astype(np.float32)).to(dev)
    M = torch.zeros(n + 4, device=dev)
    V = torch.zeros(n + 4, device=dev)
    B = torch.zeros(n + 4, dtype=torch.int16, device=dev)
    t = zs.ShardTensor([G[0][1:1 + n], G[1][2:2 + n]], P[3:3 + n], M[:n], V[1:1 + n], B[:n])
    hostG = [G[0][1:1 + n].cpu().numpy().view(np.uint16), G[1][2:2 + n].cpu().numpy().view(np.uint16)]
    hostP = P[3:3 + n].cpu().numpy()
    zs.reduce_adam_list([t], N, HP, 1)
    rP, rM, rV, rB = orc.step(hostG, hostP, np.zeros(n, np.float32), np.zeros(n, np.float32), HP, 1)
    got = dict(P=P[3:3 + n].cpu().numpy(), M=M[:n].cpu().numpy(), V=V[1:1 + n].cpu().numpy(),
               B=B[:n].cpu().numpy().view(np.uint16))
    assert parity.bit_identical(got, dict(P=rP, M=rM, V=rV, B=rB))


def test_list_rejects_overlap_on_gpu(env):
    torch, zs, dev = env["torch"], env["zs"], env["dev"]
    buf = torch.zeros(10_000, device=dev)
    g = torch.zeros(10_000, dtype=torch.bfloat16, device=dev)
    b = torch.zeros(10_000, dtype=torch.int16, device=dev)
    t0 = zs.ShardTensor([g[:100]], buf[:100], buf[1000:1100], buf[2000:2100], b[:100])
    t1 = zs.ShardTensor([g[100:200]], buf[50:150], buf[3000:3100], buf[4000:4100], b[100:200])
    with pytest.raises(zs.ZShardError) as ei:
        zs.ListPlan([t0, t1], 1)
    assert ei.value.name == "ZS_ERR_ALIAS"


def oracle_list_groups(orc, w, host, offsets, t, hps, groups):
    """The oracle tensor by tensor, tensor k with hps[groups[k]]; gaps keep their inputs."""
    L = host["P"].size
    P, M, V = host["P"].copy(), host["M"].copy(), host["V"].copy()
    B = np.full(L, 0x7FBF, dtype=np.uint16)
    for k, (o, n) in enumerate(zip(offsets, w.sizes)):
        sl = slice(int(o), int(o) + int(n))
        p, m, v, b = P[sl].copy(), M[sl].copy(), V[sl].copy(), B[sl].copy()
        orc.step_inplace([g[sl] for g in host["G"]], p, m, v, b, hps[groups[k]], t)
        P[sl], M[sl], V[sl], B[sl] = p, m, v, b
    return dict(P=P, M=M, V=V, B=B)


@pytest.mark.parametrize("N,n_groups", [(3, 3), (16, 8), (8, 1)])
def test_list_plan_hyperparameter_groups(env, orc, N, n_groups):
    """Tensors in hyperparameter groups (different lr and weight decay per
    group, e.g. no decay on norms and biases), one launch, against the oracle
    per tensor with its group's set; then the single-set call again applies
    its one set to every tensor."""
    torch, zs = env["torch"], env["zs"]
    w = small_ragged(N, 120, seed=300 + N, zero_frac=0.01)
    host, d, offsets, L = arena_case(env, w)
    groups = [(k * 7 + 3) % n_groups for k in range(len(w.sizes))]
    hps = [dict(lr=1e-3 * (1 + g), beta1=0.9, beta2=0.999 - 0.0001 * g, eps=1e-8, weight_decay=0.1 * (g % 2))
           for g in range(n_groups)]
    with zs.ListPlan.from_arenas(w.sizes, offsets, d["G"], d["P"], d["M"], d["V"], d["B"]) as plan:
        plan.set_groups(groups, n_groups)
        plan.step_groups(hps, 4)
        torch.cuda.synchronize()
        got = dict(P=d["P"].cpu().numpy(), M=d["M"].cpu().numpy(), V=d["V"].cpu().numpy(),
                   B=d["B"].cpu().numpy().view(np.uint16))
        ref = oracle_list_groups(orc, w, host, offsets, 4, hps, groups)
        parity.assert_step(got, ref, f"groups N={N}")
        assert parity.bit_identical(got, ref)
        plan.step(HP, 5)   # one set for every tensor, whatever the groups
        torch.cuda.synchronize()
    got2 = dict(P=d["P"].cpu().numpy(), M=d["M"].cpu().numpy(), V=d["V"].cpu().numpy(),
                B=d["B"].cpu().numpy().view(np.uint16))
    ref2 = oracle_list(orc, w, dict(G=host["G"], P=ref["P"], M=ref["M"], V=ref["V"]), offsets, 5, HP)
    assert parity.bit_identical(got2, ref2)


@pytest.mark.parametrize("N", [8, 64])
def test_tensors_at_every_tile_phase(env, orc, N):
    """Tensors that start at different phases of the 512-element tile grid: each
    tensor's groups before its next 512-element boundary form a partial tile of
    their own (the whole tensor when it ends before that boundary), and every
    later tile starts on the boundary.  Phase 3 also needs a 61-element head peel."""
    from synth import workloads as W

    torch, zs, dev = env["torch"], env["zs"], env["dev"]
    cases = [(8, 100), (8, 504), (8, 505), (64, 448 + 512 * 9 + 3), (448, 64 + 512 * 20 + 100), (0, 5000),
             (3, 3000), (504, 8), (256, 512 * 9)]
    offsets = np.array([16384 * k + ph for k, (ph, _) in enumerate(cases)], dtype=np.int64)
    sizes = tuple(n for _, n in cases)
    L = int(offsets[-1] + sizes[-1] + 64)
    w = W.Workload(f"phases-N{N}", N=N, step=11, weight_decay=0.1, warm=True, sizes=sizes, seed=77 + N)
    host = W.host_inputs(w, 0, L)
    d = dict(G=[torch.from_numpy(g.view(np.int16)).to(dev) for g in host["G"]],
             P=torch.from_numpy(host["P"]).to(dev), M=torch.from_numpy(host["M"]).to(dev),
             V=torch.from_numpy(host["V"]).to(dev), B=torch.full((L,), 0x7FBF, dtype=torch.int16, device=dev))
    with zs.ListPlan.from_arenas(sizes, offsets, d["G"], d["P"], d["M"], d["V"], d["B"]) as plan:
        plan.step(w.hp(), w.step)
        torch.cuda.synchronize()
    got = dict(P=d["P"].cpu().numpy(), M=d["M"].cpu().numpy(), V=d["V"].cpu().numpy(),
               B=d["B"].cpu().numpy().view(np.uint16))
    ref = oracle_list(orc, w, host, offsets, w.step, w.hp())
    parity.assert_step(got, ref, f"tile phases N={N}")
    assert parity.bit_identical(got, ref)
