"""Checkpoint and resume: k steps, the fp32 state (master, m, v) and the bf16
working copy saved to host memory, the device buffers (and for lists the
plan) thrown away, the state loaded into fresh device buffers, and the run
continued with the step index carried on.  The result must be bit-identical
to an uninterrupted run, and to the oracle run step by step.

The library keeps no state between calls (the step index is an argument), so
a checkpoint is the caller's arrays plus the step index.  The pages' only save
knob is the DeepSpeed config's gather_16bit_weights_on_model_save ("Почему
training 70B модели требует optimizer sharding (ZeRO-3)?", §8), which gathers
the 16-bit working copy; resuming needs the fp32 master, m and v as well."""
import numpy as np
import pytest

from tests import parity

pytestmark = pytest.mark.gpu

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1)


def grad_key(t: int, r: int) -> int:
    """Counter-based stream of replica r's gradients at step t (seed = step)."""
    import synth

    return synth.key(t, synth.KIND_GRAD, r)


def replicas(rng, N, n):
    """Fresh bf16 gradients for one step (N replicas of n), as uint16 bits."""
    x = (rng.standard_normal((N, n)) * 1e-3).astype(np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def initial_state(rng, n):
    P = (rng.standard_normal(n) * 0.02).astype(np.float32)
    return P, np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.uint16)


def to_dev(torch, host):
    P, M, V, B = host
    dev = torch.device("cuda:0")
    return [torch.from_numpy(P.copy()).to(dev), torch.from_numpy(M.copy()).to(dev),
            torch.from_numpy(V.copy()).to(dev), torch.from_numpy(B.view(np.int16).copy()).to(dev)]


def to_host(state):
    P, M, V, B = state
    return (P.cpu().numpy().copy(), M.cpu().numpy().copy(), V.cpu().numpy().copy(),
            B.cpu().numpy().view(np.uint16).copy())


@pytest.mark.parametrize("N,n", [(4, 100_003), (64, (1 << 25) + 3_707)])
def test_flat_resume_is_bit_identical(orc, N, n):
    """(64, 2^25 + 3,707) takes the windowed kernel; (4, 100,003) the one-tile kernel.  Each step draws
    new replicas on the device from the counter-based generator; the oracle redraws them on the host."""
    import torch

    import sharded_mixed_precision_rank_amd as zs
    import synth

    zs.set_grid_blocks(0)
    steps = 4 if N == 64 else 6
    half = steps // 2
    kP = synth.key(N, synth.KIND_P)
    P0 = torch.empty(n, dtype=torch.float32, device="cuda")
    synth.dev_fill_normal_f32(P0, kP, 0, 0.02)
    init = (P0.cpu().numpy(), np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.uint16))
    del P0
    G = [torch.empty(n, dtype=torch.bfloat16, device="cuda") for _ in range(N)]

    def run(state, ts):
        P, M, V, B = state
        for t in ts:
            for r in range(N):
                synth.dev_fill_normal_bf16(G[r], grad_key(t, r), 0, 1e-3)
            zs.reduce_adam_flat(G, P, M, V, B, HP, t)
        torch.cuda.synchronize()

    a = to_dev(torch, init)
    run(a, range(1, steps + 1))
    straight = to_host(a)
    del a
    # interrupted: save after `half` steps, drop the buffers, load into fresh ones, go on
    b = to_dev(torch, init)
    run(b, range(1, half + 1))
    ckpt = to_host(b)
    del b
    torch.cuda.empty_cache()
    c = to_dev(torch, ckpt)
    run(c, range(half + 1, steps + 1))
    resumed = to_host(c)
    del c, G
    names = ("P", "M", "V", "B")
    assert parity.bit_identical(dict(zip(names, resumed)), dict(zip(names, straight)))
    # and the oracle, step by step from the same initial state (the tail slice at the large size)
    lo = 0 if n < 1 << 20 else n - 300_000
    P, M, V = (x[lo:].copy() for x in init[:3])
    for t in range(1, steps + 1):
        Gh = np.stack([synth.normal_bf16(grad_key(t, r), lo, n - lo, 1e-3) for r in range(N)])
        P, M, V, B = orc.step(Gh, P, M, V, HP, t)
    ref = dict(P=P, M=M, V=V, B=B)
    got = {k: x[lo:] for k, x in zip(names, resumed)}
    parity.assert_step(got, ref, f"resumed N={N} n={n}")
    assert parity.bit_identical(got, ref)
    torch.cuda.empty_cache()


def test_list_plan_resume_is_bit_identical(orc):
    import torch

    import sharded_mixed_precision_rank_amd as zs

    zs.set_grid_blocks(0)
    rng = np.random.default_rng(99)
    N = 3
    sizes = np.array([1, 9, 4097, 100_003, 64, 0, 20_001], dtype=np.int64)
    offsets = np.zeros_like(sizes)
    offsets[1:] = np.cumsum((sizes[:-1] + 7) // 8 * 8 + 8)   # 8-element gaps between tensors
    L = int(offsets[-1] + sizes[-1] + 8)
    init = initial_state(rng, L)
    grads = {t: replicas(rng, N, L) for t in range(1, 7)}

    def run(state, steps):
        P, M, V, B = state
        for t in steps:
            G = [torch.from_numpy(g.view(np.int16)).to(P.device) for g in grads[t]]
            plan = zs.ListPlan.from_arenas(sizes, offsets, G, P, M, V, B)
            plan.step(HP, t)
            torch.cuda.synchronize()
            plan.close()

    a = to_dev(torch, init)
    run(a, range(1, 7))
    straight = to_host(a)
    b = to_dev(torch, init)
    run(b, range(1, 4))
    ckpt = to_host(b)
    del b
    c = to_dev(torch, ckpt)
    run(c, range(4, 7))
    resumed = to_host(c)
    names = ("P", "M", "V", "B")
    assert parity.bit_identical(dict(zip(names, resumed)), dict(zip(names, straight)))
    # the oracle, tensor by tensor; the gaps keep their initial values
    inside = np.zeros(L, dtype=bool)
    for o, s in zip(offsets.tolist(), sizes.tolist()):
        if s == 0:
            continue
        P, M, V = (x[o:o + s].copy() for x in init[:3])
        for t in range(1, 7):
            P, M, V, B = orc.step(np.ascontiguousarray(grads[t][:, o:o + s]), P, M, V, HP, t)
        got = {k: x[o:o + s] for k, x in zip(names, resumed)}
        assert parity.bit_identical(got, dict(P=P, M=M, V=V, B=B)), f"tensor at {o} of {s}"
        inside[o:o + s] = True
    for k, x, x0 in zip(names, resumed, init):
        assert np.array_equal(x[~inside].view(np.uint8), x0[~inside].view(np.uint8)), f"gap of {k} was written"
