"""GPU + CPU optimizer-offload step: bit-identical to the fused device step."""
import numpy as np
import pytest

from tests import parity

pytestmark = pytest.mark.gpu

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1)


@pytest.mark.parametrize("n,N,chunk", [(1, 1, 2048), (5000, 2, 2048), (100_003, 8, 16_384), (1_000_001, 64, 262_144)])
def test_offload_equals_fused(n, N, chunk):
    import torch

    import sharded_mixed_precision_rank_amd as zs

    dev = torch.device("cuda:0")
    rng = np.random.default_rng(n + N)
    G = [torch.from_numpy(((rng.standard_normal(n) * 1e-3).astype(np.float32).view(np.uint32) >> 16)
                          .astype(np.uint16).view(np.int16)).to(dev) for _ in range(N)]
    P = (rng.standard_normal(n) * 0.02).astype(np.float32)
    M = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    V = np.abs(rng.standard_normal(n) * 1e-6).astype(np.float32)
    # device reference: the fused step, three steps
    Pd, Md, Vd = (torch.from_numpy(x.copy()).to(dev) for x in (P, M, V))
    Bd = torch.zeros(n, dtype=torch.int16, device=dev)
    for t in (1, 2, 3):
        zs.reduce_adam_flat(G, Pd, Md, Vd, Bd, HP, t)
    # offload: host state (pinned torch tensors), device working copy
    Ph, Mh, Vh = (torch.from_numpy(x.copy()).pin_memory() for x in (P, M, V))
    Bo = torch.zeros(n, dtype=torch.int16, device=dev)
    with zs.Offload(chunk, 4) as off:
        for t in (1, 2, 3):
            off.step(G, Ph, Mh, Vh, Bo, HP, t)
    torch.cuda.synchronize()
    ref = dict(P=Pd.cpu().numpy(), M=Md.cpu().numpy(), V=Vd.cpu().numpy(), B=Bd.cpu().numpy().view(np.uint16))
    got = dict(P=Ph.numpy(), M=Mh.numpy(), V=Vh.numpy(), B=Bo.cpu().numpy().view(np.uint16))
    assert parity.bit_identical(got, ref)


def test_offload_misaligned_grads():
    import torch

    import sharded_mixed_precision_rank_amd as zs

    dev = torch.device("cuda:0")
    rng = np.random.default_rng(3)
    n, N = 30_001, 3
    G = [torch.from_numpy(((rng.standard_normal(n + 3) * 1e-3).astype(np.float32).view(np.uint32) >> 16)
                          .astype(np.uint16).view(np.int16)).to(dev)[r:r + n] for r in range(N)]
    P = (rng.standard_normal(n) * 0.02).astype(np.float32)
    Z = np.zeros(n, np.float32)
    Pd, Md, Vd = (torch.from_numpy(x.copy()).to(dev) for x in (P, Z, Z))
    Bd = torch.zeros(n, dtype=torch.int16, device=dev)
    zs.reduce_adam_flat(G, Pd, Md, Vd, Bd, HP, 1)
    Ph, Mh, Vh = P.copy(), Z.copy(), Z.copy()
    Bo = torch.zeros(n, dtype=torch.int16, device=dev)
    with zs.Offload(4096, 2) as off:
        off.step(G, Ph, Mh, Vh, Bo, HP, 1)
    torch.cuda.synchronize()
    assert parity.bit_identical(dict(P=Ph, M=Mh, V=Vh, B=Bo.cpu().numpy().view(np.uint16)),
                                dict(P=Pd.cpu().numpy(), M=Md.cpu().numpy(), V=Vd.cpu().numpy(),
                                     B=Bd.cpu().numpy().view(np.uint16)))


@pytest.mark.parametrize("n,N,t,chunk", [(70_001, 4, 1, 8192), (300_017, 16, 9, 65_536)])
def test_offload_against_oracle(orc, n, N, t, chunk):
    """The offload step checked directly against the CPU oracle on the same seeded inputs."""
    import torch

    import sharded_mixed_precision_rank_amd as zs

    dev = torch.device("cuda:0")
    rng = np.random.default_rng(1000 + n)
    G = np.stack([((rng.standard_normal(n) * 1e-3).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
                  for _ in range(N)])
    P = (rng.standard_normal(n) * 0.02).astype(np.float32)
    M = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    V = np.abs(rng.standard_normal(n) * 1e-6).astype(np.float32)
    Pr, Mr, Vr, Br = orc.step(G, P, M, V, HP, t)
    Gd = [torch.from_numpy(np.ascontiguousarray(g).view(np.int16)).to(dev) for g in G]
    Ph, Mh, Vh = (torch.from_numpy(x.copy()).pin_memory() for x in (P, M, V))
    Bo = torch.full((n,), 0x7FBF, dtype=torch.int16, device=dev)
    with zs.Offload(chunk, 8) as off:
        off.step(Gd, Ph, Mh, Vh, Bo, HP, t)
    torch.cuda.synchronize()
    got = dict(P=Ph.numpy(), M=Mh.numpy(), V=Vh.numpy(), B=Bo.cpu().numpy().view(np.uint16))
    ref = dict(P=Pr, M=Mr, V=Vr, B=Br)
    parity.assert_step(got, ref, f"offload n={n} N={N}")
    assert parity.bit_identical(got, ref)


def test_offload_copies_follow_earlier_work_on_the_stream(orc):
    """Work already on the caller's stream that writes the working copy (here a
    bounded spin, then a fill) lands before the step's bf16 copies, not after."""
    import torch

    import sharded_mixed_precision_rank_amd as zs

    dev = torch.device("cuda:0")
    rng = np.random.default_rng(77)
    n, N, t = 50_000, 2, 4
    G = np.stack([((rng.standard_normal(n) * 1e-3).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
                  for _ in range(N)])
    P = (rng.standard_normal(n) * 0.02).astype(np.float32)
    Z = np.zeros(n, np.float32)
    Gd = [torch.from_numpy(np.ascontiguousarray(g).view(np.int16)).to(dev) for g in G]
    Ph, Mh, Vh = (torch.from_numpy(x.copy()).pin_memory() for x in (P, Z, Z))
    Bo = torch.zeros(n, dtype=torch.int16, device=dev)
    torch.cuda.synchronize()
    if hasattr(torch.cuda, "_sleep"):
        torch.cuda._sleep(20_000_000)  # a few milliseconds of spinning on the current stream
    Bo.fill_(0x1234)
    with zs.Offload(8192, 2) as off:
        off.step(Gd, Ph, Mh, Vh, Bo, HP, t)
    torch.cuda.synchronize()
    _, _, _, Br = orc.step(G, P, Z, Z, HP, t)
    assert np.array_equal(Bo.cpu().numpy().view(np.uint16), Br)
