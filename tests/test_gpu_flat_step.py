"""The prepared flat step (FlatStep) against reduce_adam_flat and the oracle:
the same bits over three steps, with a frozen AdamHP (packed once) and a dict
(packed per call), on torch's current stream and on a fixed side stream."""
import numpy as np
import pytest

from tests import parity
from tests.test_gpu_flat import HP, download, rand_host, upload

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("N,n,fixed_stream", [(2, 100_003, False), (8, 1 << 20, True), (3, 7, False)])
def test_flat_step_matches_the_plain_call_and_the_oracle(orc, N, n, fixed_stream):
    import torch

    import sharded_mixed_precision_rank_amd as zs

    dev = torch.device("cuda:0")
    host = rand_host(np.random.default_rng(N * 1000 + n % 997), N, n)
    a = upload(torch, dev, host)
    b = upload(torch, dev, host)
    for d in (a, b):
        d["B"] = torch.zeros(n, dtype=torch.int16, device=dev)
    hp_frozen = zs.AdamHP(**HP)
    side = torch.cuda.Stream(device=dev) if fixed_stream else None
    if side is not None:
        side.wait_stream(torch.cuda.current_stream())
    step = zs.FlatStep(b["G"], b["P"], b["M"], b["V"], b["B"], stream=side)
    P, M, V = host["P"].copy(), host["M"].copy(), host["V"].copy()
    for t, hp in ((1, hp_frozen), (2, hp_frozen), (3, dict(HP))):
        zs.reduce_adam_flat(a["G"], a["P"], a["M"], a["V"], a["B"], hp, t)
        step(hp, t)
        torch.cuda.synchronize()
        P, M, V, B = orc.step(host["G"], P, M, V, HP, t)
        ref = dict(P=P, M=M, V=V, B=B)
        assert parity.bit_identical(download(b), download(a)), f"step {t}: prepared against plain"
        assert parity.bit_identical(download(b), ref), f"step {t}: prepared against the oracle"


def test_flat_step_checks_its_arguments_once():
    """The checks of reduce_adam_flat run at construction: wrong dtypes and sizes are refused there."""
    import torch

    import sharded_mixed_precision_rank_amd as zs

    dev = torch.device("cuda:0")
    n = 1000
    G = [torch.zeros(n, dtype=torch.int16, device=dev) for _ in range(2)]
    P, M, V = (torch.zeros(n, dtype=torch.float32, device=dev) for _ in range(3))
    B = torch.zeros(n, dtype=torch.int16, device=dev)
    zs.FlatStep(G, P, M, V, B)
    with pytest.raises(TypeError):
        zs.FlatStep(G, P.double(), M, V, B)
    with pytest.raises(ValueError):
        zs.FlatStep(G, P, M[:-1], V, B)
    with pytest.raises(ValueError):
        zs.FlatStep([G[0], G[1][:-1]], P, M, V, B)
