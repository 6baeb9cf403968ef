"""The step under HIP graph capture: the library enqueues no memsets and no
host synchronisation, so the fused step, and the whole fp16 step of the
two-pass form (pass 1 with the device loss scale, pass 2, the device scaler
update), can be captured once and replayed.  Each replay is checked against
the same step run eagerly on a copy of the state, with eager work and
synchronisation between the replays.  The step index is a kernel argument,
fixed at capture."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1)


def _state(torch, rng, n, dev):
    return [torch.from_numpy(x).to(dev) for x in ((rng.standard_normal(n) * 0.02).astype(np.float32),
                                                  (rng.standard_normal(n) * 1e-4).astype(np.float32),
                                                  np.abs(rng.standard_normal(n) * 1e-6).astype(np.float32))]


def test_fused_step_in_a_graph(orc):
    import torch

    import sharded_mixed_precision_rank_amd as zs

    dev = torch.device("cuda:0")
    rng = np.random.default_rng(8)
    n, N = 300_007, 8
    G = [torch.from_numpy(((rng.standard_normal(n) * 1e-3).astype(np.float32).view(np.uint32) >> 16)
                          .astype(np.uint16).view(np.int16)).to(dev) for _ in range(N)]
    P, M, V = _state(torch, rng, n, dev)
    B = torch.zeros(n, dtype=torch.int16, device=dev)
    Pe, Me, Ve, Be = P.clone(), M.clone(), V.clone(), B.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # a first call outside capture settles the library's one-time queries
        zs.reduce_adam_flat(G, P, M, V, B, HP, 5)
    torch.cuda.current_stream().wait_stream(side)
    zs.reduce_adam_flat(G, Pe, Me, Ve, Be, HP, 5)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        zs.reduce_adam_flat(G, P, M, V, B, HP, 5)
    for replay in range(4):
        graph.replay()
        zs.reduce_adam_flat(G, Pe, Me, Ve, Be, HP, 5)  # eager work between the replays
        torch.cuda.synchronize()
        for a, b in ((P, Pe), (M, Me), (V, Ve), (B, Be)):
            assert torch.equal(a, b), f"replay {replay}"


def test_fp16_two_pass_step_with_device_scaler_in_a_graph(orc):
    import torch

    import sharded_mixed_precision_rank_amd as zs

    dev = torch.device("cuda:0")
    rng = np.random.default_rng(9)
    n, N = 100_003, 4
    G = [torch.from_numpy(orc.f16((rng.standard_normal(n) * 1e-3 * 2 ** 12).astype(np.float32)).view(np.int16))
         .to(dev) for _ in range(N)]
    ws_bytes = zs.two_pass_workspace_bytes(n)
    runs = []
    for _ in range(2):  # [0] replayed from the graph, [1] eager
        P, M, V = (x.clone() for x in _state(torch, np.random.default_rng(10), n, dev))
        runs.append(dict(P=P, M=M, V=V, B=torch.zeros(n, dtype=torch.float16, device=dev),
                         ws=torch.empty(ws_bytes, dtype=torch.uint8, device=dev),
                         sq=torch.empty(1, dtype=torch.float64, device=dev),
                         sc=zs.LossScaler(2.0 ** 12, 1.0, 2, 1).to_device(dev)))

    def step(r):
        zs.reduce_grads_flat_device_scale(G, r["ws"], r["sq"], r["sc"], "fp16")
        zs.adam_from_grads_flat(r["ws"], n, r["P"], r["M"], r["V"], r["B"], HP, 3, r["sq"], 1.0, "fp16")
        r["sc"].update(r["sq"])

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(runs[0])
    torch.cuda.current_stream().wait_stream(side)
    step(runs[1])
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(runs[0])
    for replay in range(4):
        graph.replay()
        step(runs[1])
        torch.cuda.synchronize()
        for k in ("P", "M", "V", "B", "sq"):
            assert torch.equal(runs[0][k], runs[1][k]), f"replay {replay}: {k}"
        assert runs[0]["sc"].state() == runs[1]["sc"].state(), f"replay {replay}: scaler"
