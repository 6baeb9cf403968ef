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


def _grads(torch, rng, N, n, dev):
    return [torch.from_numpy(((rng.standard_normal(n) * 1e-3).astype(np.float32).view(np.uint32) >> 16)
                             .astype(np.uint16).view(np.int16)).to(dev) for _ in range(N)]


def test_device_step_matches_host_step_and_skips_outside_the_table(orc):
    import torch

    import sharded_mixed_precision_rank_amd as zs

    dev = torch.device("cuda:0")
    rng = np.random.default_rng(12)
    n, N = 70_001, 3
    G = _grads(torch, rng, N, n, dev)
    P, M, V = _state(torch, rng, n, dev)
    B = torch.zeros(n, dtype=torch.int16, device=dev)
    Ph, Mh, Vh, Bh = P.clone(), M.clone(), V.clone(), B.clone()
    src = zs.StepSource(HP, 5, 10, dev, start=7)
    zs.reduce_adam_flat_devstep(G, P, M, V, B, src)
    zs.reduce_adam_flat(G, Ph, Mh, Vh, Bh, HP, 7)
    torch.cuda.synchronize()
    for a, b in ((P, Ph), (M, Mh), (V, Vh), (B, Bh)):
        assert torch.equal(a, b)
    assert src.status == 0
    # a step outside the table (5 .. 14) changes nothing and is reported
    src.step_t.fill_(15)
    before = [x.clone() for x in (P, M, V, B)]
    zs.reduce_adam_flat_devstep(G, P, M, V, B, src)
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip((P, M, V, B), before))
    assert src.status == 1


def test_graph_replays_advance_the_step(orc):
    """[fused step with the device step, advance] captured once and replayed
    five times equals five host-driven steps t = 1..5, replay by replay."""
    import torch

    import sharded_mixed_precision_rank_amd as zs

    dev = torch.device("cuda:0")
    rng = np.random.default_rng(13)
    n, N = 200_003, 4
    G = _grads(torch, rng, N, n, dev)
    P, M, V = _state(torch, rng, n, dev)
    B = torch.zeros(n, dtype=torch.int16, device=dev)
    Pe, Me, Ve, Be = P.clone(), M.clone(), V.clone(), B.clone()
    src = zs.StepSource(HP, 1, 100, dev)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside capture on scratch copies (one-time library queries)
        Pw, Mw, Vw, Bw = P.clone(), M.clone(), V.clone(), B.clone()
        zs.reduce_adam_flat_devstep(G, Pw, Mw, Vw, Bw, src)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        zs.reduce_adam_flat_devstep(G, P, M, V, B, src)
        src.advance()
    for t in range(1, 6):
        graph.replay()
        zs.reduce_adam_flat(G, Pe, Me, Ve, Be, HP, t)
        torch.cuda.synchronize()
        for a, b in ((P, Pe), (M, Me), (V, Ve), (B, Be)):
            assert torch.equal(a, b), f"replay for step {t}"
        assert src.step == t + 1


def test_fp16_graph_replays_with_device_step_and_scaler(orc):
    """The fp16 step [pass 1 with the device scale, pass 2 with the device step,
    scaler update, advance] captured once and replayed six times equals the
    host-driven oracle run of steps 1..6, including overflow steps (an Inf
    replica at steps 2 and 5, written into the replica buffer between
    replays)."""
    import torch

    import sharded_mixed_precision_rank_amd as zs

    dev = torch.device("cuda:0")
    rng = np.random.default_rng(14)
    n, N = 30_011, 4
    x = [(rng.standard_normal(n) * 1e-3).astype(np.float32) for _ in range(N)]
    Gd = [torch.empty(n, dtype=torch.int16, device=dev) for _ in range(N)]
    P0, M0, V0 = (np.asarray(t.cpu()) for t in _state(torch, rng, n, dev))
    P, M, V = (torch.from_numpy(a.copy()).to(dev) for a in (P0, M0, V0))
    B = torch.zeros(n, dtype=torch.float16, device=dev)
    ws = torch.empty(zs.two_pass_workspace_bytes(n), dtype=torch.uint8, device=dev)
    sq = torch.empty(1, dtype=torch.float64, device=dev)
    scaler = zs.LossScaler(2.0 ** 10, 1.0, 2, 1).to_device(dev)
    src = zs.StepSource(HP, 1, 50, dev)
    ref_sc = orc.scaler(2.0 ** 10, 1.0, 2, 1)

    def fill(t):  # the replicas of step t at the oracle scaler's current scale (input preparation)
        Gh = [orc.f16(xi * np.float32(ref_sc.scale)) for xi in x]
        if t in (2, 5):
            Gh[1][9] = 0x7C00
        for d, h in zip(Gd, Gh):
            d.copy_(torch.from_numpy(h.view(np.int16)))
        return Gh

    def step():
        zs.reduce_grads_flat_device_scale(Gd, ws, sq, scaler, "fp16")
        zs.adam_from_grads_flat_devstep(ws, n, P, M, V, B, src, sq, 1.0, "fp16")
        scaler.update(sq)
        src.advance()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside capture, on scratch state and a scratch step source
        fill(1)
        w_src = zs.StepSource(HP, 1, 50, dev)
        w_sc = zs.LossScaler(2.0 ** 10, 1.0, 2, 1).to_device(dev)
        Pw, Mw, Vw, Bw = P.clone(), M.clone(), V.clone(), B.clone()
        zs.reduce_grads_flat_device_scale(Gd, ws, sq, w_sc, "fp16")
        zs.adam_from_grads_flat_devstep(ws, n, Pw, Mw, Vw, Bw, w_src, sq, 1.0, "fp16")
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    Pr, Mr, Vr, Br = P0.copy(), M0.copy(), V0.copy(), np.zeros(n, np.uint16)
    for t in range(1, 7):
        Gh = fill(t)
        torch.cuda.synchronize()
        graph.replay()
        g = orc.reduce_unscale(Gh, 1, ref_sc.scale)
        tsq = orc.sqnorm(g)
        Pr, Mr, Vr, B1, taken = orc.adam_from_gbar(g, Pr, Mr, Vr, HP, t, tsq, 1.0, out_fmt=1)
        if taken:
            Br = B1
        orc.scaler_update(ref_sc, not np.isfinite(tsq))
        torch.cuda.synchronize()
        assert scaler.state()["scale"] == ref_sc.scale, t
        got = dict(P=P.cpu().numpy(), M=M.cpu().numpy(), V=V.cpu().numpy())
        for k, r in (("P", Pr), ("M", Mr), ("V", Vr)):
            assert np.array_equal(got[k].view(np.uint32), r.view(np.uint32)), (t, k)
        assert np.array_equal(B.view(torch.int16).cpu().numpy().view(np.uint16), Br), t
    assert src.step == 7


def test_list_plan_graph_replays_advance_the_step(orc):
    """A ragged list plan's step with the device step, [step, advance] captured
    once and replayed four times, against the oracle per tensor at t = 1..4."""
    import torch

    import sharded_mixed_precision_rank_amd as zs
    from tests.test_gpu_list import arena_case, oracle_list, small_ragged

    dev = torch.device("cuda:0")
    env = dict(torch=torch, zs=zs, dev=dev)
    w = small_ragged(8, 80, seed=55)
    host, d, offsets, L = arena_case(env, w)
    src = zs.StepSource(HP, 1, 10, dev)
    with zs.ListPlan.from_arenas(w.sizes, offsets, d["G"], d["P"], d["M"], d["V"], d["B"]) as plan:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):  # warm-up outside capture: an out-of-range step updates nothing
            w_src = zs.StepSource(HP, 1, 10, dev, start=11)
            plan.step_devstep(w_src)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        assert w_src.status == 1
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            plan.step_devstep(src)
            src.advance()
        state = dict(G=host["G"], P=host["P"], M=host["M"], V=host["V"])
        for t in range(1, 5):
            graph.replay()
            torch.cuda.synchronize()
            ref = oracle_list(orc, w, state, offsets, t, HP)
            state = dict(G=host["G"], P=ref["P"], M=ref["M"], V=ref["V"])
            got = dict(P=d["P"].cpu().numpy(), M=d["M"].cpu().numpy(), V=d["V"].cpu().numpy(),
                       B=d["B"].cpu().numpy().view(np.uint16))
            for k in "PMV":
                assert np.array_equal(got[k].view(np.uint32), ref[k].view(np.uint32)), (t, k)
            assert np.array_equal(got["B"], ref["B"]), t
