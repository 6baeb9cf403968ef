"""GPU parity of the two-pass form (clipping, fp16 loss scaling) against the oracle."""
import numpy as np
import pytest

from tests import parity

pytestmark = pytest.mark.gpu

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1)


@pytest.fixture(scope="module")
def env():
    import torch

    import sharded_mixed_precision_rank_amd as zs

    zs.set_grid_blocks(0)
    return dict(torch=torch, zs=zs, dev=torch.device("cuda:0"))


def rand_case(rng, N, n, fmt="bf16", scale=1.0, gscale=1e-3, orc=None):
    x = (rng.standard_normal((N, n)) * gscale * scale).astype(np.float32)
    if fmt == "bf16":
        G = (x.view(np.uint32) >> 16).astype(np.uint16)
    else:
        G = orc.f16(x)
    P = (rng.standard_normal(n) * 0.02).astype(np.float32)
    M = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    V = np.abs(rng.standard_normal(n) * 1e-6).astype(np.float32)
    return dict(G=G, P=P, M=M, V=V)


def run(env, host, hp, t, max_norm=0.0, loss_scale=1.0, gfmt="bf16", pfmt="bf16", offset=0):
    torch, zs, dev = env["torch"], env["zs"], env["dev"]
    n = host["P"].size
    pad = offset
    G = [torch.from_numpy(np.concatenate([np.zeros(pad, np.uint16), g]).view(np.int16)).to(dev)[pad:]
         for g in host["G"]]
    P = torch.from_numpy(np.concatenate([np.zeros(pad, np.float32), host["P"]])).to(dev)[pad:]
    M = torch.from_numpy(np.concatenate([np.zeros(pad, np.float32), host["M"]])).to(dev)[pad:]
    V = torch.from_numpy(np.concatenate([np.zeros(pad, np.float32), host["V"]])).to(dev)[pad:]
    B = torch.zeros(n + pad, dtype=torch.int16, device=dev)[pad:]
    ws = torch.empty(zs.two_pass_workspace_bytes(n), dtype=torch.uint8, device=dev)
    sq = torch.empty(1, dtype=torch.float64, device=dev)
    zs.reduce_grads_flat(G, ws, sq, loss_scale, gfmt)
    torch.cuda.synchronize()
    start = (256 - ws.data_ptr() % 256) % 256
    gbar = ws[start:start + 4 * n].cpu().numpy().view(np.float32).copy()
    sqv = float(sq.cpu().item())
    zs.adam_from_grads_flat(ws, n, P, M, V, B, hp, t, sq, max_norm, pfmt)
    torch.cuda.synchronize()
    got = dict(P=P.cpu().numpy(), M=M.cpu().numpy(), V=V.cpu().numpy(), B=B.cpu().numpy().view(np.uint16))
    return gbar, sqv, got


def oracle_pass2(orc, host, ref_g, sqv, hp, t, max_norm, out_fmt=0):
    """Pass 2 of the oracle on its own mean gradient and its own squared norm.
    The GPU's norm (sqv) is only compared: within 1e-12 relative (the two sum
    the same doubles in different orders) and giving the same fp32 clip
    coefficient."""
    ref_sq = orc.sqnorm(ref_g)
    assert abs(sqv - ref_sq) <= 1e-12 * ref_sq, (sqv, ref_sq)
    assert orc.clip_coef(sqv, max_norm) == orc.clip_coef(ref_sq, max_norm)
    return orc.adam_from_gbar(ref_g, host["P"], host["M"], host["V"], hp, t, ref_sq, max_norm, out_fmt=out_fmt)


@pytest.mark.parametrize("N", [1, 3, 8, 64])
@pytest.mark.parametrize("n", [1, 2047, 2048, 100_003])
def test_two_pass_equals_fused_and_oracle(env, orc, N, n):
    torch, zs, dev = env["torch"], env["zs"], env["dev"]
    rng = np.random.default_rng(N * 1000 + n)
    host = rand_case(rng, N, n)
    gbar, sqv, got = run(env, host, HP, 12)
    # pass 1 against the oracle: the gradient bit for bit, the norm to double rounding
    ref_g = orc.reduce_unscale(host["G"], 0, 1.0)
    assert np.array_equal(gbar.view(np.uint32), ref_g.view(np.uint32))
    ref_sq = orc.sqnorm(ref_g)
    assert abs(sqv - ref_sq) <= 1e-12 * ref_sq
    # pass 2 against the oracle and against the fused step
    P1, M1, V1, B1, taken = oracle_pass2(orc, host, ref_g, sqv, HP, 12, 0.0)
    assert taken
    assert parity.bit_identical(got, dict(P=P1, M=M1, V=V1, B=B1))
    fP, fM, fV, fB = orc.step(host["G"], host["P"], host["M"], host["V"], HP, 12)
    assert parity.bit_identical(got, dict(P=fP, M=fM, V=fV, B=fB))


@pytest.mark.parametrize("shrink", [2.0, 7.0, 1000.0])
def test_clipping_matches_oracle(env, orc, shrink):
    rng = np.random.default_rng(int(shrink))
    host = rand_case(rng, 8, 50_001)
    ref_g = orc.reduce_unscale(host["G"], 0, 1.0)
    norm = orc.sqnorm(ref_g) ** 0.5
    gbar, sqv, got = run(env, host, HP, 300, max_norm=norm / shrink)
    assert np.array_equal(gbar.view(np.uint32), ref_g.view(np.uint32))
    assert orc.clip_coef(orc.sqnorm(ref_g), norm / shrink) < 1.0  # clipping is active
    P1, M1, V1, B1, taken = oracle_pass2(orc, host, ref_g, sqv, HP, 300, norm / shrink)
    ref = dict(P=P1, M=M1, V=V1, B=B1)
    parity.assert_step(got, ref, f"clip /{shrink}")
    assert parity.bit_identical(got, ref)


@pytest.mark.parametrize("loss_scale", [1.0, 2.0 ** 8, 2.0 ** 16])
def test_fp16_loss_scaled_grads_and_fp16_copy(env, orc, loss_scale):
    rng = np.random.default_rng(int(np.log2(loss_scale)) + 5)
    host = rand_case(rng, 4, 30_000, fmt="fp16", scale=loss_scale, orc=orc)
    gbar, sqv, got = run(env, host, HP, 40, max_norm=1.0, loss_scale=loss_scale, gfmt="fp16", pfmt="fp16")
    ref_g = orc.reduce_unscale(host["G"], 1, loss_scale)
    assert np.array_equal(gbar.view(np.uint32), ref_g.view(np.uint32))
    P1, M1, V1, B1, taken = oracle_pass2(orc, host, ref_g, sqv, HP, 40, 1.0, out_fmt=1)
    ref = dict(P=P1, M=M1, V=V1, B=B1)
    for k in "PMV":
        parity.assert_f32(got[k], ref[k], k)
    assert np.array_equal(got["B"], B1), "fp16 working copy"
    for k in "PMV":
        assert np.array_equal(got[k].view(np.uint32), ref[k].view(np.uint32)), k


def test_fp16_overflow_skips_the_step(env, orc):
    rng = np.random.default_rng(9)
    host = rand_case(rng, 4, 10_000, fmt="fp16", scale=2.0 ** 16, orc=orc)
    host["G"][2, 1234] = 0x7C00  # +Inf in one replica
    gbar, sqv, got = run(env, host, HP, 7, max_norm=1.0, loss_scale=2.0 ** 16, gfmt="fp16", pfmt="fp16")
    assert not np.isfinite(sqv)
    assert np.array_equal(got["P"], host["P"]) and np.array_equal(got["M"], host["M"])
    assert np.array_equal(got["V"], host["V"]) and np.all(got["B"] == 0)


def test_misaligned_two_pass(env, orc):
    """Offsets 1..63 put up to 63 elements in the head partial of the norm;
    clipping is active, so a wrong head partial would change every update."""
    rng = np.random.default_rng(11)
    host = rand_case(rng, 3, 9_999)
    ref_g = orc.reduce_unscale(host["G"], 0, 1.0)
    max_norm = orc.sqnorm(ref_g) ** 0.5 / 3
    assert orc.clip_coef(orc.sqnorm(ref_g), max_norm) < 0.5
    for off in (1, 3, 8, 40, 63):
        gbar, sqv, got = run(env, host, HP, 2, max_norm=max_norm, offset=off)
        assert np.array_equal(gbar.view(np.uint32), ref_g.view(np.uint32))
        P1, M1, V1, B1, _ = oracle_pass2(orc, host, ref_g, sqv, HP, 2, max_norm)
        assert parity.bit_identical(got, dict(P=P1, M=M1, V=V1, B=B1)), off


def test_norm_does_not_depend_on_launch_size(env):
    torch, zs, dev = env["torch"], env["zs"], env["dev"]
    rng = np.random.default_rng(13)
    n, N = 1_000_003, 8
    G = [torch.from_numpy(((rng.standard_normal(n) * 1e-3).astype(np.float32).view(np.uint32) >> 16)
                          .astype(np.uint16).view(np.int16)).to(dev) for _ in range(N)]
    ws = torch.empty(zs.two_pass_workspace_bytes(n), dtype=torch.uint8, device=dev)
    vals = []
    try:
        for blocks in (0, 1, 7, 333):
            zs.set_grid_blocks(blocks)
            sq = torch.empty(1, dtype=torch.float64, device=dev)
            zs.reduce_grads_flat(G, ws, sq)
            torch.cuda.synchronize()
            vals.append(sq.item())
    finally:
        zs.set_grid_blocks(0)
    assert len(set(vals)) == 1, vals


def test_empty_shard_norm_is_zero(env):
    torch, zs, dev = env["torch"], env["zs"], env["dev"]
    sq = torch.full((1,), 5.0, dtype=torch.float64, device=dev)
    e = torch.empty(0, dtype=torch.bfloat16, device=dev)
    zs.reduce_grads_flat([e, e], torch.empty(0, dtype=torch.uint8, device=dev), sq)
    torch.cuda.synchronize()
    assert sq.item() == 0.0


def test_clipped_step_convenience(env, orc):
    torch, zs, dev = env["torch"], env["zs"], env["dev"]
    rng = np.random.default_rng(17)
    host = rand_case(rng, 2, 5000)
    G = [torch.from_numpy(g.view(np.int16)).to(dev) for g in host["G"]]
    P, M, V = (torch.from_numpy(host[k]).to(dev) for k in "PMV")
    B = torch.zeros(5000, dtype=torch.int16, device=dev)
    sq = zs.clipped_step_flat(G, P, M, V, B, HP, 3, max_norm=0.01)
    torch.cuda.synchronize()
    ref_g = orc.reduce_unscale(host["G"], 0, 1.0)
    P1, M1, V1, B1, _ = oracle_pass2(orc, host, ref_g, sq.item(), HP, 3, 0.01)
    got = dict(P=P.cpu().numpy(), M=M.cpu().numpy(), V=V.cpu().numpy(), B=B.cpu().numpy().view(np.uint16))
    assert parity.bit_identical(got, dict(P=P1, M=M1, V=V1, B=B1))


def test_clipped_step_on_a_side_stream(env, orc):
    """clipped_step_flat on a non-default stream, with its workspace allocated
    by the call: allocations made on the current stream right after it must not
    take that workspace while the side stream still has the passes queued."""
    torch, zs, dev = env["torch"], env["zs"], env["dev"]
    rng = np.random.default_rng(19)
    n = 3_000_017
    host = rand_case(rng, 8, n)
    G = [torch.from_numpy(g.view(np.int16)).to(dev) for g in host["G"]]
    P, M, V = (torch.from_numpy(host[k]).to(dev) for k in "PMV")
    B = torch.zeros(n, dtype=torch.int16, device=dev)
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    # keep the side stream busy first, so both passes are still queued when the call returns
    big = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    with torch.cuda.stream(side):
        for _ in range(8):
            big.mul_(1.0)
    sq = zs.clipped_step_flat(G, P, M, V, B, HP, 4, max_norm=0.05, stream=side)
    # allocations of the workspace's size on the current stream, filled at once
    junk = [torch.full((zs.two_pass_workspace_bytes(n) // 4,), float("nan"), device=dev) for _ in range(3)]
    torch.cuda.synchronize()
    del junk, big
    ref_g = orc.reduce_unscale(host["G"], 0, 1.0)
    P1, M1, V1, B1, _ = oracle_pass2(orc, host, ref_g, sq.item(), HP, 4, 0.05)
    got = dict(P=P.cpu().numpy(), M=M.cpu().numpy(), V=V.cpu().numpy(), B=B.cpu().numpy().view(np.uint16))
    assert parity.bit_identical(got, dict(P=P1, M=M1, V=V1, B=B1))


def _scaler_state(st) -> dict:
    return {k: getattr(st, k) for k in ("scale", "min_scale", "window", "hysteresis", "overflows", "clean")}


def test_device_loss_scaler_follows_the_oracle(env, orc):
    """The device scaler against the oracle's scaler, step by step, on a random
    overflow sequence (an Inf or NaN global norm is an overflow)."""
    torch, zs, dev = env["torch"], env["zs"], env["dev"]
    rng = np.random.default_rng(21)
    ds = zs.LossScaler(2.0 ** 16, 1.0, 7, 2).to_device(dev)
    ref = orc.scaler(2.0 ** 16, 1.0, 7, 2)
    taken = torch.zeros(1, dtype=torch.int32, device=dev)
    for k in range(200):
        u = rng.random()
        value = float("inf") if u < 0.15 else float("nan") if u < 0.2 else float(rng.random() * 10)
        sq = torch.tensor([value], dtype=torch.float64, device=dev)
        ds.update(sq, taken)
        ref_taken = orc.scaler_update(ref, not np.isfinite(value))
        assert ds.state() == _scaler_state(ref), k
        assert int(taken.item()) == int(ref_taken), k


@pytest.mark.parametrize("scale", [1.0, 2.0 ** 8, 2.0 ** 16, 3.0])
def test_device_scale_pass1_equals_host_scale(env, orc, scale):
    torch, zs, dev = env["torch"], env["zs"], env["dev"]
    rng = np.random.default_rng(int(scale) + 40)
    n = 50_001
    host = rand_case(rng, 3, n, fmt="fp16", scale=scale, orc=orc)
    G = [torch.from_numpy(g.view(np.int16)).to(dev) for g in host["G"]]
    outs = []
    for device_scale in (False, True):
        ws = torch.zeros(zs.two_pass_workspace_bytes(n), dtype=torch.uint8, device=dev)
        sq = torch.zeros(1, dtype=torch.float64, device=dev)
        if device_scale:
            zs.reduce_grads_flat_device_scale(G, ws, sq, zs.LossScaler(scale, 1.0, 10, 2).to_device(dev), "fp16")
        else:
            zs.reduce_grads_flat(G, ws, sq, scale, "fp16")
        torch.cuda.synchronize()
        start = (256 - ws.data_ptr() % 256) % 256
        outs.append((ws[start:start + 4 * n].cpu().numpy().copy(), float(sq.item())))
    assert np.array_equal(outs[0][0], outs[1][0]) and outs[0][1] == outs[1][1]
    ref_g = orc.reduce_unscale(host["G"], 1, scale)
    assert np.array_equal(outs[1][0].view(np.float32).view(np.uint32), ref_g.view(np.uint32))


def test_fp16_steps_without_host_round_trips(env, orc):
    """Six fp16 steps, each pass 1 with the device scale, pass 2 with clipping
    and overflow skip, then the device scaler update, with no host
    synchronisation between them; steps 2 and 4 carry an Inf replica.  The
    final state and scale equal the oracle's run of the same sequence."""
    torch, zs, dev = env["torch"], env["zs"], env["dev"]
    rng = np.random.default_rng(77)
    n, N = 20_003, 4
    P = (rng.standard_normal(n) * 0.02).astype(np.float32)
    M = np.zeros(n, np.float32)
    V = np.zeros(n, np.float32)
    scaler = zs.LossScaler(2.0 ** 15, 1.0, 2, 1)
    ds = scaler.to_device(dev)
    ref_sc = orc.scaler(2.0 ** 15, 1.0, 2, 1)
    Pd, Md, Vd = (torch.from_numpy(x.copy()).to(dev) for x in (P, M, V))
    Bd = torch.zeros(n, dtype=torch.float16, device=dev)
    ws = torch.empty(zs.two_pass_workspace_bytes(n), dtype=torch.uint8, device=dev)
    sq = torch.empty(1, dtype=torch.float64, device=dev)
    Pr, Mr, Vr, Br = P.copy(), M.copy(), V.copy(), np.zeros(n, np.uint16)
    for t in range(1, 7):
        x = (rng.standard_normal((N, n)) * 1e-3).astype(np.float32)
        # the replicas the device sees are scaled by the scale the oracle's scaler holds at this step
        Gh = orc.f16(x * np.float32(ref_sc.scale))
        if t in (2, 4):
            Gh[1, 77] = 0x7C00
        G = [torch.from_numpy(g.view(np.int16)).to(dev) for g in Gh]
        zs.reduce_grads_flat_device_scale(G, ws, sq, ds, "fp16")
        zs.adam_from_grads_flat(ws, n, Pd, Md, Vd, Bd, HP, t, sq, 1.0, "fp16")
        ds.update(sq)
        # the oracle, driven from the host
        g = orc.reduce_unscale(Gh, 1, ref_sc.scale)
        tsq = orc.sqnorm(g)
        Pr, Mr, Vr, B1, taken = orc.adam_from_gbar(g, Pr, Mr, Vr, HP, t, tsq, 1.0, out_fmt=1)
        if taken:
            Br = B1
        orc.scaler_update(ref_sc, not np.isfinite(tsq))
    torch.cuda.synchronize()
    assert ds.state() == _scaler_state(ref_sc)
    got = dict(P=Pd.cpu().numpy(), M=Md.cpu().numpy(), V=Vd.cpu().numpy(), B=Bd.view(torch.int16).cpu().numpy().view(np.uint16))
    for k, r in (("P", Pr), ("M", Mr), ("V", Vr)):
        assert np.array_equal(got[k].view(np.uint32), r.view(np.uint32)), k
    assert np.array_equal(got["B"], Br)
