"""Pins: checks that tie the CPU oracle to something other than itself.

Each pin takes an object with the ``oracle.Oracle`` interface and raises
AssertionError when the oracle disagrees with what the pages or the
mathematics fix.  ``test_oracle_pins.py`` runs them on the oracle;
``test_oracle_mutants.py`` runs them on deliberately broken copies of it to
show each plausible mistake is caught.

  P1  N identical replicas average to that replica, bit for bit, and the whole
      step equals the one-replica step (the averaging equation of "Data
      Parallelism 数据并行（二）", section 数据并行训练（DP）).
  P2  First step from zero moments moves every weight by -lr*g/(|g|+eps)
      (closed form of bias-corrected Adam at t = 1), m' = 0.1 g, v' = 0.001 g^2.
  P3  Zero gradient at t = 1 without decay leaves the weight exactly alone.
  P4  Zero gradient and zero moments with decay scale the weight by 1 - lr*wd
      (decoupled, learning-rate-scaled weight decay).
  P5  A constant gradient for 10,000 steps from zero state: m_t = (1-b1^t) g,
      v_t = (1-b2^t) g^2 and each step moves the weight by lr*g/(|g|+eps).
  P6  State bytes per parameter = 16, as the pages print (golden file).
  P7  Random tiny inputs agree with a float64 evaluation within a rigorous
      running forward-error bound.
  P8  Replicas are summed in rank order 0..N-1 (cases whose sum differs under
      reversed or pairwise order).
  P9  bf16 re-cast = round to nearest even (hand cases + torch's CPU cast).
  P10 Agreement with torch.optim.AdamW in float64 within the P7 bound.
  P11 Folded scalars are the doubles rounded once to fp32.
"""
from __future__ import annotations

import math
import os
import struct

import numpy as np

from tests import f64_bruteforce as bf

U = 2.0 ** -24
HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0)
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def f32(x: float) -> float:
    return struct.unpack("f", struct.pack("f", x))[0]


def bits(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def bf16_bits_trunc(x) -> np.ndarray:
    return (np.ascontiguousarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def widen(h) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def ulp32(x) -> np.ndarray:
    x = np.abs(np.asarray(x, dtype=np.float32))
    return np.spacing(np.maximum(x, np.float32(1.17549435e-38))).astype(np.float64)


def rand_bf16(rng, n, scale=1e-3) -> np.ndarray:
    return bf16_bits_trunc((rng.standard_normal(n) * scale).astype(np.float32))


# ----------------------------------------------------------------------- P1
def pin_identical_replicas(o):
    rng = np.random.default_rng(101)
    mags = 2.0 ** rng.integers(-130, 120, 4096)
    g = bf16_bits_trunc((rng.standard_normal(4096) * mags).astype(np.float32))
    g[:4] = [0x0000, 0x8000, 0x0001, 0x8001]          # +0, -0, smallest subnormals
    P = (rng.standard_normal(4096) * 0.02).astype(np.float32)
    M = (rng.standard_normal(4096) * 1e-4).astype(np.float32)
    V = np.abs(rng.standard_normal(4096) * 1e-6).astype(np.float32)
    ref = o.step([g], P, M, V, HP, 7, threads=1)
    for N in (1, 2, 3, 5, 7, 8, 12, 48, 64):
        gbar = o.reduce_mean([g] * N, threads=1)
        assert np.array_equal(bits(gbar), bits(widen(g))), f"P1: mean of {N} identical replicas != replica"
        out = o.step([g] * N, P, M, V, HP, 7, threads=1)
        for a, b, name in zip(out, ref, "PMVB"):
            assert np.array_equal(np.asarray(a).view(np.uint8), np.asarray(b).view(np.uint8)), \
                f"P1: step with {N} identical replicas differs from one replica in {name}"


# ----------------------------------------------------------------------- P2
def pin_first_step(o):
    rng = np.random.default_rng(102)
    n = 8192
    scale = np.concatenate([np.full(n // 2, 1e-3), 10.0 ** rng.uniform(-7, 2, n // 2)])
    g = rand_bf16(rng, n, 1.0)
    g = bf16_bits_trunc(widen(g) * scale.astype(np.float32))
    g[(g & 0x7FFF) == 0] = 0x3A83                         # no zero grads here
    P = (rng.standard_normal(n) * 0.02).astype(np.float32)
    Z = np.zeros(n, dtype=np.float32)
    lr, eps = HP["lr"], HP["eps"]
    P1, M1, V1, B1 = o.step([g], P, Z, Z, HP, 1, threads=1)
    gd = widen(g).astype(np.float64)
    delta = -lr * gd / (np.abs(gd) + eps)
    err = np.abs((P1.astype(np.float64) - P) - delta)
    tol = 12 * U * np.abs(delta) + U * np.abs(P1.astype(np.float64)) + U * np.abs(P.astype(np.float64))
    assert np.all(err <= tol), f"P2: first step is not -lr*g/(|g|+eps): worst {np.max(err - tol):.3e}"
    big = np.abs(delta) > 8 * ulp32(P)
    assert np.all(np.sign(P1[big].astype(np.float64) - P[big]) == -np.sign(gd[big])), "P2: step not against g"
    assert np.all(np.abs(M1 - 0.1 * gd) <= 2 * U * np.abs(0.1 * gd)), "P2: m' != (1-beta1) g"
    assert np.all(np.abs(V1 - 0.001 * gd * gd) <= 4 * U * 0.001 * gd * gd + 1e-45), "P2: v' != (1-beta2) g^2"


# ----------------------------------------------------------------------- P3
def pin_zero_grad(o):
    rng = np.random.default_rng(103)
    n = 1024
    G = [np.where(rng.random(n) < 0.5, 0x0000, 0x8000).astype(np.uint16) for _ in range(4)]
    P = (rng.standard_normal(n) * 0.02).astype(np.float32)
    Z = np.zeros(n, dtype=np.float32)
    P1, M1, V1, B1 = o.step(G, P, Z, Z, HP, 1, threads=1)
    assert np.array_equal(bits(P1), bits(P)), "P3: zero grad moved the weight"
    assert np.all(M1 == 0) and np.all(V1 == 0), "P3: zero grad gave non-zero moments"
    assert not np.any(np.isnan(P1)), "P3: NaN from 0/eps"


# ----------------------------------------------------------------------- P4
def pin_decoupled_decay(o):
    rng = np.random.default_rng(104)
    n = 4096
    P = (rng.standard_normal(n) * 0.02).astype(np.float32)
    Z = np.zeros(n, dtype=np.float32)
    zg = np.zeros(n, dtype=np.uint16)
    for wd in (0.1, 0.01):
        for t in (1, 5000):
            hp = dict(HP, weight_decay=wd)
            P1, M1, V1, B1 = o.step([zg, zg], P, Z, Z, hp, t, threads=1)
            exact = (1.0 - hp["lr"] * wd) * P.astype(np.float64)
            assert np.all(np.abs(P1 - exact) <= 2 * U * np.abs(exact)), \
                f"P4: zero-grad step with wd={wd}, t={t} is not p*(1-lr*wd)"
            assert np.all(M1 == 0) and np.all(V1 == 0)


# ----------------------------------------------------------------------- P5
def pin_constant_grad_run(o, T: int = 10_000):
    rng = np.random.default_rng(105)
    n = 64
    g = bf16_bits_trunc((np.sign(rng.standard_normal(n)) * 10.0 ** rng.uniform(-5, -1, n)).astype(np.float32))
    gd = widen(g).astype(np.float64)
    P = np.zeros(n, dtype=np.float32)
    M = np.zeros(n, dtype=np.float32)
    V = np.zeros(n, dtype=np.float32)
    B = np.zeros(n, dtype=np.uint16)
    b1, b2, lr, eps = HP["beta1"], HP["beta2"], HP["lr"], HP["eps"]
    tol_m = (3 / (1 - b1) + 4) * U
    tol_v = (3 / (1 - b2) + 8) * U
    tol_d = (4 / (1 - b1) + 2 / (1 - b2) + 32) * U
    check = {1, 2, 3, 10, 100, 1000, 5000, T}
    for t in range(1, T + 1):
        Pprev = P.copy()
        o.step_inplace([g], P, M, V, B, HP, t, threads=1)
        if t in check:
            mt = (1 - b1 ** t) * gd
            vt = (1 - b2 ** t) * gd * gd
            assert np.all(np.abs(M - mt) <= tol_m * np.abs(mt)), f"P5: m_t wrong at t={t}"
            assert np.all(np.abs(V - vt) <= tol_v * vt), f"P5: v_t wrong at t={t}"
            step = P.astype(np.float64) - Pprev
            exact = -lr * gd / (np.abs(gd) + eps)
            bound = tol_d * np.abs(exact) + ulp32(P) + ulp32(Pprev)
            assert np.all(np.abs(step - exact) <= bound), f"P5: step size wrong at t={t}"


# ----------------------------------------------------------------------- P6
def read_golden_memory():
    out = {}
    with open(os.path.join(GOLDEN, "memory_accounting.txt"), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, value, _src = [s.strip() for s in line.split("|", 2)]
            out[name] = float(value)
    return out


def pin_memory_accounting(o):
    gold = read_golden_memory()
    assert o.state_bytes_per_param() == gold["state_bytes_per_param_bf16"] == gold["state_bytes_per_param_fp16"]
    assert o.sharded_state_bytes(70e9, 1) > gold["state_bytes_70B_exceeds"]
    assert o.sharded_state_bytes(1.0, 1) == gold["sharded_state_bytes_formula_psi"]
    assert math.isclose(o.sharded_state_bytes(70e9, 64), 16 * 70e9 / 64)
    # fp16 parameters alone are 2 of the 16 bytes: 140/N GB
    assert round(o.sharded_state_bytes(70e9, 64) * 2 / 16 / 1e9, 1) == gold["fp16_param_shard_GB_N64"]
    assert o.sharded_state_bytes(70e9, 8) * 2 / 16 / 1e9 == gold["fp16_param_shard_GB_N8"]
    # traffic of one step: each replica's bf16 grad read once, fp32 state read and written, bf16 copy written
    for N in (1, 2, 8, 64):
        assert o.step_traffic_bytes(N, 1000) == (2 * N + 26) * 1000


# ----------------------------------------------------------------------- P7
def random_case(rng, N, n, warm, t, wd, hp=None):
    if hp is None:
        hp = dict(lr=float(10 ** rng.uniform(-5, -2)), beta1=float(rng.uniform(0.5, 0.99)),
                  beta2=float(rng.uniform(0.9, 0.9999)), eps=float(10 ** rng.uniform(-10, -6)),
                  weight_decay=wd)
    G = np.stack([rand_bf16(rng, n, float(10 ** rng.uniform(-4, -2))) for _ in range(N)])
    P = (rng.standard_normal(n) * 0.02).astype(np.float32)
    if warm:
        M = (rng.standard_normal(n) * 1e-4).astype(np.float32)
        V = np.abs(rng.standard_normal(n) * 1e-6).astype(np.float32)
    else:
        M = np.zeros(n, dtype=np.float32)
        V = np.zeros(n, dtype=np.float32)
    return G, P, M, V, hp, t


def check_against_f64(o, G, P, M, V, hp, t, what="P7"):
    out = o.step(G, P, M, V, hp, t, threads=1)
    gbar = o.reduce_mean(G, threads=1)
    x64, err = bf.step_f64(G, P, M, V, hp, t)
    for name, got in (("g", gbar), ("P", out[0]), ("M", out[1]), ("V", out[2])):
        d = np.abs(got.astype(np.float64) - x64[name])
        lim = err[name] * (1 + 1e-6) + 1e-300
        bad = ~(d <= lim)
        assert not np.any(bad), f"{what}: {name} outside the fp32 error bound at {np.flatnonzero(bad)[:5]}"
    assert np.array_equal(out[3], o.bf16(out[0]))
    return out, x64, err


def pin_f64_bound(o):
    rng = np.random.default_rng(107)
    for N in (1, 2, 3, 5, 8, 16, 64):
        for t in (1, 2, 7, 100, 5000):
            for warm in (False, True):
                wd = float(rng.choice([0.0, 0.01, 0.1]))
                check_against_f64(o, *random_case(rng, N, 512 if N == 64 else 2048, warm, t, wd))


# ----------------------------------------------------------------------- P8
def pin_rank_order(o):
    one, tiny, mone, zero = 0x3F80, 0x3380, 0xBF80, 0x0000  # 1, 2^-24, -1, 0 as bf16
    cases = [([one, tiny, mone, zero], 0.0, "in order 0..N-1 sums to 0"),
             ([zero, mone, tiny, one], 2.0 ** -26, "rank 0 first"),
             ([one, tiny, tiny, mone], 0.0, "sequential, not pairwise"),
             ([mone, tiny, tiny, one], 2.0 ** -23 / 4, "sequential left to right")]
    for chunks, want, why in cases:
        G = [np.array([c], dtype=np.uint16) for c in chunks]
        got = float(o.reduce_mean(G, threads=1)[0])
        assert got == want, f"P8: {why}: got {got!r}, want {want!r}"


# ----------------------------------------------------------------------- P9
def pin_bf16_cast(o):
    cases = {0x3F808000: 0x3F80, 0x3F818000: 0x3F82, 0x3F80FFFF: 0x3F81, 0x3F807FFF: 0x3F80,
             0x7F800000: 0x7F80, 0xFF800000: 0xFF80, 0x7F7FC99E: 0x7F80, 0x00000000: 0x0000,
             0x80000000: 0x8000, 0x00008000: 0x0000, 0x00018000: 0x0002, 0x7F7F7FFF: 0x7F7F}
    x = np.array(list(cases), dtype=np.uint32).view(np.float32)
    got = o.bf16(x)
    want = np.array(list(cases.values()), dtype=np.uint16)
    assert np.array_equal(got, want), f"P9: bf16 cases {got} != {want}"
    nan = o.bf16(np.array([0x7F800001, 0xFFC00000, 0x7FFFFFFF], dtype=np.uint32).view(np.float32))
    assert np.all((nan & 0x7F80) == 0x7F80) and np.all(nan & 0x007F), "P9: NaN must stay NaN"
    import torch

    rng = np.random.default_rng(109)
    r = rng.integers(0, 2 ** 32, 10_000_000, dtype=np.uint64).astype(np.uint32)
    r = r[(r & 0x7F800000) != 0x7F800000]
    xs = r.view(np.float32)
    ref = torch.from_numpy(xs).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(o.bf16(xs), ref), "P9: differs from torch's bf16 cast"


# ---------------------------------------------------------------------- P10
def torch_adamw_f64(G, P, M, V, hp, t):
    import torch

    gbar = bf.bf16_to_f64(G).sum(axis=0) / len(G)        # exact: bf16 sums of <= 64 terms fit a double
    p = torch.nn.Parameter(torch.from_numpy(P.astype(np.float64)))
    opt = torch.optim.AdamW([p], lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]), eps=hp["eps"],
                            weight_decay=hp["weight_decay"], foreach=False, fused=False)
    st = opt.state[p]
    st["step"] = torch.tensor(float(t - 1), dtype=torch.float64)
    st["exp_avg"] = torch.from_numpy(M.astype(np.float64))
    st["exp_avg_sq"] = torch.from_numpy(V.astype(np.float64))
    p.grad = torch.from_numpy(gbar)
    opt.step()
    return p.detach().numpy(), st["exp_avg"].numpy(), st["exp_avg_sq"].numpy()


def pin_torch_adamw(o):
    rng = np.random.default_rng(110)
    for N in (1, 4):
        for wd in (0.0, 0.1):
            for t in (1, 100, 5000):
                for warm in (False, True):
                    G, P, M, V, hp, t_ = random_case(rng, N, 2048, warm, t, wd,
                                                     hp=dict(HP, weight_decay=wd))
                    out, x64, err = check_against_f64(o, G, P, M, V, hp, t_, what="P10")
                    tp, tm, tv = torch_adamw_f64(G, P, M, V, hp, t_)
                    for name, ref in (("P", tp), ("M", tm), ("V", tv)):
                        # the float64 evaluation is torch's AdamW, to a millionth of the fp32 bound ...
                        assert np.all(np.abs(x64[name] - ref) <= 1e-12 * np.abs(ref) + 1e-6 * err[name]), \
                            f"P10: f64 vs torch {name}"
                    for got, ref, e, name in ((out[0], tp, err["P"], "P"), (out[1], tm, err["M"], "M"),
                                              (out[2], tv, err["V"], "V")):
                        # ... and the oracle's fp32 result lies within the fp32 bound of torch's
                        d = np.abs(got.astype(np.float64) - ref)
                        assert np.all(d <= e * (1 + 1e-6) + 1e-12 * np.abs(ref) + 1e-300), f"P10: oracle vs torch {name}"


# ---------------------------------------------------------------------- P11
def pin_folded_scalars(o):
    for wd in (0.0, 0.1):
        for t in (1, 100, 1000, 5000, 10000):
            hp = dict(HP, weight_decay=wd)
            b1, b2 = hp["beta1"], hp["beta2"]
            want = [b1, 1.0 - b1, b2, 1.0 - b2, hp["eps"], hp["lr"] / (1.0 - b1 ** t),
                    1.0 / math.sqrt(1.0 - b2 ** t), 1.0 - hp["lr"] * wd]
            got = o.fold(hp, t)
            assert [float(x) for x in got] == [f32(w) for w in want], f"P11: folded scalars wrong at t={t}, wd={wd}"


# ---------------------------------------------------------------------- P12
def pin_f16_casts(o):
    """binary16 <-> binary32: every one of the 65536 encodings decodes as numpy's
    float16 does; encoding matches numpy's round-to-nearest-even cast."""
    allh = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    want = allh.view(np.float16).astype(np.float32)
    got = o.f16_to_f32(allh)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan) and np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))
    rng = np.random.default_rng(112)
    r = rng.integers(0, 2 ** 32, 4_000_000, dtype=np.uint64).astype(np.uint32)
    r = r[(r & 0x7F800000) != 0x7F800000]
    specials = np.array([0x477FEFFF, 0x477FF000, 0x477FE000, 0x33000000, 0x33000001, 0x387FC000, 0x38800000,
                         0x387FFFFF, 0x7F800000, 0xFF800000, 0x80000000, 0x00000001], dtype=np.uint32)
    xs = np.concatenate([r, specials]).view(np.float32)
    with np.errstate(over="ignore"):
        ref = xs.astype(np.float16).view(np.uint16)
    assert np.array_equal(o.f16(xs), ref), "P12: fp16 cast differs from numpy's"
    nanh = o.f16(np.array([np.nan], dtype=np.float32))
    assert (nanh[0] & 0x7C00) == 0x7C00 and (nanh[0] & 0x3FF)


# ---------------------------------------------------------------------- P13
def pin_two_pass_equals_fused(o):
    """Without loss scaling or clipping, pass 1 + pass 2 is the fused step, bit for bit."""
    rng = np.random.default_rng(113)
    for N in (1, 3, 8):
        G, P, M, V, hp, t = random_case(rng, N, 4096, True, 17, 0.1, hp=dict(HP, weight_decay=0.1))
        g = o.reduce_unscale(G, 0, 1.0, threads=1)
        assert np.array_equal(bits(g), bits(o.reduce_mean(G, threads=1)))
        ts = o.sqnorm(g)
        two = o.adam_from_gbar(g, P, M, V, hp, t, ts, 0.0, 0)
        fused = o.step(G, P, M, V, hp, t, threads=1)
        assert two[4] and all(np.array_equal(np.asarray(a).view(np.uint8), np.asarray(b).view(np.uint8))
                              for a, b in zip(two[:4], fused)), "P13: two-pass != fused"


def pin_unscale_and_fp16_grads(o):
    """Power-of-two loss scales unscale exactly; fp16 replicas average like bf16 ones."""
    rng = np.random.default_rng(114)
    xs = (rng.standard_normal((4, 4096)) * 1e-2).astype(np.float32)
    H = o.f16(xs)
    g1 = o.reduce_unscale(H, 1, 1.0, threads=1)
    for k in (1, 8, 16, 24):
        gk = o.reduce_unscale(H, 1, float(2 ** k), threads=1)
        assert np.array_equal(bits(gk), bits(g1 * np.float32(2.0 ** -k))), f"P13: unscale by 2^{k} not exact"
    dec = np.stack([o.f16_to_f32(h) for h in H]).astype(np.float64)
    exact = dec.sum(axis=0) / 4                       # fp16 sums of 4 terms are exact in double
    assert np.all(np.abs(g1 - exact) <= 4 * U * np.abs(dec).sum(axis=0) / 4 + 1e-45)
    one = o.reduce_unscale([H[0]] * 5, 1, 1.0, threads=1)
    assert np.array_equal(bits(one), bits(dec[0].astype(np.float32))), "P13: identical fp16 replicas"


# ---------------------------------------------------------------------- P14
def pin_sqnorm(o):
    import math

    rng = np.random.default_rng(115)
    g = (rng.standard_normal(100_003) * 1e-3).astype(np.float32)
    exact = math.fsum(float(x) * float(x) for x in g)      # correctly rounded sum of exact squares
    got = o.sqnorm(g)
    assert abs(got - exact) <= g.size * 2.0 ** -53 * exact, "P14: squared norm"
    c = np.full(1000, np.float32(0.5))
    assert o.sqnorm(c) == 250.0
    assert math.isinf(o.sqnorm(np.array([1.0, np.inf], np.float32)))
    assert math.isnan(o.sqnorm(np.array([1.0, np.nan], np.float32)))


# ---------------------------------------------------------------------- P15
def pin_clipping(o):
    """Clipping by global norm: coefficient 1 below the threshold (the update is
    then the unclipped one, bit for bit); above it, agreement with
    torch.nn.utils.clip_grad_norm_ followed by AdamW, in float64."""
    import torch

    rng = np.random.default_rng(116)
    G, P, M, V, hp, t = random_case(rng, 4, 4096, True, 100, 0.1, hp=dict(HP, weight_decay=0.1))
    g = o.reduce_unscale(G, 0, 1.0, threads=1)
    ts = o.sqnorm(g)
    norm = ts ** 0.5
    assert o.clip_coef(ts, 2 * norm) == 1.0 and o.clip_coef(ts, 0.0) == 1.0
    a = o.adam_from_gbar(g, P, M, V, hp, t, ts, 2 * norm)
    b = o.adam_from_gbar(g, P, M, V, hp, t, ts, 0.0)
    assert all(np.array_equal(np.asarray(x).view(np.uint8), np.asarray(y).view(np.uint8)) for x, y in zip(a[:4], b[:4]))
    max_norm = norm / 7
    k = o.clip_coef(ts, max_norm)
    want = max_norm / (norm + 1e-6)
    assert abs(k - want) <= U * want, "P15: clip coefficient"
    out = o.adam_from_gbar(g, P, M, V, hp, t, ts, max_norm)
    # torch: clip the float64 average, then AdamW
    p = torch.nn.Parameter(torch.from_numpy(P.astype(np.float64)))
    p.grad = torch.from_numpy(g.astype(np.float64))
    torch.nn.utils.clip_grad_norm_([p], max_norm)
    opt = torch.optim.AdamW([p], lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]), eps=hp["eps"],
                            weight_decay=hp["weight_decay"], foreach=False, fused=False)
    st = opt.state[p]
    st["step"] = torch.tensor(float(t - 1), dtype=torch.float64)
    st["exp_avg"] = torch.from_numpy(M.astype(np.float64))
    st["exp_avg_sq"] = torch.from_numpy(V.astype(np.float64))
    opt.step()
    gk = (g * np.float32(k)).astype(np.float64)
    for got, ref, scale in ((out[1], st["exp_avg"].numpy(), np.abs(M) + np.abs(gk)),
                            (out[2], st["exp_avg_sq"].numpy(), np.abs(V) + gk * gk)):
        assert np.all(np.abs(got - ref) <= 8 * U * scale + 1e-30), "P15: clipped moments differ from torch"
    step_ref = p.detach().numpy() - P.astype(np.float64)
    step_got = out[0].astype(np.float64) - P
    assert np.all(np.abs(step_got - step_ref) <= 64 * U * np.abs(step_ref) + 2 * ulp32(out[0]) + 2 * ulp32(P)), \
        "P15: clipped update differs from torch"


# ---------------------------------------------------------------------- P16
def pin_overflow_skips(o):
    rng = np.random.default_rng(117)
    G, P, M, V, hp, t = random_case(rng, 2, 1024, True, 5, 0.0)
    g = o.reduce_unscale(G, 0, 1.0, threads=1)
    g[7] = np.inf
    ts = o.sqnorm(g)
    P1, M1, V1, B1, taken = o.adam_from_gbar(g, P, M, V, hp, t, ts, 1.0)
    assert not taken and np.array_equal(P1, P) and np.array_equal(M1, M) and np.array_equal(V1, V)


# ---------------------------------------------------------------------- P17
def pin_loss_scaler(o):
    """The dynamic loss scale of the DeepSpeed fp16 block: start 2^16, window
    1000, hysteresis 2, minimum 1.  Scripted sequence with hand-derived
    states.  hysteresis is a DeepSpeed knob the page sets but does not define;
    the reading taken is DeepSpeed's default one: the overflow budget is spent
    by overflows and restored only when the scale grows, so once it is spent
    every further overflow halves.  The steps marked (*) separate that reading
    from two others: a budget restored at every halving, and a budget restored
    by any clean step."""
    s = o.scaler(2.0 ** 16, 1.0, 1000, 2)
    for _ in range(999):
        assert o.scaler_update(s, False)
    assert s.scale == 2.0 ** 16
    assert o.scaler_update(s, False) and s.scale == 2.0 ** 17          # 1000 clean steps: grow
    assert not o.scaler_update(s, True) and s.scale == 2.0 ** 17       # first overflow: the budget holds
    assert o.scaler_update(s, False) and s.scale == 2.0 ** 17          # one clean step ...
    assert not o.scaler_update(s, True) and s.scale == 2.0 ** 16       # (*) ... does not restore it: halve
    assert not o.scaler_update(s, True) and s.scale == 2.0 ** 15       # (*) a halving does not restore it
    assert not o.scaler_update(s, True) and s.scale == 2.0 ** 14       # every overflow now halves
    for _ in range(40):
        o.scaler_update(s, True)
    assert s.scale == 1.0                                             # never below the minimum
    for _ in range(500):
        o.scaler_update(s, False)
    assert not o.scaler_update(s, True) and s.scale == 1.0            # the clean run restarts
    for _ in range(999):
        assert o.scaler_update(s, False) and s.scale == 1.0
    assert o.scaler_update(s, False) and s.scale == 2.0               # growth ...
    assert not o.scaler_update(s, True) and s.scale == 2.0            # (*) ... restores the budget
    assert not o.scaler_update(s, True) and s.scale == 1.0
    # hysteresis 1: every overflow halves; hysteresis 3: the third halves
    s1 = o.scaler(8.0, 1.0, 1000, 1)
    assert not o.scaler_update(s1, True) and s1.scale == 4.0
    assert not o.scaler_update(s1, True) and s1.scale == 2.0
    s3 = o.scaler(8.0, 1.0, 4, 3)
    assert not o.scaler_update(s3, True) and s3.scale == 8.0
    assert not o.scaler_update(s3, True) and s3.scale == 8.0
    assert not o.scaler_update(s3, True) and s3.scale == 4.0
    for _ in range(3):
        assert o.scaler_update(s3, False) and s3.scale == 4.0
    assert o.scaler_update(s3, False) and s3.scale == 8.0            # window 4: grow, budget restored
    assert not o.scaler_update(s3, True) and s3.scale == 8.0
    assert not o.scaler_update(s3, True) and s3.scale == 8.0
    assert not o.scaler_update(s3, True) and s3.scale == 4.0


TWO_PASS = [pin_f16_casts, pin_two_pass_equals_fused, pin_unscale_and_fp16_grads, pin_sqnorm, pin_clipping,
            pin_overflow_skips, pin_loss_scaler]

ALL = [pin_identical_replicas, pin_first_step, pin_zero_grad, pin_decoupled_decay, pin_constant_grad_run,
       pin_memory_accounting, pin_f64_bound, pin_rank_order, pin_bf16_cast, pin_torch_adamw, pin_folded_scalars] + TWO_PASS
