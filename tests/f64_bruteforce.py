"""Double-precision evaluation of the shard step with a running forward-error bound.

Independent of the C++ oracle (different language, different evaluation): it
evaluates the exact-arithmetic result of the step in float64 from the same
bf16/fp32 inputs and the unrounded hyperparameters, and, alongside every
intermediate, a bound E on how far an fp32 evaluation (one round-to-nearest
per operation, unit roundoff u = 2^-24, scalars rounded once to fp32) may sit
from it.  Running error analysis in the style of Higham, "Accuracy and
Stability of Numerical Algorithms", ch. 3: for z = x op y computed from
perturbed operands (|dx| <= Ex, |dy| <= Ey)

    add/sub : Ez = Ex + Ey + u (|z| + Ex + Ey)
    mul     : Ez = |x| Ey + |y| Ex + Ex Ey + u (|z| + |x| Ey + |y| Ex + Ex Ey)
    div     : Ez = (Ex + |z| Ey) / (|y| - Ey) + u (|z| + (Ex + |z| Ey) / (|y| - Ey))
    sqrt    : Ez = min(Ex / sqrt(x), sqrt(Ex)) + u (|z| + min(...))

The bound is first-order rigorous; float64's own error (2^-53 per operation)
is covered by a 1e-6 relative slack the callers add.
"""
from __future__ import annotations

import numpy as np

U = 2.0 ** -24


def bf16_to_f64(G) -> np.ndarray:
    G = np.asarray(G, dtype=np.uint16)
    return (G.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _add(x, ex, y, ey):
    z = x + y
    return z, ex + ey + U * (np.abs(z) + ex + ey)


def _mul(x, ex, y, ey):
    z = x * y
    e = np.abs(x) * ey + np.abs(y) * ex + ex * ey
    return z, e + U * (np.abs(z) + e)


def _div(x, ex, y, ey):
    z = x / y
    e = (ex + np.abs(z) * ey) / (np.abs(y) - ey)
    return z, e + U * (np.abs(z) + e)


def _sqrt(x, ex):
    z = np.sqrt(x)
    with np.errstate(divide="ignore", invalid="ignore"):
        lin = np.where(x > 0, ex / np.sqrt(np.where(x > 0, x, 1.0)), np.inf)
    e = np.minimum(lin, np.sqrt(ex))
    return z, e + U * (np.abs(z) + e)


def _const(c):
    return c, U * abs(c)


def step_f64(G, P, M, V, hp: dict, t: int):
    """Returns dict(g, P, M, V) of float64 results and dict(g, P, M, V) of bounds."""
    lr, b1, b2, eps = hp["lr"], hp["beta1"], hp["beta2"], hp["eps"]
    wd = hp.get("weight_decay", 0.0)
    g_r = bf16_to_f64(G)
    N = g_r.shape[0]
    P = np.asarray(P, dtype=np.float32).astype(np.float64)
    M = np.asarray(M, dtype=np.float32).astype(np.float64)
    V = np.asarray(V, dtype=np.float32).astype(np.float64)
    zero = np.zeros_like(P)

    s, es = g_r[0].copy(), zero.copy()
    for r in range(1, N):
        s, es = _add(s, es, g_r[r], zero)
    g, eg = _div(s, es, np.float64(N), 0.0)

    cb1, ecb1 = _const(b1)
    cc1, ecc1 = _const(1.0 - b1)
    cb2, ecb2 = _const(b2)
    cc2, ecc2 = _const(1.0 - b2)
    ce, ece = _const(eps)
    css, ecss = _const(lr / (1.0 - b1 ** t))
    crb, ecrb = _const(1.0 / np.sqrt(1.0 - b2 ** t))
    cdk, ecdk = _const(1.0 - lr * wd)

    a, ea = _mul(cb1, ecb1, M, zero)
    b, eb = _mul(cc1, ecc1, g, eg)
    m1, em1 = _add(a, ea, b, eb)

    a, ea = _mul(cb2, ecb2, V, zero)
    gg, egg = _mul(g, eg, g, eg)
    b, eb = _mul(cc2, ecc2, gg, egg)
    v1, ev1 = _add(a, ea, b, eb)

    sq, esq = _sqrt(v1, ev1)
    a, ea = _mul(sq, esq, crb, ecrb)
    d, ed = _add(a, ea, ce, ece)
    q, eq = _div(m1, em1, d, ed)

    a, ea = _mul(cdk, ecdk, P, zero)
    b, eb = _mul(css, ecss, q, eq)
    p1, ep1 = _add(a, ea, -b, eb)
    return dict(g=g, P=p1, M=m1, V=v1), dict(g=eg, P=ep1, M=em1, V=ev1)
