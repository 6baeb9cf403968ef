"""The CPU oracle against what the pages and the mathematics fix (pins P1-P11)."""
import numpy as np
import pytest

from tests import pins


@pytest.mark.parametrize("pin", pins.ALL, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)


def test_nonfinite_grads_propagate(orc):
    """A non-finite replica gradient is neither skipped nor clipped: Inf makes
    the moments Inf and the weight NaN; NaN makes everything NaN."""
    n = 4
    G = [np.array([0x7F80, 0xFF80, 0x7FC0, 0x3A83], dtype=np.uint16), np.full(n, 0x3A83, dtype=np.uint16)]
    P = np.full(n, 0.01, dtype=np.float32)
    Z = np.zeros(n, dtype=np.float32)
    P1, M1, V1, B1 = orc.step(G, P, Z, Z, pins.HP, 1, threads=1)
    assert np.isinf(M1[0]) and np.isinf(V1[0]) and np.isnan(P1[0])
    assert np.isinf(M1[1]) and M1[1] < 0 and np.isnan(P1[1])
    assert np.isnan(M1[2]) and np.isnan(P1[2]) and (B1[2] & 0x7FFF) > 0x7F80
    assert np.isfinite(P1[3])


def test_thread_count_does_not_change_bits(orc):
    rng = np.random.default_rng(5)
    G, P, M, V, hp, t = pins.random_case(rng, 8, 100_003, True, 100, 0.1)
    ref = orc.step(G, P, M, V, hp, t, threads=1)
    for th in (2, 3, 8):
        out = orc.step(G, P, M, V, hp, t, threads=th)
        for a, b in zip(out, ref):
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8))


def test_bad_arguments_rejected(orc):
    g = np.zeros(4, dtype=np.uint16)
    P = np.zeros(4, dtype=np.float32)
    with pytest.raises(ValueError):
        orc.step([g], P, P, P, pins.HP, 0)
