"""The seeded input generator: counter-based, position-addressable, right moments."""
import numpy as np

import synth
from synth import workloads as W


def test_slices_and_gathers_agree():
    k = synth.key(0, synth.KIND_P)
    full = synth.normal_f32(k, 0, 10_000, 0.02)
    assert np.array_equal(full[4321:], synth.normal_f32(k, 4321, 10_000 - 4321, 0.02))
    idx = np.array([0, 17, 9999, 5000, 5000], dtype=np.int64)
    assert np.array_equal(synth.normal_f32_at(k, idx, 0.02), full[idx])
    kg = synth.key(0, synth.KIND_GRAD, 3)
    km = synth.key(0, synth.KIND_MASK)
    th = synth.mask_threshold(0.01)
    gb = synth.normal_bf16(kg, 0, 10_000, 1e-3, km, th)
    assert np.array_equal(synth.normal_bf16_at(kg, idx, 1e-3, km, th), gb[idx])


def test_streams_differ_and_repeat():
    a = synth.normal_f32(synth.key(0, synth.KIND_GRAD, 0), 0, 1000, 1.0)
    b = synth.normal_f32(synth.key(0, synth.KIND_GRAD, 1), 0, 1000, 1.0)
    c = synth.normal_f32(synth.key(1, synth.KIND_GRAD, 0), 0, 1000, 1.0)
    assert not np.array_equal(a, b) and not np.array_equal(a, c)
    assert np.array_equal(a, synth.normal_f32(synth.key(0, synth.KIND_GRAD, 0), 0, 1000, 1.0))


def test_moments():
    x = synth.normal_f32(synth.key(7, synth.KIND_P), 0, 4_000_000, 0.02).astype(np.float64)
    assert abs(x.mean()) < 1e-4 and abs(x.std() / 0.02 - 1) < 3e-3
    assert np.max(np.abs(x)) <= 6 * 0.02 * (1 + 1e-6)
    v = synth.normal_f32(synth.key(7, synth.KIND_V), 0, 1_000_000, 1e-6, absval=True)
    assert np.all(v >= 0)
    g = synth.normal_bf16(synth.key(7, synth.KIND_GRAD), 0, 2_000_000, 1e-3,
                          synth.key(7, synth.KIND_MASK), synth.mask_threshold(0.001))
    zero = np.mean(g == 0)
    assert 0.0008 < zero < 0.0012
    gf = (g.astype(np.uint32) << 16).view(np.float32)
    assert abs(gf.std() / 1e-3 - 1) < 5e-3


def test_workload_sizes():
    llama = W.list_llama7b_dp8_n8()
    assert len(llama.sizes) == 288 and llama.n_params == 809_533_440
    ragged = W.list_ragged_20000_n16()
    assert len(ragged.sizes) == 20_000 and min(ragged.sizes) >= 64 and max(ragged.sizes) <= 1 << 20
    assert 2.0e9 < ragged.n_params < 2.3e9       # log-uniform 64..2^20 has mean ~108k
    offs, L = ragged.layout()
    assert np.all(offs % 8 == 0) and L >= ragged.n_params
    assert W.FLAT_70B_DP64_N64.n_params == 70_000_000_000 // 64
    l70 = W.list_llama70b_dp64_n64()
    # 80 layers of (2 h^2 + 2 h kv + 3 h ffn + 2 h) / 64 with h = 8192, kv = 1024, ffn = 28672
    assert len(l70.sizes) == 720 and l70.N == 64
    assert l70.n_params == 80 * (2 * 8192 ** 2 + 2 * 8192 * 1024 + 3 * 8192 * 28672 + 2 * 8192) // 64 == 1_069_568_000


def test_host_inputs_at_matches_slices():
    w = W.FLAT_1M_N2.with_(warm=True, zero_frac=0.01)
    a = W.host_inputs(w, 100, 300)
    b = W.host_inputs_at(w, np.arange(100, 300))
    for k in "GPMV":
        assert np.array_equal(a[k], b[k])
