"""The device input generator draws the same bits as the host generator."""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("offset", [0, 123_456_789_012])
def test_device_fill_matches_host(offset):
    import torch

    dev = torch.device("cuda:0")
    n = 1_000_003
    k = synth.key(0, synth.KIND_P)
    x = torch.empty(n, dtype=torch.float32, device=dev)
    synth.dev_fill_normal_f32(x, k, offset, 0.02)
    a = torch.empty(n, dtype=torch.float32, device=dev)
    synth.dev_fill_normal_f32(a, synth.key(0, synth.KIND_V), offset, 1e-6, absval=True)
    g = torch.empty(n, dtype=torch.bfloat16, device=dev)
    km = synth.key(0, synth.KIND_MASK)
    th = synth.mask_threshold(0.01)
    synth.dev_fill_normal_bf16(g, synth.key(0, synth.KIND_GRAD, 5), offset, 1e-3, km, th)
    torch.cuda.synchronize()
    assert np.array_equal(x.cpu().numpy().view(np.uint32), synth.normal_f32(k, offset, n, 0.02).view(np.uint32))
    assert np.array_equal(a.cpu().numpy().view(np.uint32),
                          synth.normal_f32(synth.key(0, synth.KIND_V), offset, n, 1e-6, True).view(np.uint32))
    assert np.array_equal(g.view(torch.int16).cpu().numpy().view(np.uint16),
                          synth.normal_bf16(synth.key(0, synth.KIND_GRAD, 5), offset, n, 1e-3, km, th))
