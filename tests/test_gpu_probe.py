"""The measurement probe on the GPU: the read-only pattern leaves every array
as it was, and the read+write patterns (stores as each tile is done, and stores
grouped in device-clock windows) touch exactly the full tiles and write the
same values."""
import ctypes
import os

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def test_probe_modes():
    import torch

    import sharded_mixed_precision_rank_amd as zs

    lib = ctypes.CDLL(os.path.join(os.path.dirname(zs.LIB_PATH), "libzshard_probe.so"))
    f = lib.zs_probe_pattern
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int32, ctypes.c_int64] + [ctypes.c_void_p] * 4 + \
        [ctypes.c_int32, ctypes.c_void_p]
    dev = torch.device("cuda:0")
    N, n = 8, 12 * 512 + 100   # twelve full 512-parameter tiles and a partial one
    gen = torch.Generator().manual_seed(5)
    G = [torch.randint(-2 ** 15, 2 ** 15, (n,), dtype=torch.int16, generator=gen).to(dev) for _ in range(N)]
    P, M, V = (torch.randn(n, generator=gen).to(dev) for _ in range(3))
    B = torch.zeros(n, dtype=torch.int16, device=dev)
    before = [x.clone() for x in (P, M, V, B)]
    tab = (ctypes.c_void_p * N)(*[g.data_ptr() for g in G])
    s = torch.cuda.current_stream().cuda_stream
    assert f(tab, N, n, P.data_ptr(), M.data_ptr(), V.data_ptr(), B.data_ptr(), 0, s) == 0
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip((P, M, V, B), before)), "read-only probe wrote"
    assert f(tab, N, n, P.data_ptr(), M.data_ptr(), V.data_ptr(), B.data_ptr(), 1, s) == 0
    torch.cuda.synchronize()
    full = 12 * 512
    for a, b in zip((P, M, V, B), before):
        assert torch.equal(a[full:], b[full:]), "the probe wrote past the full tiles"
    assert not torch.equal(M[:full], before[1][:full])
    assert np.any(B[:full].cpu().numpy() != 0)
    after = [x.clone() for x in (P, M, V, B)]
    # the windowed pattern from the same starting state writes the same values
    for x, b0 in zip((P, M, V, B), before):
        x.copy_(b0)
    fw = lib.zs_probe_pattern_windowed
    fw.restype = ctypes.c_int
    fw.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int32, ctypes.c_int64] + [ctypes.c_void_p] * 4 + \
        [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    assert fw(tab, N, n, P.data_ptr(), M.data_ptr(), V.data_ptr(), B.data_ptr(), 256, 32, s) == 0
    torch.cuda.synchronize()
    # bit patterns: the random 16-bit replicas include NaN encodings, and NaN != NaN
    bits = lambda x: x.view(torch.int32) if x.dtype == torch.float32 else x
    for a, b in zip((P, M, V, B), after):
        assert torch.equal(bits(a), bits(b)), "the windowed pattern wrote other values than the plain one"
