"""The measurement probe on the GPU: the read-only pattern leaves every array
as it was, and the read+write patterns (stores as each tile is done, and stores
grouped in device-clock windows) touch exactly the full tiles and write the
same values."""
import ctypes

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def test_probe_modes():
    import torch

    import bench_probe

    lib = bench_probe.load()
    f = lib.zs_probe_pattern
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
    assert fw(tab, N, n, P.data_ptr(), M.data_ptr(), V.data_ptr(), B.data_ptr(), 256, 32, s) == 0
    torch.cuda.synchronize()
    # bit patterns: the random 16-bit replicas include NaN encodings, and NaN != NaN
    bits = lambda x: x.view(torch.int32) if x.dtype == torch.float32 else x
    for a, b in zip((P, M, V, B), after):
        assert torch.equal(bits(a), bits(b)), "the windowed pattern wrote other values than the plain one"


@pytest.mark.parametrize("n", [0, 1, 511, 512, 513, 12 * 512 + 100, 3_000_001])
def test_probe_copy(n):
    """The copy kernel copies every element, full tiles and the tail, and nothing past them."""
    import torch

    import bench_probe

    lib = bench_probe.load()
    dev = torch.device("cuda:0")
    src = torch.randn(n + 64, generator=torch.Generator().manual_seed(n)).to(dev)
    dst = torch.full((n + 64,), -7.0, device=dev)
    assert lib.zs_probe_copy(src.data_ptr(), dst.data_ptr(), n, torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    assert torch.equal(dst[:n], src[:n])
    assert torch.all(dst[n:] == -7.0)


def test_probe_copy_in_several_launches():
    """Past 3e9 bytes the copy runs as consecutive launches; the boundary between them is exact."""
    import torch

    import bench_probe

    lib = bench_probe.load()
    n = 400_000_123   # 3.2 GB of traffic: two launches, the second starting at tile 732,421
    src = torch.arange(n, dtype=torch.int32, device="cuda").view(torch.float32)
    dst = torch.zeros(n, dtype=torch.float32, device="cuda")
    assert lib.zs_probe_copy(src.data_ptr(), dst.data_ptr(), n, torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    assert torch.equal(dst.view(torch.int32), src.view(torch.int32))
    del src, dst
    torch.cuda.empty_cache()


def test_probe_phased_pattern():
    """The phased pattern (the library's super-chunk loop with its AdamW replaced by the write = 1
    values) covers the whole super-chunks, writes there what the per-tile pattern writes, and nothing
    past them."""
    import torch

    import bench_probe

    lib = bench_probe.load()
    dev = torch.device("cuda:0")
    N = 64
    n = 256 * 12 * 8 * 512 + 5_000   # one super-chunk on a 256-workgroup grid, and a rest
    gen = torch.Generator().manual_seed(9)
    G = [torch.randint(-2 ** 14, 2 ** 14, (n,), dtype=torch.int16, generator=gen).to(dev) for _ in range(N)]
    P, M, V = (torch.randn(n, generator=gen).to(dev) for _ in range(3))
    B = torch.zeros(n, dtype=torch.int16, device=dev)
    before = [x.clone() for x in (P, M, V, B)]
    tab = (ctypes.c_void_p * N)(*[g.data_ptr() for g in G])
    s = torch.cuda.current_stream().cuda_stream
    covered = torch.zeros(1, dtype=torch.int64, device=dev)
    assert lib.zs_probe_pattern_phased(tab, N, n, P.data_ptr(), M.data_ptr(), V.data_ptr(), B.data_ptr(),
                                       covered.data_ptr(), s) == 0
    torch.cuda.synchronize()
    c = int(covered.item())
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    assert c == (n // 512) // (cus * 12 * 8) * (cus * 12 * 8) * 512 and c > 0
    for a, b in zip((P, M, V, B), before):
        assert torch.equal(a[c:], b[c:]), "the phased pattern wrote past its super-chunks"
    got = [x[:c].clone() for x in (P, M, V, B)]
    for x, b0 in zip((P, M, V, B), before):
        x.copy_(b0)
    f = lib.zs_probe_pattern
    assert f(tab, N, n, P.data_ptr(), M.data_ptr(), V.data_ptr(), B.data_ptr(), 1, s) == 0
    torch.cuda.synchronize()
    bits = lambda x: x.view(torch.int32) if x.dtype == torch.float32 else x  # noqa: E731
    for a, b in zip(got, (P, M, V, B)):
        assert torch.equal(bits(a), bits(b[:c])), "the phased pattern wrote other values than the per-tile one"
    del G, P, M, V, B
    torch.cuda.empty_cache()
