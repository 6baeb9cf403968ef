"""The no-allocation list step (zs_reduce_adam_list_static) against the
one-shot list step that allocates its plan (zs_reduce_adam_list), through the
C ABI: two calls in a row on the same device, the second on a smaller list (its
table rewrites a prefix of the fixed array the first filled), each
bit-identical to the allocating call on the same inputs; and the size limit
is refused before any GPU work."""
import ctypes

import numpy as np
import pytest

from tests import parity

pytestmark = pytest.mark.gpu

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1)


def make_list(torch, rng, sizes, N):
    """Tensors in buffers of their own (one starting 3 elements into its buffer), drawn on the host."""
    dev = torch.device("cuda:0")
    host, dev_t = [], []
    for k, n in enumerate(sizes):
        off = 3 if k == 1 else 0
        G = [(((rng.standard_normal(n) * 1e-3).astype(np.float32).view(np.uint32)) >> 16).astype(np.uint16)
             for _ in range(N)]
        P = (rng.standard_normal(n) * 0.02).astype(np.float32)
        M = (rng.standard_normal(n) * 1e-4).astype(np.float32)
        V = np.abs(rng.standard_normal(n) * 1e-6).astype(np.float32)
        host.append(dict(G=G, P=P, M=M, V=V))

        def put(a, dt):
            buf = torch.zeros(n + off, dtype=dt, device=dev)
            buf[off:].copy_(torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a))
            return buf[off:]

        dev_t.append(dict(G=[put(g, torch.int16) for g in G], P=put(P, torch.float32), M=put(M, torch.float32),
                          V=put(V, torch.float32), B=torch.zeros(n, dtype=torch.int16, device=dev)))
    return host, dev_t


def c_table(zs, dev_t):
    keep = []
    tab = (zs.TensorStruct * len(dev_t))()
    for i, t in enumerate(dev_t):
        g = (ctypes.c_void_p * len(t["G"]))(*[x.data_ptr() for x in t["G"]])
        keep.append(g)
        tab[i] = zs.TensorStruct(t["P"].numel(), t["P"].data_ptr(), t["M"].data_ptr(), t["V"].data_ptr(),
                                 t["B"].data_ptr(), ctypes.cast(g, ctypes.POINTER(ctypes.c_void_p)))
    return tab, keep


def state(dev_t):
    return [dict(P=t["P"].cpu().numpy(), M=t["M"].cpu().numpy(), V=t["V"].cpu().numpy(),
                 B=t["B"].cpu().numpy().view(np.uint16)) for t in dev_t]


def test_static_list_step_matches_the_allocating_one():
    import torch

    import sharded_mixed_precision_rank_amd as zs

    lib = zs.library()
    h = zs.AdamHPStruct(HP["lr"], HP["beta1"], HP["beta2"], HP["eps"], HP["weight_decay"])
    s = torch.cuda.current_stream().cuda_stream
    for call, (sizes, N, t) in enumerate((([100_003, 4_097, 1, 9, 20_000_011, 0, 64], 8, 11),
                                          ([3_001, 77, 5_000], 3, 12))):
        print(f"static list step, call {call}: {len(sizes)} tensors, N={N}", flush=True)
        rng = np.random.default_rng(600 + call)
        host, a = make_list(torch, rng, sizes, N)
        _, b = make_list(torch, np.random.default_rng(600 + call), sizes, N)
        ta, ka = c_table(zs, a)
        tb, kb = c_table(zs, b)
        assert lib.zs_reduce_adam_list_static(ta, len(sizes), N, ctypes.byref(h), t, s) == 0, \
            lib.zs_last_error().decode() if lib.zs_last_error() else ""
        assert lib.zs_reduce_adam_list(tb, len(sizes), N, ctypes.byref(h), t, s) == 0
        torch.cuda.synchronize()
        got, ref = state(a), state(b)
        for k in range(len(sizes)):
            assert parity.bit_identical(got[k], ref[k]), f"call {call}, tensor {k}"
        # and the oracle on the small tensors
        import oracle

        o = oracle.load()
        for k, hk in enumerate(host):
            if 0 < hk["P"].size <= 200_000:
                P, M, V, B = o.step(np.stack(hk["G"]), hk["P"], hk["M"], hk["V"], HP, t)
                assert parity.bit_identical(got[k], dict(P=P, M=M, V=V, B=B)), f"call {call}, tensor {k} (oracle)"
        del a, b, ka, kb
        torch.cuda.empty_cache()
