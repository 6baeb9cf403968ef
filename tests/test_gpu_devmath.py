"""The device's fp32 square root and division, built with libzshard's flags,
against the host's IEEE binary32 operations (numpy's float32 sqrt and divide,
which round correctly and keep subnormals).

The AdamW update takes one square root and one division per parameter, and
the bit-exact parity of the whole step rests on both being correctly rounded
(-fhip-fp32-correctly-rounded-divide-sqrt).  The step's own parity tests only
reach the narrow range of values an optimizer produces; these pin the two
operations directly:
  * the square root of every non-negative encoding (2^31 of them, NaNs
    included), and of the negative zero, subnormals, normals, -Inf and NaNs;
  * 2^30 quotients: random encodings over every exponent, values in the
    update's own range (momentum over a root of the variance plus epsilon),
    subnormal operands, power-of-two divisors whose quotients land on
    subnormal ties, and every pair of special values.
NaN results must be NaN (payloads are free); everything else must have the
same encoding."""
import ctypes
import os

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "devmath", "libzs_devmath.so")


@pytest.fixture(scope="module")
def dm():
    import torch

    if not os.path.exists(LIB):
        pytest.fail(f"{LIB} is missing: build it with __graft_entry__.build()")
    lib = ctypes.CDLL(LIB)
    vp, i64, u32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint32
    lib.zs_devmath_sqrt.restype = ctypes.c_int
    lib.zs_devmath_sqrt.argtypes = [u32, i64, vp, vp]
    lib.zs_devmath_div.restype = ctypes.c_int
    lib.zs_devmath_div.argtypes = [vp, vp, i64, vp, vp]
    return lib, torch


def host_is_ieee():
    """The host keeps subnormals and rounds ties to even (no flush-to-zero)."""
    tiny = np.float32(2.0 ** -140)
    assert np.float32(tiny / np.float32(2.0)) == np.float32(2.0 ** -141)
    dmin = np.float32(2.0 ** -149)
    assert np.float32(dmin / np.float32(2.0)) == 0.0                      # tie: to even (zero)
    assert np.float32(np.float32(3 * 2.0 ** -149) / np.float32(2.0)) == np.float32(2 * 2.0 ** -149)


def mismatches(torch, got, ref) -> int:
    """Positions (device tensors) whose results differ; NaN matches any NaN."""
    gn, rn = torch.isnan(got), torch.isnan(ref)
    bad = (gn != rn) | (~gn & (got.view(torch.int32) != ref.view(torch.int32)))
    return int(bad.sum().item())


def test_sqrt_every_nonnegative_encoding(dm):
    lib, torch = dm
    host_is_ieee()
    chunk = 1 << 28
    s = torch.cuda.current_stream().cuda_stream
    out = torch.empty(chunk, dtype=torch.float32, device="cuda")
    ref_d = torch.empty_like(out)
    ref_h = torch.empty(chunk, dtype=torch.float32).pin_memory()
    idx = np.arange(chunk, dtype=np.uint32)
    x = np.empty(chunk, dtype=np.uint32)
    ranges = [(c * chunk, chunk) for c in range(8)]            # encodings 0x00000000 .. 0x7FFFFFFF
    ranges += [(0x80000000, 1 << 24), (0xBF800000, 1 << 24),  # -0, negative subnormals, normals; from -1 down
               (0xFF800000, 1 << 23)]                          # -Inf and negative NaNs
    for first, n in ranges:
        print(f"sqrt: encodings {first:#010x}..{first + n - 1:#010x}", flush=True)
        assert lib.zs_devmath_sqrt(first, n, out.data_ptr(), s) == 0
        np.add(idx[:n], np.uint32(first), out=x[:n])
        with np.errstate(all="ignore"):
            np.sqrt(x[:n].view(np.float32), out=ref_h.numpy()[:n])
        ref_d[:n].copy_(ref_h[:n])
        assert mismatches(torch, out[:n], ref_d[:n]) == 0, f"encodings from {first:#010x}"
    del out, ref_d
    torch.cuda.empty_cache()


def div_operands(torch, g, n: int, first_chunk: bool):
    """n pairs (a, b) of float32 device tensors, drawn on the device: a mix of the kinds in the module
    docstring, chosen per pair."""
    dev = "cuda"
    i32 = torch.int32
    kind = torch.randint(0, 100, (n,), device=dev, generator=g, dtype=i32)

    def bits(lo, hi):
        return torch.randint(lo, hi, (n,), device=dev, generator=g, dtype=torch.int64)

    def enc(x):  # int64 encodings below 2^32 -> float32
        return x.to(i32).view(torch.float32)

    # random encodings over every exponent, finite: an exponent field of 255 loses its top bit
    a, b = bits(0, 1 << 32), bits(0, 1 << 32)
    a = torch.where((a >> 23) & 0xFF == 0xFF, a & 0xBFFFFFFF, a)
    b = torch.where((b >> 23) & 0xFF == 0xFF, b & 0xBFFFFFFF, b)
    af, bf = enc(a).clone(), enc(b).clone()
    # the update's own range: m1 ~ N(0, 1e-4) over sqrt(|N(0, 1e-6)|) * rb + eps
    sel = (kind >= 40) & (kind < 70)
    m = torch.randn(n, device=dev, generator=g) * 1e-4
    v = (torch.randn(n, device=dev, generator=g) * 1e-6).abs()
    rb = 1.0 + torch.rand(n, device=dev, generator=g) * 30.0
    af = torch.where(sel, m, af)
    bf = torch.where(sel, torch.sqrt(v) * rb + 1e-8, bf)
    # a subnormal numerator or denominator: exponent field 0, random mantissa and sign
    sel = (kind >= 70) & (kind < 85)
    sub = enc(bits(0, 1 << 23) | (bits(0, 2) << 31))
    which = bits(0, 2) == 1
    af = torch.where(sel & which, sub, af)
    bf = torch.where(sel & ~which, sub, bf)
    # power-of-two divisors 2^k with quotients in the subnormal range that drop t = 1..3 bits, the
    # dropped bits exactly one half: ties, to be rounded to even
    sel = kind >= 85
    t = bits(1, 4)
    ea = bits(1, 125)                                  # numerator's biased exponent
    mant = ((bits(0, 1 << 20) << t) | (1 << (t - 1))) & 0x7FFFFF
    sign = bits(0, 2) << 31
    k = ea + t - 1                                     # quotient's biased exponent 1 - t: t bits dropped
    af = torch.where(sel, enc(sign | (ea << 23) | mant), af)
    bf = torch.where(sel, enc((k + 127) << 23), bf)
    if first_chunk:  # every pair of special values
        sp = torch.tensor([0.0, -0.0, float("inf"), float("-inf"), float("nan"), 2.0 ** -149, -(2.0 ** -149),
                           2.0 ** -126, 3.4028235e38, -3.4028235e38, 1.0, -1.0, 3.0, 2.0 ** -127, 1e-8],
                          dtype=torch.float32)
        pa, pb = torch.meshgrid(sp, sp, indexing="ij")
        af[:pa.numel()] = pa.reshape(-1).to(dev)
        bf[:pb.numel()] = pb.reshape(-1).to(dev)
    return af.contiguous(), bf.contiguous()


def test_division_2_30_pairs(dm):
    lib, torch = dm
    host_is_ieee()
    chunk, chunks = 1 << 27, 8
    s = torch.cuda.current_stream().cuda_stream
    out = torch.empty(chunk, dtype=torch.float32, device="cuda")
    ref_d = torch.empty_like(out)
    a_h, b_h, ref_h = (torch.empty(chunk, dtype=torch.float32).pin_memory() for _ in range(3))
    g = torch.Generator(device="cuda").manual_seed(20261202)
    for c in range(chunks):
        print(f"division: pairs {c * chunk}..{(c + 1) * chunk - 1}", flush=True)
        af, bf = div_operands(torch, g, chunk, c == 0)
        assert lib.zs_devmath_div(af.data_ptr(), bf.data_ptr(), chunk, out.data_ptr(), s) == 0
        a_h.copy_(af)
        b_h.copy_(bf)
        with np.errstate(all="ignore"):
            np.divide(a_h.numpy(), b_h.numpy(), out=ref_h.numpy())
        ref_d.copy_(ref_h)
        bad = mismatches(torch, out, ref_d)
        if bad:
            gn, rn = torch.isnan(out), torch.isnan(ref_d)
            idx = torch.nonzero((gn != rn) | (~gn & (out.view(torch.int32) != ref_d.view(torch.int32))))[:5, 0]
            pytest.fail(f"chunk {c}: {bad} quotients differ, e.g. " + ", ".join(
                f"{a_h[j].item()!r}/{b_h[j].item()!r}: device {out[j].item()!r} host {ref_h[j].item()!r}"
                for j in idx.tolist()))
        del af, bf
    del out, ref_d
    torch.cuda.empty_cache()
