"""Element-by-element comparison of the GPU results with the CPU oracle.

The bar: fp32 master / momentum / variance within a relative error of 1e-6
(|x - ref| / |ref|; a zero reference needs a zero result; NaN positions must
match, payloads are free), bf16 working copy within 1 ulp (distance between the
encodings in value order; NaN positions must match).
"""
from __future__ import annotations

import numpy as np

F32_REL_TOL = 1e-6
BF16_ULP_TOL = 1


def f32_report(got, ref) -> dict:
    g = np.asarray(got, dtype=np.float32)
    r = np.asarray(ref, dtype=np.float32)
    assert g.shape == r.shape
    gn, rn = np.isnan(g), np.isnan(r)
    nan_mismatch = int(np.count_nonzero(gn != rn))
    ok = ~rn & ~gn
    g64, r64 = g[ok].astype(np.float64), r[ok].astype(np.float64)
    inf = np.isinf(r64) | np.isinf(g64)
    inf_mismatch = int(np.count_nonzero(inf & (g64 != r64)))
    fin = ~inf
    d = np.abs(g64[fin] - r64[fin])
    den = np.abs(r64[fin])
    zero = den == 0
    zero_mismatch = int(np.count_nonzero(zero & (d != 0)))
    rel = np.where(zero, 0.0, d / np.where(zero, 1.0, den))
    bitdiff = int(np.count_nonzero(g.view(np.uint32)[ok] != r.view(np.uint32)[ok]))
    return dict(max_rel=float(rel.max()) if rel.size else 0.0, nan_mismatch=nan_mismatch,
                inf_mismatch=inf_mismatch, zero_mismatch=zero_mismatch, bitdiff=bitdiff, n=int(g.size))


def bf16_order(b) -> np.ndarray:
    b = np.asarray(b, dtype=np.uint16).astype(np.int64)
    return np.where(b & 0x8000, 0x8000 - (b & 0x7FFF), b + 0x8000)


def bf16_report(got, ref) -> dict:
    g = np.asarray(got).view(np.uint16)
    r = np.asarray(ref).view(np.uint16)
    gn = ((g & 0x7F80) == 0x7F80) & ((g & 0x7F) != 0)
    rn = ((r & 0x7F80) == 0x7F80) & ((r & 0x7F) != 0)
    ok = ~gn & ~rn
    dist = np.abs(bf16_order(g[ok]) - bf16_order(r[ok]))
    return dict(max_ulp=int(dist.max()) if dist.size else 0, nan_mismatch=int(np.count_nonzero(gn != rn)),
                bitdiff=int(np.count_nonzero(g[ok] != r[ok])), n=int(g.size))


def assert_f32(got, ref, what: str) -> dict:
    rep = f32_report(got, ref)
    assert rep["nan_mismatch"] == 0 and rep["inf_mismatch"] == 0 and rep["zero_mismatch"] == 0, f"{what}: {rep}"
    assert rep["max_rel"] <= F32_REL_TOL, f"{what}: {rep}"
    return rep


def assert_bf16(got, ref, what: str) -> dict:
    rep = bf16_report(got, ref)
    assert rep["nan_mismatch"] == 0 and rep["max_ulp"] <= BF16_ULP_TOL, f"{what}: {rep}"
    return rep


def assert_step(got: dict, ref: dict, what: str) -> dict:
    """got/ref: dict with P, M, V (float32) and B (uint16 bits)."""
    out = {k: assert_f32(got[k], ref[k], f"{what} {k}") for k in "PMV"}
    out["B"] = assert_bf16(got["B"], ref["B"], f"{what} B")
    return out


def _same_bits_f32(a, b) -> bool:
    a = np.asarray(a, dtype=np.float32)
    b = np.asarray(b, dtype=np.float32)
    both_nan = np.isnan(a) & np.isnan(b)                 # NaN payloads are free
    return bool(np.array_equal(a.view(np.uint32)[~both_nan], b.view(np.uint32)[~both_nan]))


def _same_bits_bf16(a, b) -> bool:
    a = np.asarray(a).view(np.uint16)
    b = np.asarray(b).view(np.uint16)
    nan = lambda x: ((x & 0x7F80) == 0x7F80) & ((x & 0x7F) != 0)
    both_nan = nan(a) & nan(b)
    return bool(np.array_equal(a[~both_nan], b[~both_nan]))


def bit_identical(got: dict, ref: dict) -> bool:
    """Same encodings everywhere (NaN payloads aside)."""
    return all(_same_bits_f32(got[k], ref[k]) for k in "PMV") and _same_bits_bf16(got["B"], ref["B"])
