"""Comparison rules between the HIP path and the oracle.

Floating point (non-integer inputs): every element must satisfy
    |C - C_ref| <= 2 * ulp16(|C_ref|) + 1e-3
computed in fp64, with ulp16(x) = 2^(max(floor(log2 x), -14) - 10) and
ulp16(0) = 2^-24; an infinite C_ref must be matched by the identical infinity
and any NaN fails.  The GPU accumulates in fp32 in its own K order and then
rounds once; the oracle sums exactly (fp64) and rounds once, so several
results are correct and they may differ by about one fp16 ulp.

Integer inputs (sums exact in fp32 in any order): bit-exact, +0 and -0 equal.
"""
from __future__ import annotations

import numpy as np


def ulp16(x: np.ndarray) -> np.ndarray:
    ax = np.abs(np.asarray(x, dtype=np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    u = np.exp2(np.maximum(e, -14) - 10)
    return np.where(ax > 0, u, 2.0 ** -24)


def tolerance_report(got: np.ndarray, ref: np.ndarray, exact_sum: np.ndarray | None = None):
    """Return (ok, stats) for fp16 arrays got and ref of equal shape."""
    g = np.asarray(got, dtype=np.float16).astype(np.float64)
    r = np.asarray(ref, dtype=np.float16).astype(np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    nan = np.isnan(g) | np.isnan(r)
    inf_ref = np.isinf(r)
    inf_bad = inf_ref & (g != r)
    inf_extra = np.isinf(g) & ~inf_ref
    fin = ~(nan | inf_ref | np.isinf(g))
    err = np.zeros_like(r)
    err[fin] = np.abs(g[fin] - r[fin])
    bound = 2 * ulp16(r) + 1e-3
    bad_fin = fin & (err > bound)
    nbad = int(nan.sum() + inf_bad.sum() + inf_extra.sum() + bad_fin.sum())
    stats = {
        "n": int(r.size),
        "bad": nbad,
        "max_abs_err": float(err.max()) if err.size else 0.0,
        "max_err_ulps": float((err[fin] / ulp16(r[fin])).max()) if fin.any() else 0.0,
        "bit_identical_frac": float(np.mean(
            np.asarray(got, np.float16).view(np.uint16) == np.asarray(ref, np.float16).view(np.uint16)))
        if r.size else 1.0,
    }
    if exact_sum is not None and r.size:
        stats["mae_vs_exact"] = float(np.mean(np.abs(g - np.asarray(exact_sum, np.float64))))
    return nbad == 0, stats


def assert_within_tolerance(got, ref, what=""):
    ok, stats = tolerance_report(got, ref)
    assert ok, f"{what}: {stats}"
    return stats


def assert_bit_exact(got, ref, what=""):
    gb = np.asarray(got, np.float16).view(np.uint16).astype(np.uint32)
    rb = np.asarray(ref, np.float16).view(np.uint16).astype(np.uint32)
    gb = np.where((gb & 0x7fff) == 0, 0, gb)
    rb = np.where((rb & 0x7fff) == 0, 0, rb)
    mism = int((gb != rb).sum())
    assert mism == 0, f"{what}: {mism} of {gb.size} elements differ"
