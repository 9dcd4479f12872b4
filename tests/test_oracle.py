"""Pins for the CPU oracle, each against something other than the oracle itself.

The oracle computes C = fp16_rne(sum_k double(A[i,k]) * double(B[j,k])), the
definition on the Tilus "Hopper matmul" pages ("2. Multi-Stage Software
Pipelining" / The Full Kernel; "6. Register Reallocation, Multicast, and a
Persistent Kernel" / opening paragraphs: fp32 accumulation, fp16 output).

Each pin targets a mistake that could plausibly hide in it:
  conversions ........ exhaustive against numpy's binary16 type, and every
                       rounding midpoint against the even-neighbour rule
  summation + RNE .... brute force with exact rationals on all M, N, K <= 6
  orientation (NT) ... identity and permutation B, the swap invariant
  exact integers ..... integer matmul in int64 (a library routine)
  whole definition ... numpy fp64 matmul then astype(float16)
  single rounding .... the pages' MAE figure at K = 8192 (golden fixture),
                       with a planted fp16-accumulation mistake that fails it
  ties / overflow /
  subnormals ......... closed-form probes
"""
import itertools
import json
import os
from bisect import bisect_left
from fractions import Fraction

import numpy as np
import pytest

import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------
# helpers independent of the oracle
# --------------------------------------------------------------------------
def _all_finite_f16_bits():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = bits.view(np.float16)
    return bits[np.isfinite(vals)]


_POS_TABLE = None


def _positive_table():
    """Sorted exact values of every non-negative finite fp16, plus 65536 standing
    for +inf (its bit pattern 0x7c00 has an even fraction, so a tie between
    65504 and 65536 goes to inf exactly as IEEE overflow does)."""
    global _POS_TABLE
    if _POS_TABLE is None:
        bits = np.arange(0, 0x7c00, dtype=np.uint16)  # +0 .. 65504
        vals = [Fraction(float(v)) for v in bits.view(np.float16)]
        vals.append(Fraction(65536))
        codes = [int(b) for b in bits] + [0x7c00]
        _POS_TABLE = (vals, codes)
    return _POS_TABLE


def exact_to_f16_bits(x: Fraction) -> int:
    """Nearest fp16 to an exact rational by table search, ties to even code."""
    vals, codes = _positive_table()
    neg = x < 0
    ax = -x if neg else x
    if ax == 0:
        return 0x0000  # an exact zero sum is +0 (sum starts at +0.0)
    if ax >= vals[-1]:
        code = 0x7c00
    else:
        i = bisect_left(vals, ax)
        if vals[i] == ax:
            code = codes[i]
        else:
            lo, hi = i - 1, i
            dlo, dhi = ax - vals[lo], vals[hi] - ax
            if dlo < dhi:
                code = codes[lo]
            elif dhi < dlo:
                code = codes[hi]
            else:
                code = codes[lo] if codes[lo] % 2 == 0 else codes[hi]
    return code | (0x8000 if neg else 0)


def bits(x: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float16).view(np.uint16)


def same_up_to_zero_sign(c: np.ndarray, ref: np.ndarray) -> bool:
    cb = bits(c).astype(np.uint32)
    rb = bits(ref).astype(np.uint32)
    cb[(cb & 0x7fff) == 0] = 0
    rb[(rb & 0x7fff) == 0] = 0
    return bool(np.array_equal(cb, rb))


# --------------------------------------------------------------------------
# conversions
# --------------------------------------------------------------------------
def test_decode_every_pattern_matches_numpy(oracle_mod):
    b = _all_finite_f16_bits()
    got = oracle_mod.f16_bits_to_f64(b)
    ref = b.view(np.float16).astype(np.float64)
    assert np.array_equal(got, ref)
    assert np.array_equal(np.signbit(got), np.signbit(ref))


def test_decode_special_patterns(oracle_mod):
    got = oracle_mod.f16_bits_to_f64(np.array([0x7c00, 0xfc00, 0x7e00, 0x0001, 0x03ff, 0x0400],
                                              dtype=np.uint16))
    assert got[0] == np.inf and got[1] == -np.inf and np.isnan(got[2])
    assert got[3] == 2.0 ** -24
    assert got[4] == 1023 * 2.0 ** -24
    assert got[5] == 2.0 ** -14


def test_roundtrip_every_pattern(oracle_mod):
    b = _all_finite_f16_bits()
    back = oracle_mod.f64_to_f16_bits(oracle_mod.f16_bits_to_f64(b))
    assert np.array_equal(back, b)  # including -0


def test_every_midpoint_ties_to_even(oracle_mod):
    """Between consecutive positive fp16 values the exact midpoint must go to the
    neighbour with the even fraction; one double-ulp either side goes to the
    nearer neighbour."""
    lo = np.arange(0, 0x7bff, dtype=np.uint16)          # +0 .. one below 65504
    hi = lo + 1
    vlo = lo.view(np.float16).astype(np.float64)
    vhi = hi.view(np.float16).astype(np.float64)
    mid = (vlo + vhi) / 2.0                              # exact in fp64
    even = np.where(lo % 2 == 0, lo, hi).astype(np.uint16)
    assert np.array_equal(oracle_mod.f64_to_f16_bits(mid), even)
    assert np.array_equal(oracle_mod.f64_to_f16_bits(np.nextafter(mid, 0)), lo)
    assert np.array_equal(oracle_mod.f64_to_f16_bits(np.nextafter(mid, np.inf)), hi)
    # the same on the negative side
    assert np.array_equal(oracle_mod.f64_to_f16_bits(-mid), even | 0x8000)


def test_overflow_boundary(oracle_mod):
    x = np.array([65504.0, 65519.999, 65520.0, 1e6, -65520.0, -65519.0], dtype=np.float64)
    got = oracle_mod.f64_to_f16_bits(x)
    assert list(got) == [0x7bff, 0x7bff, 0x7c00, 0x7c00, 0xfc00, 0xfbff]


def test_random_doubles_match_numpy_cast(oracle_mod):
    rng = np.random.default_rng(7)
    # log-uniform magnitudes from far below the subnormal range to overflow
    x = np.exp2(rng.uniform(-30, 17, size=200_000)) * rng.choice([-1.0, 1.0], size=200_000)
    got = oracle_mod.f64_to_f16_bits(x)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)


# --------------------------------------------------------------------------
# the GEMM definition
# --------------------------------------------------------------------------
def _random_f16_values(rng, shape):
    """fp16 values with exponents from the subnormal range up to 2^3, plus +-0."""
    code = rng.integers(0, 0x4800, size=shape).astype(np.uint16)       # |x| < 8
    sign = (rng.integers(0, 2, size=shape).astype(np.uint16) << 15)
    v = (code | sign).view(np.float16).copy()
    zeros = rng.random(size=shape) < 0.05
    v[zeros] = np.float16(0.0)
    return v


def test_brute_force_exact_rationals_all_small_shapes(oracle_mod):
    rng = np.random.default_rng(11)
    for m, n, k in itertools.product(range(1, 7), repeat=3):
        a = _random_f16_values(rng, (m, k))
        b = _random_f16_values(rng, (n, k))
        got = bits(oracle_mod.gemm(a, b))
        fa = [[Fraction(float(v)) for v in row] for row in a]
        fb = [[Fraction(float(v)) for v in row] for row in b]
        for i in range(m):
            for j in range(n):
                s = sum((fa[i][t] * fb[j][t] for t in range(k)), Fraction(0))
                assert got[i, j] == exact_to_f16_bits(s), (m, n, k, i, j)


def test_exhaustive_single_element_times_one(oracle_mod):
    """1x1x1 with B = 1.0 over every finite fp16 A: C = A, and -0 becomes +0
    because the accumulator starts at +0.0."""
    b16 = _all_finite_f16_bits()
    a = b16.view(np.float16).reshape(-1, 1)
    one = np.ones((1, 1), dtype=np.float16)
    got = bits(oracle_mod.gemm(a, one)).reshape(-1)
    expect = b16.copy()
    expect[expect == 0x8000] = 0x0000
    assert np.array_equal(got, expect)


def test_empty_shapes(oracle_mod):
    a = np.zeros((0, 5), np.float16)
    b = np.zeros((3, 5), np.float16)
    assert oracle_mod.gemm(a, b).shape == (0, 3)
    assert oracle_mod.gemm(b, a).shape == (3, 0)
    # K = 0: the empty sum, +0 everywhere
    c = oracle_mod.gemm(np.zeros((4, 0), np.float16), np.zeros((6, 0), np.float16))
    assert c.shape == (4, 6) and np.all(bits(c) == 0)


def test_identity_b_returns_a(oracle_mod):
    a, _ = workloads.make_inputs(37, 1, 64, "uniform", 1.0, seed=3)
    eye = np.eye(64, dtype=np.float16)
    c = oracle_mod.gemm(a, eye)
    assert same_up_to_zero_sign(c, a)


def test_permutation_b_permutes_columns(oracle_mod):
    rng = np.random.default_rng(5)
    a, _ = workloads.make_inputs(29, 1, 48, "normal", 1.0, seed=4)
    perm = rng.permutation(48)
    b = np.zeros((48, 48), np.float16)
    b[np.arange(48), perm] = 1.0          # B[j, perm[j]] = 1
    c = oracle_mod.gemm(a, b)
    assert same_up_to_zero_sign(c, a[:, perm])
    # and a non-square selection: N < K, C[:, j] = A[:, sel[j]]
    sel = rng.choice(48, size=13, replace=False)
    bs = np.zeros((13, 48), np.float16)
    bs[np.arange(13), sel] = 1.0
    assert same_up_to_zero_sign(oracle_mod.gemm(a, bs), a[:, sel])


@pytest.mark.parametrize("k,expect", [(256, 256.0), (4096, 4096.0), (4160, 4160.0),
                                      (8192, 8192.0), (16384, 16384.0),
                                      (2049, 2048.0),   # tie between 2048 and 2050: even
                                      (4999, 5000.0)])  # nearest on the 4-wide grid
def test_all_ones(oracle_mod, k, expect):
    a = np.ones((3, k), np.float16)
    b = np.ones((2, k), np.float16)
    c = oracle_mod.gemm(a, b)
    assert np.all(c.astype(np.float64) == expect)


def test_small_integers_match_int64_matmul(oracle_mod):
    """Entries in {-2..2}: every sum is an integer below 2^11 * 8 here, so the
    int64 matmul (exact) rounded once must equal the oracle bit for bit."""
    a, b = workloads.make_inputs(96, 80, 512, "int2", 1.0, seed=9)
    exact = a.astype(np.int64) @ b.astype(np.int64).T
    ref = exact.astype(np.float64).astype(np.float16)
    assert same_up_to_zero_sign(oracle_mod.gemm(a, b), ref)


@pytest.mark.parametrize("shape,dist", [((64, 48, 1000), "uniform"),
                                        ((128, 96, 200), "normal"),
                                        ((33, 65, 4160), "normal")])
def test_numpy_fp64_matmul_cross_check(oracle_mod, shape, dist):
    m, n, k = shape
    a, b = workloads.make_inputs(m, n, k, dist, 1.0 / np.sqrt(k), seed=m + n + k)
    ref = (a.astype(np.float64) @ b.astype(np.float64).T).astype(np.float16)
    got = oracle_mod.gemm(a, b)
    assert same_up_to_zero_sign(got, ref)


def test_swap_invariant(oracle_mod):
    a, b = workloads.make_inputs(40, 23, 300, "normal", 0.05, seed=12)
    assert np.array_equal(bits(oracle_mod.gemm(b, a)), bits(oracle_mod.gemm(a, b)).T)


def test_power_of_two_scaling(oracle_mod):
    a, b = workloads.make_inputs(50, 60, 256, "uniform", 1.0 / 16, seed=13)
    c = oracle_mod.gemm(a, b).astype(np.float64)
    c2 = oracle_mod.gemm((a.astype(np.float64) * 4).astype(np.float16), b).astype(np.float64)
    normal = (np.abs(c) >= 2.0 ** -14) & (np.abs(c) * 4 <= 65504)
    assert normal.mean() > 0.9
    assert np.array_equal(c2[normal], 4 * c[normal])


def test_sampled_equals_full(oracle_mod):
    a, b = workloads.make_inputs(70, 90, 333, "normal", 0.1, seed=14)
    full, full_sum = oracle_mod.gemm(a, b, return_sum=True)
    rng = np.random.default_rng(1)
    r = rng.integers(0, 70, 500)
    c = rng.integers(0, 90, 500)
    s, s_sum = oracle_mod.gemm_sampled(a, b, r, c, return_sum=True)
    assert np.array_equal(bits(s), bits(full[r, c]))
    assert np.array_equal(s_sum, full_sum[r, c])


# --------------------------------------------------------------------------
# closed-form probes: ties, overflow, subnormals
# --------------------------------------------------------------------------
def test_rne_tie_probes(oracle_mod):
    # 1 + 3*2^-11 lies exactly between 1 + 2^-10 and 1 + 2^-9: even wins (1 + 2^-9);
    # truncation would give 1 + 2^-10.  1 + 0.75*2^-10 rounds up to 1 + 2^-10;
    # truncation would give 1.
    a = np.array([[1.0, 3 * 2.0 ** -11], [1.0, 0.75 * 2.0 ** -10]], dtype=np.float16)
    b = np.ones((1, 2), np.float16)
    c = oracle_mod.gemm(a, b).astype(np.float64).ravel()
    assert c[0] == 1 + 2.0 ** -9
    assert c[1] == 1 + 2.0 ** -10


def test_overflow_probe(oracle_mod):
    a = np.full((2, 256), 16.0, np.float16)
    b = np.full((2, 256), 16.0, np.float16)
    assert np.all(np.isposinf(oracle_mod.gemm(a, b).astype(np.float64)))   # 65536
    c = oracle_mod.gemm(a[:, :255].copy(), b[:, :255].copy()).astype(np.float64)
    assert np.all(c == 65280.0)


def test_subnormal_probe(oracle_mod):
    j = np.arange(1, 1024, dtype=np.float64)
    a = (j * 2.0 ** -24).astype(np.float16).reshape(31, 33)
    assert np.all(a.view(np.uint16) < 0x0400)      # all subnormal
    c = oracle_mod.gemm(a, np.eye(33, dtype=np.float16))
    assert same_up_to_zero_sign(c, a)


# --------------------------------------------------------------------------
# the pages' accuracy figure pins "fp32-or-better accumulation, one rounding"
# --------------------------------------------------------------------------
def _unit_variance_inputs(m, n, k, seed):
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((m, k)).astype(np.float16)
    b = (rng.standard_normal((n, k)) / np.sqrt(k)).astype(np.float16)
    return a, b


def _page_figures():
    with open(os.path.join(GOLDEN, "page_accuracy_k8192.json")) as f:
        return json.load(f)


def test_page_mae_single_rounding(oracle_mod):
    g = _page_figures()
    a, b = _unit_variance_inputs(128, 128, g["K"], seed=21)
    c, s = oracle_mod.gemm(a, b, return_sum=True)
    assert 0.9 < s.std() < 1.1                     # unit-variance outputs
    mae = np.mean(np.abs(c.astype(np.float64) - s))
    # 0.00014 printed with two significant digits
    assert 0.000135 <= mae <= 0.000145, mae


def test_page_mae_catches_planted_fp16_accumulation():
    """A planted mistake -- an fp16 accumulator rounded after every 16-deep MMA
    step, the pages' fp16-accumulating variant (their MMA instructions are k16
    deep, page 6 "The Full Kernel") -- lands near the pages' 0.0023, far outside
    the single-rounding band: the MAE pin tells the two apart."""
    g = _page_figures()
    a, b = _unit_variance_inputs(48, 48, g["K"], seed=22)
    af = a.astype(np.float64)
    bf = b.astype(np.float64)
    exact = af @ bf.T
    acc = np.zeros((48, 48), np.float16)
    for k0 in range(0, g["K"], 16):
        step = af[:, k0:k0 + 16] @ bf[:, k0:k0 + 16].T
        acc = (acc.astype(np.float64) + step).astype(np.float16)
    mae = np.mean(np.abs(acc.astype(np.float64) - exact))
    assert 0.5 * g["mae_fp16_accumulate"] < mae < 2.0 * g["mae_fp16_accumulate"], mae
    assert mae > 5 * g["mae_fp32_accumulate"]
