"""Parity of the HIP path (through the C ABI) with the CPU oracle.

All inputs are seeded and synthetic (workloads.py).  Non-integer inputs are
compared element by element within |C - C_ref| <= 2 ulp16(C_ref) + 1e-3;
integer inputs, identity/permutation B, all-ones, scaling and the closed-form
probes must be bit-exact.  Shapes span several tiles with ragged tails; the
five workload shapes run at full size in the launch configuration the
benchmark times, checked against the whole oracle matrix and through
size-independent properties.
"""
import sys

import numpy as np
import pytest

import workloads
from parity import assert_bit_exact, assert_within_tolerance, tolerance_report

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def g():
    import torch

    import dense_fp16_gemm_amd as lib

    lib.load()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return lib


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


def run_gpu(g, a, b, config=None, swizzle=0, grid=0, epilogue=-1, c_offset=0):
    """C = a @ b.T on the GPU through the C ABI.  c_offset shifts C by that
    many fp16 elements inside a larger buffer (to test C alignment)."""
    import torch

    _say(f"  gpu gemm {a.shape[0]}x{b.shape[0]}x{a.shape[1]} config={config} "
         f"swizzle={swizzle} grid={grid} epilogue={epilogue} c_offset={c_offset}")
    dev = torch.device("cuda:0")
    ta = torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    tb = torch.from_numpy(np.ascontiguousarray(b)).to(dev)
    m, n = a.shape[0], b.shape[0]
    # poison C so that an element the kernel never writes cannot pass
    flat = torch.full((m * n + c_offset + 8,), float("nan"), dtype=torch.float16, device=dev)
    out = flat[c_offset:c_offset + m * n].view(m, n)
    g.gemm_nt(ta, tb, out=out, config=config, swizzle=swizzle, grid=grid, epilogue=epilogue)
    torch.cuda.synchronize()
    host = flat.cpu().numpy()
    # nothing outside C may be touched
    assert np.isnan(host[:c_offset].astype(np.float32)).all()
    assert np.isnan(host[c_offset + m * n:].astype(np.float32)).all()
    return host[c_offset:c_offset + m * n].reshape(m, n)


def num_configs(g):
    return g.gemm_f16_nt_num_configs()


# ---------------------------------------------------------------------------
# small and medium shapes against the full oracle
# ---------------------------------------------------------------------------
SHAPES = [
    (256, 256, 256),      # one 256x256 tile
    (300, 260, 200),      # ragged M/N/K, two tiles each way
    (513, 385, 136),      # three tiles of 256 along M, K tail of 8
    (1, 1, 8),            # degenerate
    (33, 31, 24),         # smaller than one MFMA block
    (640, 96, 1000),      # K tail of 40, tall-skinny
    (96, 700, 72),        # N tail, K = one full slice + 8
]


@pytest.mark.parametrize("shape", SHAPES)
def test_parity_default_plan(g, oracle_mod, shape):
    m, n, k = shape
    a, b = workloads.make_inputs(m, n, k, "uniform", 1.0 / np.sqrt(k), seed=m * 7 + n + k)
    got = run_gpu(g, a, b)
    ref = oracle_mod.gemm(a, b)
    assert_within_tolerance(got, ref, f"{shape}")


@pytest.mark.parametrize("shape", [(300, 260, 200), (513, 385, 136), (33, 31, 24),
                                   (129, 65, 520)])
def test_parity_every_config(g, oracle_mod, shape):
    """Every compiled configuration, including ones the planner does not pick
    for this shape; all must agree with the oracle and be bit-identical to
    each other (the K order of an element never depends on the tiling)."""
    m, n, k = shape
    a, b = workloads.make_inputs(m, n, k, "normal", 1.0 / np.sqrt(k), seed=m + 3 * n + k)
    ref = oracle_mod.gemm(a, b)
    first = None
    for cid in range(num_configs(g)):
        if g.gemm_f16_nt_config_info(cid).layout != "nt":
            continue                                   # another operand layout's
        for epi in (0, 1):
            try:
                got = run_gpu(g, a, b, config=cid, epilogue=epi)
            except g.GemmError as e:
                assert epi == 1 and e.status == g.UNSUPPORTED   # no room to stage C
                continue
            assert_within_tolerance(got, ref, f"{shape} config {cid} epilogue {epi}")
            if first is None:
                first = got
            else:
                assert_bit_exact(got, first, f"{shape} config {cid} epilogue {epi} vs first")


@pytest.mark.parametrize("cid", [0, 1, 2, 3, 4, 5, 9, 11, 17, 18, 19, 20, 21, 22, 23, 42, 43])
@pytest.mark.parametrize("k", [8, 24, 32, 40, 64, 72, 128, 136, 160, 192, 200, 256, 264, 328])
def test_short_and_ragged_k(g, oracle_mod, cid, k):
    """K with fewer slices than stages, exactly the stages, one more, and
    tails of 8..56 beyond a whole slice."""
    a, b = workloads.make_inputs(130, 70, k, "uniform", 1.0, seed=k)
    got = run_gpu(g, a, b, config=cid)
    assert_within_tolerance(got, oracle_mod.gemm(a, b), f"k={k} config {cid}")


@pytest.mark.parametrize("cid", [0, 2, 4, 5, 11, 17, 18, 19, 20, 21, 22, 23, 42, 43])
def test_edge_m_n(g, oracle_mod, cid):
    info = g.gemm_f16_nt_config_info(cid)
    bm, bn = info.block_m, info.block_n
    for m in (1, 31, 32, 33, bm - 1, bm + 1):
        for n in (1, 33, bn - 1, bn + 1):
            a, b = workloads.make_inputs(m, n, 72, "normal", 0.1, seed=m * 1000 + n)
            got = run_gpu(g, a, b, config=cid)
            assert_within_tolerance(got, oracle_mod.gemm(a, b), f"{m}x{n}x72 config {cid}")


@pytest.mark.parametrize("c_offset", [1, 2, 3, 4])
@pytest.mark.parametrize("epi", [0, 1])
@pytest.mark.parametrize("cid", [9, 11])
def test_unaligned_c(g, oracle_mod, c_offset, epi, cid):
    """C only 2-, 4- or 8-byte aligned, and odd N: the epilogue's narrower
    store paths; every element written once, nothing outside C touched."""
    a, b = workloads.make_inputs(300, 261, 136, "normal", 0.1, seed=c_offset)
    got = run_gpu(g, a, b, config=cid, epilogue=epi, c_offset=c_offset)
    assert_within_tolerance(got, oracle_mod.gemm(a, b), f"c_offset {c_offset} epilogue {epi}")


@pytest.mark.parametrize("cid", [None, 11, 42, 43])
def test_k_zero_writes_positive_zero(g, cid):
    a = np.zeros((70, 0), np.float16)
    b = np.zeros((90, 0), np.float16)
    got = run_gpu(g, a, b, config=cid)
    assert np.all(got.view(np.uint16) == 0)


STREAM = 43   # B streamed through registers (no LDS ring)


@pytest.mark.parametrize("m", [1, 2, 7, 16, 17, 40])
@pytest.mark.parametrize("c_offset", [0, 1, 3])
def test_streaming_configuration_small_m(g, oracle_mod, m, c_offset):
    """The register-streaming configuration on a few rows of A, with N and K
    tails (K = 54 steps of 32 and 8 more) and C at 2-, 4- and 8-byte
    alignment: within tolerance of the oracle and bit-identical to the
    headline configuration (the same MFMA and K order)."""
    assert g.gemm_f16_nt_config_info(STREAM).stages == 0
    a, b = workloads.make_inputs(m, 1000, 1736, "normal", 0.05, seed=500 + m)
    got = run_gpu(g, a, b, config=STREAM, c_offset=c_offset)
    assert_within_tolerance(got, oracle_mod.gemm(a, b), f"stream m={m} c_offset={c_offset}")
    assert_bit_exact(got, run_gpu(g, a, b, config=11), f"stream m={m} vs config 11")


@pytest.mark.parametrize("shape", [(64, 1024, 2056), (40, 640, 3080), (8, 6000, 1032), (3, 8192, 1000),
                                   (4099, 1, 4104), (1000, 13, 2056), (1000, 40, 1032)])
def test_planned_streaming_shapes(g, oracle_mod, shape):
    """Shapes the plain planner streams beyond M <= 16 with a quarter of the
    CUs (up to 64 rows in one round of 16 x 16 tiles, or up to 8 rows with
    half the CUs), and with the roles swapped (a few columns of B, A
    streamed), as planned, on integer inputs: bit-exact with the oracle."""
    m, n, k = shape
    plan = g.gemm_f16_nt_plan(m, n, k, 256)
    assert g.gemm_f16_nt_config_info(plan.config_id).stages == 0
    a, b = workloads.make_inputs(m, n, k, "int2", 1.0, seed=510 + m)
    assert_bit_exact(run_gpu(g, a, b), oracle_mod.gemm(a, b), f"planned stream {shape}")


def test_m_or_n_zero_is_a_no_op(g):
    import torch

    z = torch.zeros((0, 64), dtype=torch.float16, device="cuda:0")
    b = torch.zeros((16, 64), dtype=torch.float16, device="cuda:0")
    assert tuple(g.gemm_nt(z, b).shape) == (0, 16)
    assert tuple(g.gemm_nt(b, z).shape) == (16, 0)


# ---------------------------------------------------------------------------
# bit-exact cases
# ---------------------------------------------------------------------------
def test_integer_inputs_bit_exact(g, oracle_mod):
    a, b = workloads.make_inputs(700, 500, 1032, "int2", 1.0, seed=31)
    got = run_gpu(g, a, b)
    assert_bit_exact(got, oracle_mod.gemm(a, b), "int2 700x500x1032")


def test_identity_and_permutation_b(g):
    rng = np.random.default_rng(2)
    a, _ = workloads.make_inputs(300, 1, 264, "normal", 1.0, seed=5)
    eye = np.eye(264, dtype=np.float16)
    assert_bit_exact(run_gpu(g, a, eye), a, "B = I")
    perm = rng.permutation(264)
    bp = np.zeros((264, 264), np.float16)
    bp[np.arange(264), perm] = 1.0
    assert_bit_exact(run_gpu(g, a, bp), a[:, perm], "B = permutation")


@pytest.mark.parametrize("k,expect", [(256, 256.0), (4096, 4096.0), (4160, 4160.0),
                                      (8192, 8192.0), (2056, 2056.0), (5000, 5000.0)])
def test_all_ones(g, k, expect):
    a = np.ones((260, k), np.float16)
    b = np.ones((70, k), np.float16)
    got = run_gpu(g, a, b).astype(np.float64)
    assert np.all(got == expect)


def test_rne_tie_probes(g):
    # K padded to 8 with zeros; sums 1 + 3*2^-11 (tie -> 1 + 2^-9) and
    # 1 + 0.75*2^-10 (-> 1 + 2^-10).  A truncating convert gives 1 + 2^-10 and 1.
    a = np.zeros((2, 8), np.float16)
    a[0, :2] = [1.0, 3 * 2.0 ** -11]
    a[1, :2] = [1.0, 0.75 * 2.0 ** -10]
    b = np.zeros((1, 8), np.float16)
    b[0, :2] = 1.0
    got = run_gpu(g, a, b).astype(np.float64).ravel()
    assert got[0] == 1 + 2.0 ** -9
    assert got[1] == 1 + 2.0 ** -10


def test_overflow_probe(g):
    a = np.full((3, 256), 16.0, np.float16)
    got = run_gpu(g, a, a).astype(np.float64)
    assert np.all(np.isposinf(got))
    a2 = np.zeros((3, 256), np.float16)
    a2[:, :255] = 16.0
    got2 = run_gpu(g, a2, a2).astype(np.float64)
    assert np.all(got2 == 65280.0)


def test_subnormal_probe(g):
    j = np.arange(0, 1024, dtype=np.float64)          # 0 and every subnormal j * 2^-24
    a = (j * 2.0 ** -24).astype(np.float16).reshape(32, 32)
    assert np.all(a.view(np.uint16) < 0x0400)
    eye = np.zeros((32, 32), np.float16)
    eye[np.arange(32), np.arange(32)] = 1.0
    assert_bit_exact(run_gpu(g, a, eye), a, "subnormal A, B = I")


def test_power_of_two_scaling_bit_exact(g):
    a, b = workloads.make_inputs(300, 270, 520, "uniform", 1.0 / 16, seed=41)
    c = run_gpu(g, a, b).astype(np.float64)
    c4 = run_gpu(g, (a.astype(np.float64) * 4).astype(np.float16), b).astype(np.float64)
    normal = (np.abs(c) >= 2.0 ** -14) & (np.abs(c) * 4 <= 65504)
    assert normal.mean() > 0.9
    assert np.array_equal(c4[normal], 4 * c[normal])


def test_swap_invariant_integer(g):
    a, b = workloads.make_inputs(333, 290, 264, "int2", 1.0, seed=43)
    assert_bit_exact(run_gpu(g, b, a), run_gpu(g, a, b).T, "swap")


def test_determinism_and_launch_shape_independence(g):
    a, b = workloads.make_inputs(1100, 900, 1000, "normal", 0.03, seed=47)
    first = run_gpu(g, a, b)
    for _ in range(3):
        assert_bit_exact(run_gpu(g, a, b), first, "rerun")
    for swz in (1, 3, 5):
        assert_bit_exact(run_gpu(g, a, b, config=0, swizzle=swz), first, f"swizzle {swz}")
    for grid in (1, 7, 64):
        assert_bit_exact(run_gpu(g, a, b, config=0, grid=grid), first, f"grid {grid}")


def test_gemm_nt_passes_swizzle_and_grid_without_a_config(g, monkeypatch):
    # a raster width or grid given alone must reach the library (the plain
    # entry point takes neither); results stay bit-identical
    a, b = workloads.make_inputs(700, 600, 512, "int2", 1.0, seed=53)
    first = run_gpu(g, a, b)
    seen = []
    real = g.gemm_f16_nt_with_config

    def spy(*args):
        seen.append(args[-4:])   # config, swizzle, grid, epilogue
        return real(*args)

    monkeypatch.setattr(g, "gemm_f16_nt_with_config", spy)
    assert_bit_exact(run_gpu(g, a, b, swizzle=3), first, "swizzle 3, planned config")
    assert_bit_exact(run_gpu(g, a, b, grid=5), first, "grid 5, planned config")
    assert seen == [(-1, 3, 0, -1), (-1, 0, 5, -1)]


def test_page_mae_statistic(g):
    """K = 8192 with unit-variance outputs: the mean |error| against the exact
    sum must sit at the pages' fp32-accumulation figure, 0.00014 (page 6,
    note in "Shared-Memory Epilogue"), not near the fp16-accumulation 0.0023."""
    import json
    import os

    with open(os.path.join(os.path.dirname(__file__), "golden", "page_accuracy_k8192.json")) as f:
        fig = json.load(f)
    rng = np.random.default_rng(23)
    k = fig["K"]
    a = rng.standard_normal((256, k)).astype(np.float16)
    b = (rng.standard_normal((256, k)) / np.sqrt(k)).astype(np.float16)
    import oracle

    ref, exact = oracle.gemm(a, b, return_sum=True)
    got = run_gpu(g, a, b)
    ok, stats = tolerance_report(got, ref, exact_sum=exact)
    assert ok, stats
    assert 0.000135 <= stats["mae_vs_exact"] <= 0.000145, stats


# ---------------------------------------------------------------------------
# full-size workloads, in the launch configuration the benchmark times
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", list(workloads.WORKLOADS) + list(workloads.FEW_ROWS_WORKLOADS))
def test_full_size_workload(g, oracle_mod, name):
    """Each workload at full size, in the plan the benchmark times, against
    the whole oracle matrix (8192^3 takes the oracle about 20 s on 16 host
    cores).  The one-row workload runs the register-streaming plan."""
    w = workloads.ALL_WORKLOADS[name]
    if name in workloads.FEW_ROWS_WORKLOADS:
        plan = g.gemm_f16_nt_plan(w.M, w.N, w.K, 256)
        assert g.gemm_f16_nt_config_info(plan.config_id).stages == 0
    _say(f"  workload {name}: {w.M}x{w.N}x{w.K} {w.dist} seed={w.seed}")
    a, b = workloads.workload_inputs(name)
    got = run_gpu(g, a, b)
    assert not np.isnan(got).any(), "unwritten (NaN-poisoned) output elements"
    _say(f"  oracle {name}: full {w.M}x{w.N} output")
    ref = oracle_mod.gemm(a, b)
    if w.dist == "int2":
        assert_bit_exact(got, ref, name)
    else:
        stats = assert_within_tolerance(got, ref, name)
        _say(f"  {name}: {stats}")


def test_tail_equals_padded_interior(g):
    """Ragged 4999 x 7001 x 4160: the same inputs zero-padded to whole tiles
    give bit-identical values on the original rows and columns, since each
    element's K order does not depend on its position."""
    a, b = workloads.workload_inputs("ragged4999x7001x4160")
    got = run_gpu(g, a, b)
    ap = np.zeros((5120, 4160), np.float16)
    ap[:4999] = a
    bp = np.zeros((7168, 4160), np.float16)
    bp[:7001] = b
    padded = run_gpu(g, ap, bp)
    assert_bit_exact(got, padded[:4999, :7001], "tail vs padded")
    assert np.all(padded[4999:].view(np.uint16) == 0)
    assert np.all(padded[:, 7001:].view(np.uint16) == 0)


def test_integer_workload_full_matrix(g):
    """4096^3 with entries in {-2..2}: every partial sum is an integer below
    2^24, so the whole output must equal the exactly computed integer product
    (numpy fp64 matmul is exact here)."""
    a, b = workloads.workload_inputs("square4096_int")
    got = run_gpu(g, a, b)
    exact = (a.astype(np.float64) @ b.astype(np.float64).T).astype(np.float16)
    assert_bit_exact(got, exact, "4096^3 int2 full matrix")


# ---------------------------------------------------------------------------
# the general kernel: any K, A and B at any 2-byte alignment
# ---------------------------------------------------------------------------
def run_gpu_offset(g, a, b, a_offset=0, b_offset=0, config=None):
    """As run_gpu, with A and B placed a_offset / b_offset fp16 elements into
    larger buffers (to test A and B alignment)."""
    import torch

    _say(f"  gpu gemm {a.shape[0]}x{b.shape[0]}x{a.shape[1]} a_offset={a_offset} "
         f"b_offset={b_offset} config={config}")
    dev = torch.device("cuda:0")
    m, k = a.shape
    n = b.shape[0]
    fa = torch.zeros(m * k + a_offset + 8, dtype=torch.float16, device=dev)
    fb = torch.zeros(n * k + b_offset + 8, dtype=torch.float16, device=dev)
    ta = fa[a_offset:a_offset + m * k].view(m, k)
    tb = fb[b_offset:b_offset + n * k].view(n, k)
    ta.copy_(torch.from_numpy(np.ascontiguousarray(a)))
    tb.copy_(torch.from_numpy(np.ascontiguousarray(b)))
    flat = torch.full((m * n + 8,), float("nan"), dtype=torch.float16, device=dev)
    out = flat[:m * n].view(m, n)
    g.gemm_nt(ta, tb, out=out, config=config)
    torch.cuda.synchronize()
    host = flat.cpu().numpy()
    assert np.isnan(host[m * n:].astype(np.float32)).all()
    return host[:m * n].reshape(m, n)


@pytest.mark.parametrize("k", [1, 2, 3, 7, 9, 15, 17, 33, 100, 255, 1001])
def test_general_any_k(g, oracle_mod, k):
    """K that is not a multiple of 8 runs the general kernel (tails in M, N
    and within the last 16-byte chunk of every row)."""
    a, b = workloads.make_inputs(130, 70, k, "uniform", 1.0 / np.sqrt(k), seed=k + 500)
    got = run_gpu(g, a, b)
    assert_within_tolerance(got, oracle_mod.gemm(a, b), f"k={k}")
    ai, bi = workloads.make_inputs(130, 70, k, "int2", 1.0, seed=k + 600)
    assert_bit_exact(run_gpu(g, ai, bi), oracle_mod.gemm(ai, bi), f"int k={k}")


@pytest.mark.parametrize("a_offset,b_offset", [(1, 0), (0, 1), (3, 5), (4, 4), (7, 2)])
def test_general_unaligned_a_b(g, oracle_mod, a_offset, b_offset):
    """A or B only 2-, 4- or 8-byte aligned runs the general kernel; the
    result equals the aligned direct-to-LDS path's bit for bit (same K order)."""
    a, b = workloads.make_inputs(300, 260, 136, "normal", 0.1, seed=a_offset * 8 + b_offset)
    got = run_gpu_offset(g, a, b, a_offset, b_offset)
    assert_within_tolerance(got, oracle_mod.gemm(a, b), f"offsets {a_offset},{b_offset}")
    assert_bit_exact(got, run_gpu(g, a, b), f"offsets {a_offset},{b_offset} vs aligned")


def test_general_matches_direct_path(g):
    """The general kernel forced on aligned inputs gives the default plan's
    result bit for bit."""
    general = g.gemm_f16_nt_num_configs() - 1
    a, b = workloads.make_inputs(517, 389, 264, "normal", 0.06, seed=77)
    assert_bit_exact(run_gpu(g, a, b, config=general), run_gpu(g, a, b), "general vs default")


def test_forced_direct_config_rejects_general_arguments(g):
    """A direct-to-LDS configuration forced on arguments it cannot take is an
    error, not a wrong result."""
    a, b = workloads.make_inputs(64, 64, 60, "uniform", 0.1, seed=3)
    with pytest.raises(g.GemmError) as e:
        run_gpu(g, a, b, config=11)
    assert e.value.status == g.UNSUPPORTED


def test_general_large_k(g, oracle_mod):
    """K beyond 2^21 (past the direct path's 32-bit buffer offsets)."""
    k = (1 << 21) + 24
    a, b = workloads.make_inputs(8, 9, k, "uniform", 1.0 / np.sqrt(k), seed=91)
    assert_within_tolerance(run_gpu(g, a, b), oracle_mod.gemm(a, b), f"k={k}")


# ---------------------------------------------------------------------------
# seeded random shapes across every configuration and alignment
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("case", range(24))
def test_random_shapes_every_path(g, oracle_mod, case):
    """Seeded random M, N, K (K a multiple of 8 or not), a random
    configuration that can take them, and random A/B offsets: parity with
    the oracle, and for K a multiple of 8 with aligned operands, equality
    with the default plan bit for bit."""
    rng = np.random.default_rng(9000 + case)
    m = int(rng.integers(1, 700))
    n = int(rng.integers(1, 700))
    k = int(rng.integers(1, 600))
    if case % 2 == 0:
        k = max(8, k - k % 8)
    a_off = int(rng.choice([0, 0, 8, 1, 3]))
    b_off = int(rng.choice([0, 0, 8, 2, 5]))
    general = g.gemm_f16_nt_num_configs() - 1
    fast_ok = k % 8 == 0 and a_off % 8 == 0 and b_off % 8 == 0
    nt_ids = [c for c in range(g.gemm_f16_nt_num_configs())
              if g.gemm_f16_nt_config_info(c).layout == "nt"]
    cid = int(rng.choice(nt_ids)) if fast_ok else general
    a, b = workloads.make_inputs(m, n, k, "normal", 1.0 / np.sqrt(k), seed=case)
    got = run_gpu_offset(g, a, b, a_off, b_off, config=cid)
    assert_within_tolerance(got, oracle_mod.gemm(a, b), f"case {case}: {m}x{n}x{k} config {cid}")
    if fast_ok:
        assert_bit_exact(got, run_gpu(g, a, b), f"case {case}: config {cid} vs default")
