"""Parity of the split-K entry point (through the C ABI) with the CPU oracle.

The split path computes the same C = fp16_rne(A B^T) as the plain one, with
the K sum cut into ranges whose fp32 partials are added in range order, so
non-integer inputs are held to the same tolerance against the oracle and
integer inputs (every partial sum exact) must be bit-exact.  The workspace is
poisoned before each call: its contents on entry must not matter.
"""
import sys

import numpy as np
import pytest

import workloads
from parity import assert_bit_exact, assert_within_tolerance

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


def run_splitk(g, a, b, splits=0, config=None, ws_offset=0, ws_bytes=None, poison=0xFF):
    """C through gemm_f16_nt_splitk_with_config; returns (C, effective splits)."""
    import torch

    m, n, k = a.shape[0], b.shape[0], a.shape[1]
    _say(f"  gpu splitk {m}x{n}x{k} splits={splits} config={config} ws_offset={ws_offset}")
    dev = torch.device("cuda:0")
    ta = torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    tb = torch.from_numpy(np.ascontiguousarray(b)).to(dev)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    _, eff, need = g.gemm_f16_nt_splitk_plan(m, n, k, cus, splits)
    if config is not None and splits > 1:
        # a forced configuration may cut K into more ranges than the planner's
        need = max(need, g.gemm_f16_splitk_workspace_bytes(m, n, splits))
    flat = torch.full((m * n + 8,), float("nan"), dtype=torch.float16, device=dev)
    out = flat[:m * n].view(m, n)
    ws = torch.full((need + ws_offset + 16,), poison, dtype=torch.uint8, device=dev)
    nbytes = need if ws_bytes is None else ws_bytes
    g.gemm_f16_nt_splitk_with_config(m, n, k, ta.data_ptr(), tb.data_ptr(), out.data_ptr(),
                                     splits, ws.data_ptr() + ws_offset, nbytes,
                                     torch.cuda.current_stream().cuda_stream,
                                     -1 if config is None else config)
    torch.cuda.synchronize()
    host = flat.cpu().numpy()
    assert np.isnan(host[m * n:].astype(np.float32)).all()    # nothing past C written
    return host[:m * n].reshape(m, n), eff


@pytest.mark.parametrize("shape,splits,dist,seed", [
    ((300, 260, 4104), 0, "uniform", 301),
    ((256, 256, 16384), 0, "normal", 302),
    ((77, 129, 2056), 5, "uniform", 303),
    ((64, 64, 40000), 7, "normal", 304),       # the last range ends mid-slice
    ((513, 385, 8200), 3, "uniform", 305),
    ((1, 1, 4096), 4, "uniform", 306),
    ((33, 31, 520), 64, "normal", 307),        # more requested splits than slices
    ((200, 300, 6144), 2, "uniform", 308),
])
def test_splitk_parity(g, oracle_mod, shape, splits, dist, seed):
    m, n, k = shape
    a, b = workloads.make_inputs(m, n, k, dist, 1.0 / np.sqrt(k), seed=seed)
    got, eff = run_splitk(g, a, b, splits)
    assert eff > 1, "the case must exercise the split path"
    assert_within_tolerance(got, oracle_mod.gemm(a, b), f"splitk {shape} splits {splits}")


@pytest.mark.parametrize("config", [None, 2, 4, 9, 11, 18, 21, 22, 23, 42, 43])
def test_splitk_integer_bit_exact(g, oracle_mod, config):
    a, b = workloads.make_inputs(200, 300, 6152, "int2", 1.0, seed=311)
    got, eff = run_splitk(g, a, b, 6, config=config)
    assert eff > 1
    assert_bit_exact(got, oracle_mod.gemm(a, b), f"int2 splitk config {config}")


STREAM = 43   # B streamed through registers (no LDS ring)


def _ranges(k, splits):
    """Ranges of K a split count gives the streaming configuration (K steps of 32)."""
    k_split = -(-(-(-k // splits)) // 32) * 32
    return -(-k // k_split)


@pytest.mark.parametrize("shape,splits,dist,seed", [
    ((1, 256, 8192), 0, "normal", 321),       # planned: 4 ranges of 2048
    ((16, 1000, 8200), 0, "uniform", 322),    # planned: 4 ranges, N tail, a shorter last range
    ((1, 256, 32768), 0, "normal", 326),      # planned: 16 ranges
    ((7, 33, 4136), 5, "normal", 323),        # ranges end mid-block; K tail of 8
    ((17, 100, 4096), 8, "uniform", 324),     # two tile rows of A
    ((3, 4099, 2056), 3, "normal", 325),
])
def test_splitk_streaming_parity(g, oracle_mod, shape, splits, dist, seed):
    """The streaming configuration's split instance: each unit streams one
    range of K for one 16 x 16 tile into an fp32 partial; as planned for few
    rows of A and as forced, against the oracle."""
    m, n, k = shape
    plan, eff, _ = g.gemm_f16_nt_splitk_plan(m, n, k, 256, splits)
    if splits == 0:
        assert plan.config_id == STREAM and eff > 1, "the planner must split the streaming plan"
    a, b = workloads.make_inputs(m, n, k, dist, 1.0 / np.sqrt(k), seed=seed)
    got, _ = run_splitk(g, a, b, splits, config=None if splits == 0 else STREAM)
    assert splits == 0 or _ranges(k, splits) > 1
    assert_within_tolerance(got, oracle_mod.gemm(a, b), f"stream splitk {shape} splits {splits}")


@pytest.mark.parametrize("splits", [2, 3, 16])
def test_splitk_streaming_integer_bit_exact(g, oracle_mod, splits):
    a, b = workloads.make_inputs(9, 777, 5000, "int2", 1.0, seed=327)
    got, _ = run_splitk(g, a, b, splits, config=STREAM)
    assert_bit_exact(got, oracle_mod.gemm(a, b), f"int2 stream splitk {splits}")


def test_splitk_one_split_is_the_plain_path(g):
    import torch

    a, b = workloads.make_inputs(300, 260, 4104, "normal", 0.02, seed=312)
    got, eff = run_splitk(g, a, b, 1)
    assert eff == 1
    plain = g.gemm_nt(torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda())
    torch.cuda.synchronize()
    assert_bit_exact(got, plain.cpu().numpy(), "splits=1 vs gemm_nt")


def test_splitk_deterministic_whatever_the_workspace_held(g):
    a, b = workloads.make_inputs(256, 256, 16384, "normal", 1.0 / 128, seed=313)
    first, _ = run_splitk(g, a, b, 0, poison=0xFF)
    for poison in (0x00, 0x7F, 0xFF):
        again, _ = run_splitk(g, a, b, 0, poison=poison)
        assert_bit_exact(again, first, f"rerun, workspace bytes 0x{poison:02x}")


@pytest.mark.parametrize("k", [60, 4097])
def test_splitk_general_arguments_run_the_plain_path(g, oracle_mod, k):
    import torch

    a, b = workloads.make_inputs(130, 70, k, "uniform", 1.0 / np.sqrt(k), seed=314)
    got, eff = run_splitk(g, a, b, 8)
    assert eff == 1
    plain = g.gemm_nt(torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda())
    torch.cuda.synchronize()
    assert_bit_exact(got, plain.cpu().numpy(), f"k={k} splitk vs gemm_nt")
    assert_within_tolerance(got, oracle_mod.gemm(a, b), f"k={k}")


def test_splitk_k_zero(g):
    a = np.zeros((40, 0), np.float16)
    b = np.zeros((50, 0), np.float16)
    got, eff = run_splitk(g, a, b, 4)
    assert eff == 1
    assert (got.view(np.uint16) == 0).all()


def test_splitk_workspace_errors(g):
    import torch

    a, b = workloads.make_inputs(256, 256, 16384, "uniform", 0.01, seed=315)
    dev = torch.device("cuda:0")
    ta, tb = torch.from_numpy(a).to(dev), torch.from_numpy(b).to(dev)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    _, eff, need = g.gemm_f16_nt_splitk_plan(256, 256, 16384, cus, 0)
    assert eff > 1
    c = torch.empty(256, 256, dtype=torch.float16, device=dev)
    ws = torch.empty(need + 64, dtype=torch.uint8, device=dev)
    s = torch.cuda.current_stream().cuda_stream
    lib = g.load()
    call = lambda w, nb, cc=c: lib.gemm_f16_nt_splitk(256, 256, 16384, ta.data_ptr(), tb.data_ptr(),
                                                     cc.data_ptr(), 0, w, nb, s)
    assert call(0, need) == 1                            # no workspace
    assert call(ws.data_ptr(), need - 4) == 1            # too small
    assert call(ws.data_ptr() + 4, need) == 2            # not 16-byte aligned
    assert call(c.data_ptr(), need) == 1                 # overlaps C
    assert call(ta.data_ptr(), need) == 1                # overlaps A
    assert call(ws.data_ptr(), need) == 0
    torch.cuda.synchronize()


def test_splitk_torch_wrapper(g, oracle_mod):
    import torch

    a, b = workloads.make_inputs(96, 160, 12288, "uniform", 1.0 / 111, seed=316)
    c = g.gemm_nt_splitk(torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda())
    torch.cuda.synchronize()
    assert_within_tolerance(c.cpu().numpy(), oracle_mod.gemm(a, b), "gemm_nt_splitk")


@pytest.mark.parametrize("name", list(workloads.EXTRA_WORKLOADS))
def test_full_size_underfilled_workload(g, oracle_mod, name):
    """The under-filled workload at full size, split as the benchmark's
    --splitk 0 launch splits it; sampled elements (random positions plus the
    first and last rows and the last column) against the oracle."""
    w = workloads.EXTRA_WORKLOADS[name]
    a, b = workloads.workload_inputs(name)
    got, eff = run_splitk(g, a, b, 0)
    assert eff > 1
    assert not np.isnan(got).any(), "unwritten (NaN-poisoned) output elements"
    rng = np.random.default_rng(w.seed)
    rows = [rng.integers(0, w.M, 4096), np.zeros(w.N, np.int64), np.full(w.N, w.M - 1),
            np.arange(w.M)]
    cols = [rng.integers(0, w.N, 4096), np.arange(w.N), np.arange(w.N), np.full(w.M, w.N - 1)]
    r, c = np.concatenate(rows), np.concatenate(cols)
    assert_within_tolerance(got[r, c], oracle_mod.gemm_sampled(a, b, r, c), name)


@pytest.mark.parametrize("name", list(workloads.FEW_ROWS_WORKLOADS))
def test_full_size_few_rows_workload_split(g, oracle_mod, name):
    """The one-row workload through the split entry point as planned, against
    the whole oracle row."""
    a, b = workloads.workload_inputs(name)
    got, _ = run_splitk(g, a, b, 0)
    assert_within_tolerance(got, oracle_mod.gemm(a, b), name)


# ---------------------------------------------------------------------------
# the split over K for the other operand layouts
# ---------------------------------------------------------------------------
def _operands(lay, a_mk, b_nk):
    a = np.ascontiguousarray(a_mk.T) if lay[0] == "t" else a_mk
    b = np.ascontiguousarray(b_nk.T) if lay[1] == "n" else b_nk
    return a, b


@pytest.mark.parametrize("lay", ["nn", "tn", "tt"])
@pytest.mark.parametrize("shape,splits", [((256, 256, 16384), 0), ((128, 136, 4104), 5),
                                          ((384, 256, 40000), 7)])
def test_splitk_layouts_parity(g, oracle_mod, lay, shape, splits):
    import torch

    m, n, k = shape
    a_mk, b_nk = workloads.make_inputs(m, n, k, "normal", 1.0 / np.sqrt(k), seed=320 + k)
    a, b = _operands(lay, a_mk, b_nk)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    _, eff, _ = getattr(g, f"gemm_f16_{lay}_splitk_plan")(m, n, k, cus, splits)
    assert eff > 1, "the case must exercise the split path"
    _say(f"  gpu splitk {lay} {shape} splits={splits}")
    c = g.gemm_splitk(torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda(), lay, splits=splits)
    torch.cuda.synchronize()
    assert_within_tolerance(c.cpu().numpy(), oracle_mod.gemm(a_mk, b_nk), f"splitk {lay} {shape}")


@pytest.mark.parametrize("lay", ["nn", "tn", "tt"])
def test_splitk_layouts_integer_bit_exact(g, oracle_mod, lay):
    import torch

    a_mk, b_nk = workloads.make_inputs(200, 304, 6152, "int2", 1.0, seed=331)
    a, b = _operands(lay, a_mk, b_nk)
    c = g.gemm_splitk(torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda(), lay, splits=6)
    torch.cuda.synchronize()
    assert_bit_exact(c.cpu().numpy(), oracle_mod.gemm(a_mk, b_nk), f"int2 splitk {lay}")


def test_splitk_forced_config_default_workspace(g, oracle_mod):
    """A forced configuration whose K slice differs from the planner's splits
    into more ranges than the planner's plan (here 6 against 5): the torch
    wrapper's default workspace must still cover it."""
    import torch

    m, n, k = 64, 64, 1040
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    plan, eff, _ = g.gemm_f16_nt_splitk_plan(m, n, k, cus, 8)
    assert plan.block_k == 128 and eff == 5, "the case needs a K-128 plan"
    a, b = workloads.make_inputs(m, n, k, "int2", 1.0, seed=351)
    _say(f"  gpu splitk forced config 11 {m}x{n}x{k} splits=8")
    c = g.gemm_nt_splitk(torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda(), splits=8,
                         config=11)
    torch.cuda.synchronize()
    assert_bit_exact(c.cpu().numpy(), oracle_mod.gemm(a, b), "forced config 11, 8 splits")
