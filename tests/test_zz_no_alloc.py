"""gemm_f16_nt_splitk_noalloc (through the C ABI) against gemm_f16_nt_splitk.

The no-allocation entry point keeps the split-K partials in the library's
fixed device array instead of a caller workspace; with the same plan it runs
the same kernels, so its result must carry the same bits as the workspace
entry point's, and (as that one's) match the oracle: bit-exact on integer
inputs, within the fp16 tolerance otherwise.  Two calls in a row, the second
smaller, show that what the first left in the shared array does not leak
into the second.
"""
import sys

import numpy as np
import pytest

import workloads
from parity import assert_bit_exact, assert_within_tolerance

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 64 << 20


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


def _both(g, a, b, splits):
    """(C from the no-allocation entry point, C from gemm_f16_nt_splitk with a
    poisoned workspace, effective splits, planned workspace bytes)."""
    import torch

    m, n, k = a.shape[0], b.shape[0], a.shape[1]
    dev = torch.device("cuda:0")
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    _, eff, need = g.gemm_f16_nt_splitk_plan(m, n, k, cus, splits)
    assert need <= SCRATCH_BYTES
    _say(f"  noalloc {m}x{n}x{k} splits={splits} -> {eff} ranges, {need} bytes of partials")
    ta = torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    tb = torch.from_numpy(np.ascontiguousarray(b)).to(dev)
    stream = torch.cuda.current_stream().cuda_stream
    outs = []
    for use_scratch in (True, False):
        flat = torch.full((m * n + 8,), float("nan"), dtype=torch.float16, device=dev)
        c = flat[:m * n]
        if use_scratch:
            g.gemm_f16_nt_splitk_noalloc(m, n, k, ta.data_ptr(), tb.data_ptr(), c.data_ptr(),
                                         splits, stream)
        else:
            ws = torch.full((max(need, 16),), 0xFF, dtype=torch.uint8, device=dev)
            g.gemm_f16_nt_splitk(m, n, k, ta.data_ptr(), tb.data_ptr(), c.data_ptr(), splits,
                                 ws.data_ptr(), need, stream)
        torch.cuda.synchronize()
        host = flat.cpu().numpy()
        assert np.isnan(host[m * n:].astype(np.float32)).all()   # nothing past C written
        outs.append(host[:m * n].reshape(m, n))
    return outs[0], outs[1], eff, need


def test_two_calls_in_a_row_match_the_workspace_entry_point(g, oracle_mod):
    # first call: integer inputs, the planner's split (several ranges)
    a, b = workloads.make_inputs(512, 512, 16384, "int2", 1.0, seed=71)
    c_na, c_ws, eff, need = _both(g, a, b, 0)
    assert eff > 1 and need > 0
    assert_bit_exact(c_na, c_ws, "noalloc vs workspace entry point, 512x512x16384 int")
    assert_bit_exact(c_na, oracle_mod.gemm(a, b), "noalloc vs oracle, 512x512x16384 int")
    # second call, smaller and ragged, non-integer inputs, a forced split:
    # the array still holds the first call's larger partials
    a, b = workloads.make_inputs(200, 136, 9000, "uniform", 1.0, seed=72)
    c_na, c_ws, eff, need = _both(g, a, b, 4)
    assert eff == 4
    assert_bit_exact(c_na, c_ws, "noalloc vs workspace entry point, 200x136x9000")
    assert_within_tolerance(c_na, oracle_mod.gemm(a, b), "noalloc vs oracle, 200x136x9000")


def test_streaming_split_plan(g, oracle_mod):
    # a few rows of A over a short N: the planner splits the register-streaming
    # plan over K (16 x 16 tiles, one fp32 partial per range); then a smaller
    # call with ragged N and K over what the first left in the array
    for (m, n, k, dist, seed) in [(1, 256, 32768, "int2", 75), (5, 200, 8200, "uniform", 76)]:
        a, b = workloads.make_inputs(m, n, k, dist, 1.0, seed=seed)
        plan, _, _ = g.gemm_f16_nt_splitk_plan(m, n, k, 256, 0)
        assert g.gemm_f16_nt_config_info(plan.config_id).stages == 0
        c_na, c_ws, eff, need = _both(g, a, b, 0)
        assert eff > 1 and need > 0
        assert_bit_exact(c_na, c_ws, f"noalloc vs workspace entry point, {m}x{n}x{k} streaming")
        if dist == "int2":
            assert_bit_exact(c_na, oracle_mod.gemm(a, b), f"noalloc vs oracle, {m}x{n}x{k}")
        else:
            assert_within_tolerance(c_na, oracle_mod.gemm(a, b), f"noalloc vs oracle, {m}x{n}x{k}")


def test_repeated_calls_are_bit_identical(g):
    a, b = workloads.make_inputs(300, 260, 12000, "normal", 1.0 / np.sqrt(12000), seed=73)
    first, _, eff, _ = _both(g, a, b, 6)
    assert eff > 1
    again, _, _, _ = _both(g, a, b, 6)
    assert_bit_exact(again, first, "noalloc rerun")


def test_unsplit_plan_and_empty_problems(g, oracle_mod):
    import torch

    # a plan with one split runs the plain kernel (no partials at all)
    a, b = workloads.make_inputs(256, 256, 256, "int2", 1.0, seed=74)
    c_na, c_ws, eff, need = _both(g, a, b, 1)
    assert eff == 1 and need == 0
    assert_bit_exact(c_na, oracle_mod.gemm(a, b), "noalloc unsplit vs oracle")
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    c = torch.full((8, 8), float("nan"), dtype=torch.float16, device=dev)
    # K = 0: the empty sum, +0 everywhere
    g.gemm_f16_nt_splitk_noalloc(8, 8, 0, 0, 0, c.data_ptr(), 0, stream)
    torch.cuda.synchronize()
    assert (c.cpu().numpy().view(np.uint16) == 0).all()
    # M = 0: nothing to do (B still holds N x K elements, so it is not NULL)
    tb = torch.zeros((8, 64), dtype=torch.float16, device=dev)
    g.gemm_f16_nt_splitk_noalloc(0, 8, 64, 0, tb.data_ptr(), 0, 0, stream)


def test_errors_before_any_launch(g):
    import torch

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    m = n = 4096
    k = 1024
    ta = torch.zeros((m, k), dtype=torch.float16, device=dev)
    tb = torch.zeros((n, k), dtype=torch.float16, device=dev)
    c = torch.full((m, n), 7.0, dtype=torch.float16, device=dev)
    # two ranges of a 4096 x 4096 output need 128 MiB of partials: more than
    # the array holds, a clear status, and nothing is launched
    _, eff, need = g.gemm_f16_nt_splitk_plan(m, n, k, 256, 2)
    assert eff == 2 and need > SCRATCH_BYTES
    with pytest.raises(g.GemmError) as e:
        g.gemm_f16_nt_splitk_noalloc(m, n, k, ta.data_ptr(), tb.data_ptr(), c.data_ptr(), 2,
                                     stream)
    assert e.value.status == g.SCRATCH_LIMIT
    torch.cuda.synchronize()
    assert (c.cpu().numpy() == 7.0).all()
    # argument errors come first
    with pytest.raises(g.GemmError) as e:
        g.gemm_f16_nt_splitk_noalloc(m, n, -1, ta.data_ptr(), tb.data_ptr(), c.data_ptr(), 0,
                                     stream)
    assert e.value.status == g.INVALID_ARG
    with pytest.raises(g.GemmError) as e:
        g.gemm_f16_nt_splitk_noalloc(m, n, k, ta.data_ptr(), tb.data_ptr(), c.data_ptr(), 65,
                                     stream)
    assert e.value.status == g.INVALID_ARG
