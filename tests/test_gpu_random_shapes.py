"""Seeded random shapes in every layout, through the planner's entry points
(plain and split over K), on integer inputs: every partial sum is exact in
fp32, so each result must equal the oracle bit for bit, whichever
configuration, split count and tail handling the planner picks.  The output
is NaN-poisoned first, so an element left unwritten fails too."""
import sys

import numpy as np
import pytest

import workloads
from parity import assert_bit_exact

pytestmark = pytest.mark.gpu

LAYOUTS = ["nt", "nn", "tn", "tt"]


def _shapes(seed, count):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        m, n, k = (int(x) for x in rng.integers(1, 700, 3))
        if i % 4 == 1:   # larger outputs: the 128- and 256-wide tiles
            m, n = 3 * m, 3 * n
        if i % 2 == 0:   # half with every dimension a multiple of 8: the fast kernels
            m, n, k = (max(8, x // 8 * 8) for x in (m, n, k))
        out.append((m, n, 8 * k if i % 3 == 0 else k))   # some long K for the splits
    return out


@pytest.fixture(scope="module")
def g():
    import torch

    import dense_fp16_gemm_amd as lib

    lib.load()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return lib


@pytest.mark.parametrize("lay", LAYOUTS)
@pytest.mark.parametrize("split", [False, True])
def test_random_shapes_bit_exact(g, oracle_mod, lay, split):
    import torch

    for idx, (m, n, k) in enumerate(_shapes(410 + LAYOUTS.index(lay), 16)):
        a_mk, b_nk = workloads.make_inputs(m, n, k, "int2", 1.0, seed=420 + idx)
        a = np.ascontiguousarray(a_mk.T) if lay[0] == "t" else a_mk
        b = np.ascontiguousarray(b_nk.T) if lay[1] == "n" else b_nk
        print(f"  gpu random {lay} split={split} {m}x{n}x{k}", file=sys.stderr, flush=True)
        ta, tb = torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda()
        out = torch.full((m, n), float("nan"), dtype=torch.float16, device="cuda")
        if split:
            g.gemm_splitk(ta, tb, lay, out=out)
        else:
            g.gemm(ta, tb, lay, out=out)
        torch.cuda.synchronize()
        assert_bit_exact(out.cpu().numpy(), oracle_mod.gemm(a_mk, b_nk),
                         f"{lay} split={split} {m}x{n}x{k}")


def _few_shapes(seed, count):
    """NT shapes with a few rows of A or a few columns of B (1..64), the other
    side up to a few thousand, K a multiple of 8 and sometimes long: the
    register-streaming plans and their splits over K."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        few, many = int(rng.integers(1, 65)), int(rng.integers(16, 4000))
        k = int(rng.integers(1, 600)) * 8 * (4 if i % 3 == 0 else 1)
        many = max(16, min(many, int(1.5e8 // (few * k))))   # keeps the oracle quick
        out.append((few, many, k) if i % 2 == 0 else (many, few, k))
    return out


@pytest.mark.parametrize("split", [False, True])
def test_random_few_rows_or_columns_bit_exact(g, oracle_mod, split):
    import torch

    streamed = 0
    for idx, (m, n, k) in enumerate(_few_shapes(450 + int(split), 16)):
        plan = (g.gemm_f16_nt_splitk_plan(m, n, k, g.gemm_f16_device_cus(), 0)[0] if split
                else g.gemm_f16_nt_plan(m, n, k, g.gemm_f16_device_cus()))
        streamed += g.gemm_f16_nt_config_info(plan.config_id).stages == 0
        a, b = workloads.make_inputs(m, n, k, "int2", 1.0, seed=460 + idx)
        print(f"  gpu few rows/columns split={split} {m}x{n}x{k} config {plan.config_id}",
              file=sys.stderr, flush=True)
        ta, tb = torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda()
        out = torch.full((m, n), float("nan"), dtype=torch.float16, device="cuda")
        if split:
            g.gemm_splitk(ta, tb, "nt", out=out)
        else:
            g.gemm(ta, tb, "nt", out=out)
        torch.cuda.synchronize()
        assert_bit_exact(out.cpu().numpy(), oracle_mod.gemm(a, b),
                         f"few rows/columns split={split} {m}x{n}x{k}")
    assert streamed >= 4, "the sample must exercise the streaming plans"


@pytest.mark.parametrize("lay, shape, tile", [
    ("nt", (2000, 3000, 776), (256, 128)),
    ("nn", (2000, 3000, 776), (256, 128)),
    ("tn", (2000, 3000, 776), (256, 128)),
    ("tt", (2000, 3000, 776), (256, 128)),
    ("nt", (1000, 3000, 1000), (128, 128)),
])
def test_plans_the_time_model_overrides(g, oracle_mod, lay, shape, tile):
    # shapes where the planner's time model replaces the area rule's tile:
    # the plain entry point runs the model's configuration, bit-exact
    import torch

    m, n, k = shape
    plan = getattr(g, f"gemm_f16_{lay}_plan")(m, n, k, g.gemm_f16_device_cus())
    assert (plan.block_m, plan.block_n) == tile
    a_mk, b_nk = workloads.make_inputs(m, n, k, "int2", 1.0, seed=433)
    a = np.ascontiguousarray(a_mk.T) if lay[0] == "t" else a_mk
    b = np.ascontiguousarray(b_nk.T) if lay[1] == "n" else b_nk
    print(f"  gpu planned {lay} {m}x{n}x{k} config {plan.config_id}", file=sys.stderr, flush=True)
    ta, tb = torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda()
    out = torch.full((m, n), float("nan"), dtype=torch.float16, device="cuda")
    g.gemm(ta, tb, lay, out=out)
    torch.cuda.synchronize()
    assert_bit_exact(out.cpu().numpy(), oracle_mod.gemm(a_mk, b_nk), f"{lay} {m}x{n}x{k}")
