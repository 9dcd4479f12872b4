"""Autotuning on the GPU: gemm_f16_autotune through the C ABI.

Every candidate the tuner times (each configuration of a layout, unsplit and
with each split count) is first run on its own on integer inputs, whose sums
are exact in fp32 in any order, and must equal the oracle bit for bit.  Then
the tuner itself: the output it leaves is the fastest candidate's, within the
oracle tolerance, replaying its choice gives the same bits, its timings are
consistent, and arguments only the general kernel takes leave that kernel as
the one candidate.
"""
import sys

import numpy as np
import pytest

import workloads
from parity import assert_bit_exact, assert_within_tolerance

pytestmark = pytest.mark.gpu

LAYOUTS = ["nt", "nn", "tn", "tt"]


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


def _operands(lay, a_mk, b_nk):
    a = np.ascontiguousarray(a_mk.T) if lay[0] == "t" else a_mk
    b = np.ascontiguousarray(b_nk.T) if lay[1] == "n" else b_nk
    return a, b


def _cus():
    import torch

    return torch.cuda.get_device_properties(0).multi_processor_count


@pytest.mark.parametrize("lay", LAYOUTS)
def test_every_candidate_bit_exact_on_integer_inputs(g, oracle_mod, lay):
    import torch

    m, n, k = 200, 304, 6152
    a_mk, b_nk = workloads.make_inputs(m, n, k, "int2", 1.0, seed=341)
    ref = oracle_mod.gemm(a_mk, b_nk)
    a, b = _operands(lay, a_mk, b_nk)
    ta, tb = torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda()
    cand, need = g.gemm_f16_autotune_candidates(g.LAYOUT_CODES[lay], m, n, k, _cus(), True,
                                                1 << 40)
    assert any(e.splits > 1 for e in cand), "the case must exercise split candidates"
    ws = torch.full((max(need, 16),), 0xFF, dtype=torch.uint8, device="cuda")
    out = torch.empty((m, n), dtype=torch.float16, device="cuda")
    for e in cand:
        _say(f"  gpu candidate {lay} {m}x{n}x{k} config={e.config_id} splits={e.splits}")
        out.fill_(float("nan"))
        g.gemm_splitk(ta, tb, lay, splits=e.splits, config=e.config_id, out=out, workspace=ws)
        torch.cuda.synchronize()
        assert_bit_exact(out.cpu().numpy(), ref,
                         f"int2 {lay} config {e.config_id} splits {e.splits}")


@pytest.mark.parametrize("lay", LAYOUTS)
def test_autotune_leaves_the_fastest_result(g, oracle_mod, lay):
    import torch

    m, n, k = 296, 264, 4104
    a_mk, b_nk = workloads.make_inputs(m, n, k, "uniform", 1.0 / np.sqrt(k), seed=342)
    a, b = _operands(lay, a_mk, b_nk)
    ta, tb = torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda()
    _say(f"  gpu autotune {lay} {m}x{n}x{k}")
    tuned = g.autotune(ta, tb, lay, iters=3)
    torch.cuda.synchronize()
    assert_within_tolerance(tuned.out.cpu().numpy(), oracle_mod.gemm(a_mk, b_nk),
                            f"autotune {lay}")
    cand, _ = g.gemm_f16_autotune_candidates(g.LAYOUT_CODES[lay], m, n, k, _cus(), True, 1 << 40)
    assert [(e["config_id"], e["splits"]) for e in tuned.entries] == \
        [(e.config_id, e.splits) for e in cand], "every candidate timed, in order"
    assert all(e["status"] == 0 and e["ms"] > 0 for e in tuned.entries)
    assert tuned.ms == min(e["ms"] for e in tuned.entries)
    assert (tuned.config, tuned.splits) in [(e["config_id"], e["splits"]) for e in tuned.entries]
    # replaying the choice gives the same bits (deterministic kernels)
    again = tuned(ta, tb)
    torch.cuda.synchronize()
    assert torch.equal(again.view(torch.int16), tuned.out.view(torch.int16))


@pytest.mark.parametrize("lay,shape,misalign", [
    ("nt", (200, 304, 4102), False),      # K not a multiple of 8
    ("nt", (200, 304, 4104), True),       # A one element off 16-byte alignment
    ("nn", (200, 301, 4104), False),      # N not a multiple of 8 with B stored [K, N]
    ("tn", (203, 304, 4104), True),
])
def test_autotune_general_arguments(g, oracle_mod, lay, shape, misalign):
    import torch

    m, n, k = shape
    a_mk, b_nk = workloads.make_inputs(m, n, k, "normal", 1.0 / np.sqrt(k), seed=343)
    a, b = _operands(lay, a_mk, b_nk)
    ta = torch.from_numpy(a).cuda()
    if misalign:
        buf = torch.empty(a.size + 8, dtype=torch.float16, device="cuda")
        ta = buf[1:1 + a.size].view(a.shape)
        ta.copy_(torch.from_numpy(a).cuda())
    tb = torch.from_numpy(b).cuda()
    _say(f"  gpu autotune general {lay} {shape} misalign={misalign}")
    tuned = g.autotune(ta, tb, lay, iters=2)
    torch.cuda.synchronize()
    assert len(tuned.entries) == 1 and tuned.splits == 1
    info = g.gemm_f16_nt_config_info(tuned.config)
    assert info.layout == lay
    assert_within_tolerance(tuned.out.cpu().numpy(), oracle_mod.gemm(a_mk, b_nk),
                            f"autotune general {lay}")


def test_autotune_empty_problems(g):
    import torch

    a = torch.zeros((0, 64), dtype=torch.float16, device="cuda")
    b = torch.zeros((64, 64), dtype=torch.float16, device="cuda")
    tuned = g.autotune(a, b, "nt")
    assert tuned.config == -1 and tuned.splits == 1 and tuned.entries == []
    # K = 0: C is the empty sum, +0
    a = torch.zeros((96, 0), dtype=torch.float16, device="cuda")
    b = torch.zeros((80, 0), dtype=torch.float16, device="cuda")
    out = torch.full((96, 80), float("nan"), dtype=torch.float16, device="cuda")
    tuned = g.autotune(a, b, "nt", out=out)
    torch.cuda.synchronize()
    assert tuned.config == -1 and tuned.entries == []
    assert (out.view(torch.int16) == 0).all()


def test_autotune_workspace_bound(g, oracle_mod):
    """A workspace smaller than the largest split leaves those splits out."""
    import torch

    m, n, k = 256, 256, 16384
    a, b = workloads.make_inputs(m, n, k, "int2", 1.0, seed=344)
    ta, tb = torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda()
    bound = 4 * m * n * 4
    ws = torch.empty(bound, dtype=torch.uint8, device="cuda")
    _say(f"  gpu autotune bound {m}x{n}x{k} workspace={bound}")
    tuned = g.autotune(ta, tb, "nt", iters=2, workspace=ws)
    torch.cuda.synchronize()
    assert max(e["splits"] for e in tuned.entries) == 4
    assert_bit_exact(tuned.out.cpu().numpy(), oracle_mod.gemm(a, b), "autotune bound")


@pytest.mark.parametrize("name", list(workloads.EXTRA_WORKLOADS))
def test_autotune_full_size_underfilled(g, oracle_mod, name):
    """The under-filled workload at full size: the tuner picks a split (the
    unsplit grid fills 16 of 256 CUs), and the result matches the oracle on
    sampled elements."""
    import torch

    w = workloads.EXTRA_WORKLOADS[name]
    a, b = workloads.workload_inputs(name)
    ta, tb = torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda()
    _say(f"  gpu autotune {name}")
    tuned = g.autotune(ta, tb, "nt", iters=3)
    torch.cuda.synchronize()
    _say(f"  chose config {tuned.config} splits {tuned.splits} ({tuned.ms:.4f} ms)")
    assert tuned.splits > 1
    got = tuned.out.cpu().numpy()
    rng = np.random.default_rng(w.seed)
    r = np.concatenate([rng.integers(0, w.M, 4096), np.arange(w.M)])
    c = np.concatenate([rng.integers(0, w.N, 4096), np.full(w.M, w.N - 1)])
    assert_within_tolerance(got[r, c], oracle_mod.gemm_sampled(a, b, r, c), name)
