"""The other operand layouts (gemm_f16_nn, gemm_f16_tn, gemm_f16_tt) against
the oracle.

The oracle computes C = fp16_rne(sum_k a(i, k) b(k, j)) for A [M, K] and
B [N, K]; the tests hand the layouts the same data transposed with numpy
(pure data movement).  Every layout keeps each element's K order, so each
must also equal gemm_f16_nt on the untransposed data bit for bit, for every
configuration of that layout.
"""
import sys

import numpy as np
import pytest

import workloads
from parity import assert_bit_exact, assert_within_tolerance

pytestmark = pytest.mark.gpu

LAYOUTS = ["nn", "tn", "tt"]


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


def configs_of(g, lay):
    return [c for c in range(g.gemm_f16_nt_num_configs())
            if g.gemm_f16_nt_config_info(c).layout == lay]


def operands(lay, a_mk, b_nk):
    """The NT operands a [M, K], b [N, K] stored as the layout wants them."""
    a = np.ascontiguousarray(a_mk.T) if lay[0] == "t" else a_mk
    b = np.ascontiguousarray(b_nk.T) if lay[1] == "n" else b_nk
    return a, b


def run_layout(g, lay, a, b, config=None, epilogue=-1):
    """C through the layout's entry point; C poisoned with NaN first."""
    import torch

    m = a.shape[1] if lay[0] == "t" else a.shape[0]
    n = b.shape[1] if lay[1] == "n" else b.shape[0]
    _say(f"  gpu gemm_{lay} {tuple(a.shape)} x {tuple(b.shape)} config={config} epilogue={epilogue}")
    dev = torch.device("cuda:0")
    ta = torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    tb = torch.from_numpy(np.ascontiguousarray(b)).to(dev)
    flat = torch.full((m * n + 8,), float("nan"), dtype=torch.float16, device=dev)
    out = flat[:m * n].view(m, n)
    g.gemm(ta, tb, lay, out=out, config=config, epilogue=epilogue)
    torch.cuda.synchronize()
    host = flat.cpu().numpy()
    assert np.isnan(host[m * n:].astype(np.float32)).all()
    return host[:m * n].reshape(m, n)


def run_nt(g, a_mk, b_nk):
    import torch

    c = g.gemm_nt(torch.from_numpy(np.ascontiguousarray(a_mk)).cuda(),
                  torch.from_numpy(np.ascontiguousarray(b_nk)).cuda())
    torch.cuda.synchronize()
    return c.cpu().numpy()


# M, N, K multiples of 8 (each layout needs them for its contiguous dimension)
SHAPES = [(256, 256, 256), (304, 264, 200), (512, 392, 136), (32, 40, 24), (128, 64, 520),
          (1000, 1000, 1000), (64, 1024, 2056), (776, 136, 72)]


@pytest.mark.parametrize("lay", LAYOUTS)
@pytest.mark.parametrize("shape", SHAPES)
def test_layout_parity_every_config(g, oracle_mod, lay, shape):
    m, n, k = shape
    a_mk, b_nk = workloads.make_inputs(m, n, k, "normal", 1.0 / np.sqrt(k), seed=500 + m + n + k)
    a, b = operands(lay, a_mk, b_nk)
    ref = oracle_mod.gemm(a_mk, b_nk)
    nt = run_nt(g, a_mk, b_nk)
    for cid in configs_of(g, lay):
        for epi in (0, 1):
            try:
                got = run_layout(g, lay, a, b, config=cid, epilogue=epi)
            except g.GemmError as e:
                assert epi == 1 and e.status == g.UNSUPPORTED   # no room to stage C
                continue
            assert_within_tolerance(got, ref, f"{lay} {shape} config {cid} epilogue {epi}")
            assert_bit_exact(got, nt, f"{lay} {shape} config {cid} epilogue {epi} vs nt")


@pytest.mark.parametrize("lay", LAYOUTS)
def test_layout_integer_bit_exact(g, oracle_mod, lay):
    a_mk, b_nk = workloads.make_inputs(704, 504, 1032, "int2", 1.0, seed=511)
    a, b = operands(lay, a_mk, b_nk)
    assert_bit_exact(run_layout(g, lay, a, b), oracle_mod.gemm(a_mk, b_nk), f"int2 {lay}")


@pytest.mark.parametrize("lay", LAYOUTS)
def test_layout_identity_and_permutation(g, lay):
    rng = np.random.default_rng(512)
    a_mk = rng.standard_normal((96, 256)).astype(np.float16)
    eye = np.eye(256, dtype=np.float16)
    perm = rng.permutation(256)
    for b_nk, want, what in [(eye, a_mk, "B = I"), (eye[perm], a_mk[:, perm], "B = permutation")]:
        a, b = operands(lay, a_mk, b_nk)
        assert_bit_exact(run_layout(g, lay, a, b), want, f"{lay} {what}")


@pytest.mark.parametrize("lay", LAYOUTS)
def test_layout_k_zero(g, lay):
    a, b = operands(lay, np.zeros((40, 0), np.float16), np.zeros((48, 0), np.float16))
    got = run_layout(g, lay, a, b)
    assert got.shape == (40, 48) and (got.view(np.uint16) == 0).all()


@pytest.mark.parametrize("lay", LAYOUTS)
@pytest.mark.parametrize("shape", [(61, 70, 45), (33, 31, 24), (130, 257, 1001), (7, 9, 3),
                                   (200, 136, 64), (129, 64, 520)])
def test_layout_general_sizes(g, oracle_mod, lay, shape):
    """M, N or K not multiples of 8 (and, for comparison, shapes that are):
    the layout's general kernel where the direct-to-LDS ones cannot run."""
    m, n, k = shape
    a_mk, b_nk = workloads.make_inputs(m, n, k, "normal", 1.0 / np.sqrt(k), seed=600 + m + n + k)
    a, b = operands(lay, a_mk, b_nk)
    got = run_layout(g, lay, a, b)
    assert_within_tolerance(got, oracle_mod.gemm(a_mk, b_nk), f"{lay} {shape}")
    assert_bit_exact(got, run_nt(g, a_mk, b_nk), f"{lay} {shape} vs nt")


@pytest.mark.parametrize("lay", LAYOUTS)
@pytest.mark.parametrize("a_off,b_off", [(1, 0), (0, 3), (4, 4), (7, 2)])
def test_layout_general_unaligned(g, oracle_mod, lay, a_off, b_off):
    """A or B only 2-, 4- or 8-byte aligned: the layout's general kernel, with
    the same bits as the aligned call."""
    import torch

    m, n, k = 136, 200, 264
    a_mk, b_nk = workloads.make_inputs(m, n, k, "uniform", 1.0 / np.sqrt(k), seed=610)
    a, b = operands(lay, a_mk, b_nk)
    dev = torch.device("cuda:0")
    fa = torch.zeros(a.size + 8, dtype=torch.float16, device=dev)
    fb = torch.zeros(b.size + 8, dtype=torch.float16, device=dev)
    fa[a_off:a_off + a.size] = torch.from_numpy(a.ravel()).to(dev)
    fb[b_off:b_off + b.size] = torch.from_numpy(b.ravel()).to(dev)
    ta = fa[a_off:a_off + a.size].view(a.shape)
    tb = fb[b_off:b_off + b.size].view(b.shape)
    _say(f"  gpu gemm_{lay} unaligned a_off={a_off} b_off={b_off}")
    got = g.gemm(ta, tb, lay)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    assert_within_tolerance(got, oracle_mod.gemm(a_mk, b_nk), f"{lay} offsets {a_off},{b_off}")
    assert_bit_exact(got, run_layout(g, lay, a, b), f"{lay} offsets {a_off},{b_off} vs aligned")


def test_layout_forced_fast_config_rejects_general_arguments(g):
    import torch

    a = torch.zeros((64, 60), dtype=torch.float16, device="cuda")     # K = 60 for nn
    b = torch.zeros((60, 64), dtype=torch.float16, device="cuda")
    fast = [c for c in configs_of(g, "nn") if g.gemm_f16_nt_config_info(c).block_k == 64][0]
    with pytest.raises(g.GemmError) as e:
        g.gemm(a, b, "nn", config=fast)
    assert e.value.status == g.UNSUPPORTED


@pytest.mark.parametrize("lay", LAYOUTS)
@pytest.mark.parametrize("name", ["square8192", "skinny128x16384x16384", "square4096_int"])
def test_layout_full_size_equals_nt(g, lay, name):
    """At full size, in the launch configuration the planner picks, each
    layout's result equals the NT result on the same data bit for bit (the NT
    path is parity-tested against the oracle at these sizes)."""
    import torch

    a_mk, b_nk = workloads.workload_inputs(name)
    ta = torch.from_numpy(a_mk).cuda()
    tb = torch.from_numpy(b_nk).cuda()
    nt = g.gemm_nt(ta, tb)
    a = ta.t().contiguous() if lay[0] == "t" else ta
    b = tb.t().contiguous() if lay[1] == "n" else tb
    got = g.gemm(a, b, lay)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), nt.view(torch.int16)), f"{lay} {name}"


@pytest.mark.parametrize("ta,tb", [(False, False), (False, True), (True, False), (True, True)])
def test_matmul_picks_the_layout_from_strides(g, oracle_mod, ta, tb):
    """matmul(a, b) on row-major operands and transposed views: bit-exact on
    integer inputs, in every layout."""
    import torch

    m, n, k = 200, 304, 520
    a_mk, b_nk = workloads.make_inputs(m, n, k, "int2", 1.0, seed=361)
    ga = torch.from_numpy(a_mk.T.copy()).cuda().t() if ta else torch.from_numpy(a_mk).cuda()
    gb = torch.from_numpy(b_nk.copy()).cuda().t() if tb else torch.from_numpy(b_nk.T.copy()).cuda()
    _say(f"  gpu matmul ta={ta} tb={tb}")
    c = g.matmul(ga, gb)
    torch.cuda.synchronize()
    assert_bit_exact(c.cpu().numpy(), oracle_mod.gemm(a_mk, b_nk), f"matmul ta={ta} tb={tb}")


@pytest.mark.parametrize("ta,tb", [(False, False), (False, True), (True, False), (True, True)])
@pytest.mark.parametrize("side_stream", [False, True])
def test_matmul_splits_an_underfilled_long_k(g, oracle_mod, ta, tb, side_stream):
    """Few output tiles and a long K: matmul runs the split over K (workspace
    from torch's allocator), bit-exact on integer inputs, on the current
    stream or on a stream passed in."""
    import torch

    m, n, k = 256, 256, 16384
    a_mk, b_nk = workloads.make_inputs(m, n, k, "int2", 1.0, seed=367)
    ga = torch.from_numpy(a_mk.T.copy()).cuda().t() if ta else torch.from_numpy(a_mk).cuda()
    gb = torch.from_numpy(b_nk.copy()).cuda().t() if tb else torch.from_numpy(b_nk.T.copy()).cuda()
    lay = g.matmul_layout(ga, gb)[0]
    assert g.matmul_splits(lay, m, n, k, ga) > 1
    _say(f"  gpu matmul split {lay} side_stream={side_stream}")
    if side_stream:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        c = g.matmul(ga, gb, stream=s)
        s.synchronize()
    else:
        c = g.matmul(ga, gb)
    torch.cuda.synchronize()
    assert_bit_exact(c.cpu().numpy(), oracle_mod.gemm(a_mk, b_nk), f"matmul split {lay}")
