"""Host side of autotuning: the candidate list gemm_f16_autotune times
(gemm_f16_autotune_candidates, a pure host function of the C ABI).

What is pinned: every candidate is a configuration of the requested layout
that the layout's entry points accept for these arguments; the unsplit run of
each configuration comes first and split counts are distinct, increasing
effective counts (whole K slices per range, at least 256 of K per range)
bounded by the grid rule; split candidates need at most the stated workspace
and none beyond the caller's bound; arguments only the general kernel takes
give it alone; the planner's own choice is always among the candidates.
"""
import ctypes

import pytest

import dense_fp16_gemm_amd as g

CUS = 256


def cdiv(a, b):
    return -(-a // b)


def configs():
    return [g.gemm_f16_nt_config_info(i) for i in range(g.gemm_f16_nt_num_configs())]


def plan_fn(lay):
    return getattr(g, f"gemm_f16_{lay}_plan")


SHAPES = [(8192, 8192, 8192), (1024, 1024, 65536), (4992, 7000, 4160), (128, 16384, 16384),
          (256, 256, 256), (200, 304, 6152), (64, 64, 1024)]


@pytest.mark.parametrize("lay", list(g.LAYOUT_CODES))
@pytest.mark.parametrize("shape", SHAPES)
def test_candidates_well_formed(lay, shape):
    m, n, k = shape
    code = g.LAYOUT_CODES[lay]
    info = configs()
    cand, need = g.gemm_f16_autotune_candidates(code, m, n, k, CUS, True, 1 << 40)
    assert cand, "no candidates"
    pairs = [(e.config_id, e.splits) for e in cand]
    assert len(set(pairs)) == len(pairs)
    stride_bytes = cdiv(m * n, 64) * 64 * 4
    seen = []
    largest = 0
    for e in cand:
        c = info[e.config_id]
        assert c.layout == lay
        assert e.status == 0 and e.ms == -1.0
        if e.config_id not in seen:
            assert e.splits == 1, "a configuration's unsplit run comes first"
            assert not seen or e.config_id > seen[-1], "configurations in id order"
            seen.append(e.config_id)
            last = 1
            continue
        tiles = cdiv(m, c.block_m) * cdiv(n, c.block_n)
        assert e.splits > last
        last = e.splits
        assert tiles < 4 * CUS and tiles * e.splits <= 16 * CUS
        ks = cdiv(k, e.splits)
        ks = cdiv(ks, c.block_k) * c.block_k          # ranges of whole K slices
        assert cdiv(k, ks) == e.splits, "effective counts replay to themselves"
        assert cdiv(k, e.splits) >= 256
        largest = max(largest, e.splits * stride_bytes)
    assert need == largest
    # the planner's unsplit choice is a candidate
    planned = plan_fn(lay)(m, n, k, CUS).config_id
    assert (planned, 1) in pairs


@pytest.mark.parametrize("lay", list(g.LAYOUT_CODES))
def test_candidates_cover_every_configuration_of_the_layout(lay):
    code = g.LAYOUT_CODES[lay]
    # the register-streaming kernel (no LDS ring) only for a few rows of A
    for m, stream in ((1024, False), (64, True), (16, True)):
        cand, _ = g.gemm_f16_autotune_candidates(code, m, 1024, 4096, CUS, True, 0)
        ids = {e.config_id for e in cand}
        want = {i for i, c in enumerate(configs())
                if c.layout == lay and (stream or c.stages > 0)}
        assert ids == want
        assert all(e.splits == 1 for e in cand), "no workspace: no split candidates"


def test_workspace_bound_drops_only_the_larger_splits():
    full, need = g.gemm_f16_autotune_candidates(0, 1024, 1024, 65536, CUS, True, 1 << 40)
    stride_bytes = 1024 * 1024 * 4
    bound = 8 * stride_bytes
    part, need2 = g.gemm_f16_autotune_candidates(0, 1024, 1024, 65536, CUS, True, bound)
    assert need2 == need > bound
    assert [(e.config_id, e.splits) for e in part] == \
        [(e.config_id, e.splits) for e in full if e.splits * stride_bytes <= bound]


@pytest.mark.parametrize("lay,shape,aligned", [
    ("nt", (200, 304, 6150), True),       # K not a multiple of 8
    ("nt", (200, 304, 6152), False),      # A or B not 16-byte aligned
    ("nn", (200, 301, 6152), True),       # N not a multiple of 8 for B stored [K, N]
    ("tn", (203, 304, 6152), True),       # M not a multiple of 8 for A stored [K, M]
    ("tt", (200, 304, 6152), False),
])
def test_general_arguments_give_the_general_kernel_alone(lay, shape, aligned):
    cand, need = g.gemm_f16_autotune_candidates(g.LAYOUT_CODES[lay], *shape, CUS, aligned,
                                                1 << 40)
    assert len(cand) == 1 and cand[0].splits == 1 and need == 0
    # the same configuration the layout's entry point runs for such arguments
    assert cand[0].config_id == plan_fn(lay)(*shape, CUS).config_id or not aligned
    assert configs()[cand[0].config_id].layout == lay


@pytest.mark.parametrize("shape", [(0, 64, 64), (64, 0, 64), (64, 64, 0)])
def test_empty_problems_have_no_candidates(shape):
    cand, need = g.gemm_f16_autotune_candidates(0, *shape, CUS, True, 1 << 40)
    assert cand == [] and need == 0


def test_candidates_count_beyond_the_buffer():
    lib = g.load()
    n, need = ctypes.c_int32(), ctypes.c_int64()
    buf = (g.TuneEntry * 3)()
    assert lib.gemm_f16_autotune_candidates(0, 1024, 1024, 65536, CUS, 1, 1 << 40, buf, 3,
                                            ctypes.byref(n), ctypes.byref(need)) == 0
    full, _ = g.gemm_f16_autotune_candidates(0, 1024, 1024, 65536, CUS, True, 1 << 40)
    assert n.value == len(full) > 3
    assert [(e.config_id, e.splits) for e in buf] == [(e.config_id, e.splits) for e in full[:3]]


@pytest.mark.parametrize("args", [
    (4, 64, 64, 64, CUS, 1, 0),       # layout outside 0..3
    (-1, 64, 64, 64, CUS, 1, 0),
    (0, -1, 64, 64, CUS, 1, 0),
    (0, 64, 64, -8, CUS, 1, 0),
    (0, 64, 64, 64, 0, 1, 0),          # no compute units
    (0, 64, 64, 64, CUS, 1, -1),       # negative workspace bound
])
def test_candidates_invalid_arguments(args):
    lib = g.load()
    n, need = ctypes.c_int32(), ctypes.c_int64()
    assert lib.gemm_f16_autotune_candidates(*args, None, 0, ctypes.byref(n),
                                            ctypes.byref(need)) == g.INVALID_ARG
    # NULL outputs
    assert lib.gemm_f16_autotune_candidates(0, 64, 64, 64, CUS, 1, 0, None, 0, None,
                                            ctypes.byref(need)) == g.INVALID_ARG
    assert lib.gemm_f16_autotune_candidates(0, 64, 64, 64, CUS, 1, 0, None, 4,
                                            ctypes.byref(n), ctypes.byref(need)) == g.INVALID_ARG


def test_autotune_rejects_bad_arguments_without_a_device():
    """Argument checks come before any device call."""
    lib = g.load()
    best, n = g.TuneEntry(), ctypes.c_int32()
    A, B, C = 0x10000, 0x20000000, 0x40000000
    for layout, iters, bp in ((4, 10, ctypes.byref(best)), (0, 0, ctypes.byref(best)),
                              (0, 10001, ctypes.byref(best)), (0, 10, None)):
        assert lib.gemm_f16_autotune(layout, 64, 64, 64, A, B, C, None, 0, iters, None, bp,
                                     None, 0, ctypes.byref(n)) == g.INVALID_ARG
    # the GEMM's own argument checks: C overlapping A
    assert lib.gemm_f16_autotune(0, 64, 64, 64, A, B, A, None, 0, 10, None,
                                 ctypes.byref(best), None, 0, ctypes.byref(n)) == g.INVALID_ARG
    # a workspace size without a workspace
    assert lib.gemm_f16_autotune(0, 64, 64, 64, A, B, C, None, 1024, 10, None,
                                 ctypes.byref(best), None, 0, ctypes.byref(n)) == g.INVALID_ARG


def test_splitk_workspace_bytes_bounds_every_configuration():
    """The bound covers the effective split count of every configuration of
    every layout (each splits K into ranges of its own K slice)."""
    for (m, n, k) in ((1024, 1024, 65536), (300, 200, 1000), (64, 64, 1048576), (8, 8, 520)):
        for splits in (2, 3, 5, 7, 16, 64):
            bound = g.gemm_f16_splitk_workspace_bytes(m, n, splits)
            assert bound == splits * cdiv(m * n, 64) * 64 * 4
            for c in configs():
                if c.block_k == 32:
                    continue
                ks = cdiv(cdiv(k, splits), c.block_k) * c.block_k
                assert cdiv(k, ks) * cdiv(m * n, 64) * 64 * 4 <= bound
    assert g.gemm_f16_splitk_workspace_bytes(100, 100, 1) == 0
    assert g.gemm_f16_splitk_workspace_bytes(100, 100, 0) == 0
    for bad in ((-1, 4, 2), (4, 4, 65), (4, 4, -1)):
        with pytest.raises(g.GemmError):
            g.gemm_f16_splitk_workspace_bytes(*bad)
