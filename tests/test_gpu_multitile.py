"""Persistent workgroups that own several tiles, against the full oracle.

A workgroup of the persistent grid walks its tiles one after another (Tilus
"Hopper matmul" page "6. Register Reallocation, Multicast, and a Persistent
Kernel", Persistent Tile Loop): the next tile's ring prefill is issued
before the current tile's epilogue, and after an interior tile the LDS-staged
epilogue's C stores are left in flight through the next tile's first wait.
Those hand-offs only run when a workgroup owns more than one tile, so every
configuration with the staged epilogue is forced onto grids of 1, 3 and 7
workgroups over a shape of interior and edge tiles, and the whole output is
compared with the oracle: bit-exact on integer inputs, within the fp16
tolerance otherwise.  Every layout's configurations are covered, on the same
data transposed as the layout stores it.
"""
import sys

import numpy as np
import pytest

import workloads
from parity import assert_bit_exact, assert_within_tolerance

pytestmark = pytest.mark.gpu

# 1096 x 904: with 256 x 256 tiles 5 x 4 tiles, 12 of them interior; M, N and
# K multiples of 8, as the k-outermost layouts' direct-to-LDS kernels need
M, N, K = 1096, 904, 1000
GRIDS = (1, 3, 7)


@pytest.fixture(scope="module")
def g():
    import torch

    import dense_fp16_gemm_amd as lib

    lib.load()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return lib


@pytest.fixture(scope="module")
def int_case(oracle_mod):
    a, b = workloads.make_inputs(M, N, K, "int2", 1.0, seed=81)
    return a, b, oracle_mod.gemm(a, b)


@pytest.fixture(scope="module")
def float_case(oracle_mod):
    a, b = workloads.make_inputs(M, N, K, "normal", 1.0 / np.sqrt(K), seed=82)
    return a, b, oracle_mod.gemm(a, b)


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


def _run(g, lay, a_mk, b_nk, config, grid, epilogue):
    """C through gemm_f16_<lay>_with_config on the layout's storage of the NT
    operands; C poisoned with NaN so an unwritten element cannot pass."""
    import torch

    _say(f"  gpu gemm_{lay} {M}x{N}x{K} config={config} grid={grid} epilogue={epilogue}")
    a = np.ascontiguousarray(a_mk.T) if lay[0] == "t" else a_mk
    b = np.ascontiguousarray(b_nk.T) if lay[1] == "n" else b_nk
    dev = torch.device("cuda:0")
    ta = torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    tb = torch.from_numpy(np.ascontiguousarray(b)).to(dev)
    flat = torch.full((M * N + 8,), float("nan"), dtype=torch.float16, device=dev)
    out = flat[:M * N].view(M, N)
    g.gemm(ta, tb, lay, out=out, config=config, grid=grid, epilogue=epilogue)
    torch.cuda.synchronize()
    host = flat.cpu().numpy()
    assert np.isnan(host[M * N:].astype(np.float32)).all()
    return host[:M * N].reshape(M, N)


def test_every_configuration_on_small_grids(g, int_case):
    """Every configuration of every layout, with the staged epilogue where it
    has room for it and direct stores otherwise."""
    a, b, ref = int_case
    staged = 0
    for cid in range(g.gemm_f16_nt_num_configs()):
        lay = g.gemm_f16_nt_config_info(cid).layout
        epi = 1
        for grid in GRIDS:
            try:
                got = _run(g, lay, a, b, cid, grid, epi)
            except g.GemmError as e:
                assert e.status == g.UNSUPPORTED and epi == 1 and grid == GRIDS[0]
                epi = 0                            # no room to stage C
                got = _run(g, lay, a, b, cid, grid, epi)
            assert_bit_exact(got, ref, f"{lay} config {cid} grid {grid} epilogue {epi}")
            staged += epi
    assert staged >= 3 * 20


@pytest.mark.parametrize("lay,cid", [("nt", 11), ("nt", 18), ("nn", 24), ("tt", 30),
                                     ("tn", 33)])
def test_headline_configurations_on_small_grids_float(g, float_case, lay, cid):
    a, b, ref = float_case
    first = None
    for grid in GRIDS + (0,):
        for epi in (1, 0):
            got = _run(g, lay, a, b, cid, grid, epi)
            assert_within_tolerance(got, ref, f"{lay} config {cid} grid {grid} epilogue {epi}")
            if first is None:
                first = got
            else:
                # the K order of an element never depends on the launch shape
                assert_bit_exact(got, first, f"{lay} config {cid} grid {grid} epilogue {epi}")
