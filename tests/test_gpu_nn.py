"""C = A B with B stored [K, N] (gemm_f16_nn) against the oracle.

The oracle computes C = fp16_rne(sum_k A[i][k] B[k][j]); the test hands it
B transposed to [N, K] with numpy (pure data movement).  The NN kernels keep
each element's K order, so they must also equal gemm_f16_nt on the transposed
B bit for bit, for every configuration.
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


def nn_configs(g):
    return [c for c in range(g.gemm_f16_nt_num_configs()) if g.gemm_f16_nt_config_info(c).b_layout == 1]


def run_nn(g, a, b_kn, config=None, epilogue=-1):
    """C = a @ b_kn through gemm_f16_nn_with_config; C poisoned with NaN first."""
    import torch

    m, k = a.shape
    n = b_kn.shape[1]
    _say(f"  gpu gemm_nn {m}x{n}x{k} config={config} epilogue={epilogue}")
    dev = torch.device("cuda:0")
    ta = torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    tb = torch.from_numpy(np.ascontiguousarray(b_kn)).to(dev)
    flat = torch.full((m * n + 8,), float("nan"), dtype=torch.float16, device=dev)
    out = flat[:m * n].view(m, n)
    g.gemm_nn(ta, tb, out=out, config=config, epilogue=epilogue)
    torch.cuda.synchronize()
    host = flat.cpu().numpy()
    assert np.isnan(host[m * n:].astype(np.float32)).all()
    return host[:m * n].reshape(m, n)


def run_nt(g, a, b_nk):
    import torch

    c = g.gemm_nt(torch.from_numpy(np.ascontiguousarray(a)).cuda(),
                  torch.from_numpy(np.ascontiguousarray(b_nk)).cuda())
    torch.cuda.synchronize()
    return c.cpu().numpy()


SHAPES = [(256, 256, 256), (300, 264, 200), (513, 392, 136), (33, 32, 24), (129, 64, 520),
          (1000, 1000, 1000), (64, 1024, 2056), (777, 136, 72)]


@pytest.mark.parametrize("shape", SHAPES)
def test_nn_parity_every_config(g, oracle_mod, shape):
    m, n, k = shape
    a, b_nk = workloads.make_inputs(m, n, k, "normal", 1.0 / np.sqrt(k), seed=500 + m + n + k)
    b_kn = np.ascontiguousarray(b_nk.T)
    ref = oracle_mod.gemm(a, b_nk)
    nt = run_nt(g, a, b_nk)
    for cid in nn_configs(g):
        for epi in (0, 1):
            got = run_nn(g, a, b_kn, config=cid, epilogue=epi)
            assert_within_tolerance(got, ref, f"{shape} nn config {cid} epilogue {epi}")
            assert_bit_exact(got, nt, f"{shape} nn config {cid} epilogue {epi} vs nt")


def test_nn_integer_bit_exact(g, oracle_mod):
    a, b_nk = workloads.make_inputs(700, 504, 1032, "int2", 1.0, seed=511)
    got = run_nn(g, a, np.ascontiguousarray(b_nk.T))
    assert_bit_exact(got, oracle_mod.gemm(a, b_nk), "int2 nn 700x504x1032")


def test_nn_identity_and_permutation(g):
    rng = np.random.default_rng(512)
    a = rng.standard_normal((96, 256)).astype(np.float16)
    eye = np.eye(256, dtype=np.float16)                 # [K, N] identity
    assert_bit_exact(run_nn(g, a, eye), a, "B = I")
    perm = rng.permutation(256)
    bp = eye[:, perm]                                   # C[:, j] = A[:, perm[j]]
    assert_bit_exact(run_nn(g, a, bp), a[:, perm], "B = permutation")


def test_nn_k_zero(g):
    got = run_nn(g, np.zeros((40, 0), np.float16), np.zeros((0, 48), np.float16))
    assert (got.view(np.uint16) == 0).all()


def test_nn_unsupported_arguments(g):
    import torch

    a = torch.zeros((64, 64), dtype=torch.float16, device="cuda")
    for b, why in [(torch.zeros((64, 60), dtype=torch.float16, device="cuda"), "N % 8"),
                   (torch.zeros((1, 64 * 64 + 4), dtype=torch.float16, device="cuda")[0, 4:]
                    .view(64, 64), "B 8-byte aligned")]:
        with pytest.raises(g.GemmError) as e:
            g.gemm_nn(a, b)
        assert e.value.status == g.UNSUPPORTED, why


@pytest.mark.parametrize("name", ["square8192", "skinny128x16384x16384", "square4096_int"])
def test_nn_full_size_equals_nt(g, name):
    """At full size, in the launch configuration the planner picks: the NN
    result equals the NT result on the same data bit for bit (the NT path is
    parity-tested against the oracle at these sizes)."""
    import torch

    w = workloads.WORKLOADS[name]
    a, b_nk = workloads.workload_inputs(name)
    ta = torch.from_numpy(a).cuda()
    tb = torch.from_numpy(b_nk).cuda()
    nt = g.gemm_nt(ta, tb)
    nn = g.gemm_nn(ta, tb.t().contiguous())
    torch.cuda.synchronize()
    assert torch.equal(nn.view(torch.int16), nt.view(torch.int16)), name
