"""Operands of more than 2^31 bytes.  The fast kernels address each tile
from a 64-bit base with 32-bit offsets inside it, and an operand stored
k-outermost runs them only while K X 2 stays below 2^31; beyond that the
layout's general kernel takes it with 64-bit addressing.  Integer inputs, so
a block of C at the matrix edges, at tile boundaries and around the 2^31-byte
mark must equal the oracle bit for bit."""
import sys

import numpy as np
import pytest

import workloads
from parity import assert_bit_exact

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def g():
    import torch

    import dense_fp16_gemm_amd as lib

    lib.load()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return lib


def _picks(n, extra, seed):
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 255, 256, n // 2, n - 257, n - 256, n - 2, n - 1] + list(extra)
    return np.unique(np.clip(np.concatenate([fixed, rng.integers(0, n, 16)]), 0, n - 1))


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


def test_nt_a_beyond_2gb(g, oracle_mod):
    import torch

    m, n, k = 135168, 256, 8192                    # A: 2.2 GB
    a = workloads.int2_matrix((m, k), 371)
    b = workloads.int2_matrix((n, k), 372)
    assert a.nbytes > 2 ** 31
    rows = _picks(m, [2 ** 31 // (2 * k) - 1, 2 ** 31 // (2 * k)], 373)   # rows around 2^31 bytes
    cols = _picks(n, [], 374)
    _say(f"  gpu large nt {m}x{n}x{k} config {g.gemm_f16_nt_plan(m, n, k, 256).config_id}")
    c = g.gemm_nt(torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda())
    torch.cuda.synchronize()
    got = c[torch.from_numpy(rows).cuda()][:, torch.from_numpy(cols).cuda()].cpu().numpy()
    assert_bit_exact(got, oracle_mod.gemm(a[rows], b[cols]), "nt, A beyond 2^31 bytes")


@pytest.mark.parametrize("n,general", [(131064, False), (135168, True)])
def test_nn_b_at_and_beyond_the_fast_limit(g, oracle_mod, n, general):
    """B stored [K, N]: K N 2 just below 2^31 (direct-to-LDS) and above it
    (the general kernel)."""
    import torch

    m, k = 256, 8192
    a = workloads.int2_matrix((m, k), 375)
    b_kn = workloads.int2_matrix((k, n), 376)
    plan = g.gemm_f16_nn_plan(m, n, k, 256)
    assert bool(g.gemm_f16_nt_config_info(plan.config_id).block_k == 32) == general
    rows = _picks(m, [], 377)
    cols = _picks(n, [2 ** 30 // k - 1, 2 ** 30 // k], 378)
    _say(f"  gpu large nn {m}x{n}x{k} config {plan.config_id}")
    c = g.gemm(torch.from_numpy(a).cuda(), torch.from_numpy(b_kn).cuda(), "nn")
    torch.cuda.synchronize()
    got = c[torch.from_numpy(rows).cuda()][:, torch.from_numpy(cols).cuda()].cpu().numpy()
    ref = oracle_mod.gemm(a[rows], np.ascontiguousarray(b_kn[:, cols].T))
    assert_bit_exact(got, ref, f"nn, B [K, N] of {b_kn.nbytes} bytes")


def test_tn_a_beyond_the_fast_limit(g, oracle_mod):
    """A stored [K, M] above 2^31 bytes: TN's general kernel."""
    import torch

    m, n, k = 135168, 256, 8192
    a_km = workloads.int2_matrix((k, m), 379)
    b_kn = workloads.int2_matrix((k, n), 380)
    plan = g.gemm_f16_tn_plan(m, n, k, 256)
    assert g.gemm_f16_nt_config_info(plan.config_id).block_k == 32, "general kernel"
    rows = _picks(m, [2 ** 30 // k - 1, 2 ** 30 // k], 381)
    cols = _picks(n, [], 382)
    _say(f"  gpu large tn {m}x{n}x{k} config {plan.config_id}")
    c = g.gemm(torch.from_numpy(a_km).cuda(), torch.from_numpy(b_kn).cuda(), "tn")
    torch.cuda.synchronize()
    got = c[torch.from_numpy(rows).cuda()][:, torch.from_numpy(cols).cuda()].cpu().numpy()
    ref = oracle_mod.gemm(np.ascontiguousarray(a_km[:, rows].T), np.ascontiguousarray(b_kn[:, cols].T))
    assert_bit_exact(got, ref, "tn, A [K, M] beyond 2^31 bytes")
