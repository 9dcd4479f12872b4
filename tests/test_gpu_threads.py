"""Entry points called from several host threads at once, each thread on its
own stream (default priority), mixing layouts, shapes and the split over K
(each thread with its own workspace).  The library's only shared state is the
per-device property cache; every result must still equal the oracle bit for
bit (integer inputs)."""
import sys
import threading

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


def test_concurrent_calls_from_threads(g, oracle_mod):
    import torch

    cases = []
    for t in range(4):
        lay = ["nt", "nn", "tn", "tt"][t]
        for idx, (m, n, k) in enumerate([(200, 304, 6152), (512, 392, 1032), (64, 640, 8200)]):
            a_mk, b_nk = workloads.make_inputs(m, n, k, "int2", 1.0, seed=500 + 10 * t + idx)
            a = np.ascontiguousarray(a_mk.T) if lay[0] == "t" else a_mk
            b = np.ascontiguousarray(b_nk.T) if lay[1] == "n" else b_nk
            cases.append((t, lay, idx % 2 == 1, torch.from_numpy(a).cuda(),
                          torch.from_numpy(b).cuda(), oracle_mod.gemm(a_mk, b_nk)))
    torch.cuda.synchronize()
    results, errors = {}, []

    def worker(t):
        try:
            stream = torch.cuda.Stream()
            with torch.cuda.stream(stream):
                for rep in range(5):
                    for ci, (tt, lay, split, ta, tb, _) in enumerate(cases):
                        if tt != t:
                            continue
                        if split:
                            out = g.gemm_splitk(ta, tb, lay, splits=3, stream=stream)
                        else:
                            out = g.gemm(ta, tb, lay, stream=stream)
                        results[(ci, rep)] = out
            stream.synchronize()
        except Exception as e:   # reported in the main thread
            errors.append(repr(e))

    print("  gpu threads: 4 threads x 3 shapes x 5 repeats", file=sys.stderr, flush=True)
    threads = [threading.Thread(target=worker, args=(t,)) for t in range(4)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not any(th.is_alive() for th in threads), "a worker did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    assert len(results) == len(cases) * 5
    for (ci, rep), out in results.items():
        _, lay, split, _, _, ref = cases[ci]
        assert_bit_exact(out.cpu().numpy(), ref, f"thread case {ci} {lay} split={split} rep {rep}")
