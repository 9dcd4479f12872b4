"""Both entry points under HIP graph capture.

Callers in serving loops capture the GEMM into a graph and replay it.  The
library issues only kernel launches on the caller's stream (no allocation, no
memset, no host synchronisation), so a captured call must give on every replay
exactly what the eager call gives.  Each test replays several times with eager
work and synchronisations in between and checks every replay bit for bit.
"""
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


def _inputs(m, n, k, seed):
    import torch

    a, b = workloads.make_inputs(m, n, k, "normal", 1.0 / np.sqrt(k), seed=seed)
    return torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda()


@pytest.mark.parametrize("shape", [(300, 260, 200), (1024, 768, 2048), (77, 129, 64)])
def test_graph_replay_plain(g, shape):
    import torch

    m, n, k = shape
    a, b = _inputs(m, n, k, 401)
    eager = g.gemm_nt(a, b)
    torch.cuda.synchronize()
    ref = eager.cpu().numpy()
    out = torch.full((m, n), float("nan"), dtype=torch.float16, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        g.gemm_nt(a, b, out=out, stream=s)          # warm the stream outside capture
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=s):
            g.gemm_nt(a, b, out=out, stream=s)
    for rep in range(4):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert_bit_exact(out.cpu().numpy(), ref, f"replay {rep}")
        g.gemm_nt(b[:, :k], a)                       # unrelated eager work in between
        torch.cuda.synchronize()


def test_graph_replay_splitk(g):
    import torch

    m, n, k = 256, 256, 16384
    a, b = _inputs(m, n, k, 402)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    _, splits, need = g.gemm_f16_nt_splitk_plan(m, n, k, cus)
    assert splits > 1
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    eager = g.gemm_nt_splitk(a, b, workspace=ws)
    torch.cuda.synchronize()
    ref = eager.cpu().numpy()
    out = torch.full((m, n), float("nan"), dtype=torch.float16, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        g.gemm_nt_splitk(a, b, out=out, workspace=ws, stream=s)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=s):
            g.gemm_nt_splitk(a, b, out=out, workspace=ws, stream=s)
    for rep in range(4):
        out.fill_(float("nan"))
        ws.fill_(0xFF)                               # the partials must be rewritten each replay
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert_bit_exact(out.cpu().numpy(), ref, f"split-K replay {rep}")
        g.gemm_nt(a[:, :64].contiguous(), b[:, :64].contiguous())
        torch.cuda.synchronize()
