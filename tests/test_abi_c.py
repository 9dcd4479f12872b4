"""The boundary from plain C: tests/abi_c_check.c includes only
include/gemm_f16_nt.h, is compiled as C99 with gcc and linked against
libgemm_f16.so, and calls the pure host entry points (no GPU).  Its output
must equal what the Python binding returns for the same calls."""
import os
import shutil
import subprocess

import pytest

import dense_fp16_gemm_amd as g

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SHAPES = [(8192, 8192, 8192), (4999, 7001, 4160), (128, 16384, 16384), (1024, 1024, 65536),
          (256, 256, 256)]


@pytest.fixture(scope="module")
def c_output(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    g.load()
    libdir = os.path.dirname(g.library_path())
    exe = str(tmp_path_factory.mktemp("abi_c") / "abi_c_check")
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror=implicit-function-declaration",
           "-D__HIP_PLATFORM_AMD__", f"-I{ROOT}/include", "-I/opt/rocm/include",
           os.path.join(ROOT, "tests", "abi_c_check.c"), f"-L{libdir}", "-lgemm_f16",
           f"-Wl,-rpath,{libdir}", "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    run = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0, (run.returncode, run.stdout, run.stderr)
    out = {}
    for line in run.stdout.splitlines():
        key, _, rest = line.partition(" ")
        out.setdefault(key, []).append(rest)
    return out


def test_c_program_sees_the_same_library(c_output):
    assert c_output["configs"] == [str(g.gemm_f16_nt_num_configs())]
    assert c_output["status"] == [f"{g.status_string(0)}|{g.status_string(2)}"]
    assert c_output["validate"] == [f"{g.OK} {g.INVALID_ARG}"]


def test_c_program_plans_match_the_binding(c_output):
    for i, (m, n, k) in enumerate(SHAPES):
        p = g.gemm_f16_nt_plan(m, n, k, 256)
        tm, tn = g.gemm_f16_nt_tile_of_slot(p, p.tiles - 1)
        assert c_output["plan"][i] == f"{m} {p.config_id} {p.block_m} {p.block_n} {p.tiles} {tm} {tn}"
        sp, splits, ws = g.gemm_f16_nt_splitk_plan(m, n, k, 256, 0)
        assert c_output["split"][i] == f"{m} {sp.config_id} {splits} {ws}"
        assert c_output["tt"][i] == f"{m} {g.gemm_f16_tt_plan(m, n, k, 256).config_id}"
        cand, need = g.gemm_f16_autotune_candidates(0, m, n, k, 256, True, 1 << 40)
        assert c_output["tune"][i] == f"{m} {len(cand)} {need}"
        assert c_output["bound"][i] == f"{m} {g.gemm_f16_splitk_workspace_bytes(m, n, 8)}"
