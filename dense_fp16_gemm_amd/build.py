"""Build libgemm_f16.so (the HIP kernels + C ABI) in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import shutil
import subprocess

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
SOURCES = [os.path.join(PKG_DIR, "csrc", "gemm_f16_nt.hip")]
HEADERS = [os.path.join(PKG_DIR, "csrc", "tile_schedule.h"),
           os.path.join(ROOT, "include", "gemm_f16_nt.h")]
LIB_PATH = os.path.join(PKG_DIR, "libgemm_f16.so")
# the benchmark's calibration kernel (not part of the GEMM library)
CALIB_SOURCES = [os.path.join(PKG_DIR, "csrc", "mfma_ceiling.hip")]
CALIB_PATH = os.path.join(PKG_DIR, "libgemm_f16_calib.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libgemm_f16.so)")


def compile_command(out: str, sources=None) -> list[str]:
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            # packed fp32 VALU ops stay off (only the device pass knows the feature)
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # the MFMA step loops must unroll fully: accumulators are indexed
            # by the loop counters, and a rolled loop would demote them to
            # scratch memory
            "-mllvm", "-pragma-unroll-threshold=1000000",
            "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG_DIR, "csrc"),
            "-o", out] + (SOURCES if sources is None else sources)


def _compile(path: str, sources, verbose: bool) -> str:
    tmp = path + ".tmp%d" % os.getpid()
    cmd = compile_command(tmp, sources)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in line and "argument unused" not in line)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)
    os.replace(tmp, path)
    return path


def build(verbose: bool = False) -> str:
    """Compile unconditionally and atomically replace the in-tree libraries:
    the GEMM library and the benchmark's calibration kernel."""
    _compile(CALIB_PATH, CALIB_SOURCES, verbose)
    return _compile(LIB_PATH, SOURCES, verbose)


if __name__ == "__main__":
    print(build(verbose=True))
