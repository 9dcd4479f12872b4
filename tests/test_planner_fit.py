"""The split-K planner's constants are the output of the committed fit.

dense_fp16_gemm_amd/planner_fit/fit_split_model.py fits the cost model of
split_cost to the committed autotuner tables (host only).  Its constants and
per-configuration rates must be the ones the library's source carries, so
the planner stays reproducible from the repository.
"""
import io
import os
import re
import sys
from contextlib import redirect_stdout

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FIT_DIR = os.path.join(ROOT, "dense_fp16_gemm_amd", "planner_fit")
SOURCE = os.path.join(ROOT, "dense_fp16_gemm_amd", "csrc", "gemm_f16_nt.hip")


def _source_constants():
    src = open(SOURCE).read()
    # the definition: the last occurrence (a declaration may precede it)
    body = src[src.rindex("static double split_cost("):]
    consts = {k: float(v) for k, v in re.findall(r"(k[A-Za-z]+) = ([0-9.e+-]+);", body[:2000])}
    tab = src[src.index("static const KernelEntry kKernels[] = {"):]
    tab = tab[:tab.index("};")]
    rates = [float(m.group(1)) for m in
             re.finditer(r"entry(?:_pc)?<Cfg<[^>]*>>\(\d+, [0-9.]+f, ([0-9.]+)f\)", tab)]
    return consts, rates


def test_fit_reproduces_the_source_constants():
    sys.path.insert(0, FIT_DIR)
    try:
        import fit_split_model
    finally:
        sys.path.pop(0)
    buf = io.StringIO()
    with redirect_stdout(buf):
        fit_split_model.main()
    out = buf.getvalue()
    fitted = {k: float(v) for k, v in re.findall(r"(k[A-Za-z]+) = ([0-9.e+-]+)", out)}
    consts, rates = _source_constants()
    for key in ("kUnitSec", "kLaunchSec", "kHbmBytesPerSec", "kActiveExp", "kReduceBytesPerSec",
                "kReduceSec"):
        assert abs(fitted[key] / consts[key] - 1) < 0.01, (key, fitted[key], consts[key])
    fitted_rates = [float(v) for v in re.findall(r"^\s+\d+\s+\S+\s+([0-9.]+)$", out, flags=re.M)]
    # configurations 0..42 (every direct-to-LDS configuration; the general
    # kernels are never split)
    assert len(fitted_rates) == 43
    for cid, (f, s) in enumerate(zip(fitted_rates, rates)):
        assert abs(f - s) <= 0.0015, (cid, f, s)
