"""Benchmark of the dense fp16 NT GEMM C = A @ B.T on one MI355X.

One step = one GEMM over the workload's inputs (the whole hot path: one
kernel launch through the C ABI).  Inputs are seeded synthetic fp16 matrices
(workloads.py), resident in HBM before the timed region starts.

Protocol (after the pages' benchmark: event timing of back-to-back launches
after a 3-second cooldown; page 6, Performance and the Warning after it): one
launch, the cooldown, W untimed warm-up launches, then exactly K launches
between two events on the launch stream, nothing else enqueued between them.
The GPU's clock ramps up over the first ~50 ms of sustained work after idle,
so by default W is sized from one launch's time to fill --warmup-ms (250 ms);
an explicit --warmup is taken as given.  The per-launch time used in the
roofline is the window over K.  As the pages report the median of three fresh
processes, the whole protocol runs in --repeat (3) fresh processes, one after
another; this process only starts them (it touches no GPU) and prints the
line of the median one, with every process's value, and times the CPU
baseline itself.

Prints ONE JSON line.  Fields beyond the common contract:
  roofline      the GEMM kernel against the MI355X dense fp16 MFMA peak
  cpu_baseline  the CPU oracle timed on a bounded block of the same workload
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP16_TFLOPS = 2500.0      # MI355X published dense fp16 MFMA peak
PEAK_HBM_GBS = 8000.0          # MI355X published HBM3E bandwidth
PAGES_H100_TFLOPS = 756.0      # the pages' best kernel at 8192^3 on H100 SXM (context)
SOURCE = os.path.join(ROOT, "dense_fp16_gemm_amd", "csrc", "gemm_f16_nt.hip")


def source_digest(paths=None) -> str:
    """Digest of the kernel sources with comments removed and whitespace
    collapsed: what the recorded HBM traffic belongs to (editing a comment
    does not change it)."""
    import re

    h = hashlib.sha256()
    for path in paths or (SOURCE, os.path.join(ROOT, "dense_fp16_gemm_amd", "csrc", "tile_schedule.h")):
        with open(path, encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update(" ".join(text.split()).encode())   # and layout
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM-side bytes per launch from the committed rocprofv3 counter summary
    (profiles/traffic_<workload>.txt, "key = value" lines), or None when there
    is none or the kernel source has changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if " = " in line:
                key, _, val = line.partition(" = ")
                fields[key.strip()] = val.strip()
    if fields.get("source_digest") != source_digest():
        return None
    try:
        return int(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(w, target_s: float):
    """The oracle, as it is, on a bounded block of the workload: the first
    m_s rows of A against all of B at the full K (a block of C), grown until
    one evaluation takes about target_s seconds."""
    import numpy as np

    import oracle
    import workloads

    threads = oracle.default_threads()
    a, b = workloads.workload_inputs(w.name)
    ns = w.N
    ms = max(1, min(w.M, threads))
    while True:
        t0 = time.perf_counter()
        oracle.gemm(np.ascontiguousarray(a[:ms]), np.ascontiguousarray(b[:ns]), threads=threads)
        dt = time.perf_counter() - t0
        if dt >= 0.5 * target_s or ms >= w.M:
            break
        ms = min(w.M, max(ms + threads, int(ms * min(8.0, 1.2 * target_s / max(dt, 1e-3)))))
    flops = 2.0 * ms * ns * w.K
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"C[0:{ms}, 0:{ns}] of {w.name} at K={w.K} "
                      f"({ms * ns} of {w.M * w.N} outputs), {dt:.1f} s"}


def copy_probe(args) -> int:
    """A plain device-to-device copy of known size, for scaling the
    FETCH_SIZE / WRITE_SIZE counters to bytes."""
    import torch

    n = args.copy_bytes // 2
    src = torch.empty(n, dtype=torch.float16, device="cuda:0").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    launches = (args.warmup or 0) + args.steps
    for _ in range(launches):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": 2 * n, "launches": launches}), flush=True)
    return 0


def power_sampler_loop() -> int:
    """Print `time power_w gfx_clock_mhz` from `amd-smi metric -p -c` every
    0.5 s until stopped.  Runs as its own process, started before the
    measuring process touches the GPU."""
    import re
    import subprocess

    parent = os.getppid()
    while os.getppid() == parent:   # ends with the measuring process
        try:
            out = subprocess.run(["amd-smi", "metric", "-p", "-c"], capture_output=True,
                                 text=True, timeout=10).stdout
        except (OSError, subprocess.SubprocessError):
            return 1
        pw = re.search(r"SOCKET_POWER:\s*([0-9.]+)\s*W", out)
        clk = re.search(r"GFX_0:\s*\n\s*CLK:\s*([0-9.]+)\s*MHz", out)
        if pw and clk:
            print(f"{time.time():.3f} {pw.group(1)} {clk.group(1)}", flush=True)
        time.sleep(0.5)
    return 0


def power_windows(proc, windows):
    """Stop the sampler process and summarise its samples taken in each
    window [t0, t1] of `windows` (None for a window without samples)."""
    proc.terminate()
    try:
        out, _ = proc.communicate(timeout=15)
    except Exception:
        proc.kill()
        out, _ = proc.communicate()
    import statistics

    samples = [tuple(float(x) for x in line.split()) for line in out.splitlines()
               if len(line.split()) == 3]
    res = []
    for t0, t1 in windows:
        pw = [p for t, p, _ in samples if t0 <= t <= t1]
        ck = [c for t, _, c in samples if t0 <= t <= t1]
        if not pw:
            res.append(None)
            continue
        res.append({"samples": len(pw), "socket_power_w_median": statistics.median(pw),
                    "socket_power_w_avg": round(sum(pw) / len(pw), 1),
                    "socket_power_w_min": min(pw), "socket_power_w_max": max(pw),
                    "gfx_clock_mhz_median": statistics.median(ck),
                    "gfx_clock_mhz_avg": round(sum(ck) / len(ck), 1), "gfx_clock_mhz_min": min(ck),
                    "gfx_clock_mhz_max": max(ck), "source": "amd-smi metric -p -c, every 0.5 s"})
    return res


def power_summary(proc, t0: float, t1: float):
    """Stop the sampler process and summarise its samples taken in [t0, t1]."""
    return power_windows(proc, [(t0, t1)])[0]


def mfma_ceiling(args, sampler) -> int:
    """The GEMM's inner loop without memory traffic (libgemm_f16_calib.so):
    16x16x32 fp16 MFMAs fed by LDS fragment reads at one wave per SIMD, 4x4
    and 8x8 result blocks per wave, random and constant operands.  For each,
    --warmup-ms of launches, then a window of --ceiling-ms; prints one JSON
    line with TFLOP/s (and socket power and GFX clock with --power-sample).
    The random-operand rate is what the board's power limit leaves for the
    GEMM's MFMA work; the GEMM's rate over it is the share it attains."""
    import ctypes

    import torch

    from dense_fp16_gemm_amd import build as libbuild

    if not os.path.exists(libbuild.CALIB_PATH):
        print(f"bench.py: {libbuild.CALIB_PATH} is missing (build first)", file=sys.stderr)
        return 1
    lib = ctypes.CDLL(libbuild.CALIB_PATH)
    fn = lib.gemm_f16_calib_mfma_loop
    i32 = ctypes.c_int32
    fn.argtypes = [i32, i32, i32, i32, ctypes.c_void_p, ctypes.c_void_p]
    fn.restype = ctypes.c_int
    dev = torch.device("cuda:0")
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    out_buf = torch.empty(cus * 256, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    rows, windows = [], []
    for fb in (8, 4):
        for constant in (0, 1):
            iters = max(1, int(4000 * 64 / (fb * fb)))   # about 20 ms per launch at 1.5 PF/s
            flops = 2.0 * 16 * 16 * 32 * 8 * fb * fb * iters * 4 * cus

            def launch():
                st = fn(fb, constant, iters, cus, out_buf.data_ptr(), stream.cuda_stream)
                if st != 0:
                    raise RuntimeError(f"gemm_f16_calib_mfma_loop returned {st}")

            e0.record(stream)
            launch()
            e1.record(stream)
            torch.cuda.synchronize()
            one = max(e0.elapsed_time(e1), 1e-3)
            for _ in range(max(1, int(args.warmup_ms / one))):
                launch()
            torch.cuda.synchronize()
            n = max(3, int(args.ceiling_ms / one))
            t0 = time.time()
            e0.record(stream)
            for _ in range(n):
                launch()
            e1.record(stream)
            torch.cuda.synchronize()
            windows.append((t0, time.time()))
            ms = e0.elapsed_time(e1) / n
            rows.append({"blocks_per_wave": f"{fb}x{fb}", "mfma_per_ds_read": fb * fb // (2 * fb),
                         "operands": "constant" if constant else "random",
                         "launches": n, "ms_per_launch": round(ms, 4),
                         "tflops": round(flops / (ms * 1e-3) / 1e12, 1)})
            print(f"bench.py: ceiling {rows[-1]}", file=sys.stderr, flush=True)
    if sampler is not None:
        for r, pw in zip(rows, power_windows(sampler, windows)):
            r["power"] = pw
    print(json.dumps({"calibration": "mfma_ceiling", "unit": "TFLOP/s",
                      "peak": PEAK_FP16_TFLOPS, "cus": cus, "rows": rows}), flush=True)
    return 0


def run_repeats(args) -> int:
    """The protocol in args.repeat fresh processes, one after another; prints
    the median process's line (the middle value; the upper middle for an even
    count) with every value, and the CPU baseline timed here."""
    import subprocess

    import workloads

    cmd = [sys.executable, os.path.abspath(__file__)] + sys.argv[1:] + [
        "--repeat", "1", "--child", "--no-cpu-baseline"]
    lines = []
    for r in range(args.repeat):
        res = subprocess.run(cmd, stdout=subprocess.PIPE, text=True)
        if res.returncode != 0:
            sys.stdout.write(res.stdout)
            return res.returncode
        found = [ln for ln in res.stdout.splitlines() if ln.startswith('{"metric"')]
        if not found:
            print("bench.py: a measuring process printed no result line", file=sys.stderr)
            return 1
        lines.append(json.loads(found[-1]))
        print(f"bench.py: process {r + 1}/{args.repeat}: {lines[-1]['value']} "
              f"{lines[-1]['unit']}", file=sys.stderr, flush=True)
    values = [d["value"] for d in lines]
    out = sorted(lines, key=lambda d: d["value"])[len(lines) // 2]
    out["repeat"] = {"processes": len(lines), "values": values, "median": out["value"],
                     "min": min(values), "max": max(values)}
    name = args.workload or workloads.HEADLINE
    out["cpu_baseline"] = (None if args.no_cpu_baseline else
                           cpu_baseline(workloads.ALL_WORKLOADS[name], args.cpu_seconds))
    print(json.dumps(out), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warm-up launches (default: enough to fill --warmup-ms)")
    ap.add_argument("--warmup-ms", type=float, default=250.0)
    ap.add_argument("--cooldown", type=float, default=3.0)
    ap.add_argument("--workload", default=None, help="workload name (default: the 8192^3 one)")
    ap.add_argument("--config", type=int, default=None, help="force a kernel configuration")
    ap.add_argument("--swizzle", type=int, default=0)
    ap.add_argument("--grid", type=int, default=0)
    ap.add_argument("--epilogue", type=int, default=-1,
                    help="-1: library choice, 0: direct stores, 1: staged through LDS")
    ap.add_argument("--splitk", type=int, default=None,
                    help="time gemm_f16_nt_splitk with this many K splits (0: the library's "
                         "choice); a step is then the split GEMM and its reduction")
    ap.add_argument("--layout", default="nt", choices=("nt", "nn", "tn", "tt"),
                    help="operand layout timed: A [K, M] for tn/tt, B [K, N] for nn/tn "
                         "(transposed before anything is timed; same result bits as nt)")
    ap.add_argument("--nn", action="store_true", help="the same as --layout nn")
    ap.add_argument("--autotune", action="store_true",
                    help="before anything is timed, time every configuration and split count "
                         "of the layout on these operands (gemm_f16_autotune), then time the "
                         "fastest")
    ap.add_argument("--tune-iters", type=int, default=10,
                    help="timed calls per autotuning candidate")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--power-sample", action="store_true",
                    help="sample socket power and the GFX clock with amd-smi every 0.5 s during "
                         "the timed window (give it a window of several seconds via --steps)")
    ap.add_argument("--repeat", type=int, default=3,
                    help="fresh processes, one after another, each running the whole "
                         "protocol; the line is the median one's (1: measure in this process)")
    ap.add_argument("--child", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--power-sampler-loop", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--mfma-ceiling", action="store_true",
                    help="instead of the GEMM, time the GEMM's MFMA + LDS-read inner loop "
                         "without memory traffic, random and constant operands (the power "
                         "ceiling of its MFMA work)")
    ap.add_argument("--ceiling-ms", type=float, default=2000.0,
                    help="timed window per --mfma-ceiling case")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="instead of the GEMM, run a plain device copy of this many bytes "
                         "(calibrates the HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: measures one GPU only (asked for --gpus {args.gpus}); "
              "the GEMM shards into independent output tiles, see the design notes.",
              file=sys.stderr)
        return 2
    if args.power_sampler_loop:
        return power_sampler_loop()
    if args.repeat > 1 and not args.child and args.copy_bytes <= 0 and not args.mfma_ceiling:
        return run_repeats(args)
    sampler = None
    if args.power_sample:
        # its own process, started before this one touches the GPU
        import subprocess

        import atexit

        sampler = subprocess.Popen([sys.executable, os.path.abspath(__file__),
                                    "--power-sampler-loop"], stdout=subprocess.PIPE, text=True)
        atexit.register(sampler.terminate)   # whatever path this process leaves by

    import numpy as np
    import torch

    import dense_fp16_gemm_amd as g
    import workloads

    g.load()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    if args.copy_bytes > 0:
        return copy_probe(args)
    if args.mfma_ceiling:
        return mfma_ceiling(args, sampler)
    name = args.workload or workloads.HEADLINE
    w = workloads.ALL_WORKLOADS[name]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    a_np, b_np = workloads.workload_inputs(name)
    a = torch.from_numpy(a_np).to(dev)
    b = torch.from_numpy(b_np).to(dev)
    c = torch.empty((w.M, w.N), dtype=torch.float16, device=dev)
    del a_np, b_np
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    plan = g.gemm_f16_nt_plan(w.M, w.N, w.K, cus).as_dict()
    if args.config is not None:
        info = g.gemm_f16_nt_config_info(args.config).as_dict()
        plan.update({k: info[k] for k in ("config_id", "block_m", "block_n", "block_k", "waves",
                                          "stages", "lds_bytes")})
    if args.epilogue >= 0:
        plan["epilogue"] = args.epilogue

    stream = torch.cuda.current_stream(dev)

    lay = "nn" if args.nn else args.layout
    if args.autotune and (args.config is not None or args.splitk is not None):
        print("bench.py: --autotune chooses the configuration and split itself", file=sys.stderr)
        return 2
    # operands as the layout stores them, prepared before anything is timed
    xa = a.t().contiguous() if lay[0] == "t" else a
    xb = b.t().contiguous() if lay[1] == "n" else b
    tune = None
    if args.autotune:
        # the search and its workspace come before anything is timed
        code = g.LAYOUT_CODES[lay]
        _, ws_bytes = g.gemm_f16_autotune_candidates(code, w.M, w.N, w.K, cus, True, 0)
        ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
        t0 = time.perf_counter()
        tuned = g.autotune(xa, xb, lay, iters=args.tune_iters, out=c, workspace=ws,
                           stream=stream)
        torch.cuda.synchronize()
        tune = {"config_id": tuned.config, "splits": tuned.splits,
                "tuned_ms": round(tuned.ms, 5), "candidates": len(tuned.entries),
                "search_s": round(time.perf_counter() - t0, 2)}
        plan = g.gemm_f16_nt_config_info(tuned.config).as_dict()
        plan.update({"splits": tuned.splits, "workspace_bytes": ws_bytes})
        split_fn = getattr(g, f"gemm_f16_{lay}_splitk_with_config")

        def launch():
            split_fn(w.M, w.N, w.K, xa.data_ptr(), xb.data_ptr(), c.data_ptr(), tuned.splits,
                     ws.data_ptr(), ws_bytes, stream.cuda_stream, tuned.config)
    elif lay != "nt" and args.splitk is None:
        plan = getattr(g, f"gemm_f16_{lay}_plan")(w.M, w.N, w.K, cus).as_dict()
        if args.config is not None:
            info = g.gemm_f16_nt_config_info(args.config).as_dict()
            plan.update({k: info[k] for k in ("config_id", "block_m", "block_n", "block_k",
                                              "waves", "stages", "lds_bytes", "a_layout",
                                              "b_layout")})

        def launch():
            g.gemm(xa, xb, lay, out=c, config=args.config, swizzle=args.swizzle, grid=args.grid,
                   stream=stream, epilogue=args.epilogue)
    elif args.splitk is not None:
        # the workspace is allocated once, before anything is timed
        sk_plan, splits, ws_bytes = getattr(g, f"gemm_f16_{lay}_splitk_plan")(
            w.M, w.N, w.K, cus, args.splitk)
        plan = sk_plan.as_dict()
        plan.update({"splits": splits, "workspace_bytes": ws_bytes})
        ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
        split_fn = getattr(g, f"gemm_f16_{lay}_splitk_with_config")

        def launch():
            split_fn(w.M, w.N, w.K, xa.data_ptr(), xb.data_ptr(), c.data_ptr(), args.splitk,
                     ws.data_ptr(), ws_bytes, stream.cuda_stream,
                     -1 if args.config is None else args.config)
    else:
        def launch():
            g.gemm_nt(a, b, out=c, config=args.config, swizzle=args.swizzle, grid=args.grid,
                      stream=stream, epilogue=args.epilogue)

    # cooldown first (the pages' protocol), then the warm-up launches bring
    # the clock back up from idle before the timed window opens
    launch()
    torch.cuda.synchronize()
    if args.cooldown > 0:
        time.sleep(args.cooldown)
    win0 = torch.cuda.Event(enable_timing=True)
    win1 = torch.cuda.Event(enable_timing=True)
    warmup = args.warmup
    if warmup is None:
        # one (cold) launch sizes the warm-up; it is a warm-up launch itself
        win0.record(stream)
        launch()
        win1.record(stream)
        torch.cuda.synchronize()
        cold_ms = max(win0.elapsed_time(win1), 1e-3)
        warmup = 1 + min(max(int(args.warmup_ms / cold_ms), 20), 20000)
        todo = warmup - 1
    else:
        todo = warmup
    for _ in range(todo):
        launch()
    torch.cuda.synchronize()

    # timed region: exactly `steps` launches, back to back
    t_start = time.time()
    win0.record(stream)
    for _ in range(args.steps):
        launch()
    win1.record(stream)
    torch.cuda.synchronize()
    power = power_summary(sampler, t_start, time.time()) if sampler is not None else None
    ms_per_step = win0.elapsed_time(win1) / args.steps
    kernel_avg_ms = ms_per_step

    tflops = w.flops / (ms_per_step * 1e-3) / 1e12
    compute_bound = w.flops / w.algorithmic_bytes > (PEAK_FP16_TFLOPS * 1e12) / (PEAK_HBM_GBS * 1e9)
    traffic = measured_traffic(name + ("" if lay == "nt" else "_" + lay) +
                               ("_splitk" if args.splitk is not None else "") +
                               ("_autotune" if args.autotune else ""))
    if compute_bound:
        achieved = w.flops / (kernel_avg_ms * 1e-3) / 1e12
        roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_FP16_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP16_TFLOPS, 4),
                    "traffic": traffic}
    else:
        achieved = w.algorithmic_bytes / (kernel_avg_ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                    "traffic": traffic}

    out = {
        "metric": "TFLOP/s and % of fp16 MFMA peak, fp16 NT GEMM M=N=K=8192, 1 GPU",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        # no published MI355X figure exists for this metric; the pages' H100
        # number is context only (below), never the baseline
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": name, "M": w.M, "N": w.N, "K": w.K, "layout": lay,
                   "inputs": w.note,
                   "seed": w.seed, "accumulate": "f32", "plan": plan,
                   "autotune": tune,
                   "power": power,
                   "kernel_ms_avg": round(kernel_avg_ms, 5),
                   # the pages' best kernel at 8192^3 ran on other hardware
                   # (H100 SXM): the ratio is context, not a target
                   "context_pages_h100": (
                       {"tflops": PAGES_H100_TFLOPS, "ratio": round(tflops / PAGES_H100_TFLOPS, 3)}
                       if name == workloads.HEADLINE and lay == "nt" and args.splitk is None
                       and not args.autotune else None),
                   "source_digest": source_digest()},
        "roofline": roofline,
        "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline(w, args.cpu_seconds),
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
