"""Fit of the split-K planner's cost model (split_cost in csrc/gemm_f16_nt.hip)
to measured times.  Host only: reads the kernel table from the source and
the measurements in autotune_tables.jsonl, runs no GPU code.

autotune_tables.jsonl: one MI355X (256 CUs), every configuration x split
count that gemm_f16_autotune tried on 28 shapes per operand layout (under-
filled grids, long and short K): one record per shape, entries
[config_id, splits, status, ms].  Configurations 0..42 (every direct-to-LDS
configuration, the producer/consumer one included) are fitted here; the
general kernels are never split.

The model (times in seconds, per launch):
  compute  = rounds x (unit flops / (rate_c x CU peak) + f1)
  operands = (M + N) K 2 / (bh x busy^a),  busy = min(units, CUs) / CUs
  t        = max(compute, operands) + 0.1 min(compute, operands) + f0 + 2 M N / bh
             + [split] (2 s M N 4 + 2 M N) / br + f2
with one rate per configuration and f0, f1, bh, br, f2, a shared.  The fit
minimises the squared log error.  Its output is the constants in split_cost
(kUnitSec = f1, kLaunchSec = f0, kHbmBytesPerSec = bh, kActiveExp = a,
kReduceBytesPerSec = br, kReduceSec = f2) and each configuration's
split_rate in the kernel table.

usage: python3 fit_split_model.py
"""
from __future__ import annotations

import json
import math
import os
import re

import numpy as np
from scipy.optimize import least_squares

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(os.path.dirname(HERE), "csrc", "gemm_f16_nt.hip")
TABLES = os.path.join(HERE, "autotune_tables.jsonl")
CU_PEAK = 2.5e15 / 256   # dense fp16 flop/s of one CU
OVERLAP = 0.1


def kernel_table():
    """(block_m, block_n, block_k) of every entry of kKernels, in id order."""
    src = open(SOURCE).read()
    tab = src[src.index("static const KernelEntry kKernels[] = {"):]
    tab = tab[:tab.index("};")]
    out = []
    for m in re.finditer(r"entry(?:_general|_pc)?<Cfg<([^>]*)>", tab):
        a = [int(x) for x in m.group(1).split(",")]
        out.append((a[0], a[1], a[2]))
    return out


def cdiv(a, b):
    return -(-a // b)


def split_len(bk, k, s):
    return cdiv(cdiv(k, s), bk) * bk


def load_rows(cfgs, max_id=43):
    recs = [json.loads(line) for line in open(TABLES)]
    rows = []
    for ri, r in enumerate(recs):
        m, n, k = r["shape"]
        for cid, s, status, ms in r["entries"]:
            if ms <= 0 or cid >= max_id:
                continue
            bm, bn, bk = cfgs[cid]
            ks = split_len(bk, k, s) if s > 1 else k
            units = cdiv(m, bm) * cdiv(n, bn) * s
            rows.append(dict(ri=ri, cid=cid, s=s, R=cdiv(units, r["cus"]), F=bm * bn * ks * 2.0,
                             HB=(m + n) * k * 2.0, CB=m * n * 2.0,
                             RB=(2 * s * m * n * 4.0 + m * n * 2.0) if s > 1 else 0.0,
                             T=ms * 1e-3, act=min(units, r["cus"]) / r["cus"]))
    return recs, rows


def main():
    cfgs = kernel_table()
    recs, rows = load_rows(cfgs)
    ids = sorted({x["cid"] for x in rows})
    idx = {c: i for i, c in enumerate(ids)}
    A = {key: np.array([x[key] for x in rows]) for key in rows[0]}
    ci = np.array([idx[x["cid"]] for x in rows])
    npar = len(ids)

    def model(p):
        rates = np.exp(p[:npar])
        f0, f1, bh, br, f2 = np.exp(p[npar:npar + 5])
        a = p[npar + 5]
        comp = A["R"] * A["F"] / (rates[ci] * CU_PEAK) + A["R"] * f1
        hbm = A["HB"] / (bh * A["act"] ** a)
        t = np.maximum(comp, hbm) + OVERLAP * np.minimum(comp, hbm) + f0 + A["CB"] / bh
        return t + np.where(A["s"] > 1, A["RB"] / br + f2, 0.0)

    p0 = np.concatenate([np.log(np.full(npar, 0.5)), np.log([3e-6, 1e-6, 4e12, 4e12, 3e-6]), [0.3]])
    p = least_squares(lambda q: np.log(model(q)) - np.log(A["T"]), p0).x
    f0, f1, bh, br, f2 = np.exp(p[npar:npar + 5])
    rms = float(np.sqrt(np.mean((np.log(model(p)) - np.log(A["T"])) ** 2)))
    print(f"{len(recs)} shapes, {len(rows)} timings, rms log error {rms:.4f}")
    print(f"kUnitSec = {f1:.3g}  kLaunchSec = {f0:.3g}  kHbmBytesPerSec = {bh:.3g}  "
          f"kActiveExp = {p[npar + 5]:.3f}  kReduceBytesPerSec = {br:.3g}  kReduceSec = {f2:.3g}")
    print("split_rate per configuration:")
    for c, v in zip(ids, np.exp(p[:npar])):
        print(f"  {c:2d}  {cfgs[c][0]}x{cfgs[c][1]}x{cfgs[c][2]}  {v:.3f}")
    # how the model's pick compares with the best measured entry, per shape
    pred = model(p)
    worst, logs = 0.0, []
    for ri in range(len(recs)):
        sel = [i for i, x in enumerate(rows) if x["ri"] == ri]
        if not sel:
            continue
        best = min(A["T"][i] for i in sel)
        pick = sel[int(np.argmin(pred[sel]))]
        ratio = A["T"][pick] / best
        logs.append(math.log(ratio))
        worst = max(worst, ratio)
    print(f"model's pick over the best measured time: geometric mean {math.exp(np.mean(logs)):.3f}, "
          f"worst {worst:.3f} (over every timed entry; the library also weighs the plain plan)")


if __name__ == "__main__":
    main()
