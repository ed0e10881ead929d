#!/usr/bin/env python3
"""Benchmark of the QuIP-family layer-quantization pass on one MI355X.

A step is one whole pass over one synthetic layer with everything resident in
HBM when the timed region starts: proxy Hessian + damping, two-sided random
Hadamard transform of H and of W, LDL, per-row scale search, LDLQ, inverse
transforms and the proxy loss. The workload is the 4096 x 4096 attention
projection layer (2-bit grid, RHT on both sides, lazy block 128, 4096
calibration rows); the metric is quantized weights per second.

Also reported: per-phase times (HIP events on the pass's stream), the RHT
bandwidth per one-sided pass, the roofline of the dominant kernel (the fp32
matrix-core Hessian contraction, one launch per step, bracketed by its own
events), HBM traffic from rocprofv3 counters when a counter summary is
present under profiles/, and the CPU oracle timed on a bounded sample.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
FP32_MFMA_PEAK_TFLOPS = 157.3


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="c2")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=4096, help="rows of W in the oracle LDLQ sample")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="end with one plain device copy of COPY_MIB MiB (counter calibration)")
    # summaries of rocprofv3 result databases (host only, no GPU)
    ap.add_argument("--summarize-trace", metavar="DB")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DB", "WRITE_DB"))
    ap.add_argument("--kernel", default=DOMINANT_KERNEL)
    ap.add_argument("--command", default="")
    ap.add_argument("--out")
    return ap.parse_args()


DOMINANT_KERNEL = "gemm_kernel<128, 128, true, false, 0>"  # the Hessian contraction
COPY_MIB = 256
COPY_KERNEL = "MulFunctor"  # torch.mul(src, 1.0, out=dst): reads and writes COPY_MIB MiB


def _kernel_rows(db):
    import re
    import sqlite3

    con = sqlite3.connect(db)
    out = []
    for name, start, end in con.execute("select name, start, end from kernels"):
        nm = name.replace("(anonymous namespace)::", "").replace("void ", "")
        nm = re.sub(r"\(.*", "", nm)
        out.append((nm, (end - start) / 1e3))
    return out


def summarize_trace(db, command, out):
    rows = _kernel_rows(db)
    agg = {}
    for nm, d in rows:
        a = agg.setdefault(nm, [0.0, 0])
        a[0] += d
        a[1] += 1
    tot = sum(v[0] for v in agg.values())
    lines = ["# rocprofv3 kernel trace: quantization pass, 4096 x 4096 layer (2-bit, RHT, B = 128)", "",
             f"Command: `{command}`", "",
             "| kernel | calls | total us | avg us | % |", "|---|---:|---:|---:|---:|"]
    for k, (t, c) in sorted(agg.items(), key=lambda kv: -kv[1][0]):
        lines.append(f"| `{k}` | {c} | {t:.1f} | {t / c:.2f} | {100 * t / tot:.1f} |")
    text = "\n".join(lines) + "\n"
    if out:
        with open(out, "w") as f:
            f.write(text)
    print(text)


def _counter(db, counter):
    import re
    import sqlite3

    con = sqlite3.connect(db)
    per = {}
    for name, value in con.execute(
            "select kernel_name, value from counters_collection where counter_name = ?", (counter,)):
        nm = name.replace("(anonymous namespace)::", "").replace("void ", "")
        nm = re.sub(r"\(.*", "", nm)
        per.setdefault(nm, []).append(float(value))
    return per


def summarize_counters(fetch_db, write_db, kernel, command, out):
    """HBM bytes per launch of `kernel` from FETCH_SIZE / WRITE_SIZE (KiB per
    dispatch), each scaled by what the counter reads for a plain copy of
    COPY_MIB MiB (read and written once)."""
    import hashlib

    fetch = _counter(fetch_db, "FETCH_SIZE")
    write = _counter(write_db, "WRITE_SIZE")

    def pick(per, key):
        hits = [v for k, v in per.items() if key in k]
        if not hits:
            raise SystemExit(f"no dispatch of {key} in the counter database")
        vals = max(hits, key=len)
        return float(np.mean(vals)), len(vals)

    kf, nf = pick(fetch, kernel)
    kw, nw = pick(write, kernel)
    cf, _ = pick(fetch, COPY_KERNEL)
    cw, _ = pick(write, COPY_KERNEL)
    nbytes = COPY_MIB * 2 ** 20
    f_read = nbytes / (cf * 1024.0)
    f_write = nbytes / (cw * 1024.0)
    rd = kf * 1024.0 * f_read
    wr = kw * 1024.0 * f_write
    src = os.path.join(ROOT, "post_weight_quantization_quip_amd", "csrc", "gemm.hip")
    with open(src, "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()[:16]
    d = {"kernel_prefix": "gemm_kernel", "kernel": kernel, "source_sha": sha,
         "fetch_kib_per_dispatch": kf, "write_kib_per_dispatch": kw, "dispatches": [nf, nw],
         "copy_fetch_kib": cf, "copy_write_kib": cw, "copy_bytes_each_way": nbytes,
         "scale_read": f_read, "scale_write": f_write,
         "read_bytes_per_launch": rd, "write_bytes_per_launch": wr,
         "bytes_per_launch": rd + wr, "command": command}
    text = json.dumps(d, indent=1)
    if out:
        with open(out, "w") as f:
            f.write(text + "\n")
    print(text)


def traffic_from_profiles(kernel_prefix: str):
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary (profiles/hessian_syrk_c2_counters.json), or None."""
    path = os.path.join(ROOT, "profiles", "hessian_syrk_c2_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_prefix") != kernel_prefix or d.get("source_sha") is None:
        return None
    src = os.path.join(ROOT, "post_weight_quantization_quip_amd", "csrc", "gemm.hip")
    import hashlib
    with open(src, "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()[:16]
    if sha != d["source_sha"]:
        return None  # the kernel changed since the counters were taken
    return d.get("bytes_per_launch")


def cpu_baseline(cfg_name: str, rows: int) -> dict:
    """The oracle as it stands, on the host cores: the Hessian, incoherence and
    LDL of the full layer, the scale search and LDLQ on `rows` rows of W~
    (rows are independent given U, D and the scales), extrapolated linearly to
    all rows."""
    import oracle as O
    import workloads as wl

    L = wl.make_layer(cfg_name)
    cfg = L.cfg
    t = {}
    t0 = time.perf_counter()
    H = O.damp(O.proxy_hessian(L.X), cfg.alpha)
    t["hessian"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    Ht = O.incoherence_H(H, L.right)
    t["incoherence_H"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    Wt = O.incoherence_W(L.W, L.left, L.right)
    t["incoherence_W"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    U, D = O.udu_cholesky(Ht)
    t["ldl"] = time.perf_counter() - t0
    sel = np.random.default_rng(0).choice(cfg.m, size=min(rows, cfg.m), replace=False)
    Ws = Wt[np.sort(sel)]
    Lv = 1 << cfg.bits
    t0 = time.perf_counter()
    s, _, _ = O.uniform_scale_search(Ws, Lv)
    t_scale = time.perf_counter() - t0
    t0 = time.perf_counter()
    _, What_s = O.ldlq(Ws, U, O.uniform_quantizer(s, Lv))
    t_ldlq = time.perf_counter() - t0
    frac = cfg.m / len(sel)
    t["scale"] = t_scale * frac
    t["ldlq"] = t_ldlq * frac
    total = sum(t.values())
    try:
        threads = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        threads = os.cpu_count()
    return {
        "value": cfg.m * cfg.n / total,
        "unit": "weights/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"{cfg_name}: Hessian, incoherence and LDL on the full layer; scale search and "
                   f"LDLQ on {len(sel)} of {cfg.m} rows, extrapolated x{frac:.0f} (rows are "
                   f"independent given U and the scales); float64 numpy"),
        "seconds": {k: round(v, 4) for k, v in t.items()},
        "measured_seconds": round(t["hessian"] + t["incoherence_H"] + t["incoherence_W"] + t["ldl"]
                                  + t_scale + t_ldlq, 3),
    }


def main():
    args = parse()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.command, args.out)
        return
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters, args.kernel, args.command, args.out)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the pass is single-GPU here; see DESIGN.md for how it would shard)", file=sys.stderr)
        sys.exit(2)

    import torch

    import post_weight_quantization_quip_amd as Q
    import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = "cuda"
    L = wl.make_layer(args.config)
    cfg = L.cfg
    W = torch.from_numpy(L.W).to(dev)
    X = torch.from_numpy(L.X).to(dev)
    left = Q.SideSpec.from_numpy(L.left, dev)
    right = Q.SideSpec.from_numpy(L.right, dev)
    lp = Q.LayerPass(cfg.m, cfg.n, left, right, quant=cfg.quant, bits=cfg.bits, B=cfg.B, g=cfg.g,
                     alpha=cfg.alpha, device=dev)
    stream = torch.cuda.current_stream()

    for _ in range(args.warmup):
        lp.run(W, X)
    torch.cuda.synchronize()
    info = int(lp.buffers["info"].item())
    if info:
        print(f"LDL failed at pivot {info - 1}", file=sys.stderr)
        sys.exit(1)

    events = {}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        lp.run(W, X, events=events)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps

    order = ["hessian", "incoherence_H", "incoherence_W", "ldl", "ldlq", "postprocess", "loss", "end"]
    phases = {}
    for a, b in zip(order[:-1], order[1:]):
        phases[a] = float(np.mean([ea.elapsed_time(eb) for ea, eb in zip(events[a], events[b])]))
    phases["step_events"] = float(np.mean([ea.elapsed_time(eb) for ea, eb in
                                           zip(events["hessian"], events["end"])]))
    mn = cfg.m * cfg.n
    value = mn / (ms_per_step / 1e3)
    from_resident = (phases["incoherence_H"] + phases["incoherence_W"] + phases["ldl"]
                     + phases["ldlq"])

    # dominant kernel: the Hessian contraction (one launch per step, events around it)
    syrk_ms = phases["hessian"]
    hs = []
    for _ in range(args.steps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        Q.quip_hessian(X, lp.buffers["H"])
        e1.record(stream)
        hs.append((e0, e1))
    torch.cuda.synchronize()
    syrk_ms = float(np.mean([a.elapsed_time(b) for a, b in hs]))
    syrk_flops = cfg.N * cfg.n * (cfg.n + 1)
    achieved = syrk_flops / (syrk_ms / 1e3) / 1e12
    traffic = traffic_from_profiles("gemm_kernel")
    if traffic is not None:
        traffic = round(traffic / 1e6, 1)  # MB per launch
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": FP32_MFMA_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / FP32_MFMA_PEAK_TFLOPS, 4),
                "traffic": traffic, "traffic_unit": "MB per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                "kernel": "gemm_kernel<128,128,transA,!transB> (Hessian X^T X)",
                "algorithmic_flops_per_launch": syrk_flops, "avg_launch_ms": round(syrk_ms, 4)}

    # RHT bandwidth per one-sided pass (W, 4096 x 4096)
    def timed(fn, reps):
        es = []
        for _ in range(reps):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            es.append((a, b))
        torch.cuda.synchronize()
        return float(np.mean([x.elapsed_time(y) for x, y in es]))

    tmp = torch.empty_like(W)
    rht = {}
    if left.is_rht and right.is_rht:
        r_ms = timed(lambda: Q.quip_rht(W, tmp, right.signs, Q.RIGHT), args.steps)
        l_ms = timed(lambda: Q.quip_rht(W, tmp, left.signs, Q.LEFT), args.steps)
        t_ms = timed(lambda: Q.quip_rht2(W, tmp, left.signs, right.signs), args.steps)
        nbytes = 8.0 * cfg.m * cfg.n
        rht = {"right_pass_GBps": round(nbytes / r_ms / 1e6, 1),
               "left_pass_GBps": round(nbytes / l_ms / 1e6, 1),
               "two_sided_effective_GBps": round(2 * nbytes / t_ms / 1e6, 1),
               "right_ms": round(r_ms, 4), "left_ms": round(l_ms, 4), "two_sided_ms": round(t_ms, 4),
               "frac_of_hbm_peak_right": round(nbytes / r_ms / 1e6 / HBM_PEAK_GBS, 3)}

    line = {
        "metric": "quantized weights/sec for a 4096x4096 layer (LDLQ+RHT, 2-bit); RHT GB/s",
        "value": round(value, 1),
        "unit": "weights/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: {cfg.description}", "m": cfg.m, "n": cfg.n,
                   "calibration_rows": cfg.N, "bits": cfg.bits, "B": cfg.B,
                   "parallelism": "single GPU"},
        "phases_ms": {k: round(v, 4) for k, v in phases.items()},
        "weights_per_s_from_resident_H_W": round(mn / (from_resident / 1e3), 1),
        "rht": rht,
        "roofline": roofline,
    }
    if args.calibrate_copy:
        src = torch.ones(COPY_MIB * 2 ** 20 // 4, device=dev)
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(args.config, args.cpu_rows)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
