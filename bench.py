#!/usr/bin/env python3
"""Benchmark of the QuIP-family layer-quantization pass on one MI355X.

A step is one whole pass over one synthetic layer with everything resident in
HBM when the timed region starts: proxy Hessian + damping, two-sided random
Hadamard transform of H and of W, LDL, per-row scale search, LDLQ with the
proxy loss, inverse transforms. The workload is the 4096 x 4096 attention
projection layer (2-bit grid, RHT on both sides, lazy block 128, 4096
calibration rows); the metric is quantized weights per second.

Also reported: per-phase times (HIP events on the pass's stream), per-kernel
family times and algorithmic work from the library's own timing (the dispatch
of every kernel stamps an event pair; the same figures rocprofv3 reports), the
roofline of the family with the most time per step, HBM traffic from the
committed rocprofv3 counter summary of that family (when its source is
unchanged), the RHT bandwidth per one-sided pass, and the CPU oracle timed on
a bounded sample. Beside the pass: the E8 codebook's MSE on a Gaussian source,
the inference product's rates on packed codes, and the QuIP variants (the
permutation inside the Kronecker multiply, LDLQ-RG's order) on a 4096 x 11008
layer.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-variants] [--no-extras]
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
FP32_MFMA_PEAK_TFLOPS = 157.3   # dense fp32 matrix cores
FP32_VECTOR_PEAK_TFLOPS = 157.3  # 256 CUs x 2.4 GHz x 256 fp32 flop/clock (vector ALUs)
FP16_MFMA_PEAK_TFLOPS = 2500.0   # dense fp16 matrix cores

# source file of each kernel family (the counter summaries are tied to its hash)
FAMILY_SOURCES = [("gemm:", "gemm.hip"), ("gemm_tail_reduce", "gemm.hip"),
                  ("ldl_block_kernel", "ldl.hip"), ("ldlq_sweep_kernel", "ldlq.hip"),
                  ("grid_scale_kernel", "ldlq.hip"), ("e8_", "ldlq.hip"), ("rht_", "rht.hip"),
                  ("qmatvec_kernel", "qmatvec.hip"), ("tcq_", "tcq.hip"), ("permute_", "permute.hip")]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="c2")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-variants", action="store_true", help="skip the QuIP-variant passes")
    ap.add_argument("--no-extras", action="store_true",
                    help="the pass only: skip the Gaussian-source VQ, inference and variant figures "
                         "(profiled runs, whose per-kernel means must cover the pass's launches only)")
    ap.add_argument("--cpu-rows", type=int, default=4096, help="rows of W in the oracle LDLQ sample")
    ap.add_argument("--profile-inference", type=int, metavar="BITS", default=0,
                    help="run only the inference product on a 16384 x 16384 layer at BITS bits "
                         "(20 products; for rocprofv3 runs of that kernel alone) and exit")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="end with one plain device copy of COPY_MIB MiB (counter calibration)")
    # summaries of rocprofv3 result databases (host only, no GPU)
    ap.add_argument("--summarize-trace", metavar="DB")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DB", "WRITE_DB"))
    ap.add_argument("--summarize-mfma", metavar="DB",
                    help="matrix-core busy table from a SQ_VALU_MFMA_BUSY_CYCLES + GRBM_GUI_ACTIVE run")
    ap.add_argument("--kernel", help="rocprofv3 kernel-name substring of the family's dispatches")
    ap.add_argument("--family", help="library timing family the counters belong to")
    ap.add_argument("--command", default="")
    ap.add_argument("--title", help="title of a --summarize-trace summary")
    ap.add_argument("--out")
    return ap.parse_args()


COPY_MIB = 256
COPY_KERNEL = "MulFunctor"  # torch.mul(src, 1.0, out=dst): reads and writes COPY_MIB MiB


def _short_name(name: str) -> str:
    """Kernel name without namespace noise and arguments. rocprofv3 leaves
    names with a _Float16 parameter (mangled DF16_) mangled; they are
    demangled here with the older half-precision code (Dh) in its place."""
    import re
    import subprocess

    if name.startswith("_Z"):
        try:
            r = subprocess.run(["c++filt"], input=name.replace("DF16_", "Dh"), capture_output=True,
                               text=True, timeout=10)
            if r.returncode == 0 and r.stdout.strip():
                name = r.stdout.strip()
        except (OSError, subprocess.SubprocessError):
            pass
    nm = name.replace("(anonymous namespace)::", "").replace("void ", "")
    return re.sub(r"\(.*", "", nm)


def _kernel_rows(db):
    import sqlite3

    con = sqlite3.connect(db)
    out = []
    names = {}
    for name, start, end in con.execute("select name, start, end from kernels"):
        if name not in names:
            names[name] = _short_name(name)
        out.append((names[name], (end - start) / 1e3))
    return out


def summarize_trace(db, command, out, title=None):
    rows = _kernel_rows(db)
    agg = {}
    probes = 0
    for nm, d in rows:
        if nm.startswith("quip::peak_"):  # the attainable-rate probes the bench also runs
            probes += 1
            continue
        a = agg.setdefault(nm, [0.0, 0])
        a[0] += d
        a[1] += 1
    tot = sum(v[0] for v in agg.values())
    title = title or "quantization pass, 4096 x 4096 layer (2-bit, RHT, B = 128)"
    lines = [f"# rocprofv3 kernel trace: {title}", "",
             f"Command: `{command}`", ""]
    if probes:
        lines += [f"The attainable-rate probes (`quip::peak_*`, {probes} dispatches) that the "
                  "bench runs beside the pass are left out.", ""]
    lines += ["| kernel | calls | total us | avg us | % |", "|---|---:|---:|---:|---:|"]
    for k, (t, c) in sorted(agg.items(), key=lambda kv: -kv[1][0]):
        lines.append(f"| `{k}` | {c} | {t:.1f} | {t / c:.2f} | {100 * t / tot:.1f} |")
    text = "\n".join(lines) + "\n"
    if out:
        with open(out, "w") as f:
            f.write(text)
    print(text)


def _counter(db, counter):
    import sqlite3

    con = sqlite3.connect(db)
    per = {}
    names = {}
    for name, value in con.execute(
            "select kernel_name, value from counters_collection where counter_name = ?", (counter,)):
        if name not in names:
            names[name] = _short_name(name)
        per.setdefault(names[name], []).append(float(value))
    return per


def family_source(family: str) -> str:
    for prefix, src in FAMILY_SOURCES:
        if family.startswith(prefix):
            return src
    raise SystemExit(f"no source file known for kernel family {family}")


def source_sha(src: str) -> str:
    import hashlib
    with open(os.path.join(ROOT, "post_weight_quantization_quip_amd", "csrc", src), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def counters_path(family: str) -> str:
    return os.path.join(ROOT, "profiles", "counters_" + family.replace(":", "_") + "_c2.json")


def summarize_mfma(db, command, out, title=None):
    """Matrix-core busy fraction per kernel from one rocprofv3 --pmc run of
    SQ_VALU_MFMA_BUSY_CYCLES, SQ_BUSY_CYCLES and GRBM_GUI_ACTIVE. The ratio
    MFMA-busy / GPU-active of each kernel is divided by the same ratio for the
    fp32 matrix-core probe (quip_peak_compute kind 0, measured at ~99% of the
    fp32 peak), so 1.0 means the matrix cores as busy as in that loop."""
    import sqlite3

    con = sqlite3.connect(db)
    disp = {}
    names = {}
    for did, name, cname, value in con.execute(
            "select dispatch_id, kernel_name, counter_name, value from counters_collection"):
        if name not in names:
            names[name] = _short_name(name)
        d = disp.setdefault(did, {"name": names[name]})
        d[cname] = d.get(cname, 0.0) + float(value)
    agg = {}
    for d in disp.values():
        a = agg.setdefault(d["name"], [0, 0.0, 0.0, 0.0])
        a[0] += 1
        a[1] += d.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0)
        a[2] += d.get("SQ_BUSY_CYCLES", 0.0)
        a[3] += d.get("GRBM_GUI_ACTIVE", 0.0)
    probe = agg.get("quip::peak_mfma_f32_kernel")
    if not probe or probe[3] <= 0 or probe[1] <= 0:
        raise SystemExit("no fp32 matrix-core probe dispatch in the counter database")
    ref = probe[1] / probe[3]
    title = title or "quantization pass, 4096 x 4096 layer (2-bit, RHT, B = 128)"
    lines = [f"# Matrix-core busy fraction: {title}", "",
             f"Command: `{command}`", "",
             "Busy = (SQ_VALU_MFMA_BUSY_CYCLES / GRBM_GUI_ACTIVE) of the kernel over the same "
             f"ratio for the fp32 matrix-core probe ({ref:.2f}). Kernels with no matrix-core "
             "work are left out.", "",
             "| kernel | dispatches | MFMA busy | GPU-active cycles per dispatch |",
             "|---|---:|---:|---:|"]
    rows = [(k, a) for k, a in agg.items() if a[1] > 0 and a[3] > 0]
    for k, a in sorted(rows, key=lambda kv: -kv[1][3]):
        lines.append(f"| `{k}` | {a[0]} | {a[1] / a[3] / ref:.3f} | {a[3] / a[0]:.0f} |")
    text = "\n".join(lines) + "\n"
    if out:
        with open(out, "w") as f:
            f.write(text)
    print(text)


def summarize_counters(fetch_db, write_db, kernel, family, command, out):
    """HBM bytes per launch of `kernel` (rocprofv3 name substring) from
    FETCH_SIZE / WRITE_SIZE (KiB per dispatch), each scaled by what the counter
    reads for a plain copy of COPY_MIB MiB (read and written once)."""
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
    # the calibration copy is the largest dispatch of its kernel (a run may
    # launch the same elementwise kernel for small tensors too)
    cf = max(v for k, vals in fetch.items() if COPY_KERNEL in k for v in vals)
    cw = max(v for k, vals in write.items() if COPY_KERNEL in k for v in vals)
    nbytes = COPY_MIB * 2 ** 20
    f_read = nbytes / (cf * 1024.0)
    f_write = nbytes / (cw * 1024.0)
    rd = kf * 1024.0 * f_read
    wr = kw * 1024.0 * f_write
    src = family_source(family)
    d = {"family": family, "kernel": kernel, "source": src, "source_sha": source_sha(src),
         "fetch_kib_per_dispatch": kf, "write_kib_per_dispatch": kw, "dispatches": [nf, nw],
         "copy_fetch_kib": cf, "copy_write_kib": cw, "copy_bytes_each_way": nbytes,
         "scale_read": f_read, "scale_write": f_write,
         "read_bytes_per_launch": rd, "write_bytes_per_launch": wr,
         "bytes_per_launch": rd + wr, "command": command}
    text = json.dumps(d, indent=1)
    out = out or counters_path(family)
    with open(out, "w") as f:
        f.write(text + "\n")
    print(text)


def traffic_from_profiles(family: str):
    """HBM bytes per launch of a kernel family from its committed counter
    summary under profiles/, or None (absent, or the kernel's source changed
    since the counters were taken)."""
    path = counters_path(family)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("family") != family or d.get("source_sha") != source_sha(family_source(family)):
        return None
    return d.get("bytes_per_launch")


def kernel_bound(name: str):
    """(bound, peak, unit) of a kernel family: the matrix-core products against
    the fp32 MFMA peak; the latency-bound sequential kernels (LDL block factor,
    LDLQ sweep) and the vector-ALU-bound searches (scale candidates, E8
    codewords) against the fp32 vector-ALU peak; the streaming kernels against
    HBM bandwidth."""
    if name.startswith("gemm:"):
        return "mfma", FP32_MFMA_PEAK_TFLOPS, "TFLOP/s"
    if name in ("ldl_block_kernel", "ldlq_sweep_kernel", "grid_scale_kernel", "e8_argmin_kernel",
                "e8_scale_kernel"):
        return "alu", FP32_VECTOR_PEAK_TFLOPS, "TFLOP/s"
    return "hbm", HBM_PEAK_GBS, "GB/s"


def attainable_bench(Q, dev, timed) -> dict:
    """What plain, dependency-free work attains on this card, next to the
    published peaks the roofline fractions use: a 1 GiB device copy, and
    loops of independent fp32 and f16 matrix-core instructions and fp32
    vector FMAs (the library's probe kernels, four waves per SIMD)."""
    import torch

    count = 2 ** 28  # 1 GiB of float32 each way
    src = torch.ones(count, device=dev)
    dst = torch.empty_like(src)
    ms = timed(lambda: Q.quip_peak_copy(src, dst), 5)
    copy_gbps = 8.0 * count / (ms / 1e3) / 1e9
    del src, dst
    out = torch.zeros(1, device=dev)
    rates = {}
    for kind, iters in ((0, 20000), (1, 20000), (2, 100000)):
        flops = Q.quip_peak_compute(kind, iters, out)
        ms = timed(lambda: Q.quip_peak_compute(kind, iters, out), 3)
        rates[kind] = flops / (ms / 1e3) / 1e12
    return {"hbm_copy_GBps": round(copy_gbps, 1), "hbm_published_GBps": HBM_PEAK_GBS,
            "mfma_f32_TFLOPs": round(rates[0], 1), "mfma_f32_published_TFLOPs": FP32_MFMA_PEAK_TFLOPS,
            "mfma_f16_TFLOPs": round(rates[1], 1), "mfma_f16_published_TFLOPs": FP16_MFMA_PEAK_TFLOPS,
            "valu_f32_fma_TFLOPs": round(rates[2], 1),
            "valu_f32_published_TFLOPs": FP32_VECTOR_PEAK_TFLOPS,
            "note": "published vector peak counts packed fp32 (2 FMAs per lane); the library "
                    "issues one FMA per lane and instruction"}


def gaussian_vq_bench(Q, wl, dev, timed) -> dict:
    """The E8 codebook at 2 bits per weight on an i.i.d. N(0,1) source (1024 x
    4096 weights, 524288 8-vectors), through the search of the E8
    configuration's scale step: the best mean squared error per weight over the
    32 scale candidates, against the Gaussian distortion-rate bound 2^-4; the
    QTIP page's figures (E8P 0.089, 256-D TCQ 0.068-0.071) are context."""
    import torch

    gm, gn = 1024, 4096
    G = torch.from_numpy(wl.gaussian_rows(1, gm, gn)).to(dev)
    cb = Q.quip_e8_codebook().to(dev)
    q8 = Q.quantizer(Q.Q_E8, 2)
    gsc = torch.empty(gm + 1, device=dev)
    gsse = torch.empty(32, dtype=torch.float64, device=dev)
    gws = Q.native._workspace(Q.native._ws_query(Q.native.lib.quip_scales_workspace, gm, gn,
                                                 ctypes.byref(q8)), dev)
    g_ms = timed(lambda: Q.quip_scales(G, q8, gsc, mse_out=gsse, codebook=cb, ws=gws), 3)
    nvec = gm * gn // 8
    return {"mse_per_weight": round(float(gsse.min().item()) / (gm * gn), 5),
            "distortion_rate_bound": 0.0625, "printed_e8p": 0.089,
            "printed_tcq_256d": [0.068, 0.071], "vectors": nvec, "ms": round(g_ms, 3),
            "candidate_distances_per_s": round(nvec * 65536 * 32 / (g_ms / 1e3), 1)}


def inference_bench(Q, wl, dev, timed, lp, left, right, cfg) -> dict:
    """Inference with the quantized layer, y = Q_L^T W^~ Q_R x: the pass's own
    codes packed at 2 bits, then 16384 x 16384 layers of random codes at 2 and
    4 bits, four distinct copies cycled so that the packed codes read per cycle
    (268 or 537 MB) exceed the 256 MB last-level cache."""
    import torch

    if not (left.is_rht and right.is_rht):
        return {}

    def qmv_case(codes_list, scales, sl, sr, bits, reps):
        m, n = codes_list[0].shape
        rb = Q.quip_packed_row_bytes(n, bits)
        packs = []
        for c in codes_list:
            p = torch.empty((m, rb), dtype=torch.uint8, device=dev)
            Q.quip_pack_codes(c, bits, p)
            packs.append(p)
        x = torch.from_numpy(wl.gaussian_rows(7, 1, n)[0]).to(dev)
        y = torch.empty(m, device=dev)
        ws = Q.native._workspace(Q.native._ws_query(Q.native.lib.quip_qmatvec_rht_workspace, m, n),
                                 dev)
        it = [0]

        def call():
            Q.quip_qmatvec_rht(packs[it[0] % len(packs)], n, bits, scales, sl, sr, x, y, ws=ws)
            it[0] += 1
        ms = timed(call, reps)
        Q.timing_reset()
        Q.timing_enable(True)
        for _ in range(reps):
            call()
        torch.cuda.synchronize()
        Q.timing_enable(False)
        rep = Q.timing_report()
        launches, kms, _, kbytes = rep["qmatvec_kernel"]
        Q.timing_reset()
        per_kernel_us = {k: round(1e3 * v[1] / v[0], 2) for k, v in rep.items()}
        gbps = kbytes / (kms / 1e3) / 1e9
        return {"m": m, "n": n, "bits": bits, "packed_MB": round(m * rb / 1e6, 2),
                "copies": len(packs), "product_us": round(1e3 * ms, 2),
                "qmatvec_kernel_us": round(1e3 * kms / launches, 2),
                "qmatvec_kernel_GBps": round(gbps, 1), "frac_of_hbm_peak": round(gbps / HBM_PEAK_GBS, 3),
                "weights_per_s": round(m * n / (ms / 1e3), 1), "kernels_us": per_kernel_us}

    out = {"pass_layer": qmv_case([lp.buffers["codes"]], lp.buffers["scales"], left.signs,
                                  right.signs, cfg.bits, 50)}
    big = 16384
    gen = torch.Generator(device=dev).manual_seed(11)

    def sgn():
        return torch.randint(0, 2, (big,), device=dev, generator=gen).float() * 2 - 1
    bsl, bsr = sgn(), sgn()
    bsc = torch.rand(big, device=dev, generator=gen) + 0.5
    for bits in (2, 4):
        cl = [torch.randint(0, 1 << bits, (big, big), dtype=torch.uint8, device=dev, generator=gen)
              for _ in range(4)]
        out[f"{big}x{big}_{bits}bit"] = qmv_case(cl, bsc, bsl, bsr, bits, 40)
        del cl
    torch.cuda.empty_cache()
    return out


def tcq_bench(Q, wl, dev, timed) -> dict:
    """Trellis-coded quantization with the bitshift trellis at k = 2 bits per
    step on an i.i.d. N(0,1) source: 4096 sequences of T = 256 (1M weights),
    L = 12 and 15 state bits. Reports the mean squared error per weight
    (against the distortion-rate bound at the rate k + (L - k)/T, and the
    QTIP page's 256-D TCQ figures 0.068-0.071 as context), the time, and the
    forward kernel's edge-relaxation rate from the library timing."""
    import torch

    rows, T = 4096, 256
    X = torch.from_numpy(wl.gaussian_rows(3, rows, T)).to(dev)
    st = torch.empty((rows, T), dtype=torch.int16, device=dev)
    cost = torch.empty(rows, device=dev)
    out = {"sequences": rows, "T": T, "k": 2, "printed_tcq_256d": [0.068, 0.071]}
    for L in (12, 15):
        ws = Q.native._workspace(Q.native._ws_query(Q.native.lib.quip_tcq_workspace, rows, T, L), dev)
        ms = timed(lambda: Q.quip_tcq_quantize(X, L, st, cost, ws=ws), 2)
        Q.timing_reset()
        Q.timing_enable(True)
        Q.quip_tcq_quantize(X, L, st, cost, ws=ws)
        torch.cuda.synchronize()
        Q.timing_enable(False)
        rep = Q.timing_report()
        Q.timing_reset()
        launches, fms, edges, _ = rep["tcq_forward_kernel"]
        _, tms, _, _ = rep["tcq_traceback_kernel"]
        rate = 2 + (L - 2) / T
        out[f"L{L}"] = {"mse_per_weight": round(float(cost.double().sum().item()) / (rows * T), 5),
                        "bits_per_weight": round(rate, 4),
                        "distortion_rate_bound": round(2.0 ** (-2 * rate), 5),
                        "ms": round(ms, 3), "weights_per_s": round(rows * T / (ms / 1e3), 1),
                        "forward_ms": round(fms, 3), "traceback_ms": round(tms, 3),
                        "edge_relaxations_per_s": round(edges / (fms / 1e3), 1)}
        del ws
    return out


def profile_inference(Q, dev, bits: int, calibrate_copy: bool) -> None:
    """20 products y = Q_L^T W^~ Q_R x on one 16384 x 16384 layer of random
    codes at `bits` bits (four copies cycled, as in the inference figures)."""
    import torch

    big = 16384
    gen = torch.Generator(device=dev).manual_seed(11)
    sl = torch.randint(0, 2, (big,), device=dev, generator=gen).float() * 2 - 1
    sr = torch.randint(0, 2, (big,), device=dev, generator=gen).float() * 2 - 1
    sc = torch.rand(big, device=dev, generator=gen) + 0.5
    rb = Q.quip_packed_row_bytes(big, bits)
    packs = []
    for _ in range(4):
        codes = torch.randint(0, 1 << bits, (big, big), dtype=torch.uint8, device=dev, generator=gen)
        p = torch.empty((big, rb), dtype=torch.uint8, device=dev)
        Q.quip_pack_codes(codes, bits, p)
        packs.append(p)
        del codes
    x = torch.randn(big, device=dev, generator=gen)
    y = torch.empty(big, device=dev)
    ws = Q.native._workspace(Q.native._ws_query(Q.native.lib.quip_qmatvec_rht_workspace, big, big), dev)
    for i in range(20):
        Q.quip_qmatvec_rht(packs[i % 4], big, bits, sc, sl, sr, x, y, ws=ws)
    torch.cuda.synchronize()
    if calibrate_copy:
        src = torch.ones(COPY_MIB * 2 ** 20 // 4, device=dev)
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
    print(json.dumps({"profile_inference": {"bits": bits, "products": 20}}))


def configs_bench(Q, wl, dev) -> dict:
    """One warm-up and one timed pass of every configuration (their shapes,
    bit widths and transforms as the workloads define them): ms per pass and
    quantized weights per second."""
    import torch

    out = {}
    for name in ("c1", "c2", "c3a", "c3b", "c3p", "c4a", "c4b", "c4c", "c5"):
        L = wl.make_layer(name)
        cfg = L.cfg
        W = torch.from_numpy(L.W).to(dev)
        X = torch.from_numpy(L.X).to(dev)
        del L
        lp = Q.LayerPass(cfg.m, cfg.n, Q.SideSpec.from_numpy(wl.side_inputs(cfg, cfg.left, cfg.m, "left"), dev),
                         Q.SideSpec.from_numpy(wl.side_inputs(cfg, cfg.right, cfg.n, "right"), dev),
                         quant=cfg.quant, bits=cfg.bits, B=cfg.B, g=cfg.g, alpha=cfg.alpha,
                         device=dev, rg_order=cfg.rg_order)
        lp.run(W, X)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        lp.run(W, X)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3
        out[name] = {"m": cfg.m, "n": cfg.n, "N": cfg.N, "bits": cfg.bits, "quant": cfg.quant,
                     "ms_per_pass": round(ms, 3), "weights_per_s": round(cfg.m * cfg.n / (ms / 1e3), 1),
                     "info": int(lp.buffers["info"].item())}
        del lp, W, X
        torch.cuda.empty_cache()
    return out


def e8_config_bench(Q, wl, dev, steps: int) -> dict:
    """The E8 configuration (4096 x 4096, BlockLDLQ with g = 8 and the 65536-point
    E8 codebook at 2 bits per weight): time per pass, its phases, and the E8
    search kernels' rates: dot-product flops (2 x 8 per vector and codeword),
    and the matrix-core fraction of the split half-precision products that
    compute them (twice those flops) against the dense fp16 peak."""
    import torch

    L = wl.make_layer("c5")
    cfg = L.cfg
    W = torch.from_numpy(L.W).to(dev)
    X = torch.from_numpy(L.X).to(dev)
    lp = Q.LayerPass(cfg.m, cfg.n, Q.SideSpec.from_numpy(L.left, dev), Q.SideSpec.from_numpy(L.right, dev),
                     quant=cfg.quant, bits=cfg.bits, B=cfg.B, g=cfg.g, alpha=cfg.alpha, device=dev)
    lp.run(W, X)
    torch.cuda.synchronize()
    events = {}
    t0 = time.perf_counter()
    for _ in range(steps):
        lp.run(W, X, events=events)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    order = ["hessian", "incoherence_H", "incoherence_W", "ldl", "ldlq", "postprocess", "end"]
    phases = {a: round(float(np.mean([ea.elapsed_time(eb) for ea, eb in zip(events[a], events[b])])), 3)
              for a, b in zip(order[:-1], order[1:])}
    Q.timing_reset()
    Q.timing_enable(True)
    lp.run(W, X)
    torch.cuda.synchronize()
    Q.timing_enable(False)
    rep = Q.timing_report()
    Q.timing_reset()
    kern = {}
    for k, (launches, kms, flops, _) in sorted(rep.items(), key=lambda kv: -kv[1][1])[:6]:
        v = {"launches": launches, "ms": round(kms, 3)}
        if k in ("e8_scale_kernel", "e8_argmin_kernel") and flops > 0:
            # flops = 16 per vector and codeword (the 8-dim dot product); the
            # matrix cores run it as a split half product (K = 16: twice the
            # flops) against the dense fp16 peak
            tf = flops / (kms / 1e3) / 1e12
            v.update({"dot_TFLOPs": round(tf, 2),
                      "frac_of_fp16_mfma_peak": round(2 * tf / FP16_MFMA_PEAK_TFLOPS, 4)})
        kern[k] = v
    return {"workload": f"c5: {cfg.description}", "ms_per_pass": round(ms, 3),
            "weights_per_s": round(cfg.m * cfg.n / (ms / 1e3), 1), "phases_ms": phases,
            "proxy_loss": float(lp.buffers["loss"].item()), "top_kernels": kern}


def variants_bench(Q, wl, dev, steps: int) -> dict:
    """The QuIP variants on the 4096 x 11008 MLP layer (3-bit, RHT left,
    Kronecker 64 x 172 right): without them, with the random permutation inside
    the Kronecker multiply, with LDLQ-RG's diag(H) order, and with both. Per
    variant: time per pass (wall clock over `steps` passes), the proxy loss, and
    the permutation kernels' own times and rates from the library timing."""
    import torch

    L = wl.make_layer("c3p")
    cfg = L.cfg
    W = torch.from_numpy(L.W).to(dev)
    X = torch.from_numpy(L.X).to(dev)
    out = {"workload": f"{cfg.m}x{cfg.n}, {cfg.bits}-bit, RHT left, Kron 64x172 right, N = {cfg.N}"}
    for name, perm, rg in (("plain", False, False), ("perm", True, False), ("rg", False, True),
                           ("perm_rg", True, True)):
        right = dict(L.right)
        if not perm:
            right.pop("perm")
        lp = Q.LayerPass(cfg.m, cfg.n, Q.SideSpec.from_numpy(L.left, dev),
                         Q.SideSpec.from_numpy(right, dev), quant=cfg.quant, bits=cfg.bits, B=cfg.B,
                         alpha=cfg.alpha, device=dev, rg_order=rg)
        lp.run(W, X)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            lp.run(W, X)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        Q.timing_reset()
        Q.timing_enable(True)
        lp.run(W, X)
        torch.cuda.synchronize()
        Q.timing_enable(False)
        rep = Q.timing_report()
        Q.timing_reset()
        v = {"ms_per_pass": round(ms, 3), "proxy_loss": float(lp.buffers["loss"].item()),
             "info": int(lp.buffers["info"].item())}
        for k in ("permute_gather_kernel", "permute_scatter_kernel", "diag_rank_kernel",
                  "diag_order_finish_kernel"):
            if k in rep:
                launches, kms, _, kbytes = rep[k]
                v[k] = {"launches": launches, "us": round(1e3 * kms, 2)}
                if k.startswith("permute"):
                    v[k]["GBps"] = round(kbytes / (kms / 1e3) / 1e9, 1)
        out[name] = v
        del lp
        torch.cuda.empty_cache()
    return out


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


def pass_targets(kernels: dict, phases: dict, rht: dict, cfg) -> dict:
    """The phase-level figures the pass is held to, each next to its target:
    the two-sided random-sign Hadamard transform against the HBM peak (>= 60 %,
    on matrices read from and written to HBM; the cache-resident figures are
    reported beside them),
    the proxy-Hessian product and the LDLQ trailing update (the per-batch
    outer product; the feedback inside a batch is taken by the sweep kernel
    itself) against the fp32 matrix-core peak (>= 50 %), and the LDL and LDLQ
    phases (n^3 / 3 and m n (n - 1) flops over their wall time; reported, no
    target)."""

    def family_frac(names):
        fl = sum(kernels[n]["algorithmic_flops_per_launch"] * kernels[n]["launches_per_step"]
                 for n in names if n in kernels)
        ms = sum(kernels[n]["ms_per_step"] for n in names if n in kernels)
        return (fl / (ms / 1e3) / 1e12 / FP32_MFMA_PEAK_TFLOPS if ms > 0 else None), ms

    out = {}
    if rht:
        # against the HBM peak with the bytes coming from and going to HBM
        # (six matrices in turn); the same passes on one matrix that stays in
        # the last-level cache are reported beside them
        hr = rht.get("hbm_resident") or rht
        out["rht_two_sided_frac_of_hbm"] = {
            "measured": round(hr["two_sided_effective_GBps"] / HBM_PEAK_GBS, 3), "target": 0.60}
        out["rht_right_pass_frac_of_hbm"] = {
            "measured": round(hr["right_pass_GBps"] / HBM_PEAK_GBS, 3), "target": 0.60}
        out["rht_left_pass_frac_of_hbm"] = {
            "measured": round(hr["left_pass_GBps"] / HBM_PEAK_GBS, 3), "target": 0.60}
        if "hbm_resident" in rht:
            out["rht_two_sided_frac_of_hbm_cache_resident"] = {
                "measured": round(rht["two_sided_effective_GBps"] / HBM_PEAK_GBS, 3), "target": None}
            out["rht_right_pass_frac_of_hbm_cache_resident"] = {
                "measured": round(rht["right_pass_GBps"] / HBM_PEAK_GBS, 3), "target": None}
            out["rht_left_pass_frac_of_hbm_cache_resident"] = {
                "measured": round(rht["left_pass_GBps"] / HBM_PEAK_GBS, 3), "target": None}
    f, ms = family_frac(["gemm:hessian"])
    if f is not None:
        out["hessian_frac_of_mfma"] = {"measured": round(f, 3), "target": 0.50, "ms": round(ms, 4)}
    f, ms = family_frac(["gemm:ldlq_inner", "gemm:ldlq_outer"])
    if f is not None:
        out["ldlq_trailing_update_frac_of_mfma"] = {"measured": round(f, 3), "target": 0.50,
                                                    "ms": round(ms, 4)}
    n = float(cfg.n)
    if phases.get("ldl"):
        out["ldl_phase_frac_of_mfma"] = {
            "measured": round(n ** 3 / 3 / (phases["ldl"] / 1e3) / 1e12 / FP32_MFMA_PEAK_TFLOPS, 4),
            "target": None, "ms": round(phases["ldl"], 4)}
    if phases.get("ldlq"):
        # every feedback product of LDLQ: m n (n - 1) flops over the phase
        # (the scale search, the sweeps with the in-batch feedback they take
        # on the matrix cores, and the outer products)
        out["ldlq_phase_ms"] = {"measured": round(phases["ldlq"], 4), "target": None}
        out["ldlq_phase_frac_of_mfma"] = {
            "measured": round(float(cfg.m) * n * (n - 1) / (phases["ldlq"] / 1e3) / 1e12
                              / FP32_MFMA_PEAK_TFLOPS, 4), "target": None}
    for v in out.values():
        if v.get("target") is not None:
            v["meets"] = bool(v["measured"] >= v["target"])
    return out


def main():
    args = parse()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.command, args.out, args.title)
        return
    if args.summarize_mfma:
        summarize_mfma(args.summarize_mfma, args.command, args.out, args.title)
        return
    if args.summarize_counters:
        if not args.kernel or not args.family:
            raise SystemExit("--summarize-counters needs --kernel and --family")
        summarize_counters(*args.summarize_counters, args.kernel, args.family, args.command, args.out)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the pass runs on one GPU; the per-shard kernels are the same at any GPU count)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import post_weight_quantization_quip_amd as Q
    import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = "cuda"
    if args.profile_inference:
        profile_inference(Q, dev, args.profile_inference, args.calibrate_copy)
        return
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

    order = ["hessian", "incoherence_H", "incoherence_W", "ldl", "ldlq", "postprocess", "end"]
    phases = {}
    for a, b in zip(order[:-1], order[1:]):
        phases[a] = float(np.mean([ea.elapsed_time(eb) for ea, eb in zip(events[a], events[b])]))
    phases["step_events"] = float(np.mean([ea.elapsed_time(eb) for ea, eb in
                                           zip(events["hessian"], events["end"])]))
    mn = cfg.m * cfg.n
    value = mn / (ms_per_step / 1e3)
    from_resident = (phases["incoherence_H"] + phases["incoherence_W"] + phases["ldl"]
                     + phases["ldlq"])

    # per-kernel figures: the same passes again with the library's event timing
    # on (two HIP events around every launch, on the pass's stream); the
    # roofline is that of the kernel family with the most time per step
    Q.timing_reset()
    Q.timing_enable(True)
    for _ in range(args.steps):
        lp.run(W, X)
    torch.cuda.synchronize()
    Q.timing_enable(False)
    rep = Q.timing_report()
    Q.timing_reset()
    kernels = {}
    for name, (launches, ms, flops, nbytes) in rep.items():
        bound, peak, unit = kernel_bound(name)
        per_step = ms / args.steps
        if bound == "hbm":
            achieved = nbytes / (ms / 1e3) / 1e9 if ms > 0 else 0.0
        else:
            achieved = flops / (ms / 1e3) / 1e12 if ms > 0 else 0.0
        kernels[name] = {"ms_per_step": round(per_step, 4), "launches_per_step": launches / args.steps,
                         "avg_launch_us": round(1e3 * ms / launches, 2), "bound": bound,
                         "achieved": round(achieved, 3), "unit": unit, "peak": peak,
                         "frac": round(achieved / peak, 4),
                         "algorithmic_flops_per_launch": round(flops / launches),
                         "algorithmic_bytes_per_launch": round(nbytes / launches)}
    dom = max(kernels, key=lambda k: kernels[k]["ms_per_step"])
    k = kernels[dom]
    traffic = traffic_from_profiles(dom)
    if traffic is not None:
        traffic = round(traffic / 1e6, 3)  # MB per launch
    roofline = {"bound": k["bound"], "achieved": k["achieved"], "peak": k["peak"], "unit": k["unit"],
                "frac": k["frac"], "traffic": traffic,
                "traffic_unit": "MB per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                "kernel": dom, "avg_launch_ms": round(k["avg_launch_us"] / 1e3, 5),
                "launches_per_step": k["launches_per_step"],
                "algorithmic_flops_per_launch": k["algorithmic_flops_per_launch"],
                "algorithmic_bytes_per_launch": k["algorithmic_bytes_per_launch"]}

    # RHT bandwidth per one-sided pass (W, 4096 x 4096): `reps` calls back to
    # back between one pair of events (per-call events would also count the
    # host's time to issue each call)
    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

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
               "frac_of_hbm_peak_right": round(nbytes / r_ms / 1e6 / HBM_PEAK_GBS, 3),
               "note": ("the same matrix transformed back to back: the 64 MB source and "
                        "result stay in the 256 MB last-level cache")}
        # the same passes with the source and result taken in turn from six
        # distinct matrices (384 MB, more than the last-level cache), so that
        # the bytes come from and go to HBM
        mats = [torch.empty_like(W).copy_(W) for _ in range(6)]
        cyc = {"j": 0}

        def cold(fn):
            def run():
                j = cyc["j"]
                cyc["j"] = (j + 1) % 6
                fn(mats[j], mats[(j + 3) % 6])
            return run

        reps = 6 * max(args.steps // 6, 5)
        rc_ms = timed(cold(lambda a, o: Q.quip_rht(a, o, right.signs, Q.RIGHT)), reps)
        lc_ms = timed(cold(lambda a, o: Q.quip_rht(a, o, left.signs, Q.LEFT)), reps)
        tc_ms = timed(cold(lambda a, o: Q.quip_rht2(a, o, left.signs, right.signs)), reps)
        rht["hbm_resident"] = {
            "right_pass_GBps": round(nbytes / rc_ms / 1e6, 1),
            "left_pass_GBps": round(nbytes / lc_ms / 1e6, 1),
            "two_sided_effective_GBps": round(2 * nbytes / tc_ms / 1e6, 1),
            "right_ms": round(rc_ms, 4), "left_ms": round(lc_ms, 4), "two_sided_ms": round(tc_ms, 4)}
        del mats

    attainable = attainable_bench(Q, dev, timed)
    targets = pass_targets(kernels, phases, rht, cfg)

    # beside the pass: Gaussian-source VQ, the inference product, the variants
    gaussian_vq, inference, variants, tcq, e8c, allcfg = {}, {}, {}, {}, {}, {}
    if not args.no_extras:
        allcfg = configs_bench(Q, wl, dev)
        e8c = e8_config_bench(Q, wl, dev, 2)
        gaussian_vq = gaussian_vq_bench(Q, wl, dev, timed)
        tcq = tcq_bench(Q, wl, dev, timed)
        inference = inference_bench(Q, wl, dev, timed, lp, left, right, cfg)
        if not args.no_variants:
            variants = variants_bench(Q, wl, dev, max(2, args.steps // 3))

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
        "configs": allcfg,
        "e8_config": e8c,
        "gaussian_vq": gaussian_vq,
        "tcq": tcq,
        "inference": inference,
        "variants": variants,
        "roofline": roofline,
        "targets": targets,
        "attainable": attainable,
        "kernels": dict(sorted(kernels.items(), key=lambda kv: -kv[1]["ms_per_step"])),
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
