#!/usr/bin/env python3
"""Benchmark of the fused SwiGLU gate/up stage on one MI355X.

Prints ONE JSON line on stdout (progress goes to stderr).

Headline workload: one training step of the fused stage at M=8192 tokens,
K=4096, N=14336 in bf16 (fp32 accumulation): the fused forward
h = SiLU(x Wg^T) * (x Wu^T) followed by the backward (dX, dWg, dWu).
value = algorithmic TFLOP/s of that step, 12 M N K flops per step (4 M N K
forward, 8 M N K for dX and dW; the recompute of g and u in the backward is
not credited).  Inputs are synthetic (seed 0) and resident in HBM before the
timed region starts; --warmup steps, then --steps timed steps, eager.

After the headline, every workload of the stage is measured with the
protocol of "Fused SwiGLU benchmark" (AstrAI docs/developer/swiglu_benchmark.md,
opening section): per variant one HIP graph of --iters calls over rotated
buffers, --graph-warmup eager calls first, then --trials trials in
A-B-C-C-B-A order across the variants of a leg, device time from HIP events
around each graph launch; every sample is kept with p50/p90/p99 per call,
eager per-call times beside them, the kernel launches per call, and the
error of one call's output against the fp64 oracle (max / mean absolute
error, cosine).  The oracle's own time on the host cores is recorded per
configuration (the headline's on a row sample, extrapolated and labelled).
Legs:
  train_fwd   forward variants at the headline shape (SwiGLU, GeGLU, both
              with the FP8-quantised output, and SwiGLU with gate and up
              multipliers), TFLOP/s;
  train_bwd   the backward (SwiGLU, GeGLU), TFLOP/s on 8 M N K;
  decode      M = 1, 2, 4, 8 at (N, K) = (6912, 1536), (11008, 4096),
              (13824, 5120), (24576, 6144) with rotated weight copies well
              past the 256 MB Infinity Cache, GB/s, beside the kernel's
              read-only twin and a dual-stream read of the same buffers; the
              floor is the faster of the two; GeGLU beside SwiGLU at M = 1, 8;
  act_quant   elementwise SwiGLU + 1x32 FP8 quantisation of [4001, 3584] fp32
              (clamp off, L = 7 with count, GELU-tanh), beside the
              quantiser's load/store twin, GB/s; the non-quantised forward
              (fp32 and bf16 h);
  act_bwd     the elementwise backward (fp32 with clamp, fp32 with row
              weights and weight_grad, bf16 with clamp, and E4M3 dgate/dup
              from fp32 and from bf16 inputs), GB/s;
  fp32        the IEEE-fp32 dual GEMM at M=4001, K=2048, N=3584 and its
              backward, TFLOP/s;
  tiny_fp32   forward + backward at x[4, 64], W[128, 64].
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time
import traceback

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6     # dense bf16 MFMA, MI355X
PEAK_FP32_TFLOPS = 157.3      # dense fp32 matrix, MI355X
PEAK_HBM_GBS = 8000.0         # HBM3E, MI355X

M4, N4, K4 = 8192, 14336, 4096
DECODE_SHAPES = ((6912, 1536, 16), (11008, 4096, 4), (13824, 5120, 2), (24576, 6144, 2))   # (N, K, copies)
AQ_R, AQ_C = 4001, 3584
F32_M, F32_N, F32_K = 4001, 3584, 2048

# Kernel launches per library call (from the entry points' code): the bf16
# backward runs the recompute, two weight transposes, the dX product, the x
# transpose and the dW product; the fp32 one transposes D as well.
LAUNCHES = {"fwd": 1, "bwd_bf16": 6, "bwd_f32": 7, "gemv": 1, "act_quant_count": 2, "act_quant": 1,
            "act_fwd_count": 2, "act_fwd": 1, "act_bwd": 1}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--trials", type=int, default=10, help="A-B-C-C-B-A trials per leg")
    p.add_argument("--iters", type=int, default=100, help="calls per graph (decode and elementwise legs)")
    p.add_argument("--gemm-iters", type=int, default=20, help="calls per graph of the 8192x14336x4096 and fp32 legs")
    p.add_argument("--graph-warmup", type=int, default=20, help="eager calls per variant before capture")
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="target host time of the headline oracle sample")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extra", action="store_true", help="headline only")
    p.add_argument("--only", default=None,
                   choices=["step", "fwd", "train_fwd", "train_bwd", "decode", "act_quant", "act_bwd", "fp32", "tiny",
                            "fwd_k_sweep", "traffic", "traffic_bwd", "traffic_decode", "traffic_act_quant", "traffic_act_fwd",
                            "traffic_act_bwd"],
                   help="profiling aid: run one leg only (no JSON contract); 'traffic*' runs a kernel and a 1 GiB "
                        "copy (the counter calibration) for the --pmc runs")
    p.add_argument("--digest-cycles", nargs=2, metavar=("NAME", "PMC_CSV"), default=None,
                   help="read the counter_collection.csv of a rocprofv3 --pmc run with GRBM_GUI_ACTIVE (and "
                        "SQ_VALU_MFMA_BUSY_CYCLES) and record NAME's cycles per launch in profiles/cycles.json")
    p.add_argument("--digest-traffic", nargs=3, metavar=("NAME", "FETCH_CSV", "WRITE_CSV"), default=None,
                   help="read the counter_collection.csv files of two rocprofv3 --pmc runs of a 'traffic*' leg "
                        "(FETCH_SIZE, then WRITE_SIZE) and record NAME in profiles/traffic.json")
    return p.parse_args()


# ------------------------------------------------------------------ traffic

COPY_BYTES = 1 << 30            # calibration copy: reads and writes this many bytes per launch
COPY_KERNEL_TAG = "copy"

# The translation unit of the forward dual GEMM: the kernel file and the
# headers it includes.
FWD_KERNEL_SOURCES = ("common.hpp", "fp8.hpp", "gemm.hip", "gemm.hpp")

# name -> (name fragments of the kernel -- mangled, and as the profiler
# demangles it --, its translation unit, algorithmic bytes per launch[, grid
# size in work-items, where one kernel serves several measured shapes])
TRAFFIC_KERNELS = {
    "fwd_dual_gemm_bf16_8192x14336x4096": (
        ("gemm_dma_kernelIDF16bLNS0_3EpiE0E",), FWD_KERNEL_SOURCES,
        (M4 * K4 + 2 * N4 * K4 + M4 * N4) * 2),
    # The recompute of the backward: x, Wg, Wu and dh read once; D = [dg | du]
    # [M, 2N] and its transpose written once (N is a multiple of 64 here, so
    # neither carries padding).
    "bwd_recompute_bf16_8192x14336x4096": (
        ("gemm_dma_kernelIDF16bLNS0_3EpiE2E",), FWD_KERNEL_SOURCES,
        (M4 * K4 + 2 * N4 * K4 + M4 * N4 + 2 * (2 * M4 * N4)) * 2),
    "gemv_bf16_M8_11008x4096": (
        ("gemv_mfma_kernelILNS_3ActE0ELb0ELb0E", "gemv_mfma_kernel<(swg::Act)0, false, false>"), ("common.hpp", "gemv.hip", "gemm.hpp"),
        2 * 11008 * 4096 * 2 + 8 * 4096 * 2 + 8 * 11008 * 2, 11008 // 16 * 512),
    "gemv_bf16_M1_11008x4096": (
        ("gemv_kernelILi1ELNS_3ActE0ELb0E", "gemv_kernel<1, (swg::Act)0, false>"), ("common.hpp", "gemv.hip", "gemm.hpp"),
        2 * 11008 * 4096 * 2 + 4096 * 2 + 11008 * 2),
    "gemv_bf16_M8_24576x6144": (
        ("gemv_mfma_kernelILNS_3ActE0ELb0ELb0E", "gemv_mfma_kernel<(swg::Act)0, false, false>"), ("common.hpp", "gemv.hip", "gemm.hpp"),
        2 * 24576 * 6144 * 2 + 8 * 6144 * 2 + 8 * 24576 * 2, 24576 // 16 * 512),
    "act_quant_4001x3584": (
        ("act_quant_kernelILNS_3ActE0ELb0ELb0ELb0ELb0E", "act_quant_kernel<(swg::Act)0, false, false, false, false>"),
        ("common.hpp", "fp8.hpp", "act_quant.hip", "gemm.hpp"),
        2 * AQ_R * AQ_C * 4 + AQ_R * AQ_C + AQ_R * AQ_C // 32),
    "act_fwd_bf16_4001x3584": (
        ("act_fwd_kernelILNS_3ActE0EDF16bLb0ELb0E", "act_fwd_kernel<(swg::Act)0, __bf16, false, false>"),
        ("common.hpp", "fp8.hpp", "act_fwd.hip", "gemm.hpp"),
        2 * AQ_R * AQ_C * 4 + AQ_R * AQ_C * 2),
    "act_bwd_f32_4001x3584": (
        ("act_bwd_flat_kernelIfLb1ELb0E", "act_bwd_flat_kernel<float, true, false, false>"),
        ("common.hpp", "act_bwd.hip", "gemm.hpp"),
        5 * AQ_R * AQ_C * 4),
}


def kernel_source_hash(files=FWD_KERNEL_SOURCES) -> str:
    """Hash of a kernel's translation unit with comments and blank space
    removed, so a counter measurement stays valid across comment-only edits
    and changes to other kernels."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "swiglu_mlp_fwd_amd", "csrc")
    for fn in files:
        with open(os.path.join(csrc, fn), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        text = " ".join(text.split())
        h.update(fn.encode() + text.encode())
    return h.hexdigest()[:16]


def digest_traffic(name: str, fetch_csv: str, write_csv: str) -> None:
    """HBM bytes per launch of one kernel from two --pmc runs: its FETCH_SIZE /
    WRITE_SIZE counters (KiB per dispatch), each scaled by (known bytes /
    counter reading) of a plain 1 GiB copy measured in the same run."""
    import csv
    tags, files, algo = TRAFFIC_KERNELS[name][:3]
    grid = TRAFFIC_KERNELS[name][3] if len(TRAFFIC_KERNELS[name]) > 3 else None

    def per_kernel(path, counter):
        vals = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            kname = r["Kernel_Name"]
            mine = any(t in kname for t in tags) and (grid is None or int(r["Grid_Size"]) == grid)
            key = "k" if mine else ("copy" if COPY_KERNEL_TAG in kname else None)
            if key is None:
                continue
            vals.setdefault(key, {}).setdefault(r["Dispatch_Id"], 0.0)
            vals[key][r["Dispatch_Id"]] += float(r["Counter_Value"])
        # The kernel: mean over its dispatches.  The calibration: the 1 GiB
        # copies, the largest copy dispatches (a leg's own buffer clones are
        # copies too, and smaller).
        copies = sorted(vals.get("copy", {}).values())
        top = [v for v in copies if v >= 0.9 * copies[-1]]
        return {"k": sum(vals["k"].values()) / len(vals["k"]), "copy": sum(top) / len(top)}

    f = per_kernel(fetch_csv, "FETCH_SIZE")
    w = per_kernel(write_csv, "WRITE_SIZE")
    sf = COPY_BYTES / (f["copy"] * 1024.0)
    sw = COPY_BYTES / (w["copy"] * 1024.0)
    fetch_b = f["k"] * 1024.0 * sf
    write_b = w["k"] * 1024.0 * sw
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as fh:
            out = json.load(fh)
    except (OSError, ValueError):
        out = {}
    out[name] = {
        "source_hash": kernel_source_hash(files),
        "bytes_per_launch": round(fetch_b + write_b),
        "fetch_bytes": round(fetch_b), "write_bytes": round(write_b),
        "fetch_kib_raw": round(f["k"], 1), "write_kib_raw": round(w["k"], 1),
        "copy_fetch_kib_raw": round(f["copy"], 1), "copy_write_kib_raw": round(w["copy"], 1),
        "fetch_scale": round(sf, 4), "write_scale": round(sw, 4),
        "algorithmic_bytes": algo}
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1, sort_keys=True)
        fh.write("\n")
    print(json.dumps({name: out[name]}))


def load_traffic(name: str):
    """HBM traffic per launch measured by rocprofv3 counters for `name`, if the
    committed measurement was taken on the current sources of that kernel."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(p) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(name)
    files = TRAFFIC_KERNELS[name][1] if name in TRAFFIC_KERNELS else FWD_KERNEL_SOURCES
    if not e or e.get("source_hash") != kernel_source_hash(files):
        return None
    return e.get("bytes_per_launch")


# MI355X: 8 XCDs (GRBM_GUI_ACTIVE counts per XCD), 256 CUs of 4 SIMDs.
N_XCD, N_SIMD = 8, 1024
NOMINAL_SCLK_GHZ = 2.4        # the clock the published peaks assume


def digest_cycles(name: str, csv_path: str) -> None:
    """Shader-clock cycles per launch of one kernel from a --pmc run that
    collected GRBM_GUI_ACTIVE (and, if present, SQ_VALU_MFMA_BUSY_CYCLES):
    the mean over its dispatches, per XCD (and per SIMD for the MFMA count)."""
    import csv
    tags, files = TRAFFIC_KERNELS[name][:2]
    grid = TRAFFIC_KERNELS[name][3] if len(TRAFFIC_KERNELS[name]) > 3 else None
    per = {}
    for r in csv.DictReader(open(csv_path)):
        if not any(t in r["Kernel_Name"] for t in tags) or (grid is not None and int(r["Grid_Size"]) != grid):
            continue
        d = per.setdefault(r["Dispatch_Id"], {})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    if not per or any("GRBM_GUI_ACTIVE" not in d for d in per.values()):
        raise SystemExit(f"{csv_path}: no GRBM_GUI_ACTIVE for {name}")
    n = len(per)
    entry = {"source_hash": kernel_source_hash(files), "dispatches": n,
             "cycles_per_launch": round(sum(d["GRBM_GUI_ACTIVE"] for d in per.values()) / n / N_XCD)}
    if all("SQ_VALU_MFMA_BUSY_CYCLES" in d for d in per.values()):
        entry["mfma_busy_cycles_per_simd"] = round(sum(d["SQ_VALU_MFMA_BUSY_CYCLES"] for d in per.values()) / n / N_SIMD)
    path = os.path.join(ROOT, "profiles", "cycles.json")
    try:
        with open(path) as fh:
            out = json.load(fh)
    except (OSError, ValueError):
        out = {}
    out[name] = entry
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1, sort_keys=True)
        fh.write("\n")
    print(json.dumps({name: entry}))


def clock_adjusted(name: str, achieved_tflops: float, launch_s: float):
    """The roofline at the clock the kernel actually ran at.  A launch of this
    kernel takes a nearly fixed number of shader cycles whatever the clock
    (the counter runs put it within 4 % over 1.46-1.92 GHz), so the mean
    clock of a timed launch is those cycles over its measured duration, and
    the dense-bf16 peak at that clock is the published one scaled by
    clock / 2.4 GHz.  None unless the cycles were counted on the current
    sources of the kernel."""
    p = os.path.join(ROOT, "profiles", "cycles.json")
    try:
        with open(p) as f:
            e = json.load(f).get(name)
    except (OSError, ValueError):
        return None
    if not e or e.get("source_hash") != kernel_source_hash(TRAFFIC_KERNELS[name][1]) or launch_s <= 0:
        return None
    ghz = e["cycles_per_launch"] / launch_s / 1e9
    peak = PEAK_BF16_TFLOPS * ghz / NOMINAL_SCLK_GHZ
    out = {"sclk_GHz": round(ghz, 3), "peak": round(peak, 1), "frac": round(achieved_tflops / peak, 4),
           "cycles_per_launch": e["cycles_per_launch"]}
    if "mfma_busy_cycles_per_simd" in e:
        out["mfma_busy_frac"] = round(e["mfma_busy_cycles_per_simd"] / e["cycles_per_launch"], 4)
    return out


def traffic_table():
    """Every counter-measured kernel whose sources are unchanged since the
    measurement: HBM bytes per launch against its algorithmic bytes."""
    out = {}
    for name, entry in TRAFFIC_KERNELS.items():
        algo = entry[2]
        b = load_traffic(name)
        if b is not None:
            out[name] = {"bytes": b, "algorithmic": algo, "ratio": round(b / algo, 3)}
    return out


# ------------------------------------------------------------------ timing protocol

def pct(xs, q):
    s = sorted(xs)
    if not s:
        return None
    k = (len(s) - 1) * q / 100.0
    lo, hi = math.floor(k), math.ceil(k)
    return s[lo] + (s[hi] - s[lo]) * (k - lo)


class Protocol:
    """A-B-C-C-B-A trials over one HIP graph per variant."""

    def __init__(self, torch, trials, graph_warmup):
        self.torch = torch
        self.trials = trials
        self.graph_warmup = graph_warmup

    def _graph(self, calls):
        torch = self.torch
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            calls[0]()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for c in calls:
                c()
        return g

    def run(self, variants: dict) -> dict:
        """variants: name -> list of closures, each launching one library call
        (the list is one graph's calls, rotating over buffers).  Returns
        per-call statistics in microseconds per variant."""
        torch = self.torch
        names = list(variants)
        for n in names:                                  # eager warm-up
            calls = variants[n]
            for i in range(self.graph_warmup):
                calls[i % len(calls)]()
        torch.cuda.synchronize()
        graphs = {n: self._graph(variants[n]) for n in names}
        for n in names:
            graphs[n].replay()
        torch.cuda.synchronize()
        samples = {n: [] for n in names}
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(2 * len(names))]
        for _ in range(self.trials):
            order = names + names[::-1]
            for k, n in enumerate(order):
                ev[k][0].record()
                graphs[n].replay()
                ev[k][1].record()
            torch.cuda.synchronize()
            for k, n in enumerate(order):
                samples[n].append(ev[k][0].elapsed_time(ev[k][1]) * 1e3 / len(variants[n]))
        eager = {n: [] for n in names}
        for _ in range(3):
            for n in names:
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for c in variants[n]:
                    c()
                e1.record()
                torch.cuda.synchronize()
                eager[n].append(e0.elapsed_time(e1) * 1e3 / len(variants[n]))
        del graphs
        out = {}
        for n in names:
            xs = samples[n]
            out[n] = {"p50_us": round(pct(xs, 50), 3), "p90_us": round(pct(xs, 90), 3), "p99_us": round(pct(xs, 99), 3),
                      "mean_us": round(sum(xs) / len(xs), 3), "samples_us": [round(v, 3) for v in xs],
                      "eager_p50_us": round(pct(eager[n], 50), 3), "calls_per_graph": len(variants[n])}
        return out


def err_stats(np, y, r):
    """max / mean absolute error and cosine of y against the oracle r (finite
    elements of r; non-finite positions must match)."""
    import oracle
    y = np.asarray(y, np.float64).reshape(-1)
    r = np.asarray(r, np.float64).reshape(-1)
    fin = np.isfinite(r)
    same_nonfinite = bool(np.array_equal(np.isnan(y[~fin]), np.isnan(r[~fin])))
    d = np.abs(y[fin] - r[fin])
    return {"max_abs_err": float(d.max(initial=0.0)), "mean_abs_err": float(d.mean()) if d.size else 0.0,
            "cosine": round(float(oracle.cosine(y[fin], r[fin])), 9) if d.size else 1.0,
            "normwise_rel_err": float(oracle.normwise_rel_err(y[fin], r[fin])) if d.size else 0.0,
            "nonfinite_match": same_nonfinite}


def host_cores():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    try:
        from threadpoolctl import threadpool_info
        blas = max((i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"), default=1)
    except Exception:  # noqa: BLE001
        blas = n
    return n, blas


def timed(fn):
    t = time.perf_counter()
    r = fn()
    return r, time.perf_counter() - t


# ------------------------------------------------------------------ main

def main():
    args = parse()
    if args.digest_traffic:
        digest_traffic(*args.digest_traffic)
        return
    if args.digest_cycles:
        digest_cycles(*args.digest_cycles)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library runs on one GPU and has no "
              "multi-GPU path; run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from swiglu_mlp_fwd_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    import swiglu_mlp_fwd_amd as S
    import synth

    S.lib()           # refuses a library built from other sources
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    P = Protocol(torch, args.trials, args.graph_warmup)
    ctx = dict(torch=torch, S=S, synth=synth, np=np, dev=dev, P=P, args=args)

    def to_dev_bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)
    ctx["to_dev_bf16"] = to_dev_bf16

    if args.only in ("decode", "act_quant", "act_bwd", "fp32", "tiny", "fwd_k_sweep", "traffic_decode",
                     "traffic_act_quant", "traffic_act_fwd", "traffic_act_bwd"):
        leg = {"decode": decode_leg, "act_quant": act_quant_leg, "act_bwd": act_bwd_leg, "fp32": fp32_leg,
               "tiny": tiny_leg, "fwd_k_sweep": fwd_k_sweep_leg,
               "traffic_decode": traffic_decode, "traffic_act_quant": traffic_act_quant,
               "traffic_act_fwd": traffic_act_fwd, "traffic_act_bwd": traffic_act_bwd}[args.only]
        res = leg(ctx)
        if args.only.startswith("traffic"):
            copy_calibration(torch, dev, args.steps)
        if res:
            print(json.dumps(res), flush=True)
        log("done")
        return

    # ------------------------------------------------------------ headline
    t0 = time.time()
    d4 = synth.train_bf16(M4, N4, K4, seed=0)
    x, wg, wu, dh = (to_dev_bf16(d4[k]) for k in ("x", "wg", "wu", "dh"))
    ws = torch.empty(S.bwd_workspace_bytes(torch.bfloat16, M4, N4, K4), dtype=torch.uint8, device=dev)
    h = torch.empty((M4, N4), dtype=torch.bfloat16, device=dev)
    grads = (torch.empty((M4, K4), dtype=torch.bfloat16, device=dev), torch.empty((N4, K4), dtype=torch.bfloat16, device=dev),
             torch.empty((N4, K4), dtype=torch.bfloat16, device=dev))
    torch.cuda.synchronize()
    log(f"inputs ready in {time.time() - t0:.1f}s")

    def step():
        S.fwd(x, wg, wu, out=h)
        S.bwd(x, wg, wu, dh, workspace=ws, out=grads)

    if args.only in ("step", "fwd", "traffic", "traffic_bwd"):
        for _ in range(args.warmup + args.steps):
            if args.only in ("step", "traffic_bwd"):
                step()
            else:
                S.fwd(x, wg, wu, out=h)
        if args.only in ("traffic", "traffic_bwd"):
            del ws, grads
            torch.cuda.empty_cache()
            copy_calibration(torch, dev, args.steps)
        torch.cuda.synchronize()
        log("done")
        return
    train = dict(x=x, wg=wg, wu=wu, dh=dh, ws=ws, h=h, grads=grads, d4=d4)
    if args.only in ("train_fwd", "train_bwd"):
        res = (train_fwd_leg if args.only == "train_fwd" else train_bwd_leg)(ctx, train)
        print(json.dumps(res), flush=True)
        log("done")
        return

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    fwd_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record()
    for i in range(args.steps):
        fwd_ev[i][0].record()
        S.fwd(x, wg, wu, out=h)
        fwd_ev[i][1].record()
        S.bwd(x, wg, wu, dh, workspace=ws, out=grads)
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    t_step = start.elapsed_time(end) * 1e-3 / args.steps
    fwd_samples = [a.elapsed_time(b) * 1e-3 for a, b in fwd_ev]
    t_fwd = sum(fwd_samples) / args.steps
    flops_step = 12.0 * M4 * N4 * K4
    value = flops_step / t_step / 1e12
    fwd_tflops = 4.0 * M4 * N4 * K4 / t_fwd / 1e12
    log(f"step {t_step * 1e3:.3f} ms ({value:.1f} TFLOP/s); fwd {t_fwd * 1e3:.3f} ms ({fwd_tflops:.1f} TFLOP/s); "
        f"host wall {wall:.2f}s")

    # The dense bf16 rate the chip sustains (register-only MFMA loop), as
    # context for the roofline fraction against the published peak: the best
    # of three rounds of five calls after a warm-up (the clock settles).
    sink = torch.empty(1024, dtype=torch.float32, device=dev)
    for _ in range(3):
        S.probe_mfma(4096, 1024, sink)
    torch.cuda.synchronize()
    mfma_tf = 0.0
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            mfma_flops = S.probe_mfma(4096, 1024, sink)
        e1.record()
        torch.cuda.synchronize()
        mfma_tf = max(mfma_tf, mfma_flops / (e0.elapsed_time(e1) * 1e-3 / 5) / 1e12)
    log(f"mfma probe: {mfma_tf:.1f} TFLOP/s sustained ({mfma_tf / PEAK_BF16_TFLOPS:.3f} of the published peak)")
    del sink

    traffic = load_traffic("fwd_dual_gemm_bf16_8192x14336x4096")
    ncores, blas = host_cores()
    result = {
        "metric": "fused SwiGLU TFLOP/s (M=8192) + cold GB/s (M=1..8), % of roofline",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_step * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seed 0): x~N(0,1), Wg,Wu~N(0,0.02), dh~N(0,0.01)",
        "config": {"workload": "fused SwiGLU gate/up training step (forward + backward), bf16, fp32 accumulation",
                   "M": M4, "K": K4, "N": N4, "flops_per_step": "12*M*N*K (recompute not credited)",
                   "parallelism": "single GPU"},
        "roofline": {
            "kernel": "fused dual GEMM forward (x Wg^T, x Wu^T, SiLU-gate epilogue)",
            "bound": "mfma",
            "achieved": round(fwd_tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(fwd_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "avg_launch_ms": round(t_fwd * 1e3, 4),
            "launch_ms_samples": [round(v * 1e3, 4) for v in fwd_samples],
            "mfma_probe_TFLOPs": round(mfma_tf, 1),
            "frac_of_mfma_probe": round(fwd_tflops / mfma_tf, 4),
            "clock_adjusted": clock_adjusted("fwd_dual_gemm_bf16_8192x14336x4096", fwd_tflops, t_fwd),
        },
        "fwd_ms": round(t_fwd * 1e3, 4),
        "bwd_ms": round((t_step - t_fwd) * 1e3, 4),
        "bwd_tflops_8MNK": round(8.0 * M4 * N4 * K4 / (t_step - t_fwd) / 1e12, 2),
        "host": {"cores": ncores, "blas_threads": blas},
        "protocol": {"trials": args.trials, "order": "A-B-C-C-B-A", "graph_warmup_calls": args.graph_warmup,
                     "calls_per_graph": args.iters, "calls_per_graph_gemm": args.gemm_iters,
                     "timing": "HIP events around each graph launch; per-call time = graph time / calls",
                     "eager": "3 x (calls per graph) eager calls, events around each batch"},
        "traffic_by_kernel": traffic_table(),
        "legs": {},
        "oracle": {},
    }
    def run_leg(name, fn, *fa):
        # A leg that raises is recorded with its error (and its traceback on
        # stderr); the headline line is still printed.
        try:
            result["legs"][name] = fn(*fa)
        except Exception as e:
            traceback.print_exc()
            result["legs"][name] = {"error": f"{type(e).__name__}: {e}"}
            torch.cuda.synchronize()
            torch.cuda.empty_cache()

    if not args.no_extra:
        run_leg("train_fwd", train_fwd_leg, ctx, train, result["oracle"])
        run_leg("train_bwd", train_bwd_leg, ctx, train, result["oracle"])
    del h, grads, train
    sample_inputs = {k: d4[k] for k in ("x", "wg", "wu", "dh")}
    del x, wg, wu, dh, ws, d4
    torch.cuda.empty_cache()

    # ------------------------------------------------------------ other legs
    if not args.no_extra:
        run_leg("decode", decode_leg, ctx, result["oracle"])
        run_leg("act_quant", act_quant_leg, ctx, result["oracle"])
        run_leg("act_bwd", act_bwd_leg, ctx, result["oracle"])
        run_leg("fp32", fp32_leg, ctx, result["oracle"])
        run_leg("tiny_fp32", tiny_leg, ctx, result["oracle"])

    # ------------------------------------------------------------ cpu baseline
    if not args.no_cpu_baseline:
        try:
            result["cpu_baseline"] = cpu_baseline(np, synth, sample_inputs, args.cpu_seconds, value)
        except Exception as e:
            traceback.print_exc()
            result["cpu_baseline"] = {"error": f"{type(e).__name__}: {e}"}

    print(json.dumps(result), flush=True)


def copy_calibration(torch, dev, n):
    """A plain device copy of 1 GiB, the known-size reference for the HBM counters."""
    src = torch.empty(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(max(n, 1)):
        dst.copy_(src)
    torch.cuda.synchronize()


# ------------------------------------------------------------------ legs

# Gate and up multipliers of the forward leg's multiplier variant (a gate
# scale below 1 and an up scale above, as in muP-style MLPs).
FWD_GATE_MULT, FWD_UP_MULT = 0.5, 2.0


def train_fwd_leg(ctx, t, oracle_times=None):
    """Forward variants at the headline shape; TFLOP/s and error on sampled rows."""
    torch, S, np, P, args = ctx["torch"], ctx["S"], ctx["np"], ctx["P"], ctx["args"]
    import oracle
    x, wg, wu, h = t["x"], t["wg"], t["wu"], t["h"]
    dev = x.device
    q = torch.empty((M4, N4), dtype=torch.uint8, device=dev)
    sc = torch.empty((M4, N4 // 32), dtype=torch.uint8, device=dev)
    h2 = torch.empty_like(h)
    n = args.gemm_iters
    variants = {
        "swiglu": [lambda: S.fwd(x, wg, wu, out=h)] * n,
        "geglu": [lambda: S.fwd(x, wg, wu, out=h2, act="gelu_tanh")] * n,
        "swiglu_fp8": [lambda: S.fwd_fp8(x, wg, wu, out=(q, sc, None))] * n,
        "geglu_fp8": [lambda: S.fwd_fp8(x, wg, wu, act="gelu_tanh", out=(q, sc, None))] * n,
        # projection multipliers (two more multiplies per output element)
        "swiglu_mult": [lambda: S.fwd(x, wg, wu, out=h2, gate_mult=FWD_GATE_MULT, up_mult=FWD_UP_MULT)] * n,
    }
    stats = P.run(variants)
    flops = 4.0 * M4 * N4 * K4
    for k, v in stats.items():
        v["TFLOPs_p50"] = round(flops / (v["p50_us"] * 1e-6) / 1e12, 2)
        v["frac_of_bf16_peak"] = round(v["TFLOPs_p50"] / PEAK_BF16_TFLOPS, 4)
        v["launches_per_call"] = LAUNCHES["fwd"]
        log(f"train_fwd {k}: p50 {v['p50_us'] / 1e3:.4f} ms, {v['TFLOPs_p50']:.1f} TFLOP/s "
            f"(eager {v['eager_p50_us'] / 1e3:.4f} ms)")
    # error on 64 sampled rows (the oracle computes them one by one)
    rows = np.unique(np.concatenate([[0, M4 - 1], np.random.default_rng(4).integers(0, M4, 62)]))
    d4, synth = t["d4"], ctx["synth"]
    f = {k: synth.bf16_bits_to_f32(d4[k]).astype(np.float64) for k in ("wg", "wu")}
    xr = synth.bf16_bits_to_f32(d4["x"][rows]).astype(np.float64)
    ri = torch.as_tensor(rows, device=dev)
    for act, out in (("silu", h), ("gelu_tanh", h2)):
        S.fwd(x, wg, wu, out=out, act=act)
        torch.cuda.synchronize()
        ref, secs = timed(lambda: oracle.glu_fwd(xr, f["wg"], f["wu"], act))
        key = "swiglu" if act == "silu" else "geglu"
        stats[key]["vs_oracle_sampled_rows"] = err_stats(np, out[ri].float().cpu().numpy(), ref)
        stats[key]["vs_oracle_rows"] = len(rows)
        if act == "silu" and oracle_times is not None:
            oracle_times["train_fwd_sampled"] = {"seconds": round(secs, 3), "rows": len(rows),
                                                 "seconds_full_extrapolated": round(secs * M4 / len(rows), 2),
                                                 "note": "full-size time extrapolated linearly in rows"}
    S.fwd(x, wg, wu, out=h2, gate_mult=FWD_GATE_MULT, up_mult=FWD_UP_MULT)
    torch.cuda.synchronize()
    ref = oracle.glu_fwd(xr, f["wg"], f["wu"], "silu", FWD_GATE_MULT, FWD_UP_MULT)
    stats["swiglu_mult"]["vs_oracle_sampled_rows"] = err_stats(np, h2[ri].float().cpu().numpy(), ref)
    stats["swiglu_mult"]["multipliers"] = {"gate": FWD_GATE_MULT, "up": FWD_UP_MULT}
    for act, key in (("silu", "swiglu_fp8"), ("gelu_tanh", "geglu_fp8")):
        S.fwd_fp8(x, wg, wu, act=act, out=(q, sc, None))
        torch.cuda.synchronize()
        qq = q[ri].cpu().numpy()
        ee = sc[ri].cpu().numpy().astype(np.int64) - 127
        deq = oracle.e4m3_decode(qq) * np.exp2(np.repeat(ee, 32, axis=1).astype(np.float64))
        ref = oracle.glu_fwd(xr, f["wg"], f["wu"], act)
        stats[key]["vs_oracle_sampled_rows"] = err_stats(np, deq, ref)
        stats[key]["note"] = "error of the dequantised E4M3 codes x 2^E against the exact h"
    del q, sc, h2
    return {"M": M4, "N": N4, "K": K4, "flops_per_call": "4*M*N*K", "variants": stats}


def train_bwd_leg(ctx, t, oracle_times=None):
    """The backward at the headline shape (SwiGLU, GeGLU); TFLOP/s on 8 M N K."""
    torch, S, np, P, args = ctx["torch"], ctx["S"], ctx["np"], ctx["P"], ctx["args"]
    import oracle
    x, wg, wu, dh, ws, grads = t["x"], t["wg"], t["wu"], t["dh"], t["ws"], t["grads"]
    n = args.gemm_iters
    variants = {"swiglu": [lambda: S.bwd(x, wg, wu, dh, workspace=ws, out=grads)] * n,
                "geglu": [lambda: S.bwd(x, wg, wu, dh, workspace=ws, out=grads, act="gelu_tanh")] * n}
    stats = P.run(variants)
    for k, v in stats.items():
        v["TFLOPs_8MNK_p50"] = round(8.0 * M4 * N4 * K4 / (v["p50_us"] * 1e-6) / 1e12, 2)
        v["TFLOPs_12MNK_incl_recompute_p50"] = round(12.0 * M4 * N4 * K4 / (v["p50_us"] * 1e-6) / 1e12, 2)
        v["launches_per_call"] = LAUNCHES["bwd_bf16"]
        log(f"train_bwd {k}: p50 {v['p50_us'] / 1e3:.4f} ms (eager {v['eager_p50_us'] / 1e3:.4f} ms)")
    S.bwd(x, wg, wu, dh, workspace=ws, out=grads)
    torch.cuda.synchronize()
    d4, synth = t["d4"], ctx["synth"]
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, M4 - 1], rng.integers(0, M4, 30)]))
    cols = np.unique(np.concatenate([[0, N4 - 1], rng.integers(0, N4, 30)]))
    f = {k: synth.bf16_bits_to_f32(d4[k]).astype(np.float64) for k in ("x", "wg", "wu", "dh")}
    (dxr, sx) = timed(lambda: oracle.swiglu_bwd_dx_rows(f["x"], f["wg"], f["wu"], f["dh"], rows))
    ((dwgr, dwur), sw) = timed(lambda: oracle.swiglu_bwd_dw_rows(f["x"], f["wg"], f["wu"], f["dh"], cols))
    dev = x.device
    stats["swiglu"]["vs_oracle_sampled"] = {
        "dx_rows": err_stats(np, grads[0][torch.as_tensor(rows, device=dev)].float().cpu().numpy(), dxr),
        "dwg_rows": err_stats(np, grads[1][torch.as_tensor(cols, device=dev)].float().cpu().numpy(), dwgr),
        "dwu_rows": err_stats(np, grads[2][torch.as_tensor(cols, device=dev)].float().cpu().numpy(), dwur),
        "sampled": f"{len(rows)} rows of dX, {len(cols)} rows of dWg and dWu"}
    if oracle_times is not None:
        oracle_times["train_bwd_sampled"] = {"seconds": round(sx + sw, 3),
                                             "sampled": f"{len(rows)} rows of dX, {len(cols)} rows of dWg, dWu"}
    return {"M": M4, "N": N4, "K": K4, "variants": stats}


# Launch shapes of the dual-stream read (threads, 16-byte chunks of each
# buffer in flight per lane, max workgroups); None is swiglu_probe_read2's.
READ_SHAPES = (None, (256, 8, 4096), (256, 2, 16384), (512, 1, 16384), (512, 2, 16384))


def decode_leg(ctx, oracle_times=None):
    torch, S, np, P, args, synth = ctx["torch"], ctx["S"], ctx["np"], ctx["P"], ctx["args"], ctx["synth"]
    import oracle
    dev, to_dev_bf16 = ctx["dev"], ctx["to_dev_bf16"]
    out = {"unit": "GB/s", "bytes": "2*N*K*2 + M*K*2 + M*N*2 per call", "launches_per_call": LAUNCHES["gemv"],
           "floor": ("those bytes over the faster p50 time of the read-only twin and the dual-stream read, per M; "
                     "the read in the fastest of READ_SHAPES launch shapes at each (N, K)"),
           "shapes": []}
    for (N, K, copies) in DECODE_SHAPES:
        d = synth.decode_bf16(8, N, K, seed=0)
        wg0, wu0 = to_dev_bf16(d["wg"]), to_dev_bf16(d["wu"])
        W = [(wg0.clone(), wu0.clone()) for _ in range(copies)]
        del wg0, wu0
        wgf = synth.bf16_bits_to_f32(d["wg"]).astype(np.float64)
        wuf = synth.bf16_bits_to_f32(d["wu"]).astype(np.float64)
        sink = torch.zeros(max(4096, N), dtype=torch.int32, device=dev)
        entry = {"N": N, "K": K, "copies": copies, "working_set_MB": round(copies * 2 * N * K * 2 / 1e6, 1), "per_M": []}
        reps = max(1, args.iters // copies)
        # The dual-stream read in several launch shapes; the fastest is the
        # stream side of the floor at every M of this shape.
        sweep = P.run({("default" if sh is None else "x".join(map(str, sh))):
                       [(lambda a=a, b=b, sh=sh: S.probe_read2(a, b, sink, shape=sh)) for _ in range(reps) for (a, b) in W]
                       for sh in READ_SHAPES})
        best = min(sweep, key=lambda k: sweep[k]["p50_us"])
        best_shape = dict(zip((("default" if sh is None else "x".join(map(str, sh))) for sh in READ_SHAPES), READ_SHAPES))[best]
        entry["stream_shapes_us_p50"] = {k: v["p50_us"] for k, v in sweep.items()}
        entry["stream_shape"] = best
        for M in (1, 2, 4, 8):
            x = to_dev_bf16(d["x"][:M].copy())
            outs = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _ in range(copies)]
            variants = {
                "gemv": [(lambda a=a, b=b, o=o: S.gemv_fwd(x, a, b, out=o)) for _ in range(reps) for (a, b), o in zip(W, outs)],
                "twin": [(lambda a=a, b=b: S.probe_gemv_read(x, a, b, sink)) for _ in range(reps) for (a, b) in W],
                "stream": [(lambda a=a, b=b: S.probe_read2(a, b, sink, shape=best_shape)) for _ in range(reps) for (a, b) in W],
            }
            if M in (1, 8):
                # the GELU-tanh gate (GeGLU) on the same stream of weights
                variants["gemv_geglu"] = [(lambda a=a, b=b, o=o: S.gemv_fwd(x, a, b, out=o, act="gelu_tanh"))
                                          for _ in range(reps) for (a, b), o in zip(W, outs)]
            st = P.run(variants)
            # One byte basis for all three: the decode call's algorithmic
            # bytes over each variant's time, so the floor is the faster of
            # the twin and the stream and frac_of_floor a ratio of times.
            nbytes = 2 * N * K * 2 + M * K * 2 + M * N * 2
            gbs = {k: nbytes / (v["p50_us"] * 1e-6) / 1e9 for k, v in st.items()}
            floor = max(gbs["twin"], gbs["stream"])
            S.gemv_fwd(x, W[0][0], W[0][1], out=outs[0])
            torch.cuda.synchronize()
            xf = synth.bf16_bits_to_f32(d["x"][:M]).astype(np.float64)
            ref, secs = timed(lambda: oracle.glu_fwd(xf, wgf, wuf))
            e = {"M": M, "us_p50": st["gemv"]["p50_us"], "us_p90": st["gemv"]["p90_us"], "us_p99": st["gemv"]["p99_us"],
                 "GBs": round(gbs["gemv"], 1), "floor_GBs": round(floor, 1),
                 "twin_us_p50": st["twin"]["p50_us"], "stream_us_p50": st["stream"]["p50_us"],
                 "frac_of_floor": round(gbs["gemv"] / floor, 4), "frac_of_8TBs": round(gbs["gemv"] / PEAK_HBM_GBS, 4),
                 "eager_us_p50": st["gemv"]["eager_p50_us"],
                 "vs_oracle": err_stats(np, outs[0].float().cpu().numpy(), ref),
                 "samples_us": {k: v["samples_us"] for k, v in st.items()}}
            if "gemv_geglu" in st:
                S.gemv_fwd(x, W[0][0], W[0][1], out=outs[0], act="gelu_tanh")
                torch.cuda.synchronize()
                e["geglu"] = {"us_p50": st["gemv_geglu"]["p50_us"], "GBs": round(gbs["gemv_geglu"], 1),
                              "frac_of_floor": round(gbs["gemv_geglu"] / floor, 4),
                              "vs_oracle": err_stats(np, outs[0].float().cpu().numpy(),
                                                     oracle.glu_fwd(xf, wgf, wuf, "gelu_tanh"))}
                log(f"decode N={N} K={K} M={M} GeGLU: {e['geglu']['us_p50']:.2f} us, "
                    f"{e['geglu']['frac_of_floor']:.1%} of the floor")
            entry["per_M"].append(e)
            if oracle_times is not None:
                oracle_times[f"decode_{N}x{K}_M{M}"] = {"seconds": round(secs, 4), "full": True,
                                                        "GBs": round(nbytes / secs / 1e9, 2)}
            log(f"decode N={N} K={K} M={M}: {e['us_p50']:.2f} us, {e['GBs']:.0f} GB/s ({e['frac_of_floor']:.1%} of "
                f"floor {floor:.0f}: twin {gbs['twin']:.0f}, stream {gbs['stream']:.0f}; {e['frac_of_8TBs']:.1%} of 8 TB/s)")
        out["shapes"].append(entry)
        del W, sink
        torch.cuda.empty_cache()
    return out


def act_quant_leg(ctx, oracle_times=None):
    torch, S, np, P, args, synth = ctx["torch"], ctx["S"], ctx["np"], ctx["P"], ctx["args"], ctx["synth"]
    import oracle
    dev = ctx["dev"]
    R, C = AQ_R, AQ_C
    d = synth.act_quant_f32(R, C, seed=0)
    g0, u0 = torch.from_numpy(d["gate"]).to(dev), torch.from_numpy(d["up"]).to(dev)
    copies = 4
    G = [g0.clone() for _ in range(copies)]
    U = [u0.clone() for _ in range(copies)]
    del g0, u0
    outs = [(torch.empty((R, C), dtype=torch.uint8, device=dev), torch.empty((R, C // 32), dtype=torch.uint8, device=dev),
             torch.empty(1, dtype=torch.int64, device=dev), None) for _ in range(copies)]
    nbytes = 2 * R * C * 4 + R * C + R * C // 32
    reps = max(1, args.iters // copies)
    variants = {
        "no_clamp": [(lambda i=i: S.act_quant(G[i], U[i], math.inf, out=outs[i])) for _ in range(reps) for i in range(copies)],
        "clamp_7": [(lambda i=i: S.act_quant(G[i], U[i], 7.0, out=outs[i])) for _ in range(reps) for i in range(copies)],
        # The clamp without its count: the difference to clamp_7 is what the
        # count costs (its zeroing launch and the per-workgroup atomics).
        "clamp_7_no_count": [(lambda i=i: S.act_quant(G[i], U[i], 7.0, out=(outs[i][0], outs[i][1], None, None)))
                             for _ in range(reps) for i in range(copies)],
        "no_clamp_geglu": [(lambda i=i: S.act_quant(G[i], U[i], math.inf, out=outs[i], act="gelu_tanh"))
                           for _ in range(reps) for i in range(copies)],
        "stream_twin": [(lambda i=i: S.probe_act_quant_stream(G[i], U[i], outs[i][0], outs[i][1]))
                        for _ in range(reps) for i in range(copies)],
    }
    st = P.run(variants)
    floor = nbytes / (st["stream_twin"]["p50_us"] * 1e-6) / 1e9
    res = {"rows": R, "cols": C, "copies": copies, "bytes_per_call": nbytes, "unit": "GB/s",
           "stream_floor_GBs": round(floor, 1), "variants": st}
    for k, v in st.items():
        v["GBs_p50"] = round(nbytes / (v["p50_us"] * 1e-6) / 1e9, 1)
        v["frac_of_8TBs"] = round(v["GBs_p50"] / PEAK_HBM_GBS, 4)
        v["frac_of_stream_floor"] = round(v["GBs_p50"] / floor, 4)
        v["launches_per_call"] = LAUNCHES["act_quant_count"] if k == "clamp_7" else LAUNCHES["act_quant"]
        log(f"act_quant {R}x{C} {k}: {v['p50_us']:.2f} us, {v['GBs_p50']:.0f} GB/s "
            f"({v['frac_of_stream_floor']:.1%} of the twin's {floor:.0f})")
    # against the oracle (clamp off and L = 7), from the inputs
    g64, u64 = d["gate"].astype(np.float64), d["up"].astype(np.float64)
    for key, L in (("no_clamp", math.inf), ("clamp_7", 7.0)):
        q, s, cnt, _ = S.act_quant(G[0], U[0], L, out=outs[0])
        torch.cuda.synchronize()
        (rq, rs, rc, _), secs = timed(lambda: oracle.act_quant(g64, u64, L))
        qn, sn = q.cpu().numpy(), s.cpu().numpy()
        nan = (rq & 0x7F) == 0x7F
        dist = np.abs(oracle.e4m3_ordinal(qn[~nan]) - oracle.e4m3_ordinal(rq[~nan]))
        st[key]["vs_oracle"] = {"scale_bytes_equal_frac": float((sn == rs).mean()),
                                "codes_equal_frac": float((qn == rq).mean()),
                                "max_code_ulp": int(dist.max(initial=0)),
                                "nan_positions_match": bool(np.array_equal((qn & 0x7F) == 0x7F, nan)),
                                "clamp_count_match": int(cnt.item()) == int(rc)}
        if oracle_times is not None:
            oracle_times[f"act_quant_{key}"] = {"seconds": round(secs, 3), "full": True,
                                                "GBs": round(nbytes / secs / 1e9, 3)}
    # the non-quantised forward (fp32 and bf16 h)
    fv = {}
    hs = {}
    for dt, nb in ((torch.float32, 4), (torch.bfloat16, 2)):
        key = "f32_h" if nb == 4 else "bf16_h"
        hs[key] = [torch.empty((R, C), dtype=dt, device=dev) for _ in range(copies)]
        fv[key] = [(lambda i=i, hh=hs[key]: S.act_fwd(G[i], U[i], math.inf, out=(hh[i], None)))
                   for _ in range(reps) for i in range(copies)]
    st2 = P.run(fv)
    for key, v in st2.items():
        nb = 4 if key == "f32_h" else 2
        v["bytes_per_call"] = 2 * R * C * 4 + R * C * nb
        v["GBs_p50"] = round(v["bytes_per_call"] / (v["p50_us"] * 1e-6) / 1e9, 1)
        v["frac_of_8TBs"] = round(v["GBs_p50"] / PEAK_HBM_GBS, 4)
        v["launches_per_call"] = LAUNCHES["act_fwd"]
        S.act_fwd(G[0], U[0], math.inf, out=(hs[key][0], None))
        torch.cuda.synchronize()
        ref, secs = timed(lambda: oracle.act_fwd(g64, u64, math.inf)[0])
        v["vs_oracle"] = err_stats(np, hs[key][0].float().cpu().numpy(), ref)
        if oracle_times is not None and key == "f32_h":
            oracle_times["act_fwd"] = {"seconds": round(secs, 3), "full": True}
        log(f"act_fwd {R}x{C} {key}: {v['p50_us']:.2f} us, {v['GBs_p50']:.0f} GB/s")
    res["act_fwd"] = st2
    del G, U, outs, hs
    torch.cuda.empty_cache()
    return res


def act_bwd_leg(ctx, oracle_times=None):
    torch, S, np, P, args, synth = ctx["torch"], ctx["S"], ctx["np"], ctx["P"], ctx["args"], ctx["synth"]
    import oracle
    dev = ctx["dev"]
    R, C = AQ_R, AQ_C
    d = synth.act_bwd_f32(R, C, seed=0)
    copies = 4
    reps = max(1, args.iters // copies)
    ins = [tuple(torch.from_numpy(d[k]).to(dev) for k in ("gate", "up", "dy", "weights")) for _ in range(copies)]
    ins16 = [tuple(t.to(torch.bfloat16) for t in i[:3]) for i in ins]
    outs = [(torch.empty((R, C), dtype=torch.float32, device=dev), torch.empty((R, C), dtype=torch.float32, device=dev),
             torch.empty(R, dtype=torch.float32, device=dev)) for _ in range(copies)]
    outs16 = [(torch.empty((R, C), dtype=torch.bfloat16, device=dev), torch.empty((R, C), dtype=torch.bfloat16, device=dev))
              for _ in range(copies)]
    u8 = dict(dtype=torch.uint8, device=dev)
    outs8 = [(torch.empty((R, C), **u8), torch.empty((R, C // 32), **u8), torch.empty((R, C), **u8),
              torch.empty((R, C // 32), **u8), None) for _ in range(copies)]
    variants = {
        "f32_clamp_0.5": [(lambda i=i: S.act_bwd(*ins[i][:3], 0.5, out=(outs[i][0], outs[i][1], None)))
                          for _ in range(reps) for i in range(copies)],
        "f32_weights_wgrad": [(lambda i=i: S.act_bwd(*ins[i][:3], math.inf, weights=ins[i][3], out=outs[i]))
                              for _ in range(reps) for i in range(copies)],
        "bf16_clamp_0.5": [(lambda i=i: S.act_bwd(*ins16[i], 0.5, out=(outs16[i][0], outs16[i][1], None)))
                           for _ in range(reps) for i in range(copies)],
        "f32_in_e4m3_out_clamp_0.5": [(lambda i=i: S.act_bwd_fp8(*ins[i][:3], 0.5, out=outs8[i]))
                                      for _ in range(reps) for i in range(copies)],
        "bf16_in_e4m3_out_clamp_0.5": [(lambda i=i: S.act_bwd_fp8(*ins16[i], 0.5, out=outs8[i]))
                                       for _ in range(reps) for i in range(copies)],
    }
    st = P.run(variants)
    e4m3_out = 2 * (R * C + R * C // 32)              # codes and scale bytes of dgate and dup
    nb = {"f32_clamp_0.5": 5 * R * C * 4, "f32_weights_wgrad": 5 * R * C * 4 + 2 * R * 4, "bf16_clamp_0.5": 5 * R * C * 2,
          "f32_in_e4m3_out_clamp_0.5": 3 * R * C * 4 + e4m3_out, "bf16_in_e4m3_out_clamp_0.5": 3 * R * C * 2 + e4m3_out}
    for k, v in st.items():
        v["bytes_per_call"] = nb[k]
        v["GBs_p50"] = round(nb[k] / (v["p50_us"] * 1e-6) / 1e9, 1)
        v["frac_of_8TBs"] = round(v["GBs_p50"] / PEAK_HBM_GBS, 4)
        v["launches_per_call"] = LAUNCHES["act_bwd"]
        log(f"act_bwd {R}x{C} {k}: {v['p50_us']:.2f} us, {v['GBs_p50']:.0f} GB/s")
    g, u, dy = (d[k].astype(np.float64) for k in ("gate", "up", "dy"))
    S.act_bwd(*ins[0][:3], 0.5, out=(outs[0][0], outs[0][1], None))
    torch.cuda.synchronize()
    (rg, ru, _), secs = timed(lambda: oracle.act_bwd(g, u, dy, 0.5, None))
    st["f32_clamp_0.5"]["vs_oracle"] = {"dgate": err_stats(np, outs[0][0].cpu().numpy(), rg),
                                        "dup": err_stats(np, outs[0][1].cpu().numpy(), ru)}
    if oracle_times is not None:
        oracle_times["act_bwd_f32_clamp_0.5"] = {"seconds": round(secs, 3), "full": True,
                                                 "GBs": round(nb["f32_clamp_0.5"] / secs / 1e9, 3)}
    # E4M3 outputs: the decoded blocks (code x 2^E) against the oracle's exact
    # dgate and dup, and the share of scale bytes equal to the oracle's.
    S.act_bwd_fp8(*ins[0][:3], 0.5, out=outs8[0])
    torch.cuda.synchronize()
    (rqg, rsg, rqu, rsu, _), secs8 = timed(lambda: oracle.act_bwd_fp8(g, u, dy, 0.5, None))
    vs = {}
    for name, q, sc, rs, ref in (("dgate", outs8[0][0], outs8[0][1], rsg, rg), ("dup", outs8[0][2], outs8[0][3], rsu, ru)):
        qn, scn = q.cpu().numpy(), sc.cpu().numpy()
        val = oracle.e4m3_decode(qn) * np.exp2(np.repeat(scn.astype(np.float64) - 127.0, 32, axis=1))
        vs[name] = err_stats(np, val, ref)
        vs[name]["scale_bytes_equal_frac"] = round(float(np.mean(scn == rs)), 6)
    st["f32_in_e4m3_out_clamp_0.5"]["vs_oracle"] = vs
    if oracle_times is not None:
        oracle_times["act_bwd_fp8_f32_clamp_0.5"] = {"seconds": round(secs8, 3), "full": True,
                                                     "GBs": round(nb["f32_in_e4m3_out_clamp_0.5"] / secs8 / 1e9, 3)}
    del ins, ins16, outs, outs16, outs8
    torch.cuda.empty_cache()
    return {"rows": R, "cols": C, "copies": copies, "unit": "GB/s", "variants": st}


def fp32_leg(ctx, oracle_times=None):
    torch, S, np, P, args, synth = ctx["torch"], ctx["S"], ctx["np"], ctx["P"], ctx["args"], ctx["synth"]
    import oracle
    dev = ctx["dev"]
    M, N, K = F32_M, F32_N, F32_K
    d = synth.gemm_fp32(M, N, K, seed=0)
    x, wg, wu = (torch.from_numpy(d[k]).to(dev) for k in ("x", "wg", "wu"))
    h = torch.empty((M, N), dtype=torch.float32, device=dev)
    h2 = torch.empty_like(h)
    dh = torch.from_numpy(synth.normal_f32((M, N), 1.0, 0, synth.STREAM_DH)).to(dev)
    ws = torch.empty(S.bwd_workspace_bytes(torch.float32, M, N, K), dtype=torch.uint8, device=dev)
    grads = (torch.empty((M, K), dtype=torch.float32, device=dev), torch.empty((N, K), dtype=torch.float32, device=dev),
             torch.empty((N, K), dtype=torch.float32, device=dev))
    n = args.gemm_iters
    st = P.run({"swiglu": [lambda: S.fwd(x, wg, wu, out=h)] * n,
                "geglu": [lambda: S.fwd(x, wg, wu, out=h2, act="gelu_tanh")] * n,
                "swiglu_bwd": [lambda: S.bwd(x, wg, wu, dh, workspace=ws, out=grads)] * n})
    for k, v in st.items():
        # the backward is credited with 8 M N K (dX, dWg, dWu), its recompute not
        flops = (8.0 if k.endswith("_bwd") else 4.0) * M * N * K
        v["TFLOPs_p50"] = round(flops / (v["p50_us"] * 1e-6) / 1e12, 2)
        v["frac_of_fp32_peak"] = round(v["TFLOPs_p50"] / PEAK_FP32_TFLOPS, 4)
        v["launches_per_call"] = LAUNCHES["bwd_f32"] if k.endswith("_bwd") else LAUNCHES["fwd"]
        log(f"fp32 {M}x{N}x{K} {k}: {v['p50_us'] / 1e3:.3f} ms, {v['TFLOPs_p50']:.1f} TFLOP/s")
    S.fwd(x, wg, wu, out=h)
    torch.cuda.synchronize()
    ref, secs = timed(lambda: oracle.glu_fwd(d["x"], d["wg"], d["wu"]))
    st["swiglu"]["vs_oracle"] = err_stats(np, h.cpu().numpy(), ref)
    if oracle_times is not None:
        oracle_times["fp32_fwd_4001x3584x2048"] = {"seconds": round(secs, 3), "full": True,
                                                   "TFLOPs": round(4.0 * M * N * K / secs / 1e12, 4)}
    # the backward against the oracle on 32 sampled rows of dX and of dWg, dWu
    S.bwd(x, wg, wu, dh, workspace=ws, out=grads)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([[0, M - 1], rng.integers(0, M, 30)]))
    cols = np.unique(np.concatenate([[0, N - 1], rng.integers(0, N, 30)]))
    f = {k: d[k].astype(np.float64) for k in ("x", "wg", "wu")}
    f["dh"] = dh.cpu().numpy().astype(np.float64)
    dxr = oracle.swiglu_bwd_dx_rows(f["x"], f["wg"], f["wu"], f["dh"], rows)
    dwgr, dwur = oracle.swiglu_bwd_dw_rows(f["x"], f["wg"], f["wu"], f["dh"], cols)
    ri, ci = torch.as_tensor(rows, device=dev), torch.as_tensor(cols, device=dev)
    st["swiglu_bwd"]["vs_oracle_sampled"] = {
        "dx_rows": err_stats(np, grads[0][ri].cpu().numpy(), dxr),
        "dwg_rows": err_stats(np, grads[1][ci].cpu().numpy(), dwgr),
        "dwu_rows": err_stats(np, grads[2][ci].cpu().numpy(), dwur),
        "sampled": f"{len(rows)} rows of dX, {len(cols)} rows of dWg and dWu"}
    del x, wg, wu, h, h2, dh, ws, grads
    torch.cuda.empty_cache()
    return {"M": M, "N": N, "K": K, "variants": st}


def tiny_leg(ctx, oracle_times=None):
    torch, S, np, P, args, synth = ctx["torch"], ctx["S"], ctx["np"], ctx["P"], ctx["args"], ctx["synth"]
    import oracle
    dev = ctx["dev"]
    d = synth.tiny_fp32(seed=0)
    t = {k: torch.from_numpy(v).to(dev) for k, v in d.items()}
    h = torch.empty((4, 128), dtype=torch.float32, device=dev)
    grads = (torch.empty((4, 64), dtype=torch.float32, device=dev), torch.empty((128, 64), dtype=torch.float32, device=dev),
             torch.empty((128, 64), dtype=torch.float32, device=dev))
    ws = torch.empty(S.bwd_workspace_bytes(torch.float32, 4, 128, 64), dtype=torch.uint8, device=dev)
    st = P.run({"fwd": [lambda: S.fwd(t["x"], t["wg"], t["wu"], out=h)] * args.iters,
                "bwd": [lambda: S.bwd(t["x"], t["wg"], t["wu"], t["dh"], workspace=ws, out=grads)] * args.iters})
    st["fwd"]["launches_per_call"] = LAUNCHES["fwd"]
    st["bwd"]["launches_per_call"] = LAUNCHES["bwd_f32"]
    S.fwd(t["x"], t["wg"], t["wu"], out=h)
    S.bwd(t["x"], t["wg"], t["wu"], t["dh"], workspace=ws, out=grads)
    torch.cuda.synchronize()
    f = {k: v.astype(np.float64) for k, v in d.items()}
    (rh, sf) = timed(lambda: oracle.swiglu_fwd(f["x"], f["wg"], f["wu"]))
    (rb, sb) = timed(lambda: oracle.swiglu_bwd(f["x"], f["wg"], f["wu"], f["dh"]))
    st["fwd"]["vs_oracle"] = err_stats(np, h.cpu().numpy(), rh)
    st["bwd"]["vs_oracle"] = {k: err_stats(np, y.cpu().numpy(), r) for k, y, r in zip(("dx", "dwg", "dwu"), grads, rb)}
    if oracle_times is not None:
        oracle_times["tiny_fp32_fwd_bwd"] = {"seconds": round(sf + sb, 5), "full": True}
    log(f"tiny fp32: fwd {st['fwd']['p50_us']:.2f} us, bwd {st['bwd']['p50_us']:.2f} us")
    return {"M": 4, "N": 128, "K": 64, "variants": st}


def fwd_k_sweep_leg(ctx, oracle_times=None):
    """The bf16 forward at M = 8192, N = 14336 and K = 1024 .. 8192, and the
    least-squares line t = a + b K through the p50 times: a is the part of a
    launch that does not scale with the reduction (ring prologue, epilogue,
    workgroup turnover)."""
    torch, S, np, P, args = ctx["torch"], ctx["S"], ctx["np"], ctx["P"], ctx["args"]
    dev = ctx["dev"]
    M, N = M4, N4
    g = torch.Generator(device=dev).manual_seed(0)
    times = {}
    for K in (1024, 2048, 4096, 8192):
        x = torch.randn(M, K, device=dev, generator=g).to(torch.bfloat16)
        wg = (torch.randn(N, K, device=dev, generator=g) * 0.02).to(torch.bfloat16)
        wu = (torch.randn(N, K, device=dev, generator=g) * 0.02).to(torch.bfloat16)
        h = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
        st = P.run({"fwd": [lambda: S.fwd(x, wg, wu, out=h)] * args.gemm_iters})
        times[K] = st["fwd"]["p50_us"]
        log(f"fwd K={K}: {times[K] / 1e3:.4f} ms, {4 * M * N * K / times[K] / 1e6:.1f} TFLOP/s")
        del x, wg, wu, h
        torch.cuda.empty_cache()
    ks = np.array(sorted(times), dtype=np.float64)
    b, a = np.polyfit(ks, np.array([times[int(k)] for k in ks]), 1)
    log(f"fit: t = {a:.1f} us + {b * 1000:.1f} us per 1000 K; fixed share at K = {K4}: {a / times[K4]:.3f}")
    return {"M": M, "N": N, "p50_us": times, "intercept_us": round(a, 2), "us_per_1000_K": round(b * 1000, 2)}


# ------------------------------------------------------------------ traffic legs (counter runs)

def traffic_decode(ctx):
    """gemv at (11008, 4096), M = 1 and 8 (x staged whole), 4 rotated copies,
    and at (24576, 6144), M = 8 (x staged in phases), 2 copies; a few calls
    each."""
    torch, S, synth = ctx["torch"], ctx["S"], ctx["synth"]
    for (N, K, copies, Ms) in ((11008, 4096, 4, (1, 8)), (24576, 6144, 2, (8,))):
        d = synth.decode_bf16(8, N, K, seed=0)
        wg0, wu0 = ctx["to_dev_bf16"](d["wg"]), ctx["to_dev_bf16"](d["wu"])
        W = [(wg0.clone(), wu0.clone()) for _ in range(copies)]
        del wg0, wu0
        for M in Ms:
            x = ctx["to_dev_bf16"](d["x"][:M].copy())
            o = torch.empty((M, N), dtype=torch.bfloat16, device=ctx["dev"])
            for _ in range(2):
                for a, b in W:
                    S.gemv_fwd(x, a, b, out=o)
        torch.cuda.synchronize()
        del W
        torch.cuda.empty_cache()
    return None


def _aq_inputs(ctx):
    torch, synth = ctx["torch"], ctx["synth"]
    d = synth.act_quant_f32(AQ_R, AQ_C, seed=0)
    return [(torch.from_numpy(d["gate"]).to(ctx["dev"]), torch.from_numpy(d["up"]).to(ctx["dev"])) for _ in range(4)]


def traffic_act_quant(ctx):
    torch, S = ctx["torch"], ctx["S"]
    ins = _aq_inputs(ctx)
    q = torch.empty((AQ_R, AQ_C), dtype=torch.uint8, device=ctx["dev"])
    s = torch.empty((AQ_R, AQ_C // 32), dtype=torch.uint8, device=ctx["dev"])
    for _ in range(2):
        for g, u in ins:
            S.act_quant(g, u, math.inf, out=(q, s, None, None))
    torch.cuda.synchronize()
    return None


def traffic_act_fwd(ctx):
    torch, S = ctx["torch"], ctx["S"]
    ins = _aq_inputs(ctx)
    h = torch.empty((AQ_R, AQ_C), dtype=torch.bfloat16, device=ctx["dev"])
    for _ in range(2):
        for g, u in ins:
            S.act_fwd(g, u, math.inf, out=(h, None))
    torch.cuda.synchronize()
    return None


def traffic_act_bwd(ctx):
    torch, S, synth = ctx["torch"], ctx["S"], ctx["synth"]
    d = synth.act_bwd_f32(AQ_R, AQ_C, seed=0)
    ins = [tuple(torch.from_numpy(d[k]).to(ctx["dev"]) for k in ("gate", "up", "dy")) for _ in range(4)]
    dg = torch.empty((AQ_R, AQ_C), dtype=torch.float32, device=ctx["dev"])
    du = torch.empty_like(dg)
    for _ in range(2):
        for g, u, dy in ins:
            S.act_bwd(g, u, dy, 0.5, out=(dg, du, None))
    torch.cuda.synchronize()
    return None


# ------------------------------------------------------------------ cpu baseline

def cpu_baseline(np, synth, d, target_s, gpu_value):
    """The fp64 oracle, as it stands, on the first m rows of the headline
    workload: forward for those rows and the backward contributions of those
    rows (dX rows, and dWg/dWu summed over the m rows only)."""
    import oracle
    ncores, blas = host_cores()
    wg = synth.bf16_bits_to_f32(d["wg"]).astype(np.float64)
    wu = synth.bf16_bits_to_f32(d["wu"]).astype(np.float64)

    def run(m):
        x = synth.bf16_bits_to_f32(d["x"][:m]).astype(np.float64)
        dh = synth.bf16_bits_to_f32(d["dh"][:m]).astype(np.float64)
        t = time.perf_counter()
        oracle.swiglu_fwd(x, wg, wu)
        oracle.swiglu_bwd(x, wg, wu, dh)
        return time.perf_counter() - t

    m0 = 64
    run(m0)                       # warm the BLAS thread pool
    t0 = run(m0)
    m = int(max(m0, min(M4, m0 * target_s / max(t0, 1e-3))))
    t = run(m)
    flops = 12.0 * m * N4 * K4
    v = flops / t / 1e12
    log(f"cpu oracle: {m} rows in {t:.1f}s on {blas} BLAS threads ({ncores} cores) -> {v:.4f} TFLOP/s")
    return {"value": round(v, 5), "unit": "TFLOP/s", "cores": blas, "kind": "oracle",
            "sample": f"fp64 numpy oracle forward + backward on the first {m} of {M4} rows of the headline "
                      f"workload (12*m*N*K flops credited, as for value); {t:.1f}s",
            "host_cores": ncores, "seconds": round(t, 2),
            "seconds_full_extrapolated": round(t * M4 / m, 2),
            "gpu_over_oracle": round(gpu_value / v, 1)}


if __name__ == "__main__":
    main()
