#!/usr/bin/env python3
"""Benchmark of the fused SwiGLU gate/up stage on one MI355X.

Prints ONE JSON line on stdout (progress goes to stderr).

Headline workload: one training step of the fused stage at M=8192 tokens,
K=4096, N=14336 in bf16 (fp32 accumulation): the fused forward
h = SiLU(x Wg^T) * (x Wu^T) followed by the backward (dX, dWg, dWu).
value = algorithmic TFLOP/s of that step, 12 M N K flops per step (4 M N K
forward, 8 M N K for dX and dW; the recompute of g and u in the backward is
not credited).  Inputs are synthetic (seed 0) and resident in HBM before the
timed region starts.

The same run also measures, after the timed region and outside `value`:
  decode   the M=1..8 weight-streaming forward at (N,K)=(6912,1536) with 16
           rotated weight copies and (11008,4096) with 4 copies (each call
           reads cold weights), in GB/s, beside a pure dual-stream read of
           the same buffers (the cold-read floor);
  act_quant the elementwise SwiGLU + FP8 block quantisation of [4001, 3584]
           fp32 inputs (4 rotated copies), in GB/s;
  act_bwd  the elementwise SwiGLU backward on [4001, 3584] fp32 gate/up/dy
           (4 rotated copies): clamp 0.5 without weights, and per-row weights
           with the weight gradient and no clamp, in GB/s;
  fp32     the IEEE-fp32 fused forward at M=4001, K=2048, N=3584, in TFLOP/s;
  geglu    the GeGLU forward (GELU-tanh gate) at the headline shape, in TFLOP/s;
  cpu_baseline  the fp64 oracle on a row sample of the headline workload,
           timed on the host cores.
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

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6     # dense bf16 MFMA, MI355X
PEAK_FP32_TFLOPS = 157.3      # dense fp32 matrix, MI355X
PEAK_HBM_GBS = 8000.0         # HBM3E, MI355X

M4, N4, K4 = 8192, 14336, 4096


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="target host time of the oracle sample")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extra", action="store_true", help="skip the decode / act_quant / fp32 legs")
    p.add_argument("--only", choices=["step", "fwd", "decode", "act_quant", "act_bwd", "fp32", "fwd_fp8", "traffic"], default=None,
                   help="profiling aid: run one leg only (no JSON contract); 'traffic' runs the headline "
                        "forward and a 1 GiB copy (the counter calibration) for the --pmc runs")
    p.add_argument("--digest-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"), default=None,
                   help="read the counter_collection.csv files of two rocprofv3 --pmc runs of "
                        "'--only traffic' (FETCH_SIZE, then WRITE_SIZE) and write profiles/traffic.json")
    return p.parse_args()


COPY_BYTES = 1 << 30            # calibration copy: reads and writes this many bytes per launch
FWD_KERNEL_TAG = "gemm_dma_kernelIDF16bLNS0_3EpiE0E"   # mangled-name fragment of the bf16 fused forward
COPY_KERNEL_TAG = "copy"


def digest_traffic(fetch_csv: str, write_csv: str) -> None:
    """HBM bytes per launch of the fused forward from two --pmc runs: the
    FETCH_SIZE / WRITE_SIZE counters (KiB per dispatch) of the forward kernel,
    each scaled by (known bytes / counter reading) of a plain 1 GiB copy
    measured in the same run."""
    import csv

    def per_kernel(path, counter):
        vals = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            name = r["Kernel_Name"]
            tag = "fwd" if FWD_KERNEL_TAG in name else ("copy" if COPY_KERNEL_TAG in name else None)
            if tag is None:
                continue
            vals.setdefault(tag, {}).setdefault(r["Dispatch_Id"], 0.0)
            vals[tag][r["Dispatch_Id"]] += float(r["Counter_Value"])
        return {k: sum(v.values()) / len(v) for k, v in vals.items()}

    f = per_kernel(fetch_csv, "FETCH_SIZE")
    w = per_kernel(write_csv, "WRITE_SIZE")
    sf = COPY_BYTES / (f["copy"] * 1024.0)
    sw = COPY_BYTES / (w["copy"] * 1024.0)
    fetch_b = f["fwd"] * 1024.0 * sf
    write_b = w["fwd"] * 1024.0 * sw
    out = {"fwd_dual_gemm_bf16_8192x14336x4096": {
        "source_hash": kernel_source_hash(),
        "bytes_per_launch": round(fetch_b + write_b),
        "fetch_bytes": round(fetch_b), "write_bytes": round(write_b),
        "fetch_kib_raw": round(f["fwd"], 1), "write_kib_raw": round(w["fwd"], 1),
        "copy_fetch_kib_raw": round(f["copy"], 1), "copy_write_kib_raw": round(w["copy"], 1),
        "fetch_scale": round(sf, 4), "write_scale": round(sw, 4),
        "algorithmic_bytes": (M4 * K4 + 2 * N4 * K4 + M4 * N4) * 2}}
    path = os.path.join(ROOT, "profiles", "traffic.json")
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")
    print(json.dumps(out))


# The translation unit of the forward dual GEMM: the kernel file and the
# headers it includes.
FWD_KERNEL_SOURCES = ("common.hpp", "fp8.hpp", "gemm.hip", "gemm.hpp")


def kernel_source_hash() -> str:
    """Hash of the forward kernel's sources with comments and blank space
    removed, so that a counter measurement stays valid across comment-only
    edits and changes to other kernels."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "swiglu_mlp_fwd_amd", "csrc")
    for fn in FWD_KERNEL_SOURCES:
        with open(os.path.join(csrc, fn), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        text = " ".join(text.split())
        h.update(fn.encode() + text.encode())
    return h.hexdigest()[:16]


def load_traffic(name: str):
    """HBM traffic per launch measured by rocprofv3 counters for `name`, if the
    committed measurement was taken on the current kernel sources."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(p) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(name)
    if not e or e.get("source_hash") != kernel_source_hash():
        return None
    return e.get("bytes_per_launch")


class Timer:
    """HIP events on the current stream (the stream the library launches on)."""

    def __init__(self, torch):
        self.torch = torch

    def ev(self):
        return self.torch.cuda.Event(enable_timing=True)


def graph_time_per_call(torch, calls, reps=5):
    """Capture `calls` (a list of closures launching one library call each) in
    one HIP graph, replay it `reps` times, return seconds per call."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for c in calls:  # warm once outside capture
            c()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for c in calls:
            c()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    samples = []
    for _ in range(reps):
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        samples.append(e0.elapsed_time(e1) * 1e-3 / len(calls))
    del g
    samples.sort()
    return samples[len(samples) // 2], samples


def main():
    args = parse()
    if args.digest_traffic:
        digest_traffic(*args.digest_traffic)
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

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def to_dev_bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    # ------------------------------------------------------------ headline
    t0 = time.time()
    d4 = synth.train_bf16(M4, N4, K4, seed=0)
    x, wg, wu, dh = (to_dev_bf16(d4[k]) for k in ("x", "wg", "wu", "dh"))
    ws = torch.empty(S.bwd_workspace_bytes(torch.bfloat16, M4, N4, K4), dtype=torch.uint8, device=dev)
    h = torch.empty((M4, N4), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    log(f"inputs ready in {time.time() - t0:.1f}s")

    def step():
        S.fwd(x, wg, wu, out=h)
        return S.bwd(x, wg, wu, dh, workspace=ws)

    if args.only in ("step", "fwd", "traffic"):
        for _ in range(args.warmup + args.steps):
            if args.only == "step":
                step()
            else:
                S.fwd(x, wg, wu, out=h)
        if args.only == "traffic":
            del ws
            torch.cuda.empty_cache()
            src = torch.empty(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev).fill_(1.0)
            dst = torch.empty_like(src)
            for _ in range(args.steps):
                dst.copy_(src)
        torch.cuda.synchronize()
        log("done")
        return
    if args.only == "fwd_fp8":
        fwd_fp8_leg(torch, S, x, wg, wu)
        log("done")
        return
    if args.only in ("decode", "act_quant", "act_bwd", "fp32"):  # noqa: SIM102
        del x, wg, wu, dh, ws, h
        torch.cuda.empty_cache()
        leg = {"decode": lambda: decode_leg(torch, S, synth, np, dev, to_dev_bf16),
               "act_quant": lambda: act_quant_leg(torch, S, synth, np, dev),
               "act_bwd": lambda: act_bwd_leg(torch, S, synth, np, dev),
               "fp32": lambda: fp32_leg(torch, S, synth, np, dev)}[args.only]
        leg()
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
        S.bwd(x, wg, wu, dh, workspace=ws)
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    t_step = start.elapsed_time(end) * 1e-3 / args.steps
    t_fwd = sum(a.elapsed_time(b) for a, b in fwd_ev) * 1e-3 / args.steps
    flops_step = 12.0 * M4 * N4 * K4
    value = flops_step / t_step / 1e12
    fwd_tflops = 4.0 * M4 * N4 * K4 / t_fwd / 1e12
    log(f"step {t_step * 1e3:.3f} ms ({value:.1f} TFLOP/s); fwd {t_fwd * 1e3:.3f} ms ({fwd_tflops:.1f} TFLOP/s); "
        f"host wall {wall:.2f}s")

    # The dense bf16 rate the chip sustains (register-only MFMA loop), as
    # context for the roofline fraction against the published peak.
    # The clock takes a few calls to settle under this load: the best of three
    # rounds of five calls after a warm-up.
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
            "mfma_probe_TFLOPs": round(mfma_tf, 1),
            "frac_of_mfma_probe": round(fwd_tflops / mfma_tf, 4),
        },
        "fwd_ms": round(t_fwd * 1e3, 4),
        "bwd_ms": round((t_step - t_fwd) * 1e3, 4),
        "bwd_tflops_8MNK": round(8.0 * M4 * N4 * K4 / (t_step - t_fwd) / 1e12, 2),
    }
    if not args.no_extra:
        result["geglu"] = geglu_leg(torch, S, x, wg, wu, h, dh, ws)
        result["fwd_fp8"] = fwd_fp8_leg(torch, S, x, wg, wu)
    del h
    sample_inputs = {k: d4[k] for k in ("x", "wg", "wu", "dh")}
    del x, wg, wu, dh, ws
    torch.cuda.empty_cache()

    # ------------------------------------------------------------ extra legs
    if not args.no_extra:
        result["decode"] = decode_leg(torch, S, synth, np, dev, to_dev_bf16)
        result["act_quant"] = act_quant_leg(torch, S, synth, np, dev)
        result["act_bwd"] = act_bwd_leg(torch, S, synth, np, dev)
        result["fp32"] = fp32_leg(torch, S, synth, np, dev)

    # ------------------------------------------------------------ cpu baseline
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(np, synth, sample_inputs, args.cpu_seconds)

    print(json.dumps(result), flush=True)


def decode_leg(torch, S, synth, np, dev, to_dev_bf16):
    out = {"unit": "GB/s", "bytes": "2*N*K*2 + M*K*2 + M*N*2 per call", "shapes": []}
    sink = torch.zeros(4096, dtype=torch.int32, device=dev)
    for (N, K, copies) in ((6912, 1536, 16), (11008, 4096, 4)):
        d = synth.decode_bf16(8, N, K, seed=0)
        wg0, wu0 = to_dev_bf16(d["wg"]), to_dev_bf16(d["wu"])
        W = [(wg0.clone(), wu0.clone()) for _ in range(copies)]
        del wg0, wu0
        reps_per_graph = 4
        probe_calls = [(lambda a=a, b=b: S.probe_read2(a, b, sink)) for _ in range(reps_per_graph) for (a, b) in W]
        t_probe, _ = graph_time_per_call(torch, probe_calls)
        floor = 2 * N * K * 2 / t_probe / 1e9
        entry = {"N": N, "K": K, "copies": copies,
                 "working_set_MB": round(copies * 2 * N * K * 2 / 1e6, 1),
                 "read_floor_GBs": round(floor, 1), "per_M": []}
        for M in (1, 2, 4, 8):
            x = to_dev_bf16(d["x"][:M].copy())
            outs = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _ in range(copies)]
            calls = [(lambda a=a, b=b, o=o: S.gemv_fwd(x, a, b, out=o))
                     for _ in range(reps_per_graph) for (a, b), o in zip(W, outs)]
            t, _ = graph_time_per_call(torch, calls)
            nbytes = 2 * N * K * 2 + M * K * 2 + M * N * 2
            gbs = nbytes / t / 1e9
            entry["per_M"].append({"M": M, "us": round(t * 1e6, 3), "GBs": round(gbs, 1),
                                   "frac_of_floor": round(gbs / floor, 4), "frac_of_8TBs": round(gbs / PEAK_HBM_GBS, 4)})
            log(f"decode N={N} K={K} M={M}: {t * 1e6:.2f} us, {gbs:.0f} GB/s ({gbs / floor:.1%} of read floor {floor:.0f})")
        out["shapes"].append(entry)
        del W
        torch.cuda.empty_cache()
    return out


def act_quant_leg(torch, S, synth, np, dev):
    R, C = 4001, 3584
    d = synth.act_quant_f32(R, C, seed=0)
    g0, u0 = torch.from_numpy(d["gate"]).to(dev), torch.from_numpy(d["up"]).to(dev)
    copies = 4
    G = [g0.clone() for _ in range(copies)]
    U = [u0.clone() for _ in range(copies)]
    del g0, u0
    outs = [(torch.empty((R, C), dtype=torch.uint8, device=dev), torch.empty((R, C // 32), dtype=torch.uint8, device=dev),
             torch.empty(1, dtype=torch.int64, device=dev), None) for _ in range(copies)]
    nbytes = 2 * R * C * 4 + R * C + R * C // 32
    res = {"rows": R, "cols": C, "copies": copies, "bytes_per_call": nbytes, "unit": "GB/s"}
    for act, L in (("silu", math.inf), ("silu", 7.0), ("gelu_tanh", math.inf)):
        calls = [(lambda i=i: S.act_quant(G[i], U[i], L, out=outs[i], act=act)) for _ in range(4) for i in range(copies)]
        t, _ = graph_time_per_call(torch, calls)
        gbs = nbytes / t / 1e9
        key = ("no_clamp" if math.isinf(L) else "clamp_7") + ("" if act == "silu" else "_geglu")
        res[key] = {"us": round(t * 1e6, 3), "GBs": round(gbs, 1), "frac_of_8TBs": round(gbs / PEAK_HBM_GBS, 4)}
        log(f"act_quant {R}x{C} {key}: {t * 1e6:.2f} us, {gbs:.0f} GB/s")
    # The non-quantised outputs (fp32 and bf16 h).
    for dt, nb in ((torch.float32, 4), (torch.bfloat16, 2)):
        hs = [torch.empty((R, C), dtype=dt, device=dev) for _ in range(copies)]
        calls = [(lambda i=i: S.act_fwd(G[i], U[i], math.inf, out=(hs[i], None))) for _ in range(4) for i in range(copies)]
        t, _ = graph_time_per_call(torch, calls)
        nbytes_h = 2 * R * C * 4 + R * C * nb
        gbs = nbytes_h / t / 1e9
        key = "act_fwd_" + ("f32" if nb == 4 else "bf16")
        res[key] = {"us": round(t * 1e6, 3), "GBs": round(gbs, 1), "bytes_per_call": nbytes_h,
                    "frac_of_8TBs": round(gbs / PEAK_HBM_GBS, 4)}
        log(f"act_fwd {R}x{C} {key}: {t * 1e6:.2f} us, {gbs:.0f} GB/s")
        del hs
    del G, U, outs
    torch.cuda.empty_cache()
    return res


def geglu_leg(torch, S, x, wg, wu, h, dh, ws):
    """GeGLU (GELU-tanh gate) on the headline inputs: the forward, and a
    training step (forward + backward)."""
    for _ in range(3):
        S.fwd(x, wg, wu, out=h, act="gelu_tanh")
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = 10
    e0.record()
    for _ in range(n):
        S.fwd(x, wg, wu, out=h, act="gelu_tanh")
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / n
    tf = 4.0 * M4 * N4 * K4 / t / 1e12
    log(f"geglu fwd {M4}x{N4}x{K4}: {t * 1e3:.3f} ms, {tf:.1f} TFLOP/s")

    def step():
        S.fwd(x, wg, wu, out=h, act="gelu_tanh")
        S.bwd(x, wg, wu, dh, workspace=ws, act="gelu_tanh")

    for _ in range(2):
        step()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(5):
        step()
    e1.record()
    torch.cuda.synchronize()
    ts = e0.elapsed_time(e1) * 1e-3 / 5
    log(f"geglu step {M4}x{N4}x{K4}: {ts * 1e3:.3f} ms, {12.0 * M4 * N4 * K4 / ts / 1e12:.1f} TFLOP/s (12MNK)")
    return {"M": M4, "N": N4, "K": K4, "ms": round(t * 1e3, 4), "TFLOPs": round(tf, 2),
            "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
            "step_ms": round(ts * 1e3, 4), "step_TFLOPs_12MNK": round(12.0 * M4 * N4 * K4 / ts / 1e12, 2)}


def fwd_fp8_leg(torch, S, x, wg, wu):
    """Forward with the 1x32 E4M3 quantisation of h fused into the epilogue,
    on the headline inputs (no h_out): h leaves as 1-byte codes + scales."""
    dev = x.device
    q = torch.empty((M4, N4), dtype=torch.uint8, device=dev)
    sc = torch.empty((M4, N4 // 32), dtype=torch.uint8, device=dev)
    res = {"M": M4, "N": N4, "K": K4}
    for act in ("silu", "gelu_tanh"):
        for _ in range(3):
            S.fwd_fp8(x, wg, wu, act=act, out=(q, sc, None))
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n = 10
        e0.record()
        for _ in range(n):
            S.fwd_fp8(x, wg, wu, act=act, out=(q, sc, None))
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) * 1e-3 / n
        tf = 4.0 * M4 * N4 * K4 / t / 1e12
        log(f"fwd_fp8 {act} {M4}x{N4}x{K4}: {t * 1e3:.3f} ms, {tf:.1f} TFLOP/s")
        res[act] = {"ms": round(t * 1e3, 4), "TFLOPs": round(tf, 2),
                    "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
    del q, sc
    return res


def act_bwd_leg(torch, S, synth, np, dev):
    R, C = 4001, 3584
    d = synth.act_bwd_f32(R, C, seed=0)
    copies = 4
    ins = [tuple(torch.from_numpy(d[k]).to(dev) for k in ("gate", "up", "dy", "weights")) for _ in range(copies)]
    outs = [(torch.empty((R, C), dtype=torch.float32, device=dev), torch.empty((R, C), dtype=torch.float32, device=dev),
             torch.empty(R, dtype=torch.float32, device=dev)) for _ in range(copies)]
    res = {"rows": R, "cols": C, "copies": copies, "unit": "GB/s"}
    for key, L, use_w in (("clamp_0.5", 0.5, False), ("weights_wgrad", math.inf, True)):
        nbytes = 5 * R * C * 4 + (2 * R * 4 if use_w else 0)
        calls = [(lambda i=i: S.act_bwd(ins[i][0], ins[i][1], ins[i][2], L, weights=ins[i][3] if use_w else None,
                                        out=(outs[i][0], outs[i][1], outs[i][2] if use_w else None)))
                 for _ in range(4) for i in range(copies)]
        t, _ = graph_time_per_call(torch, calls)
        gbs = nbytes / t / 1e9
        res[key] = {"us": round(t * 1e6, 3), "GBs": round(gbs, 1), "bytes_per_call": nbytes,
                    "frac_of_8TBs": round(gbs / PEAK_HBM_GBS, 4)}
        log(f"act_bwd {R}x{C} {key}: {t * 1e6:.2f} us, {gbs:.0f} GB/s")
    del ins, outs
    # bf16 tensors (weights and weight_grad fp32).
    ins = [tuple(t.to(torch.bfloat16) for t in (torch.from_numpy(d[k]).to(dev) for k in ("gate", "up", "dy")))
           for _ in range(copies)]
    outs = [(torch.empty((R, C), dtype=torch.bfloat16, device=dev), torch.empty((R, C), dtype=torch.bfloat16, device=dev))
            for _ in range(copies)]
    nbytes = 5 * R * C * 2
    calls = [(lambda i=i: S.act_bwd(ins[i][0], ins[i][1], ins[i][2], 0.5, out=(outs[i][0], outs[i][1], None)))
             for _ in range(4) for i in range(copies)]
    t, _ = graph_time_per_call(torch, calls)
    gbs = nbytes / t / 1e9
    res["bf16_clamp_0.5"] = {"us": round(t * 1e6, 3), "GBs": round(gbs, 1), "bytes_per_call": nbytes,
                             "frac_of_8TBs": round(gbs / PEAK_HBM_GBS, 4)}
    log(f"act_bwd {R}x{C} bf16_clamp_0.5: {t * 1e6:.2f} us, {gbs:.0f} GB/s")
    del ins, outs
    torch.cuda.empty_cache()
    return res


def fp32_leg(torch, S, synth, np, dev):
    M, N, K = 4001, 3584, 2048
    d = synth.gemm_fp32(M, N, K, seed=0)
    x, wg, wu = (torch.from_numpy(d[k]).to(dev) for k in ("x", "wg", "wu"))
    h = torch.empty((M, N), dtype=torch.float32, device=dev)
    for _ in range(3):
        S.fwd(x, wg, wu, out=h)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = 10
    e0.record()
    for _ in range(n):
        S.fwd(x, wg, wu, out=h)
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / n
    tf = 4.0 * M * N * K / t / 1e12
    log(f"fp32 fwd {M}x{N}x{K}: {t * 1e3:.3f} ms, {tf:.1f} TFLOP/s")
    del x, wg, wu, h
    torch.cuda.empty_cache()
    return {"M": M, "N": N, "K": K, "ms": round(t * 1e3, 4), "TFLOPs": round(tf, 2),
            "frac_of_fp32_peak": round(tf / PEAK_FP32_TFLOPS, 4)}


def cpu_baseline(np, synth, d, target_s):
    """The fp64 oracle, as it stands, on the first m rows of the headline
    workload: forward for those rows and the backward contributions of those
    rows (dX rows, and dWg/dWu summed over the m rows only)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max((i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"), default=1)
    except Exception:  # noqa: BLE001
        cores = os.cpu_count() or 1
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
    log(f"cpu oracle: {m} rows in {t:.1f}s on {cores} threads -> {flops / t / 1e12:.4f} TFLOP/s")
    return {"value": round(flops / t / 1e12, 5), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"fp64 numpy oracle forward + backward on the first {m} of {M4} rows of the headline "
                      f"workload (12*m*N*K flops credited, as for value); {t:.1f}s"}


if __name__ == "__main__":
    main()
