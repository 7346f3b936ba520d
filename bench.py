#!/usr/bin/env python3
"""Benchmark of the 4-bit quantize + W4 matmul path on one MI355X.

Headline workload (one "step"): the MXFP4 decode GEMV y = x W'^T with W
28672 x 8192 (MXFP4, 124.78 MB of codes + E8M0 scales), for the three
decode batches B = 1, 4 and 16 -- three launches, each streaming the whole
weight once.  Inputs are resident in HBM before timing.  Every launch reads
a different one of several identical weight copies, so no launch finds the
weights in the 256 MB Infinity Cache left there by the previous one.

value = weight bytes streamed per step / step time  (GB/s, higher is better)

The same JSON line carries:
  * roofline   -- the dominant GEMV launch: algorithmic bytes per launch
                  (weights + x + y) over its average duration, measured with
                  HIP events on the launch stream, against 8 TB/s;
  * cpu_baseline -- the CPU oracle (plain C quantizer/dequantizer + numpy
                  fp64 matmul) timed on the same workload on the host cores;
  * extra      -- the other workloads: weight quantization throughput, the
                  INT4 g128 GEMV, the NVFP4 W4A16 prefill GEMM, the MoE
                  grouped expert GEMM and the W4A4 MXFP4 GEMM.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # dense bf16 matrix cores
FP16_PEAK_TFLOPS = 2500.0      # dense fp16 matrix cores (the W4A4 NVFP4 kernel's)
FP4_PEAK_TFLOPS = 10100.0      # dense MXFP4 matrix cores
FP8_PEAK_TFLOPS = 5000.0       # dense FP8 matrix cores
GRAPH_STEPS = 10               # decode steps captured per HIP graph in the timed loop
IDLE_GAP_S = 0.5               # idle time before each extra workload
METRIC = "W4 GEMV weight GB/s and W4 GEMM TFLOP/s vs MI355X roofline, 1 GPU"


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--copies", type=int, default=6, help="weight copies rotated across launches")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--no-extra", action="store_true", help="headline workload only")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--only", default="", help="comma list of extra workloads to run")
    p.add_argument("--calibrate-copy", type=int, default=0, metavar="MB",
                   help="also run a plain device copy of MB megabytes three times (the reference "
                        "kernel for scaling HBM byte counters); prints nothing extra")
    return p.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class GraphTimer:
    """Average duration per launch of `fn`: `per_graph` calls are captured
    into one HIP graph (no host work between the kernels), the graph is
    replayed `replays` times between two HIP events on the replay stream."""

    def __init__(self, torch, fn, per_graph=1):
        self.torch = torch
        self.per_graph = per_graph
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(per_graph):   # warm the launch path once before capture
                fn(i)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            for i in range(per_graph):
                fn(i)
        torch.cuda.synchronize()

    def replay_ms(self, replays, warmup=3):
        t = self.torch
        for _ in range(warmup):
            self.graph.replay()
        t.cuda.synchronize()
        s, e = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(replays):
            self.graph.replay()
        e.record()
        t.cuda.synchronize()
        return s.elapsed_time(e) / replays

    def per_launch_ms(self, replays, warmup=3):
        return self.replay_ms(replays, warmup) / self.per_graph

    def per_launch_ms_each(self, replays):
        """Per-launch time of each replay separately (for a median)."""
        t = self.torch
        ev = [(t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)) for _ in range(replays)]
        for s, e in ev:
            s.record()
            self.graph.replay()
            e.record()
        t.cuda.synchronize()
        return [s.elapsed_time(e) / self.per_graph for s, e in ev]


def timed(torch, fn, iters, warmup=1, replays=3):
    """Average per-launch time of fn() from a graph of `iters` launches,
    replayed `replays` times after `warmup` untimed replays."""
    g = GraphTimer(torch, lambda i: fn(), per_graph=iters)
    return g.per_launch_ms(replays, warmup=warmup)


_MFMA_CEILING = {}


def mfma_ceiling(torch, q4, dev, kind):
    """TFLOP/s this part sustains for one kind of matrix instruction on
    random register operands (q4_mfma_probe, two waves per SIMD on every
    CU): the ceiling of a GEMM built on that instruction.  Random operands
    make the part lower its clock to stay within its power limit, so this is
    below the published dense peak.  Measured once per kind, after a short
    idle gap, over about 0.2 s of back-to-back launches."""
    if kind not in _MFMA_CEILING:
        sink = torch.zeros(q4.PROBE_MIX_SINK if kind.endswith(("_copy", "_mix")) else 1, dtype=torch.int32,
                           device=dev)
        iters = 4096 if kind.startswith("fp4") or kind == "fp8" else 8192
        flops = [0.0]

        def fn():
            flops[0] = q4.q4_mfma_probe(kind, iters, sink)

        torch.cuda.synchronize()
        time.sleep(IDLE_GAP_S)
        ms = timed(torch, fn, 20, warmup=10, replays=5)
        _MFMA_CEILING[kind] = flops[0] / (ms * 1e-3) / 1e12
    return _MFMA_CEILING[kind]


def with_ceiling(res, torch, q4, dev, kind, keys=("TFLOPs",), prefix="mfma_ceiling"):
    """Adds the measured ceiling of `kind` and each rate's fraction of it."""
    c = mfma_ceiling(torch, q4, dev, kind)
    res[f"{prefix}_TFLOPs"] = round(c, 1)
    res[f"{prefix}_kind"] = kind
    for k in keys:
        res[f"frac_{prefix}" if k == "TFLOPs" else f"frac_{prefix}_{k}"] = round(res[k] / c, 4)
    return res


def cpu_cores():
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    omp = os.environ.get("OMP_NUM_THREADS")
    return min(n, int(omp)) if omp and omp.isdigit() else n


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only (got --gpus {args.gpus}); "
              "the multi-GPU sharding of the path is described in DESIGN.md, not run.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import w4_gemm_amd as q4
    from w4_gemm_amd import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = "cuda:0"
    torch.cuda.set_device(0)
    q4.lib()  # fails loudly if the HIP library is missing

    if args.calibrate_copy:
        nbytes = args.calibrate_copy * 1000 * 1000
        src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # ---------------------------------------------------------------- headline
    log("generating the MXFP4 decode workload (28672 x 8192)")
    wl = workloads.mxfp4_gemv(seed=args.seed)
    W = wl.tensors["W"].to(dev)
    N, K = W.shape
    batches = wl.meta["batches"]
    xs = {b: wl.tensors[f"x{b}"].to(dev) for b in batches}
    q0 = q4.quantize(W, "mxfp4", layout="tiled")
    torch.cuda.synchronize()
    copies = [q0] + [q0.clone() for _ in range(args.copies - 1)]
    wbytes = q0.codes.numel() + q0.scales.numel()
    ys = {b: torch.empty((b, N), dtype=torch.bfloat16, device=dev) for b in batches}

    # one step = one GEMV per decode batch; step i uses weight copies
    # 3i, 3i+1, 3i+2 (mod the number of copies), so consecutive launches never
    # share a copy.  Steps are captured as HIP graphs and replayed: a graph of
    # GRAPH_STEPS consecutive steps (a whole number of copy-pattern periods,
    # as a decode loop captures many kernels per graph) for the bulk of the K
    # steps, one-step graphs for the remainder and the warmup.
    ncopy = len(copies)
    nb = len(batches)
    period = ncopy // __import__("math").gcd(ncopy, nb)   # steps until the copy pattern repeats
    graph_steps = period * max(1, GRAPH_STEPS // period)

    def step(i):
        for j, b in enumerate(batches):
            q4.q4_gemv(copies[(i * nb + j) % ncopy], xs[b], ys[b])

    step_graphs = [GraphTimer(torch, lambda _, i=i: step(i)) for i in range(period)]
    bulk = GraphTimer(torch, step, per_graph=graph_steps)
    for i in range(args.warmup):
        step_graphs[i % period].graph.replay()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(args.steps // graph_steps):
        bulk.graph.replay()
    for i in range(args.steps % graph_steps):
        step_graphs[i % period].graph.replay()
    t1.record()
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    ms_per_step = total_ms / args.steps
    value = nb * wbytes / (ms_per_step * 1e-3) / 1e9

    # per-kernel average launch duration: ncopy back-to-back launches of one
    # batch size on rotating copies, captured and replayed
    per_b = {}
    for b in batches:
        gt = GraphTimer(torch, lambda i, b=b: q4.q4_gemv(copies[i % ncopy], xs[b], ys[b]),
                        per_graph=ncopy * 4)
        ms = gt.per_launch_ms(max(3, args.steps // (ncopy * 4)))
        each = sorted(gt.per_launch_ms_each(9))
        alg = wbytes + b * K * 2 + b * N * 2
        per_b[b] = {"us": ms * 1e3, "us_median": each[len(each) // 2] * 1e3,
                    "weight_GBps": wbytes / (ms * 1e-3) / 1e9,
                    "alg_GBps": alg / (ms * 1e-3) / 1e9, "alg_bytes": alg}
    dom = max(batches, key=lambda b: per_b[b]["us"])
    achieved = per_b[dom]["alg_GBps"]
    traffic = None
    prof = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                        "gemv_mxfp4_28672x8192_traffic.json")
    if os.path.exists(prof):
        try:
            rec = json.load(open(prof))
            if rec.get("kernel_sha") == _kernel_sha("gemv.hip") and str(dom) in rec.get("bytes_per_launch", {}):
                traffic = rec["bytes_per_launch"][str(dom)]
        except Exception:
            traffic = None
    # the read ceiling: a plain streaming read (q4_read_probe) of a buffer of
    # the weight's size, rotating six copies past the last-level cache as the
    # GEMV does -- the rate the GEMV can approach on this part
    rbufs = [torch.full((wbytes,), i + 1, dtype=torch.uint8, device=dev) for i in range(ncopy)]
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    rgt = GraphTimer(torch, lambda i: q4.q4_read_probe(rbufs[i % ncopy], sink), per_graph=ncopy * 4)
    read_ms = rgt.per_launch_ms(max(3, args.steps // (ncopy * 4)))
    read_gbs = wbytes / (read_ms * 1e-3) / 1e9
    del rbufs, rgt
    # a measured device-to-device copy of 1 GB (1 GB read + 1 GB written),
    # reported beside the published peak as context
    csrc = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
    cdst = torch.empty_like(csrc)
    copy_ms = timed(torch, lambda: cdst.copy_(csrc), 4, warmup=1, replays=3)
    copy_gbs = 2 * csrc.numel() / (copy_ms * 1e-3) / 1e9
    del csrc, cdst
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": f"gemv_kernel<MXFP4> B={dom}", "alg_bytes_per_launch": per_b[dom]["alg_bytes"],
                "avg_launch_us": round(per_b[dom]["us"], 3),
                "read_ceiling_GBps": round(read_gbs, 1), "read_ceiling_us": round(read_ms * 1e3, 3),
                "read_ceiling_bytes": wbytes,
                "frac_of_read_ceiling": round(achieved / read_gbs, 4),
                "device_copy_GBps": round(copy_gbs, 1),
                "frac_of_device_copy": round(achieved / copy_gbs, 4)}

    extra = {"decode_gemv_per_batch": {str(b): {k: round(v, 3) for k, v in per_b[b].items()}
                                       for b in batches},
             "weight_copies": len(copies)}

    # the same GEMV on the row-major layout, for comparison
    rows_copies = [q4.quantize(W, "mxfp4")]
    rows_copies += [rows_copies[0].clone() for _ in range(args.copies - 1)]
    extra["decode_gemv_rowmajor_us"] = {}
    for b in batches:
        gt = GraphTimer(torch, lambda i, b=b: q4.q4_gemv(rows_copies[i % ncopy], xs[b], ys[b]),
                        per_graph=ncopy * 4)
        extra["decode_gemv_rowmajor_us"][str(b)] = round(gt.per_launch_ms(5) * 1e3, 3)
    del rows_copies

    # the same decode GEMV on the other tiled weight formats of the same
    # shape (INT4 g128, NVFP4, INT4 with a zero point), rotating copies
    extra["decode_gemv_tiled_other_formats_us"] = {}
    for fmt in ("int4", "nvfp4", "int4_zp"):
        fc = [q4.quantize(W, fmt, layout="tiled")]
        fc += [fc[0].clone() for _ in range(args.copies - 1)]
        fb = fc[0].nbytes
        res = {"weight_bytes": fb}
        for b in batches:
            gt = GraphTimer(torch, lambda i, b=b: q4.q4_gemv(fc[i % ncopy], xs[b], ys[b]), per_graph=ncopy * 4)
            us = gt.per_launch_ms(5) * 1e3
            res[str(b)] = {"us": round(us, 3), "weight_GBps": round(fb / (us * 1e-6) / 1e9, 1)}
        extra["decode_gemv_tiled_other_formats_us"][fmt] = res
        del fc

    # quantization of the decode weight
    empty = q4.empty_q4("mxfp4", N, K, device=dev, layout="tiled")
    ms = timed(torch, lambda: q4.q4_quantize(W, empty), 10, 3)
    qbytes = N * K * 2 + wbytes
    extra["quantize_mxfp4_28672x8192"] = {"us": round(ms * 1e3, 2),
                                          "GBps": round(qbytes / (ms * 1e-3) / 1e9, 1),
                                          "frac_hbm": round(qbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                          "bytes": qbytes}
    del empty
    # the same weight quantized to the other formats (bytes: bf16 read once
    # plus codes and scales written; NVFP4 also reads it in its tensor-amax
    # pass), and dequantized back to bf16 (codes and scales read, bf16 written)
    extra["quantize_28672x8192_other_formats"] = {}
    for fmt in ("int4", "nvfp4", "int4_zp"):
        ef = q4.empty_q4(fmt, N, K, device=dev, layout="tiled")
        fms = timed(torch, lambda ef=ef: q4.q4_quantize(W, ef), 10, 3)
        # NVFP4 reads the bf16 weight twice: the tensor-amax pass, then the
        # block pass (which needs the tensor scale first)
        reads = 2 if fmt == "nvfp4" else 1
        fbytes = reads * N * K * 2 + ef.nbytes
        extra["quantize_28672x8192_other_formats"][fmt] = {
            "us": round(fms * 1e3, 2), "GBps": round(fbytes / (fms * 1e-3) / 1e9, 1),
            "frac_hbm": round(fbytes / (fms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "bytes": fbytes,
            "weight_reads": reads}
        del ef
    # a row-major quantization of the same weight moved to the tiled layout
    # (q4_relayout: codes and scales read once and written once)
    rq = q4.quantize(W, "mxfp4", layout="rows")
    rt = q4.empty_q4("mxfp4", N, K, device=dev, layout="tiled")
    rms = timed(torch, lambda: q4.q4_relayout(rq, rt), 10, 3)
    rbytes = rq.nbytes + rt.nbytes
    extra["relayout_mxfp4_28672x8192_rows_to_tiled"] = {
        "us": round(rms * 1e3, 2), "GBps": round(rbytes / (rms * 1e-3) / 1e9, 1),
        "frac_hbm": round(rbytes / (rms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "bytes": rbytes}
    del rq, rt
    dq = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
    dms = timed(torch, lambda: q4.q4_dequant(copies[0], dq), 10, 3)
    dbytes = wbytes + N * K * 2
    extra["dequant_mxfp4_28672x8192_bf16"] = {"us": round(dms * 1e3, 2),
                                              "GBps": round(dbytes / (dms * 1e-3) / 1e9, 1),
                                              "frac_hbm": round(dbytes / (dms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                              "bytes": dbytes}
    del dq
    only = set(filter(None, args.only.split(",")))

    def want(name):
        return not args.no_extra and (not only or name in only)

    # HBM-bound workloads first, then the matrix-core-bound ones, each after
    # a short idle gap, so that no measurement inherits the power state (and
    # lower clock) of a long compute-bound run before it
    runs = [
        ("int4", "int4_g128_gemv_1024", lambda: bench_int4(torch, q4, workloads, dev, args.seed)),
        ("moe", "moe_grouped_mxfp4_64x2048x7168", lambda: bench_moe(torch, q4, workloads, dev, args.seed)),
        ("moe_layer", "moe_layer_mxfp4_64x(2x2048|7168)",
         lambda: bench_moe_layer(torch, q4, workloads, dev, args.seed)),
        ("nvfp4", "nvfp4_w4a16_gemm_4096x8192x8192", lambda: bench_nvfp4(torch, q4, workloads, dev, args.seed)),
        ("w4a4", "w4a4_mxfp4_gemm_8192", lambda: bench_w4a4(torch, q4, workloads, dev, args.seed)),
        ("w4a8", "w4a8_int4_fp8_gemm_4096x8192x8192", lambda: bench_w4a8(torch, q4, workloads, dev, args.seed)),
        ("w4a4_nvfp4", "w4a4_nvfp4_gemm_8192",
         lambda: bench_w4a4(torch, q4, workloads, dev, args.seed, "nvfp4")),
    ]
    for name, key, fn in runs:
        if want(name):
            torch.cuda.synchronize()
            time.sleep(IDLE_GAP_S)
            extra[key] = fn()

    if _MFMA_CEILING:
        extra["mfma_ceilings_TFLOPs"] = {
            k: {"measured": round(v, 1), "published_peak": {"fp4": FP4_PEAK_TFLOPS, "bf16": BF16_PEAK_TFLOPS,
                                                          "fp16": FP16_PEAK_TFLOPS, "fp8": FP8_PEAK_TFLOPS,
                                                          "fp4_copy": FP4_PEAK_TFLOPS, "fp4_mix": FP4_PEAK_TFLOPS,
                                                          "bf16_mix": BF16_PEAK_TFLOPS}[k],
                "note": "random register operands, q4_mfma_probe" + (
                    "; with the tiled W4A4 kernel's global->LDS copies" + (" and LDS fragment reads"
                                                                           if k == "fp4_mix" else "")
                    + " per 64 products per SIMD" if k.startswith("fp4_") else "") + (
                    "; with the tiled W4A16 kernel's NVFP4 dequantization, global->LDS copies and LDS"
                    " fragment reads per 16 products per wave" if k == "bf16_mix" else "")}
            for k, v in _MFMA_CEILING.items()}

    cpu = None
    if not args.no_cpu_baseline:
        del copies
        cpu = cpu_baseline(wl, wbytes, batches)

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "mxfp4_decode_gemv", "N": N, "K": K, "batches": list(batches),
                   "weight_format": "MXFP4 (E2M1 + E8M0 per 32)", "weight_layout": "tiled 16x128",
                   "accumulate": "fp32",
                   "global_batch": sum(batches), "parallelism": "none (1 GPU)"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(out), flush=True)


def _kernel_sha(name):
    import hashlib
    base = os.path.join(os.path.dirname(os.path.abspath(__file__)), "w4_gemm_amd", "csrc")
    h = hashlib.sha256()
    for f in (name, "q4_mma.h", "q4_device.h", "q4_layout.h"):
        h.update(open(os.path.join(base, f), "rb").read())
    return h.hexdigest()[:16]


def bench_int4(torch, q4, workloads, dev, seed):
    wl = workloads.int4_gemv(seed=seed)
    W = wl.tensors["W"].to(dev)
    x = wl.tensors["x"].to(dev)
    q = q4.quantize(W, "int4")
    y = torch.empty((1, W.shape[0]), dtype=torch.bfloat16, device=dev)
    ms = timed(torch, lambda: q4.q4_gemv(q, x, y), 200, 20)
    qms = timed(torch, lambda: q4.q4_quantize(W, q), 50, 5)
    return {"gemv_us": round(ms * 1e3, 3), "quantize_us": round(qms * 1e3, 3),
            "weight_bytes": q.nbytes, "note": "0.53 MB of weights: launch-bound, reported in us"}


def bench_nvfp4(torch, q4, workloads, dev, seed):
    log("generating the NVFP4 prefill workload")
    wl = workloads.nvfp4_gemm(seed=seed)
    A = wl.tensors["A"].to(dev)
    W = wl.tensors["W"].to(dev)
    M, K = A.shape
    N = W.shape[0]
    q = q4.quantize(W, "nvfp4", layout="tiled")
    C = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    ms = timed(torch, lambda: q4.q4_gemm(A, q, C), 10, 2)
    qms = timed(torch, lambda: q4.q4_quantize(W, q), 10, 2)
    tflops = 2.0 * M * N * K / (ms * 1e-3) / 1e12
    res = {"gemm_us": round(ms * 1e3, 1), "TFLOPs": round(tflops, 1),
           "frac_bf16_peak": round(tflops / BF16_PEAK_TFLOPS, 4),
           "quantize_us": round(qms * 1e3, 1),
           "quantize_GBps": round((N * K * 2 * 2 + q.nbytes) / (qms * 1e-3) / 1e9, 1)}
    with_ceiling(res, torch, q4, dev, "bf16_mix", prefix="mix_ceiling")
    return with_ceiling(res, torch, q4, dev, "bf16")


def bench_moe(torch, q4, workloads, dev, seed):
    log("generating the MoE workload (64 x 2048 x 7168)")
    wl = workloads.moe_grouped(seed=seed)
    W = wl.tensors["W"].to(dev)
    A = wl.tensors["A"].to(dev)
    r = wl.meta["routing"]
    N = wl.meta["N"]
    q = q4.quantize(W, "mxfp4", layout="tiled")
    del W
    g = torch.from_numpy(r.gather).to(dev)
    o = torch.from_numpy(r.offsets).to(dev)
    P = len(r.gather)
    C = torch.empty((P, N), dtype=torch.bfloat16, device=dev)
    ms = timed(torch, lambda: q4.q4_grouped_gemm(A, g, o, q, N, C), 20, 3)
    wbytes = q.codes.numel() + q.scales.numel()
    flops = 2.0 * P * N * wl.meta["K"]
    return {"us": round(ms * 1e3, 1), "weight_GBps": round(wbytes / (ms * 1e-3) / 1e9, 1),
            "frac_hbm": round(wbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "TFLOPs": round(flops / (ms * 1e-3) / 1e12, 2), "routed_rows": P,
            "rows_per_expert_min_max": [int(min(r.offsets[1:] - r.offsets[:-1])),
                                        int(max(r.offsets[1:] - r.offsets[:-1]))]}


def bench_moe_layer(torch, q4, workloads, dev, seed):
    """The MoE FFN layer at the MoE workload's shapes: route -> gate/up
    grouped GEMM (64 x 4096 x 7168) -> SwiGLU -> down grouped GEMM (64 x
    7168 x 2048) -> combine, 256 tokens, top-8, MXFP4 tiled weights.  The
    weights (2.8 G values) are drawn on the GPU (torch generator seeded with
    `seed`, N(0, 0.02^2)) -- drawing them on the host takes minutes; x and
    the router logits are the MoE workload's."""
    log("generating the MoE layer workload (64 experts, gate/up 4096x7168, down 7168x2048)")
    E, I, K, T, k = 64, 2048, 7168, 256, 8
    g = torch.Generator(device=dev).manual_seed(seed)
    w = (torch.randn((E * 2 * I, K), generator=g, device=dev) * 0.02).bfloat16()
    qgu = q4.quantize(w, "mxfp4", layout="tiled")
    del w
    w = (torch.randn((E * K, I), generator=g, device=dev) * 0.02).bfloat16()
    qd = q4.quantize(w, "mxfp4", layout="tiled")
    del w
    torch.cuda.empty_cache()
    x = workloads.matrix("moe/A", T, K, 1.0, seed).to(dev)
    logits = torch.from_numpy(workloads.normal_f32("moe/logits", T * E, seed).reshape(T, E)).to(dev)
    P = T * k
    r = q4.q4_moe_route(logits, k)
    gu = torch.empty((P, 2 * I), dtype=torch.bfloat16, device=dev)
    h = torch.empty((P, I), dtype=torch.bfloat16, device=dev)
    y = torch.empty((P, K), dtype=torch.bfloat16, device=dev)
    out = torch.empty((T, K), dtype=torch.bfloat16, device=dev)
    L = q4.lib()
    # the gate/up weight read as [W_gate_e; W_up_e] (unfused path) or in the
    # alternating-tile order of the fused gate/up + SwiGLU kernel: random
    # rows either way, so the two paths stream the same bytes
    steps = {
        "route": lambda: q4.q4_moe_route(logits, k),
        "gate_up_swiglu_fused": lambda: q4.q4_grouped_gemm_swiglu(x, r.gather, r.offsets, qgu, I, h),
        "gate_up": lambda: q4.q4_grouped_gemm(x, r.gather, r.offsets, qgu, 2 * I, gu),
        "swiglu": lambda: q4.q4_swiglu(gu, I, h),
        "down": lambda: q4.q4_grouped_gemm(h, None, r.offsets, qd, K, y),
        "combine": lambda: q4.q4_moe_combine(y, r, out),
    }

    def route():
        q4._check(L.q4_moe_route(q4._ptr(logits), E, T, E, k, q4._ptr(r.ids), q4._ptr(r.weights),
                                 q4._ptr(r.offsets), q4._ptr(r.gather), q4._ptr(r.inv), q4._stream(None)),
                  "q4_moe_route")

    def layer(fused):
        route()
        for name in (("gate_up_swiglu_fused",) if fused else ("gate_up", "swiglu")) + ("down", "combine"):
            steps[name]()

    ms = timed(torch, lambda: layer(True), 10, 2)
    ms_unfused = timed(torch, lambda: layer(False), 10, 2)
    per = {n: round(timed(torch, f, 10, 2) * 1e3, 1) for n, f in steps.items()}
    wbytes = qgu.nbytes + qd.nbytes
    return {"us": round(ms * 1e3, 1), "us_unfused": round(ms_unfused * 1e3, 1), "weight_bytes": wbytes,
            "weight_GBps": round(wbytes / (ms * 1e-3) / 1e9, 1),
            "frac_hbm": round(wbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "steps_us": per, "tokens": T, "topk": k}


def bench_w4a4(torch, q4, workloads, dev, seed, fmt="mxfp4"):
    """W4A4 GEMM 8192^3, both operands in `fmt`: MXFP4 on the block-scaled
    FP4 matrix cores (fraction of the FP4 peak), NVFP4 on the fp16 matrix
    cores with both operands dequantized exactly (fraction of the fp16
    peak); plus the activation quantize (NVFP4: tensor amax pass included)."""
    log(f"generating the W4A4 workload (8192^3, {fmt})")
    wl = workloads.w4a4_gemm(seed=seed)
    A = wl.tensors["A"].to(dev)
    W = wl.tensors["W"].to(dev)
    M, K = A.shape
    N = W.shape[0]
    qw = q4.quantize(W, fmt, layout="tiled")
    qa = q4.quantize(A, fmt, layout="tiled")
    C = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    ms = timed(torch, lambda: q4.q4_gemm(qa, qw, C), 10, 2)
    ams = timed(torch, lambda: q4.q4_quantize(A, qa), 10, 2)
    tflops = 2.0 * M * N * K / (ms * 1e-3) / 1e12
    peak = ("frac_fp4_peak", FP4_PEAK_TFLOPS) if fmt == "mxfp4" else ("frac_fp16_peak", FP16_PEAK_TFLOPS)
    res = {"gemm_us": round(ms * 1e3, 1), "TFLOPs": round(tflops, 1),
           peak[0]: round(tflops / peak[1], 4),
           "act_quantize_us": round(ams * 1e3, 1),
           "act_quantize_GBps": round((M * K * 2 + qa.nbytes) / (ams * 1e-3) / 1e9, 1)}
    if fmt == "mxfp4":
        # one layer of a W4A4 chain: the GEMM's output is the next layer's A.
        # Unfused: bf16 C, then a separate q4_quantize pass over it; fused:
        # the GEMM's epilogue writes C as MXFP4 codes + E8M0 scales directly
        # (q4_gemm_quantized), so the next GEMM starts from 4-bit activations
        qc = q4.empty_q4("mxfp4", M, N, device=dev, layout="tiled")

        def unfused():
            q4.q4_gemm(qa, qw, C)
            q4.q4_quantize(C, qc)

        ums = timed(torch, unfused, 10, 2)
        fms = timed(torch, lambda: q4.q4_gemm_quantized(qa, qw, qc), 10, 2)
        res["layer_with_separate_act_quantize_us"] = round(ums * 1e3, 1)
        res["layer_with_fused_act_quantize_us"] = round(fms * 1e3, 1)
        res["fused_epilogue_saves_us"] = round((ums - fms) * 1e3, 1)
        res["fused_TFLOPs"] = round(2.0 * M * N * K / (fms * 1e-3) / 1e12, 1)
        # the FP4 instruction alone, and with the kernel's copies and LDS
        # fragment reads mixed in at its rate (what its loop can approach)
        with_ceiling(res, torch, q4, dev, "fp4_mix", ("TFLOPs", "fused_TFLOPs"), prefix="mix_ceiling")
        return with_ceiling(res, torch, q4, dev, "fp4", ("TFLOPs", "fused_TFLOPs"))
    return with_ceiling(res, torch, q4, dev, "fp16")


def bench_w4a8(torch, q4, workloads, dev, seed):
    log("generating the W4A8 workload (4096 x 8192 x 8192)")
    wl = workloads.w4a8_gemm(seed=seed)
    A = wl.tensors["A"].to(dev)
    W = wl.tensors["W"].to(dev)
    M, K = A.shape
    N = W.shape[0]
    qw = q4.quantize(W, "int4", layout="tiled")
    qa = q4.quantize(A, "fp8_row", layout="tiled")
    C = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    ms = timed(torch, lambda: q4.q4_gemm(qa, qw, C), 10, 2)
    ams = timed(torch, lambda: q4.q4_quantize(A, qa), 10, 2)
    tflops = 2.0 * M * N * K / (ms * 1e-3) / 1e12
    res = {"gemm_us": round(ms * 1e3, 1), "TFLOPs": round(tflops, 1),
           "frac_fp8_peak": round(tflops / FP8_PEAK_TFLOPS, 4),
           "act_quantize_us": round(ams * 1e3, 1),
           "act_quantize_GBps": round((M * K * 2 + qa.nbytes) / (ams * 1e-3) / 1e9, 1)}
    return with_ceiling(res, torch, q4, dev, "fp8")


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(wl, wbytes, batches):
    """The oracle, as it stands, on the headline workload: for each batch it
    dequantizes the MXFP4 weight (plain C, OpenMP over rows) and takes the
    fp64 product (numpy).  Timed with every host thread the process may use
    (repeated until about 10 s of work) and with one thread (OpenMP and the
    BLAS capped at 1 by threadpoolctl; one step)."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    import oracle

    log("cpu baseline: oracle quantize (setup)")
    w = wl.tensors["W"].float().numpy()
    qr = oracle.quantize("mxfp4", w)
    del w
    xs = {b: wl.tensors[f"x{b}"].float().numpy() for b in batches}

    def run(seconds, max_steps):
        steps, t0 = 0, time.perf_counter()
        while True:
            for b in batches:
                oracle.gemv(qr, xs[b])
            steps += 1
            el = time.perf_counter() - t0
            if el > seconds or steps >= max_steps:
                return el / steps, steps

    log("cpu baseline: all threads")
    per_step, steps = run(10.0, 5)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [cpu_cores()])
    log("cpu baseline: one thread")
    with threadpool_limits(limits=1):
        per_step_1, steps_1 = run(20.0, 1)
    gbs = len(batches) * wbytes / per_step / 1e9
    gbs_1 = len(batches) * wbytes / per_step_1 / 1e9
    return {"value": round(gbs, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"full workload: 28672x8192 MXFP4 weight, B={list(batches)}, {steps} step(s) on "
                      f"{threads} threads ({per_step:.2f} s/step), {steps_1} on one thread "
                      f"({per_step_1:.2f} s/step)",
            "single_thread_GBps": round(gbs_1, 4), "single_thread_s_per_step": round(per_step_1, 3),
            "all_threads_s_per_step": round(per_step, 3),
            "cpu_model": cpu_model(), "nproc": os.cpu_count(), "affinity_cpus": cpu_cores()}


if __name__ == "__main__":
    main()
