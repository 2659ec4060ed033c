#!/usr/bin/env python3
"""Throughput of the quantized dense projection on one MI355X.

Headline (the JSON line's ``value``): weight-streaming rate of the row-scaled
FP8 GEMV on the decode / verify workload -- weight [N, K=5120] E4M3 with a
per-row F32 scale, BF16 activations, N in {6144, 17408, 152064} and
M in {1, 2, 8, 16}.  One step runs the GEMV once for every (N, M) pair;
``value`` = weight bytes read per step (N*K + 4N per call) / step time, in
GB/s, with every input already resident in HBM.  Weights rotate over copies
whose total footprint exceeds 1 GiB per shape so that the 256 MB Infinity
Cache cannot hold them.

The same line carries:
  roofline      the dominant kernel, the lm_head GEMV (N=152064) over the
                step's M mix, timed alone with HIP events on the launch
                stream, its algorithmic bytes per launch, and the fraction of
                the 8 TB/s HBM peak;
  cpu_baseline  the CPU oracle timed on a bounded sample of the same step;
  secondary     every other row of the hot path at its own workload size:
                quantizers / requantizers in GB/s against HBM, the three
                GEMMs in TFLOP/s against the MFMA peak of their data type,
                the block-scaled FP8 GEMV (128 x 128 F32 block scales)
                at the decode shapes for M in {1, 2, 4}, and the NVFP4-weight
                GEMV (W4A16) there for M in {1, 2, 8}, in GB/s;
  ablations     the W4A4 GEMM under three workgroup -> tile orders, a tile
                GEMM against the GEMV at M = 8 on the lm_head weight, and
                the int8 GEMM's two operand routes (int8 MFMA, FP16 MFMA).

  python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu] [--no-secondary]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
PEAK_TFLOPS = {"int8": 5033.0, "fp8": 5033.0, "fp4": 10066.0, "bf16": 2516.6,
               "fp16": 2516.6}
METRIC = ("TFLOP/s & %MFMA peak (GEMM M≥2048); weight GB/s & %HBM peak "
          "(GEMV M≤16)")
GEMV_SHAPES = [(6144, 5120), (17408, 5120), (152064, 5120)]
GEMV_MS = [1, 2, 8, 16]
ROTATE_BYTES = 1 << 30


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline")
    ap.add_argument("--no-secondary", action="store_true", help="GEMV step only")
    ap.add_argument("--only", default="", help="comma list of secondary items to run")
    ap.add_argument("--skip-gemv", action="store_true",
                    help="run only the secondary rows (for profiling them), after one "
                         "1 GiB copy (counter calibration); prints their JSON "
                         "dictionary instead of the headline line")
    ap.add_argument("--roofline-only", action="store_true",
                    help="for hardware-counter runs: one plain 1 GiB copy (counter "
                         "calibration), then the lm_head GEMV at each M, 5 launches each")
    return ap.parse_args()


def measured_traffic():
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary (two rocprofv3 --pmc runs, FETCH_SIZE and WRITE_SIZE, scaled by a
    1 GiB copy); None when the kernel source changed since it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "fp8_gemv_lm_head_hbm_traffic.md")
    try:
        fields = dict(l.split(": ", 1) for l in open(path).read().splitlines()
                      if l.startswith(("traffic_bytes_per_launch:", "kernel_source:",
                                       "kernel_source_sha256_16:")))
        src = os.path.join(ROOT, fields["kernel_source"].strip())
        h = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
        if h != fields["kernel_source_sha256_16"].strip():
            return None
        return int(fields["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def gemv_bytes(m, n, k):
    """Algorithmic bytes of one GEMV launch: weight, row scales, activations
    in, BF16 outputs."""
    return n * k + 4 * n + 2 * m * k + 2 * m * n


def time_launches(fn, iters, warm=2, warm_ms=30.0, graph=True):
    """Average duration (ms) of `fn` launched back to back on the current
    stream, measured with HIP events recorded on that stream.  Untimed
    launches run first for at least `warm_ms` (the shader clock ramps up over
    the first tens of milliseconds of load) and at least `warm` times.

    graph=True captures the `iters` launches in one HIP graph and times a
    replay of it, so the figure is the kernels' own time; launched one by one
    from Python, a kernel shorter than the binding's ~5 us per call would be
    timed as the host's launch rate instead."""
    import torch
    fn(0)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    fn(1)
    torch.cuda.synchronize()
    est = max(time.perf_counter() - t0, 1e-6)
    for i in range(max(warm, int(warm_ms * 1e-3 / est))):
        fn(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(iters):
                fn(i)
        # capture left the GPU idle: warm the clock again on replays
        t0 = time.perf_counter()
        g.replay()
        torch.cuda.synchronize()
        est = max(time.perf_counter() - t0, 1e-6)
        for _ in range(max(1, int(warm_ms * 1e-3 / est))):
            g.replay()
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        del g
        return e0.elapsed_time(e1) / iters
    e0.record()
    for i in range(iters):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / iters


def rot_count(nbytes):
    return max(2, -(-ROTATE_BYTES // max(1, nbytes)))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); "
              "the library has no multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import torch
    import gemv_nvfp4_int8_amd as qp
    import synth

    dev = torch.device("cuda:0")
    qp.lib()
    if args.roofline_only:
        roofline_only(qp, synth, dev)
        return
    if args.skip_gemv:
        only = set(s for s in args.only.split(",") if s)
        calibration_copy(torch, dev)
        print(json.dumps({"secondary": run_secondary(qp, synth, dev, only)}), flush=True)
        return

    # ---------------------------------------------------------- GEMV setup
    log("setting up GEMV weights")
    weights = {}     # (n,k) -> list of (wq, ws) rotating copies
    acts = {}
    for sid, (n, k) in enumerate(GEMV_SHAPES):
        wb = synth.gemv_weight_bf16(n, k, dev, shape_id=sid)
        wq = torch.empty((n, k), dtype=torch.uint8, device=dev)
        ws = torch.empty((n,), dtype=torch.float32, device=dev)
        qp.quant_rowwise_fp8(wb, wq, ws)
        del wb
        c = rot_count(n * k)
        copies = [(wq, ws)] + [(wq.clone(), ws.clone()) for _ in range(c - 1)]
        weights[(n, k)] = copies
        acts[(n, k)] = synth.gemv_acts_bf16(16, k, dev, shape_id=sid)
    outs = {(n, m): torch.empty((m, n), dtype=torch.bfloat16, device=dev)
            for (n, _) in GEMV_SHAPES for m in GEMV_MS}
    xs = {(n, m): acts[(n, k)][:m] for (n, k) in GEMV_SHAPES for m in GEMV_MS}
    torch.cuda.synchronize()

    def step(si):
        """Step si: every (N, M) pair once; call j of a weight in step si
        reads copy (len(GEMV_MS) * si + j) mod copies, so no call finds its
        weight in the 256 MB Infinity Cache."""
        for (n, k) in GEMV_SHAPES:
            copies = weights[(n, k)]
            for j, m in enumerate(GEMV_MS):
                wq, ws = copies[(len(GEMV_MS) * si + j) % len(copies)]
                qp.fp8_gemv_rowscale(xs[(n, m)], wq, ws, outs[(n, m)])

    step_weight_bytes = sum((n * k + 4 * n) for (n, k) in GEMV_SHAPES for _ in GEMV_MS)

    # Launched eagerly from Python.  With the binding at ~5 us per call the
    # host stays ahead of the GPU, so the step time is the kernels' own (the
    # per-call figures below, timed on HIP graphs, add up to it).  Replaying
    # one HIP graph per step measured ~4% slower on this stack.
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for i in range(args.steps):
        step(args.warmup + i)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = e0.elapsed_time(e1) / args.steps
    value = step_weight_bytes / (ms_per_step * 1e-3) / 1e9
    log(f"GEMV step: {ms_per_step:.4f} ms/step, {value:.1f} GB/s weight (wall {wall:.3f} s)")

    # ------------------------------------------ per-call GEMV figures (events)
    gemv_detail = []
    for (n, k) in GEMV_SHAPES:
        copies = weights[(n, k)]
        for m in GEMV_MS:
            x = acts[(n, k)][:m]
            o = outs[(n, m)]
            ms = time_launches(lambda i: qp.fp8_gemv_rowscale(
                x, copies[i % len(copies)][0], copies[i % len(copies)][1], o),
                iters=max(20, 2 * len(copies)))
            wgbs = (n * k + 4 * n) / (ms * 1e-3) / 1e9
            agbs = gemv_bytes(m, n, k) / (ms * 1e-3) / 1e9
            gemv_detail.append({"n": n, "k": k, "m": m, "us": round(ms * 1e3, 2),
                                "weight_GBs": round(wgbs, 1),
                                "algorithmic_GBs": round(agbs, 1),
                                "frac_hbm": round(agbs / HBM_PEAK_GBS, 4)})
            log(f"  gemv N={n} M={m}: {ms*1e3:.2f} us  weight {wgbs:.0f} GB/s  "
                f"({agbs / HBM_PEAK_GBS:.1%} of HBM)")
    # Dominant kernel: the lm_head GEMV (N=152064) over the step's M mix.
    dom = [d for d in gemv_detail if d["n"] == 152064]
    dom_bytes = sum(gemv_bytes(d["m"], 152064, 5120) for d in dom) / len(dom)
    dom_us = sum(d["us"] for d in dom) / len(dom)
    roofline = {"bound": "hbm",
                "kernel": "lm_head FP8 GEMV (N=152064, K=5120, M in {1,2,8,16}): "
                          "k_fp8_gemv_ksplit at M <= 2, k_fp8_gemv_rows above",
                "achieved": round(dom_bytes / (dom_us * 1e-6) / 1e9, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(dom_bytes / (dom_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                "bytes_per_launch": round(dom_bytes), "avg_launch_us": round(dom_us, 2),
                "traffic": measured_traffic()}

    rot_copies = {str(n): len(c) for (n, _), c in weights.items()}

    # ------------------------------------------------- secondary rows
    secondary = {}
    if not args.no_secondary:
        del weights
        torch.cuda.empty_cache()
        only = set(s for s in args.only.split(",") if s)
        secondary = run_secondary(qp, synth, dev, only)

    # ------------------------------------------------------ CPU baseline
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(synth)

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "fp8 row-scaled GEMV decode/verify: E4M3 weight "
                               "[N,5120] + F32 row scale, BF16 acts, "
                               "N in {6144,17408,152064} x M in {1,2,8,16}, "
                               "one call each per step",
                   "weight_bytes_per_step": step_weight_bytes,
                   "rotating_weight_copies": rot_copies},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "gemv": gemv_detail,
        "secondary": secondary,
    }
    print(json.dumps(line), flush=True)


def calibration_copy(torch, dev):
    """One device-to-device copy of exactly 1 GiB: it reads 1 GiB and writes
    1 GiB, which scales FETCH_SIZE / WRITE_SIZE to bytes in a counter run."""
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()


def roofline_only(qp, synth, dev):
    """A short program for counter runs: a device-to-device copy of exactly
    1 GiB (reads 1 GiB, writes 1 GiB: the scale for FETCH_SIZE / WRITE_SIZE),
    then 5 launches of the lm_head GEMV at each M, each on a fresh weight copy
    (two copies of 778 MB, so nothing stays cache-resident)."""
    import torch
    calibration_copy(torch, dev)
    n, k = 152064, 5120
    wb = synth.gemv_weight_bf16(n, k, dev, shape_id=2)
    wq = torch.empty((n, k), dtype=torch.uint8, device=dev)
    ws = torch.empty((n,), dtype=torch.float32, device=dev)
    qp.quant_rowwise_fp8(wb, wq, ws)
    del wb
    copies = [(wq, ws), (wq.clone(), ws.clone())]
    x = synth.gemv_acts_bf16(16, k, dev, shape_id=2)
    i = 0
    for m in GEMV_MS:
        o = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        for _ in range(5):
            qp.fp8_gemv_rowscale(x[:m], copies[i % 2][0], copies[i % 2][1], o)
            i += 1
    torch.cuda.synchronize()
    log("roofline-only run done")


def run_secondary(qp, synth, dev, only):
    import torch
    res = {}

    def want(name):
        return not only or name in only

    def quant_item(name, nbytes, make, call):
        """Time a streaming kernel over rotating buffer sets (>= 1 GiB)."""
        sets = [make() for _ in range(rot_count(nbytes))]
        torch.cuda.synchronize()
        ms = time_launches(lambda i: call(*sets[i % len(sets)]), iters=max(20, 2 * len(sets)))
        gbs = nbytes / (ms * 1e-3) / 1e9
        res[name] = {"us": round(ms * 1e3, 2), "bytes": nbytes, "GBs": round(gbs, 1),
                     "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)}
        log(f"  {name}: {ms*1e3:.2f} us  {gbs:.0f} GB/s ({gbs / HBM_PEAK_GBS:.1%} of HBM)")
        del sets
        torch.cuda.empty_cache()

    def gemm_item(name, flops, call, dtype_peak, iters=10):
        ms = time_launches(lambda i: call(), iters=iters)
        tf = flops / (ms * 1e-3) / 1e12
        ent = {"us": round(ms * 1e3, 1), "flop": flops, "TFLOPs": round(tf, 1),
               "peak_dtype": dtype_peak, "frac_peak": round(tf / PEAK_TFLOPS[dtype_peak], 4)}
        for d in ("int8", "fp8", "fp4", "bf16"):
            ent[f"frac_{d}"] = round(tf / PEAK_TFLOPS[d], 4)
        res[name] = ent
        log(f"  {name}: {ms*1e3:.1f} us  {tf:.1f} TFLOP/s ({tf / PEAK_TFLOPS[dtype_peak]:.1%} of {dtype_peak})")

    # Block-scaled FP8 GEMV (128 x 128 F32 block scales) at the decode shapes,
    # M in {1, 2, 4}; weights rotate over copies of >= 1 GiB per shape.
    if want("fp8_gemv_blockscale"):
        rows = []
        for sid, (n, k) in enumerate(GEMV_SHAPES):
            w, grid = synth.gemv_block_weight(n, k, dev, shape_id=sid)
            copies = [(w, grid)] + [(w.clone(), grid.clone())
                                    for _ in range(rot_count(n * k) - 1)]
            x = synth.gemv_acts_bf16(4, k, dev, shape_id=sid)
            for m in (1, 2, 4):
                o = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
                xm = x[:m]
                ms = time_launches(lambda i: qp.fp8_gemv_blockscale(
                    xm, copies[i % len(copies)][0], copies[i % len(copies)][1], o),
                    iters=max(20, 2 * len(copies)))
                wbytes = n * k + (n // 128) * (k // 128) * 4
                abytes = wbytes + 2 * m * k + 2 * m * n
                gbs = abytes / (ms * 1e-3) / 1e9
                rows.append({"n": n, "k": k, "m": m, "us": round(ms * 1e3, 2),
                             "weight_GBs": round(wbytes / (ms * 1e-3) / 1e9, 1),
                             "algorithmic_GBs": round(gbs, 1),
                             "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)})
                log(f"  fp8_gemv_blockscale N={n} M={m}: {ms*1e3:.2f} us  "
                    f"{gbs:.0f} GB/s ({gbs / HBM_PEAK_GBS:.1%} of HBM)")
            del w, grid, copies, x
            torch.cuda.empty_cache()
        res["fp8_gemv_blockscale"] = rows

    # NVFP4-weight GEMV (W4A16) at the decode shapes, M in {1, 2, 8}; the
    # weight is a BF16 N(0,0.02) draw quantised by quantize_bf16_nvfp4.
    if want("w4a16_gemv"):
        rows = []
        for sid, (n, k) in enumerate(GEMV_SHAPES):
            wb = synth.gemv_weight_bf16(n, k, dev, shape_id=sid)
            s2 = synth.per_tensor_scale2(wb)
            wp = torch.empty((n, k // 2), dtype=torch.uint8, device=dev)
            ws = torch.empty((n, k // 16), dtype=torch.uint8, device=dev)
            qp.quantize_bf16_nvfp4(wb, wp, ws, s2)
            del wb
            wbytes = n * k // 2 + n * k // 16
            copies = [(wp, ws)] + [(wp.clone(), ws.clone())
                                   for _ in range(rot_count(wbytes) - 1)]
            x = synth.gemv_acts_bf16(8, k, dev, shape_id=sid)
            for m in (1, 2, 8):
                o = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
                xm = x[:m]
                ms = time_launches(lambda i: qp.w4a16_gemv(
                    xm, copies[i % len(copies)][0], copies[i % len(copies)][1], s2, o),
                    iters=max(20, 2 * len(copies)))
                abytes = wbytes + 2 * m * k + 2 * m * n
                gbs = abytes / (ms * 1e-3) / 1e9
                rows.append({"n": n, "k": k, "m": m, "us": round(ms * 1e3, 2),
                             "weight_GBs": round(wbytes / (ms * 1e-3) / 1e9, 1),
                             "algorithmic_GBs": round(gbs, 1),
                             "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)})
                log(f"  w4a16_gemv N={n} M={m}: {ms*1e3:.2f} us  "
                    f"{gbs:.0f} GB/s ({gbs / HBM_PEAK_GBS:.1%} of HBM)")
            del wp, ws, copies, x
            torch.cuda.empty_cache()
        res["w4a16_gemv"] = rows

    # W4A8 prefill: NVFP4 weight 17408x5120 -> int8; acts 2048x5120.
    if want("w4a8") or want("requant_a_bf16_int8") or want("requant_w_nvfp4_int8") \
            or want("int8_gemm_blockscaled") or want("ablations") or want("int8_operand_route"):
        m, n, k = 2048, 17408, 5120
        c = synth.w4a8_prefill(dev, m, n, k)
        wp = torch.empty((n, k // 2), dtype=torch.uint8, device=dev)
        we = torch.empty((n, k // 16), dtype=torch.uint8, device=dev)
        qp.quantize_bf16_nvfp4(c.w_bf16, wp, we, c.scale2)
        w_i8 = torch.empty((n, k), dtype=torch.int8, device=dev)
        w_s = torch.empty((n, k // 32), dtype=torch.float32, device=dev)
        qp.requant_w_nvfp4_int8(wp, we, c.scale2, w_i8, w_s)
        a_i8 = torch.empty((m, k), dtype=torch.int8, device=dev)
        a_s = torch.empty((m, k // 32), dtype=torch.float32, device=dev)
        qp.requant_a_bf16_int8(c.a_bf16, a_i8, a_s)
        out = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        del c
        quant_item("requant_a_bf16_int8", m * k * 2 + m * k + m * (k // 32) * 4,
                   lambda: (synth.bf16_normal((m, k), 1.0, 7, dev),
                            torch.empty((m, k), dtype=torch.int8, device=dev),
                            torch.empty((m, k // 32), dtype=torch.float32, device=dev)),
                   lambda x, q, s: qp.requant_a_bf16_int8(x, q, s))
        quant_item("requant_w_nvfp4_int8", n * k // 2 + n * k // 16 + n * k + n * (k // 32) * 4,
                   lambda: (wp.clone(), we.clone(),
                            torch.empty((n, k), dtype=torch.int8, device=dev),
                            torch.empty((n, k // 32), dtype=torch.float32, device=dev)),
                   lambda p, e, q, s: qp.requant_w_nvfp4_int8(p, e, 1.0, q, s))
        gemm_item("int8_gemm_blockscaled", 2 * m * n * k,
                  lambda: qp.int8_gemm_blockscaled(a_i8, w_i8, a_s, w_s, out), "int8")
        # Operand-route ablation (gemm_dense_int8.rs, int8_gemm_faith2_prefill):
        # the same GEMM with P_b on FP16 MFMA over converted operands, which
        # halves the fold's vector-ALU work and doubles the matrix core's.
        if want("ablations") or want("int8_operand_route"):
            routes = {}
            for name, fn in (("int8_mfma", qp.int8_gemm_blockscaled),
                             ("fp16_mfma", qp.int8_gemm_blockscaled_f16ops)):
                ms = time_launches(lambda i: fn(a_i8, w_i8, a_s, w_s, out), iters=10)
                tf = 2 * m * n * k / (ms * 1e-3) / 1e12
                routes[name] = {"us": round(ms * 1e3, 1), "TOPs": round(tf, 1),
                                "frac_int8": round(tf / PEAK_TFLOPS["int8"], 4)}
                log(f"  ablation int8 operands {name}: {ms*1e3:.1f} us  {tf:.1f} TOP/s")
            res["ablation_int8_operand_route"] = {"shape": [m, n, k], "routes": routes}
        del wp, we, w_i8, w_s, a_i8, a_s, out
        torch.cuda.empty_cache()

    # W4A4 prefill: acts 4096x17408 -> NVFP4; NVFP4 weight 5120x17408.
    if want("w4a4") or want("quantize_bf16_nvfp4") or want("w4a4_gemm"):
        m, n, k = 4096, 5120, 17408
        c = synth.w4a4_prefill(dev, m, n, k)
        ap_ = torch.empty((m, k // 2), dtype=torch.uint8, device=dev)
        as_ = torch.empty((m, k // 16), dtype=torch.uint8, device=dev)
        wp = torch.empty((n, k // 2), dtype=torch.uint8, device=dev)
        ws = torch.empty((n, k // 16), dtype=torch.uint8, device=dev)
        qp.quantize_bf16_nvfp4(c.a_bf16, ap_, as_, 1.0)
        qp.quantize_bf16_nvfp4(c.w_bf16, wp, ws, c.scale_w2)
        out = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        a_src = c.a_bf16
        quant_item("quantize_bf16_nvfp4", m * k * 2 + m * k // 2 + m * k // 16,
                   lambda: (a_src.clone(),
                            torch.empty((m, k // 2), dtype=torch.uint8, device=dev),
                            torch.empty((m, k // 16), dtype=torch.uint8, device=dev)),
                   lambda x, p, s: qp.quantize_bf16_nvfp4(x, p, s, 1.0))
        gemm_item("w4a4_gemm", 2 * m * n * k,
                  lambda: qp.w4a4_gemm(ap_, as_, wp, ws, out, 1.0, c.scale_w2), "fp16")
        del c, a_src, ap_, as_, wp, ws, out
        torch.cuda.empty_cache()

    # Ablations (gemm_fp4.rs: w4a4_gemm's N-fast grid against
    # w4a4_gemm_mfast's M-fast grid; fp8_gemv_batch.rs: tile GEMMs that pad
    # M to their tile against the batched GEMV at M = 8).
    if want("ablations"):
        m, n, k = 4096, 5120, 17408
        c = synth.w4a4_prefill(dev, m, n, k)
        ap_ = torch.empty((m, k // 2), dtype=torch.uint8, device=dev)
        as_ = torch.empty((m, k // 16), dtype=torch.uint8, device=dev)
        wp = torch.empty((n, k // 2), dtype=torch.uint8, device=dev)
        ws = torch.empty((n, k // 16), dtype=torch.uint8, device=dev)
        qp.quantize_bf16_nvfp4(c.a_bf16, ap_, as_, 1.0)
        qp.quantize_bf16_nvfp4(c.w_bf16, wp, ws, c.scale_w2)
        out = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        orders = {}
        for name, order in (("banded_xcd", qp.QP_TILES_BANDED), ("m_fast", qp.QP_TILES_MFAST),
                            ("n_fast", qp.QP_TILES_NFAST)):
            ms = time_launches(lambda i: qp.w4a4_gemm(ap_, as_, wp, ws, out, 1.0, c.scale_w2,
                                                      tile_order=order), iters=10)
            tf = 2 * m * n * k / (ms * 1e-3) / 1e12
            orders[name] = {"us": round(ms * 1e3, 1), "TFLOPs": round(tf, 1),
                            "frac_fp16": round(tf / PEAK_TFLOPS["fp16"], 4)}
            log(f"  ablation w4a4 tiles {name}: {ms*1e3:.1f} us  {tf:.1f} TFLOP/s")
        res["ablation_w4a4_tile_order"] = {"shape": [m, n, k], "orders": orders}
        del c, ap_, as_, wp, ws, out
        torch.cuda.empty_cache()

        m, n, k = 8, 152064, 5120
        wb = synth.gemv_weight_bf16(n, k, dev, shape_id=2)
        wq = torch.empty((n, k), dtype=torch.uint8, device=dev)
        wsr = torch.empty((n,), dtype=torch.float32, device=dev)
        qp.quant_rowwise_fp8(wb, wq, wsr)
        del wb
        copies = [(wq, wsr), (wq.clone(), wsr.clone())]
        x = synth.gemv_acts_bf16(m, k, dev, shape_id=2)
        aq = torch.empty((m, k), dtype=torch.uint8, device=dev)
        asr = torch.empty((m,), dtype=torch.float32, device=dev)
        qp.quant_rowwise_fp8(x, aq, asr)
        o = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        ms_gemm = time_launches(lambda i: qp.fp8_gemm_rowscale(
            aq, asr, copies[i % 2][0], copies[i % 2][1], o), iters=20)
        ms_gemv = time_launches(lambda i: qp.fp8_gemv_rowscale(
            x, copies[i % 2][0], copies[i % 2][1], o), iters=20)
        wbytes = n * k + 4 * n
        res["ablation_m8_tile_gemm_vs_gemv"] = {
            "shape": [m, n, k],
            "tile_gemm": {"kernel": "fp8_gemm_rowscale (128x128 tiles, M padded to 128)",
                          "us": round(ms_gemm * 1e3, 1),
                          "weight_GBs": round(wbytes / (ms_gemm * 1e-3) / 1e9, 1)},
            "gemv": {"kernel": "fp8_gemv_rowscale", "us": round(ms_gemv * 1e3, 1),
                     "weight_GBs": round(wbytes / (ms_gemv * 1e-3) / 1e9, 1)}}
        log(f"  ablation M=8 lm_head: tile GEMM {ms_gemm*1e3:.1f} us "
            f"({wbytes / (ms_gemm * 1e-3) / 1e9:.0f} GB/s) vs GEMV {ms_gemv*1e3:.1f} us "
            f"({wbytes / (ms_gemv * 1e-3) / 1e9:.0f} GB/s)")
        del copies, wq, wsr, x, aq, asr, o
        torch.cuda.empty_cache()

    # The vendor library (hipBLASLt through torch) on the GEMM shapes, for
    # context beside the kernels above.  Run only when named in --only; it
    # is a measurement, never part of the library's path.
    if "vendor" in only:
        res["vendor"] = vendor_gemms(torch, dev)

    # Block FP8 -> row-wise FP8 requant + row-wise FP8 GEMM, M = 8192.
    if want("fp8") or want("requant_w_blockfp8_rowwise") or want("quant_rowwise_fp8") \
            or want("fp8_gemm_rowscale"):
        m, n, k = 8192, 12288, 5120
        c = synth.fp8_block(dev, m, n, k)
        quant_item("requant_w_blockfp8_rowwise", n * k + (n // 128) * (k // 128) * 4 + n * k + n * 4,
                   lambda: (c.w_block.clone(), c.block_grid.clone(),
                            torch.empty((n, k), dtype=torch.uint8, device=dev),
                            torch.empty((n,), dtype=torch.float32, device=dev)),
                   lambda w, g, q, s: qp.requant_w_blockfp8_rowwise(qp.QP_FP8_BLOCK128, w, g, q, s))
        quant_item("quant_rowwise_fp8", m * k * 2 + m * k + m * 4,
                   lambda: (c.a_bf16.clone(),
                            torch.empty((m, k), dtype=torch.uint8, device=dev),
                            torch.empty((m,), dtype=torch.float32, device=dev)),
                   lambda x, q, s: qp.quant_rowwise_fp8(x, q, s))
        wq = torch.empty((n, k), dtype=torch.uint8, device=dev)
        wsr = torch.empty((n,), dtype=torch.float32, device=dev)
        qp.requant_w_blockfp8_rowwise(qp.QP_FP8_BLOCK128, c.w_block, c.block_grid, wq, wsr)
        aq = torch.empty((m, k), dtype=torch.uint8, device=dev)
        asr = torch.empty((m,), dtype=torch.float32, device=dev)
        qp.quant_rowwise_fp8(c.a_bf16, aq, asr)
        out = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        gemm_item("fp8_gemm_rowscale", 2 * m * n * k,
                  lambda: qp.fp8_gemm_rowscale(aq, asr, wq, wsr, out), "fp8")
        del c, wq, wsr, aq, asr, out
        torch.cuda.empty_cache()
    return res


def vendor_gemms(torch, dev):
    """hipBLASLt (torch._scaled_mm, torch._int_mm, torch.matmul) on the GEMM
    shapes: FP8 with row-wise and tensor-wise scales on the row-scaled FP8
    shape, plain int8 (no block scales) and BF16 on the int8 shape, BF16 and
    tensor-scaled FP8 on the W4A4 shape.  Eager launches (library calls stay
    out of graph capture); random operands of the same shapes."""
    out = {}
    g = torch.Generator(device=dev)
    g.manual_seed(7)

    def item(name, flops, fn, peak):
        ms = time_launches(lambda i: fn(), iters=20, graph=False)
        tf = flops / (ms * 1e-3) / 1e12
        out[name] = {"us": round(ms * 1e3, 1), "TFLOPs": round(tf, 1), "peak_dtype": peak,
                     "frac_peak": round(tf / PEAK_TFLOPS[peak], 4)}
        log(f"  vendor {name}: {ms*1e3:.1f} us  {tf:.1f} TFLOP/s ({tf / PEAK_TFLOPS[peak]:.1%} of {peak})")

    def f8(shape):
        return (torch.randn(shape, generator=g, device=dev) * 0.5).to(torch.float8_e4m3fn)

    m, n, k = 8192, 12288, 5120
    a, w = f8((m, k)), f8((n, k))
    sa = torch.rand((m, 1), generator=g, device=dev) + 0.5
    sw = torch.rand((1, n), generator=g, device=dev) + 0.5
    one = torch.ones((), device=dev)
    item("fp8_rowwise_8192x12288x5120", 2 * m * n * k,
         lambda: torch._scaled_mm(a, w.t(), sa, sw, out_dtype=torch.bfloat16), "fp8")
    item("fp8_tensorwise_8192x12288x5120", 2 * m * n * k,
         lambda: torch._scaled_mm(a, w.t(), one, one, out_dtype=torch.bfloat16), "fp8")
    del a, w, sa, sw

    m, n, k = 2048, 17408, 5120
    ai = torch.randint(-127, 128, (m, k), generator=g, device=dev, dtype=torch.int8)
    wi = torch.randint(-127, 128, (n, k), generator=g, device=dev, dtype=torch.int8)
    item("int8_plain_2048x17408x5120", 2 * m * n * k, lambda: torch._int_mm(ai, wi.t()), "int8")
    del ai, wi
    ab = torch.randn((m, k), generator=g, device=dev).to(torch.bfloat16)
    wb = torch.randn((n, k), generator=g, device=dev).to(torch.bfloat16)
    item("bf16_2048x17408x5120", 2 * m * n * k, lambda: ab @ wb.t(), "bf16")
    del ab, wb

    m, n, k = 4096, 5120, 17408
    ab = torch.randn((m, k), generator=g, device=dev).to(torch.bfloat16)
    wb = torch.randn((n, k), generator=g, device=dev).to(torch.bfloat16)
    item("bf16_4096x5120x17408", 2 * m * n * k, lambda: ab @ wb.t(), "bf16")
    a, w = ab.to(torch.float8_e4m3fn), wb.to(torch.float8_e4m3fn)
    del ab, wb
    item("fp8_tensorwise_4096x5120x17408", 2 * m * n * k,
         lambda: torch._scaled_mm(a, w.t(), one, one, out_dtype=torch.bfloat16), "fp8")
    del a, w
    torch.cuda.empty_cache()
    return out


def cpu_baseline(synth, gemv_seconds=12.0, item_seconds=1.2):
    """The CPU oracle on bounded samples, on this host's cores.

    The headline figure is the GEMV step: for every (N, M) pair, the first
    N/R weight rows, with R chosen from a short probe so that the timed run
    takes about `gemv_seconds`; reported in the headline's unit (weight GB/s
    over the sampled rows).  Beside it, `per_config` times the oracle on
    each other step of every workload (quantizers, requants, GEMMs) over a
    row sample sized to about `item_seconds`, in the same units as the GPU
    rows (algorithmic GB/s, or GFLOP/s for the contractions)."""
    import numpy as np
    import oracle
    oracle.lib()
    threads = oracle.num_threads()

    def run(frac):
        tot_bytes, t = 0, 0.0
        for sid, (n, k) in enumerate(GEMV_SHAPES):
            rows = max(1, int(n * frac))
            w = synth.gemv_weight_bf16(rows, k, "cpu", shape_id=sid)
            wq, ws = oracle.quant_rowwise_fp8(synth.to_numpy_bits(w))
            x = synth.to_numpy_bits(synth.gemv_acts_bf16(16, k, "cpu", shape_id=sid))
            for m in GEMV_MS:
                t0 = time.perf_counter()
                oracle.fp8_gemv_rowscale(x[:m], wq, ws)
                t += time.perf_counter() - t0
                tot_bytes += rows * k + 4 * rows
        return tot_bytes, t

    probe_frac = 1.0 / 1024
    b, t = run(probe_frac)
    frac = min(1.0, probe_frac * gemv_seconds / max(t, 1e-3))
    b, t = run(frac)
    gbs = b / t / 1e9
    log(f"cpu oracle: {t:.1f} s on {threads} threads, {gbs:.4f} GB/s (fraction {frac:.4f})")
    def oracle_per_config(synth, target_s):
        """The oracle on each workload's steps other than the headline GEMV,
        every input built as the GPU rows build it; each step is timed on the
        first `u` rows of the input its cost scales with (activation rows for
        the GEMMs), u sized from a probe to take about target_s."""
        import numpy as np
        import oracle
        bits = synth.to_numpy_bits
        res = {}

        def item(name, unit, full, work, run, what):
            u = max(1, full // 2048)
            t0 = time.perf_counter()
            run(u)
            t = time.perf_counter() - t0
            u = int(min(full, max(u, u * target_s / max(t, 1e-4))))
            t0 = time.perf_counter()
            run(u)
            t = time.perf_counter() - t0
            rate = work(u) / t / 1e9
            res[name] = {"value": round(rate, 4), "unit": unit, "seconds": round(t, 3),
                         "sample": f"{what} {u} of {full}"}
            log(f"cpu oracle {name}: {rate:.4g} {unit} ({what} {u} of {full}, {t:.2f} s)")

        # W4A8 tiny (N=256, K=512, M=16), whole: requant_w + requant_a + GEMM.
        c = synth.w4a8_tiny("cpu")
        wp0, we0, a0 = bits(c.w_packed), bits(c.w_e4m3), bits(c.a_bf16)

        def tiny(_):
            wq, wsc = oracle.requant_w_nvfp4_int8(wp0, we0, c.scale2)
            aq, asc = oracle.requant_a_bf16_int8(a0)
            oracle.int8_gemm_blockscaled(aq, wq, asc, wsc)
        item("w4a8_tiny_step", "GFLOP/s", 1, lambda u: 2 * 16 * 256 * 512, tiny, "whole step,")

        # W4A8 prefill: NVFP4 weight 17408x5120 -> int8; acts 2048x5120.
        m, n, k = 2048, 17408, 5120
        c = synth.w4a8_prefill("cpu", m, n, k)
        wb, ab = bits(c.w_bf16), bits(c.a_bf16)
        wp, we = oracle.quantize_bf16_nvfp4(wb, c.scale2)
        wq, wsc = oracle.requant_w_nvfp4_int8(wp, we, c.scale2)
        aq, asc = oracle.requant_a_bf16_int8(ab)
        item("requant_a_bf16_int8", "GB/s", m, lambda u: u * k * 2 + u * k + u * (k // 32) * 4,
             lambda u: oracle.requant_a_bf16_int8(ab[:u]), "activation rows")
        item("requant_w_nvfp4_int8", "GB/s", n,
             lambda u: u * (k // 2 + k // 16 + k + (k // 32) * 4),
             lambda u: oracle.requant_w_nvfp4_int8(wp[:u], we[:u], c.scale2), "weight rows")
        item("int8_gemm_blockscaled", "GFLOP/s", m, lambda u: 2 * u * n * k,
             lambda u: oracle.int8_gemm_blockscaled(aq[:u], wq, asc[:u], wsc), "activation rows")
        del c, wb, ab, wp, we, wq, wsc, aq, asc

        # W4A4 prefill: acts 4096x17408 -> NVFP4; NVFP4 weight 5120x17408.
        m, n, k = 4096, 5120, 17408
        c = synth.w4a4_prefill("cpu", m, n, k)
        ab = bits(c.a_bf16)
        wp, wsc = oracle.quantize_bf16_nvfp4(bits(c.w_bf16), c.scale_w2)
        ap, asc = oracle.quantize_bf16_nvfp4(ab[:64], 1.0)
        item("quantize_bf16_nvfp4", "GB/s", m, lambda u: u * (k * 2 + k // 2 + k // 16),
             lambda u: oracle.quantize_bf16_nvfp4(ab[:u], 1.0), "activation rows")
        item("w4a4_gemm", "GFLOP/s", 64, lambda u: 2 * u * n * k,
             lambda u: oracle.w4a4_gemm(ap[:u], asc[:u], wp, wsc, 1.0, c.scale_w2),
             "activation rows (of the first 64)")
        del c, ab, wp, wsc, ap, asc

        # Block-FP8 -> row-wise FP8 requant + GEMM: W 12288x5120, acts 8192x5120.
        m, n, k = 8192, 12288, 5120
        c = synth.fp8_block("cpu", m, n, k)
        w, grid = bits(c.w_block), c.block_grid.numpy()
        ab = bits(c.a_bf16)
        item("requant_w_blockfp8_rowwise", "GB/s", n // 128, lambda u: 128 * u * (2 * k + 4),
             lambda u: oracle.requant_w_blockfp8_rowwise(w[:128 * u], grid[:u]),
             "128-row weight blocks")
        wq, wsc = oracle.requant_w_blockfp8_rowwise(w, grid)
        aq, asc = oracle.quant_rowwise_fp8(ab[:256])
        item("quant_rowwise_fp8", "GB/s", m, lambda u: u * (3 * k + 4),
             lambda u: oracle.quant_rowwise_fp8(ab[:u]), "activation rows")
        item("fp8_gemm_rowscale", "GFLOP/s", 256, lambda u: 2 * u * n * k,
             lambda u: oracle.fp8_gemm_rowscale(aq[:u], asc[:u], wq, wsc),
             "activation rows (of the first 256)")
        return res

    per = oracle_per_config(synth, item_seconds)
    return {"value": round(gbs, 5), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "seconds": round(t, 2),
            "host_cpus": len(os.sched_getaffinity(0)),
            "hardware_concurrency": os.cpu_count(),
            "sample": f"every (N, M) pair of the GEMV step on the first {frac:.4%} of "
                      f"weight rows ({b} weight bytes)",
            "per_config": per}


if __name__ == "__main__":
    main()
