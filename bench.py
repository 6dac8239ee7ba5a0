#!/usr/bin/env python3
"""Benchmark of the QLoRA linear hot path on one MI355X.

Headline workload: the 7B-shaped attention projection, W 4096x4096 (bf16,
N(0, 0.02^2)) quantized to NF4 with double quantization, LoRA rank 64
(alpha 16, s = 0.25), X of 2048 tokens (batch 4 x seq 512).  The frozen weight is
quantized once per input set, outside the timed region (as in QLoRA training, where
the base weight is quantized once); one step is the forward (X A, fused dequant
GEMM with the adapter term) and the backward (dY B^T, fused dequant dX GEMM, dA,
dB) on one batch.  `value` counts the forward+backward FLOPs
4 M in out + 6 M r (in + out) (no dW; dequantization not counted) per step time,
inputs already resident in HBM.  Four independent input sets are rotated so
consecutive steps do not hit in the 256 MB Infinity Cache.

Also reported:
  roofline     -- the dominant kernel's algorithmic FLOPs per launch over its
                  average duration (HIP events around every launch, in a
                  separate pass of the same steps), against 2.5 PFLOP/s bf16;
  gemv         -- the skinny-token forward at the 65B shapes (8192->22016 and
                  22016->8192, M in {1,4,16}): packed-weight GB/s against 8 TB/s,
                  rotating 6 weight copies (> 512 MB) per shape;
  quantize     -- quantize + double-quantize of the headline weight (timed apart):
                  bytes moved (bf16 in, codes and constants out) over time;
  adamw        -- one AdamW step on the adapters (fp32 state), GB/s against 8 TB/s, and
                  with the state paged out to pinned host memory (GB/s over the link);
  comparators  -- the headline step on the unquantized bf16 weight and with the weight
                  dequantized into a buffer first (torch / hipBLASLt products), as context,
                  and measured ceilings: hipBLASLt's bf16 GEMM of the forward's shape (also
                  in roofline.measured_ceiling) and torch's copy of 1 GiB;
  merge        -- adapter merge + requantize on the headline layer: times, and the
                  output error the requantization leaves;
  formats      -- quantization error (relative MSE of the dequantized weight) of the
                  NF4, FP4 and Int4 tables on the headline weight shape, and for NF4
                  blocks of 32, 64, 128, 256: error, constant bits per weight and the
                  headline step time;
  mlp_7b, stack_65b -- forward+backward TFLOP/s over the 7B MLP pair (M = 4096)
                  and over the 65B layer stack (80 layers x 7 linears, M = 2048,
                  all 33 GB of NF4 weight resident), forward layer 0 first, then
                  the backward in reverse;
  cpu_baseline -- the float64 NumPy oracle doing one full step of the headline
                  workload (dequantize, forward, backward) on the host cores.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

METRIC = "QLoRA linear fwd+bwd TFLOP/s (large M) + dequant-GEMV weight GB/s (M≤16)"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBPS = 8000.0


def flops_fwd_bwd(M, din, dout, r):
    return 4 * M * din * dout + 6 * M * r * (din + dout)


def weight_bytes(din, dout):
    n = din * dout
    nblk = -(-n // 64)
    return 32 * nblk + nblk + 4 * (-(-nblk // 256)) + 4


KERNEL_SOURCES = {
    "k_fwd_nf4_gemm": ["fwd_gemm.hip", "gemm_core.h", "common.h"],
    "k_bwd_dx_nf4_gemm": ["dx_gemm.hip", "gemm_core.h", "common.h"],
    "k_nf4_quantize": ["quant.hip", "common.h"],
    "k_fwd_nf4_gemv": ["gemv.hip", "gemm_core.h", "common.h"],
}


def measured_traffic(kernel):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE runs (scaled by a
    plain copy's counts), or None if the kernel's sources changed since the counters were taken."""
    import hashlib

    root = os.path.dirname(os.path.abspath(__file__))
    try:
        with open(os.path.join(root, "profiles", "traffic_counters.txt")) as f:
            rec = json.load(f)["kernels"][kernel]
        h = hashlib.sha256()
        for name in KERNEL_SOURCES[kernel]:
            with open(os.path.join(root, "bit_nf4_quantized_11_amd", "csrc", name), "rb") as f:
                h.update(f.read())
    except (OSError, KeyError, ValueError):
        return None
    return rec["traffic_bytes"] if h.hexdigest()[:16] == rec["sources_sha256_16"] else None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--sets", type=int, default=4, help="independent input sets rotated across steps")
    ap.add_argument("--settle-ms", type=float, default=150.0,
                    help="untimed run of the step before the warm-up steps, so the GPU reaches steady clocks")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-gemv", action="store_true")
    ap.add_argument("--gemv-iters", type=int, default=50)
    ap.add_argument("--no-layers", action="store_true", help="skip the 7B MLP pair and the 65B layer stack")
    ap.add_argument("--layer-steps", type=int, default=3, help="timed steps of the 7B MLP pair and the 65B stack")
    ap.add_argument("--only", choices=["all", "headline", "gemv", "few", "layers", "adamw", "copy"], default="all",
                    help="restrict the run (for profiling single kernels); 'copy' runs a plain device copy of "
                         "known size, the reference for scaling hardware byte counters")
    return ap.parse_args()


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark measures one GPU only; the hot path is not run across "
                                   "several GPUs (see the design notes for how it would shard)",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch

    import bit_nf4_quantized_11_amd as Q
    import workloads

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    if args.only == "copy":
        nbytes = 1 << 30
        src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "launches": args.steps}))
        return

    M, din, dout, r, alpha = 2048, 4096, 4096, 64, 16.0
    s = alpha / r
    flops = flops_fwd_bwd(M, din, dout, r)
    result = {"metric": METRIC, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
              "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
              "data": "synthetic (seeded Gaussian, LLaMA-7B layer shape)"}
    result["config"] = {"workload": "QLoRA linear 4096->4096, 2048 tokens, NF4 block 64 + double quant 256, "
                                    "LoRA r=64 alpha=16; step = forward + backward on the quantized weight",
                        "M": M, "in": din, "out": dout, "r": r, "alpha": alpha, "input_sets": args.sets,
                        "flops_per_step": flops}

    if args.only in ("all", "headline"):
        sets = []
        for i in range(args.sets):
            seed = 2000 + 100 * i
            sets.append(dict(
                W=workloads.device_normal_bf16(seed + 0, (dout, din), 0.02),
                A=workloads.device_normal_bf16(seed + 1, (din, r), 0.02),
                B=workloads.device_normal_bf16(seed + 2, (r, dout), 0.02),
                X=workloads.device_normal_bf16(seed + 3, (M, din), 1.0),
                dY=workloads.device_normal_bf16(seed + 4, (M, dout), 1.0),
                w=Q.nf4_alloc(dout, din, True, dev),
                Y=torch.empty((M, dout), dtype=torch.bfloat16, device=dev),
                T=torch.empty((M, r), dtype=torch.bfloat16, device=dev),
                dX=torch.empty((M, din), dtype=torch.bfloat16, device=dev),
                dA=torch.empty((din, r), dtype=torch.float32, device=dev),
                dB=torch.empty((r, dout), dtype=torch.float32, device=dev)))
        ws = torch.empty(max(Q.qlora_quantize_workspace(dout, din), Q.qlora_fwd_workspace(M, din, dout, r),
                             Q.qlora_bwd_workspace(M, din, dout, r)), dtype=torch.uint8, device=dev)

        def quantize(i):
            d = sets[i % len(sets)]
            Q.qlora_quantize_nf4(d["W"], True, out=d["w"], workspace=ws)

        for i in range(len(sets)):
            quantize(i)

        def step(i):
            d = sets[i % len(sets)]
            Q.qlora_linear_fwd(d["X"], d["w"], d["A"], d["B"], s, Y=d["Y"], T_save=d["T"], workspace=ws)
            Q.qlora_linear_bwd(d["dY"], d["X"], d["T"], d["w"], d["A"], d["B"], s, dX=d["dX"], dA=d["dA"],
                               dB=d["dB"], workspace=ws)

        # Bring the GPU to its steady clocks before the warm-up steps: from idle, the first
        # ~50 ms of this step run up to 50 % slower (measured: 295, 212, 204 ... 192 us per
        # step over the first 20-step batches) while the clocks ramp.  Untimed, same step.
        t_settle = time.perf_counter()
        i = 0
        while time.perf_counter() - t_settle < args.settle_ms * 1e-3:
            for _ in range(20):
                step(i)
                i += 1
            torch.cuda.synchronize()
        for i in range(args.warmup):
            step(i)
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        ev0.record()
        for i in range(args.steps):
            step(i)
        ev1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms = ev0.elapsed_time(ev1) / args.steps
        result["ms_per_step"] = ms
        result["value"] = flops / (ms * 1e-3) / 1e12
        result["wall_s_timed"] = wall

        # per-kernel durations: same steps again with HIP events around every launch
        Q.qlora_profile_enable(True)
        Q.qlora_profile_read(reset=True)
        for i in range(args.steps):
            step(i)
        torch.cuda.synchronize()
        prof = Q.qlora_profile_read(reset=True)
        Q.qlora_profile_enable(False)
        kern = {k: {"launches": n, "avg_us": 1e3 * t / n, "us_per_step": 1e3 * t / args.steps}
                for k, (n, t) in prof.items()}
        result["kernels"] = kern
        # algorithmic FLOPs per launch of the two dequantizing GEMMs
        algo = {"k_fwd_nf4_gemm": 2 * M * din * dout + 2 * M * r * dout,
                "k_bwd_dx_nf4_gemm": 2 * M * dout * din + 2 * M * r * din}
        dom = max((k for k in kern if k in algo), key=lambda k: kern[k]["us_per_step"])
        ach = algo[dom] / (kern[dom]["avg_us"] * 1e-6) / 1e12
        algo_bytes = 2 * M * din + 2 * M * dout + weight_bytes(din, dout) + 2 * r * (din + dout) + 2 * M * 64
        result["roofline"] = {"kernel": dom, "bound": "mfma", "achieved": ach, "peak": PEAK_BF16_TFLOPS,
                              "unit": "TFLOP/s", "frac": ach / PEAK_BF16_TFLOPS, "traffic": measured_traffic(dom),
                              "traffic_unit": "bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-scaled)",
                              "algorithmic_bytes": algo_bytes,
                              "flops_per_launch": algo[dom], "avg_us": kern[dom]["avg_us"]}
        fb_us = sum(v["us_per_step"] for v in kern.values())
        result["fwd_bwd_kernel_tflops"] = flops / (fb_us * 1e-6) / 1e12

        # quantize + double-quantize, timed apart (bf16 weight in; codes, 8-bit constants,
        # per-256 scales and the mean out)
        qbytes = 2 * din * dout + weight_bytes(din, dout)
        for i in range(3):
            quantize(i)
        torch.cuda.synchronize()
        ev0.record()
        for i in range(args.steps):
            quantize(i)
        ev1.record()
        torch.cuda.synchronize()
        qus = 1e3 * ev0.elapsed_time(ev1) / args.steps
        Q.qlora_profile_enable(True)
        Q.qlora_profile_read(reset=True)
        for i in range(args.steps):
            quantize(i)
        torch.cuda.synchronize()
        qprof = Q.qlora_profile_read(reset=True)
        Q.qlora_profile_enable(False)
        result["quantize"] = {"us_per_call": qus, "bytes": qbytes, "GBps": qbytes / (qus * 1e-6) / 1e9,
                              "peak_GBps": PEAK_HBM_GBPS,
                              "kernels_us": {k: 1e3 * t / n for k, (n, t) in qprof.items()}}
        del sets, ws
        torch.cuda.empty_cache()

    if args.only in ("all", "gemv") and not args.no_gemv:
        result["gemv"] = bench_gemv(Q, workloads, torch, dev, args.gemv_iters)
    if args.only in ("all", "few"):
        result["few_tokens"] = bench_few_tokens(Q, workloads, torch, dev)

    if args.only in ("all", "headline"):
        result["formats"] = bench_formats(Q, workloads, torch, dev)
        result["merge"] = bench_merge(Q, workloads, torch, dev)
        result["comparators"] = bench_comparators(Q, workloads, torch, dev, result["ms_per_step"])
        gemm = result["comparators"]["ceilings"]["hipblaslt_bf16_gemm_2048x4096x4096"]
        result["roofline"]["measured_ceiling"] = {
            "what": "hipBLASLt bf16 GEMM of the same shape without dequantization (torch.matmul)",
            "TFLOPs": gemm["TFLOPs"], "frac": result["roofline"]["achieved"] / gemm["TFLOPs"]}
        if "gemv" in result:
            cp = result["comparators"]["ceilings"]["device_copy_1GiB"]["GBps"]
            result["gemv"]["measured_ceiling"] = {"what": "torch copy of 1 GiB, bytes read + written per second",
                                                  "GBps": cp, "frac_max": result["gemv"]["weight_GBps_max"] / cp}

    if args.only in ("all", "adamw"):
        result["adamw"] = bench_adamw(Q, torch, dev)

    if args.only in ("all", "layers") and not args.no_layers:
        result["mlp_7b"] = bench_layers(Q, workloads, torch, dev, 3, args.layer_steps, 1)
        result["stack_65b"] = bench_layers(Q, workloads, torch, dev, 5, args.layer_steps, 1)

    if args.only in ("all", "headline") and not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(M, din, dout, r, alpha, flops)

    print(json.dumps(result))


def bench_gemv(Q, workloads, torch, dev, iters):
    """Skinny-token forward at the 65B shapes; weight GB/s on the packed weight."""
    out = {"unit": "GB/s", "peak": PEAK_HBM_GBPS, "bound": "hbm", "copies": 6, "cases": {}}
    r = 64
    s = 16.0 / r
    for din, dout in ((8192, 22016), (22016, 8192)):
        copies = []
        for c in range(6):
            W = workloads.device_normal_bf16(4000 + 10 * c, (dout, din), 0.02)
            copies.append(Q.qlora_quantize_nf4(W, True))
            del W
        A = workloads.device_normal_bf16(4001, (din, r), 0.02)
        B = workloads.device_normal_bf16(4002, (r, dout), 0.02)
        wb = weight_bytes(din, dout)
        for M in (1, 4, 16):
            X = workloads.device_normal_bf16(4003 + M, (M, din), 1.0)
            Y = torch.empty((M, dout), dtype=torch.bfloat16, device=dev)
            ws = torch.empty(Q.qlora_fwd_workspace(M, din, dout, r), dtype=torch.uint8, device=dev)
            for i in range(10):
                Q.qlora_linear_fwd(X, copies[i % 6], A, B, s, Y=Y, save_T=False, workspace=ws)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for i in range(iters):
                Q.qlora_linear_fwd(X, copies[i % 6], A, B, s, Y=Y, save_T=False, workspace=ws)
            e1.record()
            torch.cuda.synchronize()
            us = 1e3 * e0.elapsed_time(e1) / iters
            Q.qlora_profile_enable(True)
            Q.qlora_profile_read(reset=True)
            for i in range(iters):
                Q.qlora_linear_fwd(X, copies[i % 6], A, B, s, Y=Y, save_T=False, workspace=ws)
            torch.cuda.synchronize()
            prof = Q.qlora_profile_read(reset=True)
            Q.qlora_profile_enable(False)
            k = prof.get("k_fwd_nf4_gemv")
            kus = 1e3 * k[1] / k[0] if k else None
            out["cases"][f"{din}->{dout} M={M}"] = {
                "us_per_forward": us, "weight_GBps": wb / (us * 1e-6) / 1e9,
                "gemv_kernel_us": kus, "gemv_kernel_weight_GBps": (wb / (kus * 1e-6) / 1e9) if kus else None,
                "kernels_us": {kk: 1e3 * t / n for kk, (n, t) in prof.items()}}
        del copies
        torch.cuda.empty_cache()
    best = max(v["weight_GBps"] for v in out["cases"].values())
    worst = min(v["weight_GBps"] for v in out["cases"].values())
    out["weight_GBps_min"] = worst
    out["weight_GBps_max"] = best
    out["frac_min"] = worst / PEAK_HBM_GBPS
    return out


def bench_few_tokens(Q, workloads, torch, dev, iters=20):
    """Forward and backward of the 4096->4096, rank-64 layer for 1..1024 tokens, where the
    few 256-token panels of the large-M GEMMs would leave most compute units idle: the
    weight-streaming forward (M <= 64), the forward GEMM in K-slices (65..1024 tokens) and
    the dX GEMM in slices of the weight's rows (M <= 1024).  The 8.65 MB packed weight stays
    in the caches between calls; per-kernel times from the library's own HIP events."""
    din = dout = 4096
    r = 64
    s = 16.0 / r
    W = workloads.device_normal_bf16(5000, (dout, din), 0.02)
    w = Q.qlora_quantize_nf4(W, True)
    del W
    A = workloads.device_normal_bf16(5001, (din, r), 0.02)
    B = workloads.device_normal_bf16(5002, (r, dout), 0.02)
    out = {"shape": "4096->4096, r = 64, NF4 + double quant", "cases": {}}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for M in (1, 16, 64, 128, 256, 512, 1024):
        X = workloads.device_normal_bf16(5003 + M, (M, din), 1.0)
        dY = workloads.device_normal_bf16(5004 + M, (M, dout), 1.0)
        ws = torch.empty(max(Q.qlora_fwd_workspace(M, din, dout, r), Q.qlora_bwd_workspace(M, din, dout, r)),
                         dtype=torch.uint8, device=dev)
        Y = torch.empty((M, dout), dtype=torch.bfloat16, device=dev)
        T = torch.empty((M, r), dtype=torch.bfloat16, device=dev)
        dX = torch.empty((M, din), dtype=torch.bfloat16, device=dev)
        dA = torch.empty((din, r), dtype=torch.float32, device=dev)
        dB = torch.empty((r, dout), dtype=torch.float32, device=dev)
        calls = {"fwd": lambda: Q.qlora_linear_fwd(X, w, A, B, s, Y=Y, T_save=T, workspace=ws),
                 "bwd": lambda: Q.qlora_linear_bwd(dY, X, T, w, A, B, s, dX=dX, dA=dA, dB=dB, workspace=ws)}
        case = {}
        for name, fn in calls.items():
            for _ in range(5):
                fn()
            torch.cuda.synchronize()
            e0.record()
            for _ in range(iters):
                fn()
            e1.record()
            torch.cuda.synchronize()
            case[f"{name}_us"] = 1e3 * e0.elapsed_time(e1) / iters
            Q.qlora_profile_enable(True)
            Q.qlora_profile_read(reset=True)
            for _ in range(iters):
                fn()
            torch.cuda.synchronize()
            prof = Q.qlora_profile_read(reset=True)
            Q.qlora_profile_enable(False)
            case[f"{name}_kernels_us"] = {k: 1e3 * t / n for k, (n, t) in prof.items()}
        out["cases"][f"M={M}"] = case
    return out


def bench_layers(Q, workloads, torch, dev, cfg_idx, steps, warmup):
    """Large-token forward+backward over a whole configuration: the 7B MLP pair
    (4096->11008 and 11008->4096, 0.1% x20 outliers, M = 4096) or the 65B layer stack
    (80 layers x 7 linears, M = 2048, every NF4 weight resident).  A step is the forward
    over all linears, layer 0 first, then the backward in reverse order, each linear on
    its own seeded inputs; FLOPs 4 M in out + 6 M r (in + out) per linear."""
    cfg = workloads.CONFIGS[cfg_idx]
    lins = cfg.linears
    L = cfg.layers
    M, r = lins[0].M, lins[0].r

    if cfg_idx == 5:
        tensor = workloads.stack_tensor
        xslot = workloads.STACK_INPUT_SLOT
    else:
        def tensor(layer, j, what):
            lin = lins[j]
            sd = lambda tid: workloads.seed_for(cfg_idx, 10 * layer + j, tid)
            shape = {"W": (lin.d_out, lin.d_in), "A": (lin.d_in, r), "B": (r, lin.d_out),
                     "X": (M, lin.d_in), "dY": (M, lin.d_out)}[what]
            tid = {"W": workloads.TID_W, "A": workloads.TID_A, "B": workloads.TID_B,
                   "X": workloads.TID_X, "dY": workloads.TID_DY}[what]
            std = 0.02 if what in ("W", "A", "B") else 1.0
            op = lin.outlier_p if what == "W" else 0.0
            return workloads.device_normal_bf16(sd(tid), shape, std, dev, outlier_p=op,
                                                mask_seed=sd(workloads.TID_MASK))
        xslot = tuple(range(len(lins)))

    ws = torch.empty(max(max(Q.qlora_quantize_workspace(l.d_out, l.d_in), Q.qlora_fwd_workspace(M, l.d_in, l.d_out, r),
                             Q.qlora_bwd_workspace(M, l.d_in, l.d_out, r)) for l in lins),
                     dtype=torch.uint8, device=dev)
    wq = [[Q.nf4_alloc(l.d_out, l.d_in, True, dev) for l in lins] for _ in range(L)]
    quant_us = 0.0
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for layer in range(L):
        for j in range(len(lins)):
            W = tensor(layer, j, "W")
            e0.record()
            Q.qlora_quantize_nf4(W, True, out=wq[layer][j], workspace=ws)
            e1.record()
            torch.cuda.synchronize()
            quant_us += 1e3 * e0.elapsed_time(e1)
            del W
    AB = [[(tensor(layer, j, "A"), tensor(layer, j, "B")) for j in range(len(lins))] for layer in range(L)]
    X = [{j: tensor(layer, j, "X") for j in sorted(set(xslot))} for layer in range(L)]
    dY = [[tensor(layer, j, "dY") for j in range(len(lins))] for layer in range(L)]
    T = [[torch.empty((M, r), dtype=torch.bfloat16, device=dev) for _ in lins] for _ in range(L)]
    Y = [torch.empty((M, l.d_out), dtype=torch.bfloat16, device=dev) for l in lins]
    dX = [torch.empty((M, l.d_in), dtype=torch.bfloat16, device=dev) for l in lins]
    dA = [[torch.empty((l.d_in, r), dtype=torch.float32, device=dev) for l in lins] for _ in range(L)]
    dB = [[torch.empty((r, l.d_out), dtype=torch.float32, device=dev) for l in lins] for _ in range(L)]
    torch.cuda.synchronize()

    def step():
        for layer in range(L):
            for j, l in enumerate(lins):
                A, B = AB[layer][j]
                Q.qlora_linear_fwd(X[layer][xslot[j]], wq[layer][j], A, B, l.scale, Y=Y[j], T_save=T[layer][j],
                                   workspace=ws)
        for layer in reversed(range(L)):
            for j, l in enumerate(lins):
                A, B = AB[layer][j]
                Q.qlora_linear_bwd(dY[layer][j], X[layer][xslot[j]], T[layer][j], wq[layer][j], A, B, l.scale,
                                   dX=dX[j], dA=dA[layer][j], dB=dB[layer][j], workspace=ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    flops = L * sum(flops_fwd_bwd(M, l.d_in, l.d_out, r) for l in lins)
    Q.qlora_profile_enable(True)
    Q.qlora_profile_read(reset=True)
    step()
    torch.cuda.synchronize()
    prof = Q.qlora_profile_read(reset=True)
    Q.qlora_profile_enable(False)
    nf4_bytes = sum(w.nbytes() for row in wq for w in row)
    out = {"workload": cfg.name, "layers": L, "linears": L * len(lins), "steps": steps, "warmup": warmup,
           "ms_per_step": ms, "flops_per_step": flops, "TFLOPs": flops / (ms * 1e-3) / 1e12,
           "frac": flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, "peak": PEAK_BF16_TFLOPS,
           "nf4_resident_GB": nf4_bytes / 1e9, "hbm_allocated_GB": torch.cuda.memory_allocated() / 1e9,
           "quantize_all_ms": quant_us / 1e3,
           "kernels_ms_per_step": {k: t for k, (n, t) in prof.items()}}
    del wq, AB, X, dY, T, Y, dX, dA, dB, ws
    torch.cuda.empty_cache()
    return out


def bench_formats(Q, workloads, torch, dev, iters=20):
    """Format variants on the headline weight shape, with double quantization.

    codebooks: relative mean squared error of the dequantized bf16 weight for the three
    16-entry tables (NF4, FP4 = E2M1 / 6, Int4 = k / 7), the synthetic stand-in for the
    pages' data-type comparison.  block_sizes: for NF4 blocks of 32, 64, 128 and 256
    weights, the same error (also with 0.1 % of the entries x20), the bits of constants per
    weight from the library's buffer sizes, and the headline forward + backward step time
    with that block size ("Double quantization": smaller blocks are more precise and pay
    the per-block constant more often)."""
    W = workloads.device_normal_bf16(2500, (4096, 4096), 0.02)
    Wo = workloads.device_normal_bf16(2510, (4096, 4096), 0.02, outlier_p=0.001, mask_seed=2511)
    w, wo = W.float(), Wo.float()
    den, deno = (w * w).mean().item(), (wo * wo).mean().item()
    out = {"codebooks": {}, "block_sizes": {}}
    for name, cb in Q.CODEBOOKS.items():
        q = Q.qlora_quantize_nf4(W, True, codebook=cb)
        d = Q.qlora_dequant(q).float()
        out["codebooks"][name] = {"rel_mse": ((d - w) ** 2).mean().item() / den}
        del q, d
    out["codebooks"]["order"] = " < ".join(sorted(Q.CODEBOOKS, key=lambda k: out["codebooks"][k]["rel_mse"]))

    M, din, dout, r, s = 2048, 4096, 4096, 64, 0.25
    A = workloads.device_normal_bf16(2520, (din, r), 0.02)
    B = workloads.device_normal_bf16(2521, (r, dout), 0.02)
    X = workloads.device_normal_bf16(2522, (M, din), 1.0)
    dY = workloads.device_normal_bf16(2523, (M, dout), 1.0)
    Y = torch.empty((M, dout), dtype=torch.bfloat16, device=dev)
    T = torch.empty((M, r), dtype=torch.bfloat16, device=dev)
    dX = torch.empty((M, din), dtype=torch.bfloat16, device=dev)
    dA = torch.empty((din, r), dtype=torch.float32, device=dev)
    dB = torch.empty((r, dout), dtype=torch.float32, device=dev)
    ws = torch.empty(max(Q.qlora_fwd_workspace(M, din, dout, r), Q.qlora_bwd_workspace(M, din, dout, r)),
                     dtype=torch.uint8, device=dev)
    flops = 4 * M * din * dout + 6 * M * r * (din + dout)
    for block in (32, 64, 128, 256):
        q = Q.qlora_quantize_nf4(W, True, block=block)
        d = Q.qlora_dequant(q).float()
        qo = Q.qlora_quantize_nf4(Wo, True, block=block)
        do = Q.qlora_dequant(qo).float()
        cb_, ab, c1b, mub = Q.qlora_nf4_sizes(dout, din, True, block)
        rec = {"rel_mse": ((d - w) ** 2).mean().item() / den, "rel_mse_outliers": ((do - wo) ** 2).mean().item() / deno,
               "constant_bits_per_weight": 8.0 * (ab + c1b + mub) / (din * dout)}

        def step():
            Q.qlora_linear_fwd(X, q, A, B, s, Y=Y, T_save=T, workspace=ws)
            Q.qlora_linear_bwd(dY, X, T, q, A, B, s, dX=dX, dA=dA, dB=dB, workspace=ws)

        for _ in range(3):
            step()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            step()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / iters
        rec.update(step_ms=ms, step_TFLOPs=flops / (ms * 1e-3) / 1e12)
        out["block_sizes"][str(block)] = rec
        del q, d, qo, do
    torch.cuda.empty_cache()
    return out


def bench_comparators(Q, workloads, torch, dev, ms_qlora, iters=20):
    """Context for the headline step (never part of the library): the same forward and
    backward with (i) the unquantized bf16 weight ("LoRA without quantization") and (ii) the
    weight dequantized into a bf16 buffer first ("materialize then GEMM"), the products done
    by torch's bf16 matmul (hipBLASLt) with fp32 accumulation.  The pages put QLoRA's step at
    25-40% slower than LoRA on unquantized weights ("QLoRA: quantising the part you are not
    training", section "What it costs")."""
    M, din, dout, r, s = 2048, 4096, 4096, 64, 0.25
    W = workloads.device_normal_bf16(2700, (dout, din), 0.02)
    A = workloads.device_normal_bf16(2701, (din, r), 0.02)
    B = workloads.device_normal_bf16(2702, (r, dout), 0.02)
    X = workloads.device_normal_bf16(2703, (M, din), 1.0)
    dY = workloads.device_normal_bf16(2704, (M, dout), 1.0)
    w = Q.qlora_quantize_nf4(W, True)
    Wt, At, Bt, Xt = W.t().contiguous(), A.t().contiguous(), B.t().contiguous(), X.t().contiguous()
    Wd = torch.empty_like(W)

    def lora_step(Wb, Wbt):
        T = X @ A                                   # forward
        Y = X @ Wbt + (T * s) @ B
        G = dY @ Bt                                 # backward
        dX = dY @ Wb + (G * s) @ At
        dA = (Xt @ G) * s
        dB = (T.t().contiguous() @ dY) * s
        return Y, dX, dA, dB

    def materialize_step():
        Q.qlora_dequant(w, out=Wd)
        return lora_step(Wd, Wd.t().contiguous())

    out = {}
    for name, fn in (("lora_unquantized_bf16", lambda: lora_step(W, Wt)), ("materialize_then_gemm", materialize_step)):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / iters
        out[name] = {"ms_per_step": ms, "qlora_step_over_this": ms_qlora / ms}

    # measured ceilings: the plain bf16 GEMM of the forward's shape on hipBLASLt (no
    # dequantization), and HBM streaming rates of torch's copy and sum over 1 GiB
    def timed(fn, n):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return 1e3 * e0.elapsed_time(e1) / n   # us

    us = timed(lambda: X @ Wt, 50)
    big = torch.empty(1 << 29, dtype=torch.bfloat16, device=dev).normal_()
    dst = torch.empty_like(big)
    us_copy = timed(lambda: dst.copy_(big), 10)
    out["ceilings"] = {
        "hipblaslt_bf16_gemm_2048x4096x4096": {"us": us, "TFLOPs": 2 * M * din * dout / (us * 1e-6) / 1e12},
        "device_copy_1GiB": {"us": us_copy, "GBps": 2 * (1 << 30) / (us_copy * 1e-6) / 1e9,
                             "note": "bytes read + written per second"},
    }
    del W, A, B, X, dY, w, Wt, At, Bt, Xt, Wd, big, dst
    torch.cuda.empty_cache()
    return out


def bench_merge(Q, workloads, torch, dev, iters=10):
    """Adapter merge + requantize on the headline layer (4096x4096, r = 64, s = 0.25):
    time of qlora_merge_adapter and of requantizing its bf16 output, and the error the
    requantization leaves in the layer's output on 2048 tokens:
    |X deq(requant(W'))^T - Y| / |Y| with Y the unmerged layer (base + adapter), beside the
    size of the adapter's own contribution |Y - X deq(W)^T| / |Y|."""
    M, din, dout, r, s = 2048, 4096, 4096, 64, 0.25
    W = workloads.device_normal_bf16(2600, (dout, din), 0.02)
    A = workloads.device_normal_bf16(2601, (din, r), 0.02)
    B = workloads.device_normal_bf16(2602, (r, dout), 0.02)
    X = workloads.device_normal_bf16(2603, (M, din), 1.0)
    w = Q.qlora_quantize_nf4(W, True)
    Wm = torch.empty((dout, din), dtype=torch.bfloat16, device=dev)
    wm = Q.nf4_alloc(dout, din, True, dev)
    ws = torch.empty(Q.qlora_quantize_workspace(dout, din), dtype=torch.uint8, device=dev)
    for _ in range(2):
        Q.qlora_merge_adapter(w, A, B, s, out=Wm)
        Q.qlora_quantize_nf4(Wm, True, out=wm, workspace=ws)
    torch.cuda.synchronize()
    e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    e0.record()
    for _ in range(iters):
        Q.qlora_merge_adapter(w, A, B, s, out=Wm)
    e1.record()
    for _ in range(iters):
        Q.qlora_quantize_nf4(Wm, True, out=wm, workspace=ws)
    e2.record()
    torch.cuda.synchronize()
    Y, _ = Q.qlora_linear_fwd(X, w, A, B, s, save_T=False)
    Z = torch.zeros_like(B)
    Ym, _ = Q.qlora_linear_fwd(X, wm, A, Z, s, save_T=False)
    Yb, _ = Q.qlora_linear_fwd(X, w, A, Z, s, save_T=False)
    y, ym, yb = Y.float(), Ym.float(), Yb.float()
    ny = torch.linalg.vector_norm(y).item()
    out = {"merge_us": 1e3 * e0.elapsed_time(e1) / iters, "requantize_us": 1e3 * e1.elapsed_time(e2) / iters,
           "output_rel_err_merged_requantized": torch.linalg.vector_norm(ym - y).item() / ny,
           "output_rel_size_of_adapter_term": torch.linalg.vector_norm(y - yb).item() / ny}
    del W, A, B, X, w, Wm, wm, ws, Y, Ym, Yb, Z
    torch.cuda.empty_cache()
    return out


def bench_adamw(Q, torch, dev, iters=10):
    """AdamW step on the adapters: the 4096->4096 rank-64 adapter (A and B, 524,288
    parameters) and the whole 65B stack's adapters as one buffer (80 x 7 linears at
    rank 64: 799,539,200 parameters).  Bytes per parameter: fp32 param, grad, m, v read
    (16) and param, m, v written (12) plus the bf16 working copy (2)."""
    out = {"bytes_per_param": 30, "peak_GBps": PEAK_HBM_GBPS}
    for name, n in (("adapter_4096x4096_r64", 2 * 4096 * 64), ("stack_65b_adapters", 799_539_200)):
        g = torch.Generator(device=dev)
        g.manual_seed(3000)
        p = torch.randn(n, generator=g, device=dev, dtype=torch.float32).mul_(0.02)
        grad = torch.randn(n, generator=g, device=dev, dtype=torch.float32).mul_(1e-3)
        m = torch.zeros(n, device=dev, dtype=torch.float32)
        v = torch.zeros(n, device=dev, dtype=torch.float32)
        pb = torch.empty(n, device=dev, dtype=torch.bfloat16)
        for t in range(1, 3):
            Q.qlora_adamw_step(p, grad, m, v, t, 2e-4, weight_decay=0.01, param_bf16=pb)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for t in range(3, 3 + iters):
            Q.qlora_adamw_step(p, grad, m, v, t, 2e-4, weight_decay=0.01, param_bf16=pb)
        e1.record()
        torch.cuda.synchronize()
        us = 1e3 * e0.elapsed_time(e1) / iters
        out[name] = {"params": n, "us_per_step": us, "GBps": 30 * n / (us * 1e-6) / 1e9}
        if name == "stack_65b_adapters":
            out[name]["paged"] = bench_paging(Q, torch, [p, m, v], lambda t: Q.qlora_adamw_step(
                p, grad, m, v, t, 2e-4, weight_decay=0.01, param_bf16=pb), 3 + iters)
        del p, grad, m, v, pb
        torch.cuda.empty_cache()
    out["host_state"] = bench_adamw_host_state(Q, torch, dev, iters)
    return out


def bench_paging(Q, torch, state, step, t):
    """Paged optimizer state ("Paged optimizers"): the fp32 master, m and v paged out to pinned
    host memory and back in with qlora_state_page_out / qlora_state_page_in, each direction
    timed on its own (HIP events); the paged step is page-in + step + page-out."""
    host = [torch.empty(x.numel(), dtype=torch.float32, pin_memory=True) for x in state]
    nbytes = sum(x.nbytes for x in state)
    e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    torch.cuda.synchronize()
    e[0].record()
    for x, h in zip(state, host):
        Q.qlora_state_page_out(x, h)
    e[1].record()
    for x, h in zip(state, host):
        Q.qlora_state_page_in(h, x)
    e[2].record()
    step(t)
    e[3].record()
    torch.cuda.synchronize()
    out_ms, in_ms, step_ms = (e[i].elapsed_time(e[i + 1]) for i in range(3))
    del host
    return {"state_bytes": nbytes, "page_out_ms": out_ms, "page_in_ms": in_ms, "step_ms": step_ms,
            "paged_step_ms": out_ms + in_ms + step_ms, "page_out_GBps": nbytes / (out_ms * 1e-3) / 1e9,
            "page_in_GBps": nbytes / (in_ms * 1e-3) / 1e9}


def bench_adamw_host_state(Q, torch, dev, iters, n=32 * 1024 * 1024):
    """The same step with the fp32 master, m and v paged out to pinned host memory ("Paged
    optimizers"): the kernel reads and writes them through their mapped device addresses
    (hipHostGetDevicePointer), the gradient and the bf16 working copy stay in HBM.  24 bytes
    per parameter cross the host link."""
    import ctypes
    with open("/proc/self/maps") as f:
        paths = {line.split()[-1] for line in f if "libamdhip64.so" in line}
    if len(paths) != 1:
        return None
    hip = ctypes.CDLL(paths.pop())
    host = [torch.zeros(n, dtype=torch.float32).pin_memory() for _ in range(3)]
    ptrs = []
    for t in host:
        d = ctypes.c_void_p()
        if hip.hipHostGetDevicePointer(ctypes.byref(d), ctypes.c_void_p(t.data_ptr()), ctypes.c_uint(0)) != 0:
            return None
        ptrs.append(d)
    grad = torch.full((n,), 1e-3, device=dev, dtype=torch.float32)
    pb = torch.empty(n, device=dev, dtype=torch.bfloat16)
    lib = Q.lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def step(t):
        rc = lib.qlora_adamw_step(ptrs[0], ctypes.c_void_p(pb.data_ptr()), ctypes.c_void_p(grad.data_ptr()), ptrs[1],
                                  ptrs[2], n, t, 2e-4, 0.9, 0.999, 1e-8, 0.01, stream)
        if rc != 0:
            raise RuntimeError(f"qlora_adamw_step: status {rc}")

    step(1)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for t in range(2, 2 + iters):
        step(t)
    e1.record()
    torch.cuda.synchronize()
    us = 1e3 * e0.elapsed_time(e1) / iters
    return {"params": n, "us_per_step": us, "host_link_GBps": 24 * n / (us * 1e-6) / 1e9}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _blas_info():
    """(name, threads) of the BLAS NumPy calls, from threadpoolctl when it is importable."""
    try:
        from threadpoolctl import threadpool_info

        for i in threadpool_info():
            if i.get("user_api") == "blas":
                return f"{i.get('internal_api')} {i.get('version')}", i.get("num_threads")
    except Exception:
        pass
    return None, None


def cpu_baseline(M, din, dout, r, alpha, flops):
    """The oracle as it stands, on the host cores.

    value: one step of the headline workload (dequantize + forward + backward, the weight
    quantized beforehand, as the GPU step), averaged over up to 5 repeats (about 10 s).
    legs: every configuration once -- C1 (quantize + dequantize + forward + backward), C2
    (the quantize alone), C3 both shapes in full, C4 (each 65B-shaped weight quantized and
    dequantized once, then the forward at 1, 4 and 16 tokens), and C5 as an extrapolation:
    one linear of each of its three shapes (quantize, dequantize, forward, backward at 2048
    tokens; the 65B shapes reuse the C4 weights' quantize and dequantize times), one layer =
    4 x (8192->8192) + 2 x (8192->22016) + 1 x (22016->8192), times 80."""
    import numpy as np

    import workloads
    from oracle import linear, nf4

    def timed(fn):
        t0 = time.perf_counter()
        out = fn()
        return out, time.perf_counter() - t0

    lin = workloads.Linear("proj", M, din, dout, r, alpha)
    inp = workloads.linear_inputs(2, lin)
    q, c2_quant_s = timed(lambda: nf4.quantize(inp.W, double_quant=True))
    reps, total = 0, 0.0
    while reps < 5 and (reps == 0 or total < 10.0):   # about 10 s of CPU work
        t0 = time.perf_counter()
        Wd = nf4.dequantize(q, (dout, din))
        linear.forward(inp.X, Wd, inp.A, inp.B, lin.scale)
        linear.backward(inp.dY, inp.X, Wd, inp.A, inp.B, lin.scale)
        total += time.perf_counter() - t0
        reps += 1
    dt = total / reps
    del Wd, q, inp
    blas, blas_threads = _blas_info()

    def full(cfg, lin, backward=True):
        """quantize + dequantize + forward (+ backward) of one linear, each part timed."""
        li = workloads.linear_inputs(cfg, lin)
        qq, tq = timed(lambda: nf4.quantize(li.W, double_quant=True))
        wd, td = timed(lambda: nf4.dequantize(qq, (lin.d_out, lin.d_in)))
        _, tf = timed(lambda: linear.forward(li.X, wd, li.A, li.B, lin.scale))
        rec = {"quantize_s": tq, "dequant_s": td, "fwd_s": tf}
        if backward:
            _, tb = timed(lambda: linear.backward(li.dY, li.X, wd, li.A, li.B, lin.scale))
            rec["bwd_s"] = tb
        rec["total_s"] = sum(rec.values())
        return rec, li, wd

    legs = {}
    rec, _, _ = full(1, workloads.CONFIGS[1].linears[0])
    legs["C1"] = rec
    legs["C2"] = {"quantize_s": c2_quant_s, "dequant_fwd_bwd_s": dt}
    legs["C3"] = {l.name: full(3, l)[0] for l in workloads.CONFIGS[3].linears}
    # C4: two distinct weights (one per orientation); the forward at each token count
    c4, c5_parts = {}, {}
    for nm, di, do in (("up", 8192, 22016), ("down", 22016, 8192)):
        base = next(l for l in workloads.CONFIGS[4].linears if l.name == f"{nm}_M1")
        rec, li, wd = full(4, base, backward=False)
        for m in (1, 4, 16):
            lm = workloads.Linear(f"{nm}_M{m}", m, di, do, 64, 16.0)
            X = workloads.linear_inputs(4, lm, which=("X",)).X
            _, tf = timed(lambda: linear.forward(X, wd, li.A, li.B, lm.scale))
            c4[lm.name] = {"quantize_s": rec["quantize_s"], "dequant_s": rec["dequant_s"], "fwd_s": tf,
                           "total_s": rec["quantize_s"] + rec["dequant_s"] + tf}
        # the C5 linear of the same shape: forward + backward at 2048 tokens on this weight
        l5 = workloads.Linear(nm, 2048, di, do, 64, 16.0)
        t5 = workloads.linear_inputs(5, l5, which=("A", "B", "X", "dY"))
        _, tf = timed(lambda: linear.forward(t5.X, wd, t5.A, t5.B, l5.scale))
        _, tb = timed(lambda: linear.backward(t5.dY, t5.X, wd, t5.A, t5.B, l5.scale))
        c5_parts[(di, do)] = rec["quantize_s"] + rec["dequant_s"] + tf + tb
        del wd, li
    legs["C4"] = c4
    rec, _, _ = full(5, workloads.CONFIGS[5].linears[0])
    c5_parts[(8192, 8192)] = rec["total_s"]
    layer_s = 4 * c5_parts[(8192, 8192)] + 2 * c5_parts[(8192, 22016)] + c5_parts[(22016, 8192)]
    legs["C5"] = {"extrapolated": True, "per_linear_s": {f"{a}->{b}": v for (a, b), v in c5_parts.items()},
                  "layer_s": layer_s, "stack_80_layers_s": 80 * layer_s,
                  "note": "one linear of each shape timed (quantize + dequantize + forward + backward, M = 2048); "
                          "layer = 4 x 8192->8192 + 2 x 8192->22016 + 1 x 22016->8192; stack = 80 layers"}
    cores = blas_threads or len(os.sched_getaffinity(0))
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "cpu_model": _cpu_model(), "blas": blas, "seconds_per_step": dt, "repeats": reps,
            "sample": "value: full steps of the headline workload (dequantize + forward + backward; the weight "
                      "quantized once before), float64 NumPy, BLAS threads = cores, averaged over the repeats; "
                      "legs: every configuration timed once (C5 extrapolated from one linear per shape)",
            "legs": legs}


if __name__ == "__main__":
    main()
