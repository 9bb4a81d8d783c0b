#!/usr/bin/env python3
"""Benchmark of the block-quantized GEMM hot path on one MI355X.

A step is one pass of the whole path over one batch: kq_quantize_act (fp32
activations -> Q8_K blocks) then kq_gemm (Q4_K weights x Q8_K activations ->
fp32 out).  The default workload is the 4096 -> 14336 FFN gate/up projection
at 2048 tokens (M=2048, N=14336, K=4096, seeded synthetic data), the shape the
headline metric is quoted on.  Inputs are resident in HBM before timing; the
weight, activation and output buffers rotate over enough copies that
consecutive steps touch more than 512 MB, twice the 256 MB Infinity Cache.

Prints ONE JSON line.  `roofline` describes the GEMM kernel: algorithmic int8
ops per launch over its mean launch time (HIP events on the launch stream)
against the 5.0 POP/s dense int8 MFMA peak.  `cpu_baseline` is the plain CPU
oracle timed on a bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "effective int8 TOPS + prefill tok/s, Q4_K x Q8_K 4096x14336 GEMM; % of peak"
PEAK_INT8_TOPS = 5000.0     # MI355X dense int8 MFMA, 5.0 POP/s
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, 8 TB/s
ROTATE_BYTES = 512 << 20


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="ffn_up_q4k_2048")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle sample")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this path has no multi-GPU mode "
              "(the GEMM would shard along output rows; see DESIGN.md)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import block_quantized_matmul_act_amd as kq
    import datagen

    wl = datagen.WORKLOADS[args.workload]
    M, N, K, fmt = wl.M, wl.N, wl.K, wl.fmt
    act_fmt = kq.kq_act_fmt_for(fmt)
    dev = torch.device("cuda:0")

    log(f"[bench] generating {wl.name} M={M} N={N} K={K}")
    W_np, x_np = datagen.make_workload(wl)

    w_bytes = kq.kq_weight_bytes(fmt, N, K)
    a_bytes = kq.kq_act_bytes(act_fmt, M, K)
    x_bytes = M * K * 4
    o_bytes = M * N * 4
    per_step = w_bytes + a_bytes + x_bytes + o_bytes
    ncopy = max(1, min(16, -(-ROTATE_BYTES // per_step)))
    log(f"[bench] {ncopy} rotating buffer sets of {per_step / 2**20:.1f} MiB")
    Ws = [torch.from_numpy(W_np).to(dev) for _ in range(ncopy)]
    xs = [torch.from_numpy(x_np).to(dev) for _ in range(ncopy)]
    As = [torch.empty(a_bytes, dtype=torch.uint8, device=dev) for _ in range(ncopy)]
    Os = [torch.empty((M, N), dtype=torch.float32, device=dev) for _ in range(ncopy)]
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    def step(i, ev=None):
        j = i % ncopy
        if ev is not None:
            ev[0].record(stream)
        kq.kq_quantize_act(act_fmt, xs[j], M, K, As[j], sp)
        if ev is not None:
            ev[1].record(stream)
        kq.kq_gemm(fmt, Ws[j], As[j], M, N, K, Os[j], sp)
        if ev is not None:
            ev[2].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    quant_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    gemm_ms = np.array([e[1].elapsed_time(e[2]) for e in evs])
    step_ms = wall * 1e3 / args.steps
    ops = 2.0 * M * N * K

    gemm_mean_s = float(gemm_ms.mean()) * 1e-3
    quant_mean_s = float(quant_ms.mean()) * 1e-3
    value_tops = ops / (step_ms * 1e-3) / 1e12
    gemm_tops = ops / gemm_mean_s / 1e12

    result = {
        "metric": METRIC,
        "value": round(value_tops, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic",
        "config": {"workload": wl.name, "fmt": datagen.FMT_NAMES[fmt], "M": M, "N": N, "K": K,
                   "seed": wl.seed, "note": wl.note},
        "tok_per_s": round(M / (step_ms * 1e-3), 1),
        "gemm": {"mean_us": round(gemm_mean_s * 1e6, 2),
                 "min_us": round(float(gemm_ms.min()) * 1e3, 2),
                 "median_us": round(float(np.median(gemm_ms)) * 1e3, 2),
                 "tops": round(gemm_tops, 2),
                 "tok_per_s": round(M / gemm_mean_s, 1),
                 "frac_int8_peak": round(gemm_tops / PEAK_INT8_TOPS, 4),
                 "weight_gbs": round(w_bytes / gemm_mean_s / 1e9, 1),
                 "frac_hbm_on_weights": round(w_bytes / gemm_mean_s / 1e9 / PEAK_HBM_GBS, 4)},
        "quantize": {"mean_us": round(quant_mean_s * 1e6, 2),
                     "gbs": round((x_bytes + a_bytes) / quant_mean_s / 1e9, 1),
                     "frac_hbm": round((x_bytes + a_bytes) / quant_mean_s / 1e9 / PEAK_HBM_GBS,
                                       4)},
        "roofline": {"bound": "mfma" if M >= 256 else "hbm",
                     "kernel": kq.kq_variant_name(kq.kq_select_variant(fmt, M, N, K)),
                     "achieved": None, "peak": None, "unit": None, "frac": None,
                     "traffic": None},
        "dispatch": kq.dispatch_counts(),
    }
    if M >= 256:
        result["roofline"].update({"achieved": round(gemm_tops, 2), "peak": PEAK_INT8_TOPS,
                                   "unit": "TOP/s", "frac": round(gemm_tops / PEAK_INT8_TOPS, 4)})
    else:
        gbs = (w_bytes + a_bytes + o_bytes) / gemm_mean_s / 1e9
        result["roofline"].update({"achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                                   "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4)})

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, W_np, x_np, Os[(args.steps - 1) % ncopy],
                                              args.cpu_seconds)
    print(json.dumps(result), flush=True)


def cpu_baseline(wl, W_np, x_np, out_dev, target_s):
    """The plain CPU oracle (quantize + fp64 dequantize-and-multiply) on a
    bounded sample of the workload: all tokens, a subset of weight rows.  Also
    re-checks the GPU output on those rows."""
    import numpy as np

    from oracle import kqref

    act_fmt = kqref.ACT_FOR[wl.fmt]
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    t = time.perf_counter()
    qs, d, _ = kqref.quantize_act(act_fmt, x_np)
    tq = time.perf_counter() - t
    rng = np.random.default_rng(5)
    # calibrate on a few rows, then size the sample to ~target_s
    probe = np.sort(rng.choice(wl.N, 8, replace=False))
    t = time.perf_counter()
    kqref.gemm(wl.fmt, W_np, qs, d, wl.K, rows=probe)
    per_row = max((time.perf_counter() - t) / len(probe), 1e-6)
    nrows = int(min(wl.N, max(8, (target_s - tq) / per_row)))
    rows = np.sort(rng.choice(wl.N, nrows, replace=False))
    t = time.perf_counter()
    ref, tol = kqref.gemm(wl.fmt, W_np, qs, d, wl.K, rows=rows)
    tg = time.perf_counter() - t
    ops = 2.0 * wl.M * nrows * wl.K
    # quantize cost attributed to the sample in proportion to its share of rows
    t_sample = tg + tq * nrows / wl.N
    got = out_dev[:, torch_index(rows, out_dev)].cpu().numpy().astype(np.float64)
    ratio = float((np.abs(got - ref) / tol).max())
    return {"value": round(ops / t_sample / 1e12, 6), "unit": "TOPS", "cores": cores,
            "kind": "oracle",
            "sample": f"{wl.name}: all {wl.M} tokens x {nrows} of {wl.N} weight rows, K={wl.K}; "
                      f"plain C oracle (fp32 Q8 quantize + fp64 dequantize-and-multiply), "
                      f"gcc -O2 -fopenmp; quantize {tq:.2f} s for all rows, "
                      f"multiply {tg:.2f} s",
            "gpu_vs_oracle_max_err_over_tol": round(ratio, 4)}


def torch_index(rows, t):
    import torch
    return torch.from_numpy(rows).to(t.device)


if __name__ == "__main__":
    main()
