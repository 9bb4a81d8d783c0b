#!/usr/bin/env python3
"""Benchmark of the block-quantized GEMM hot path on one MI355X.

A step is one pass of the whole path over one batch: kq_quantize_act (fp32
activations -> Q8_K blocks) then kq_gemm (Q4_K weights x Q8_K activations ->
fp32 out), or for an expert-indexed workload kq_gemm_id over a seeded top-k
routing (throughput counts 2 * routed rows * N * K).  The default workload is the 4096 -> 14336 FFN gate/up projection
at 2048 tokens (M=2048, N=14336, K=4096, seeded synthetic data), the shape the
headline metric is quoted on.  Inputs are resident in HBM before timing; the
weight, activation and output buffers rotate over enough copies that
consecutive steps touch more than 512 MB, twice the 256 MB Infinity Cache.

Prints ONE JSON line.  `roofline` describes the GEMM kernel (the dominant
one): algorithmic int8 ops per launch (2*M*N*K) over its mean launch time,
against the 5.0 POP/s dense int8 MFMA peak (for M < 256 the kernel is bound by
streaming the weights: algorithmic bytes per launch over HBM's 8 TB/s).  The
launch time comes from HIP events recorded on the stream the kernel is
launched on, around the same K launches issued back to back right after the
timed steps; `gemm.mean_us` and `quantize.mean_us` come from event pairs
around each launch in a separate, untimed pass of the same steps (they include
the dispatch gap after the preceding kernel).  The timed steps themselves carry
no events.
`traffic` is the HBM traffic per launch measured with rocprofv3 counters for
the current kernel source (profiles/*_traffic.md), or null when those counters
were taken on a different kernel source.  `calibration` holds the device's
own rates measured in the same run by the library's calibration kernels
(int8 MFMA with constant operands, with operands changing every iteration, and
with 4-10 VALU instructions per MFMA; fp32 VALU; HBM read over 1 GiB);
`roofline.frac_measured` is `achieved` over the measured rate (changing-operand
MFMA when compute-bound, HBM read for few tokens).  `cpu_baseline` is the plain CPU
oracle timed on a bounded sample of the same workload (with the host's CPU model).

`configs` reports the other workloads in the same run (by default the 64-token
FFN projection, the 512-token projection, the Q6_K down projection and the
ternary projection): GEMM launches only, back to back between two events on
the launch stream, each with its own roofline and the variant the dispatch
counters saw run.  `device` holds the SMI's shader and memory clocks and
package power before and after the run.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--no-cpu-baseline] [--no-calib] [--cpu-seconds S] [--copy-mib N]
                       [--side W1,W2,...] [--side-launches L]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "effective int8 TOPS + prefill tok/s, Q4_K x Q8_K 4096x14336 GEMM; % of peak"
PEAK_INT8_TOPS = 5000.0     # MI355X dense int8 MFMA, 5.0 POP/s
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, 8 TB/s
ROTATE_BYTES = 512 << 20
CALIB_READ_BYTES = 1 << 30   # HBM read calibration buffer, 4x the Infinity Cache
CSRC = os.path.join(ROOT, "block_quantized_matmul_act_amd", "csrc")
# the sources each format's GEMM kernels are built from
GEMM_SOURCES = {
    "q4_k": ("kq_gemm_q4k.hip", "kq_tile.hpp", "kq_device.hpp", "kq_launch.hpp"),
    "q6_k": ("kq_gemm.hip", "kq_gemm_ring.hip", "kq_gemv.hip", "kq_tile.hpp", "kq_device.hpp", "kq_launch.hpp"),
    "tq": ("kq_gemm.hip", "kq_gemm_tq.hip", "kq_gemm_ring.hip", "kq_gemv.hip", "kq_tile.hpp", "kq_device.hpp",
           "kq_launch.hpp"),
    "tq2": ("kq_gemm.hip", "kq_gemm_ring.hip", "kq_tile.hpp", "kq_device.hpp", "kq_launch.hpp"),
    # expert-indexed workloads: the gather mode of the Q4_K tile kernel
    # (kq_gemm_q4k.hip) or of the other formats' tile kernel (kq_gemm.hip)
    "moe": ("kq_gemm.hip", "kq_gemm_q4k.hip", "kq_tile.hpp", "kq_device.hpp", "kq_hooks.hpp"),
}


# the other configurations, reported beside the main one in the same line:
# the 64-token case of the same FFN projection (bound by the weight stream),
# the 512-token projection, the Q6_K down projection at 2048 and at 512 tokens
# (a prefill chunk, K in two parts), the ternary projection
SIDE_WORKLOADS = ("ffn_up_q4k_64", "proj_q4k_4096", "ffn_down_q6k_2048", "ffn_down_q6k_512", "tern_5120_2048")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _code_tokens(text: str) -> str:
    """The source with its comments removed and its whitespace collapsed, so
    that an edit of comments or layout does not count as a kernel change (the
    sources hold no string literal with a comment marker)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash(fmt_name: str) -> str:
    """sha256 (first 16 hex digits) over the code of one format's GEMM kernel
    sources, in order (comments and layout excluded)."""
    h = hashlib.sha256()
    for name in GEMM_SOURCES[fmt_name]:
        with open(os.path.join(CSRC, name), encoding="utf-8") as f:
            h.update(_code_tokens(f.read()).encode())
            h.update(b"\0")
    return h.hexdigest()[:16]


def measured_traffic(workload: str, fmt_name: str):
    """HBM bytes per GEMM launch from profiles/<...>_<workload>_traffic.md, if
    that file was measured on the current kernel source; else None."""
    pdir = os.path.join(ROOT, "profiles")
    if not os.path.isdir(pdir):
        return None
    want = kernel_source_hash(fmt_name)
    for name in sorted(os.listdir(pdir)):
        if not name.endswith(f"{workload}_traffic.md"):
            continue
        text = open(os.path.join(pdir, name)).read()
        h = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
        b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
        if h and b and h.group(1) == want:
            return float(b.group(1))
    return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="ffn_up_q4k_2048")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-calib", action="store_true",
                    help="skip the calibration kernels (measured peak rates)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--side", default=",".join(SIDE_WORKLOADS),
                    help="comma-separated workloads timed after the main one (GEMM launches "
                         "only, each with its own roofline); empty for none")
    ap.add_argument("--side-launches", type=int, default=50)
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="after timing, run one plain device copy of this many MiB "
                         "(the reference kernel for scaling profiler byte counters)")
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

    dev_state0 = device_state()
    log(f"[bench] generating {wl.name} M={M} N={N} K={K}")
    W_np, x_np = datagen.make_workload(wl)
    # an expert-indexed workload routes M tokens to topk of E experts: R
    # routed rows, each one expert's N x K product
    E = max(wl.experts, 1)
    src_key = "moe" if wl.experts else datagen.FMT_NAMES[fmt]  # sources of the GEMM kernel
    R = M * wl.topk if wl.experts else M
    if wl.experts:
        off_np, rows_np = datagen.draw_routing(M, wl.experts, wl.topk, wl.seed)
        off_d = torch.from_numpy(off_np).to(dev)
        rows_d = torch.from_numpy(rows_np).to(dev)

    w_bytes = kq.kq_weight_bytes(fmt, N, K) * E
    a_bytes = kq.kq_act_bytes(act_fmt, M, K)
    x_bytes = M * K * 4
    o_bytes = R * N * 4
    per_step = w_bytes + a_bytes + x_bytes + o_bytes
    ncopy = max(1, min(16, -(-ROTATE_BYTES // per_step)))
    log(f"[bench] {ncopy} rotating buffer sets of {per_step / 2**20:.1f} MiB")
    Ws = [torch.from_numpy(W_np).to(dev) for _ in range(ncopy)]
    xs = [torch.from_numpy(x_np).to(dev) for _ in range(ncopy)]
    As = [torch.empty(a_bytes, dtype=torch.uint8, device=dev) for _ in range(ncopy)]
    Os = [torch.empty((R, N), dtype=torch.float32, device=dev) for _ in range(ncopy)]
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    def gemm(j):
        if wl.experts:
            kq.kq_gemm_id(fmt, Ws[j], E, As[j], M, N, K, off_d, rows_d, R, Os[j], sp)
        else:
            kq.kq_gemm(fmt, Ws[j], As[j], M, N, K, Os[j], sp)

    def step(i, ev=None):
        j = i % ncopy
        if ev is not None:
            ev[0].record(stream)
        kq.kq_quantize_act(act_fmt, xs[j], M, K, As[j], sp)
        if ev is not None:
            ev[1].record(stream)
        gemm(j)
        if ev is not None:
            ev[2].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # the timed steps: nothing but the two launches per step
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    log(f"[bench] timed {args.steps} steps in {wall:.3f} s")

    # per-kernel breakdown, in a separate pass of the same steps with events
    # around each launch (the event packets cost a few microseconds per step,
    # so they stay out of the timed steps)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()

    # The roofline's launch duration: the same GEMM launches back to back on
    # the same stream (no quantize in between), so the events bracket kernel
    # time rather than the dispatch gap that follows each quantize.
    # (Launched through the C ABI with the pointers resolved beforehand: the
    # binding's argument checks take longer on the host than the shortest
    # kernels run, and would time the host instead.)
    launch = raw_gemm_launcher(kq, fmt, Ws, As, Os, M, N, K, sp,
                               (E, off_d.data_ptr(), rows_d.data_ptr(), R) if wl.experts else None)
    b2b = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    b2b[0].record(stream)
    for i in range(args.steps):
        launch(i % ncopy)
    b2b[1].record(stream)
    torch.cuda.synchronize()
    gemm_b2b_s = b2b[0].elapsed_time(b2b[1]) * 1e-3 / args.steps

    if args.copy_mib > 0:
        src = torch.empty(args.copy_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        src.fill_(1)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] reference copy of {args.copy_mib} MiB done")

    quant_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    gemm_ms = np.array([e[1].elapsed_time(e[2]) for e in evs])
    step_ms = wall * 1e3 / args.steps
    ops = 2.0 * R * N * K

    gemm_mean_s = float(gemm_ms.mean()) * 1e-3
    quant_mean_s = float(quant_ms.mean()) * 1e-3
    value_tops = ops / (step_ms * 1e-3) / 1e12
    gemm_tops = ops / gemm_mean_s / 1e12
    gemm_alg_bytes = w_bytes + a_bytes + o_bytes

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
                   **({"experts": wl.experts, "topk": wl.topk, "routed_rows": R} if wl.experts else {}),
                   "seed": wl.seed, "note": wl.note},
        "tok_per_s": round(M / (step_ms * 1e-3), 1),
        "gemm": {"mean_us": round(gemm_mean_s * 1e6, 2),
                 "min_us": round(float(gemm_ms.min()) * 1e3, 2),
                 "median_us": round(float(np.median(gemm_ms)) * 1e3, 2),
                 "tops": round(gemm_tops, 2),
                 "tok_per_s": round(M / gemm_mean_s, 1),
                 "frac_int8_peak": round(gemm_tops / PEAK_INT8_TOPS, 4),
                 "weight_gbs": round(w_bytes / gemm_mean_s / 1e9, 1),
                 "frac_hbm_on_weights": round(w_bytes / gemm_mean_s / 1e9 / PEAK_HBM_GBS, 4),
                 "algorithmic_bytes": gemm_alg_bytes,
                 "back_to_back_us": round(gemm_b2b_s * 1e6, 2)},
        "quantize": {"mean_us": round(quant_mean_s * 1e6, 2),
                     "gbs": round((x_bytes + a_bytes) / quant_mean_s / 1e9, 1),
                     "frac_hbm": round((x_bytes + a_bytes) / quant_mean_s / 1e9 / PEAK_HBM_GBS,
                                       4)},
        "dispatch": kq.dispatch_counts(),
        "kernel_source_sha256_16": kernel_source_hash(src_key),
    }
    traffic = measured_traffic(wl.name, src_key)
    if R >= 256:
        tops = ops / gemm_b2b_s / 1e12
        result["roofline"] = {"bound": "mfma", "achieved": round(tops, 2),
                              "peak": PEAK_INT8_TOPS, "unit": "TOP/s",
                              "frac": round(tops / PEAK_INT8_TOPS, 4), "traffic": traffic}
    else:
        gbs = gemm_alg_bytes / gemm_b2b_s / 1e9
        result["roofline"] = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                              "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                              "traffic": traffic}
    if wl.experts:  # the expert-indexed variant this run dispatched
        disp = kq.dispatch_counts()
        result["roofline"]["kernel"] = max((v for v in disp if v.startswith("gemm_id")), key=disp.get)
    else:
        result["roofline"]["kernel"] = kq.kq_variant_name(kq.kq_select_variant(fmt, M, N, K))

    if not args.no_calib:
        # the device's own rates, measured now: the GEMM's fraction of them
        # sits beside the fraction of the published peak
        cal = calibrate(kq, stream)
        result["calibration"] = cal
        rl = result["roofline"]
        measured = cal["mfma_i8_toggle_tops"] if rl["bound"] == "mfma" else cal["hbm_read_gbs"]
        rl["measured_peak"] = measured
        rl["frac_measured"] = round(rl["achieved"] / measured, 4)

    side = [w for w in args.side.split(",") if w and w != wl.name]
    if side:
        # free the main workload's rotation sets before the others allocate
        cpu_out = Os[(args.steps - 1) % ncopy].cpu()
        del Ws, xs, As, Os
        torch.cuda.empty_cache()
        result["configs"] = {w: side_config(kq, w, stream, args.side_launches) for w in side}
    else:
        cpu_out = Os[(args.steps - 1) % ncopy].cpu()
    result["device"] = {"before": dev_state0, "after": device_state()}

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, W_np, x_np, cpu_out, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def raw_gemm_launcher(kq, fmt, Ws, As, Os, M, N, K, sp, routing):
    """launch(j): kq_gemm (or kq_gemm_id with routing = (experts, off, rows,
    routed rows)) on buffer set j, straight through the C ABI with the
    device pointers taken once.  The buffers were checked by earlier calls
    through the binding with the same arguments."""
    L = kq.lib()
    ptr = [(W.data_ptr(), A.data_ptr(), O.data_ptr()) for W, A, O in zip(Ws, As, Os)]
    if routing is None:
        f = L.kq_gemm

        def launch(j):
            w, a, o = ptr[j]
            rc = f(fmt, w, a, M, N, K, o, sp)
            if rc != 0:
                raise RuntimeError(f"kq_gemm failed: {rc}")
    else:
        f = L.kq_gemm_id
        E, off, rows, R = routing

        def launch(j):
            w, a, o = ptr[j]
            rc = f(fmt, w, E, a, M, N, K, off, rows, R, o, sp)
            if rc != 0:
                raise RuntimeError(f"kq_gemm_id failed: {rc}")
    return launch


def _sysfs_device_dir():
    """sysfs directory of cuda:0's PCI function, or None."""
    try:
        import torch
        p = torch.cuda.get_device_properties(0)
        path = "/sys/bus/pci/devices/%04x:%02x:%02x.0" % (p.pci_domain_id, p.pci_bus_id, p.pci_device_id)
        return path if os.path.isdir(path) else None
    except Exception:
        return None


def device_state():
    """Shader and memory clocks (the current DPM levels) and package power
    read from the driver's sysfs files of cuda:0; None where a value cannot
    be read.  (No program is started for this: a process that has
    initialised the GPU must not replace a child with another program.)"""
    st = {"sclk_mhz": None, "mclk_mhz": None, "power_w": None}
    d = _sysfs_device_dir()
    if d is None:
        return st
    for key, fname in (("sclk_mhz", "pp_dpm_sclk"), ("mclk_mhz", "pp_dpm_mclk")):
        try:
            for line in open(os.path.join(d, fname)):
                if "*" in line:
                    m = re.search(r"(\d+)\s*Mhz", line, re.I)
                    if m:
                        st[key] = float(m.group(1))
        except OSError:
            pass
    try:
        hw = os.path.join(d, "hwmon")
        for h in sorted(os.listdir(hw)):
            for fname in ("power1_average", "power1_input"):
                f = os.path.join(hw, h, fname)
                if os.path.exists(f):
                    st["power_w"] = round(int(open(f).read().strip()) / 1e6, 1)
                    break
            if st["power_w"] is not None:
                break
    except (OSError, ValueError):
        pass
    return st


def side_config(kq, name, stream, launches):
    """One more workload, GEMM launches only: its activations quantized once
    per rotating buffer set, then `launches` GEMM launches back to back
    between two events on the launch stream (mean launch time), the variant
    that ran taken from the dispatch counters, and its roofline: int8 ops
    against the 5.0 POP/s peak for M >= 256, else algorithmic bytes against
    8 TB/s (with the weight bytes alone beside them)."""
    import torch

    import datagen
    wl = datagen.WORKLOADS[name]
    M, N, K, fmt = wl.M, wl.N, wl.K, wl.fmt
    act_fmt = kq.kq_act_fmt_for(fmt)
    log(f"[bench] side config {name} M={M} N={N} K={K}")
    W_np, x_np = datagen.make_workload(wl)
    w_bytes = kq.kq_weight_bytes(fmt, N, K)
    a_bytes = kq.kq_act_bytes(act_fmt, M, K)
    o_bytes = M * N * 4
    per = w_bytes + a_bytes + o_bytes
    ncopy = max(1, min(16, -(-ROTATE_BYTES // per)))
    dev = torch.device("cuda:0")
    Ws = [torch.from_numpy(W_np).to(dev) for _ in range(ncopy)]
    x = torch.from_numpy(x_np).to(dev)
    As = [kq.quantize_act(x, act_fmt) for _ in range(ncopy)]
    Os = [torch.empty((M, N), dtype=torch.float32, device=dev) for _ in range(ncopy)]
    sp = stream.cuda_stream
    for i in range(5):
        kq.kq_gemm(fmt, Ws[i % ncopy], As[i % ncopy], M, N, K, Os[i % ncopy], sp)
    torch.cuda.synchronize()
    before = kq.dispatch_counts()
    launch = raw_gemm_launcher(kq, fmt, Ws, As, Os, M, N, K, sp, None)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(launches):
        launch(i % ncopy)
    e1.record(stream)
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / launches
    ran = {k: v - before[k] for k, v in kq.dispatch_counts().items() if v != before[k]}
    variant = max(ran, key=ran.get)
    assert ran[variant] == launches, ran
    ops = 2.0 * M * N * K
    out = {"fmt": datagen.FMT_NAMES[fmt], "M": M, "N": N, "K": K, "seed": wl.seed,
           "gemm_us": round(t * 1e6, 2), "tops": round(ops / t / 1e12, 2),
           "tok_per_s": round(M / t, 1), "launches": launches}
    if M >= 256:
        tops = ops / t / 1e12
        out["roofline"] = {"bound": "mfma", "achieved": round(tops, 2), "peak": PEAK_INT8_TOPS,
                           "unit": "TOP/s", "frac": round(tops / PEAK_INT8_TOPS, 4), "kernel": variant,
                           "traffic": measured_traffic(name, datagen.FMT_NAMES[fmt])}
    else:
        gbs = per / t / 1e9
        out["roofline"] = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                           "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "kernel": variant,
                           "weight_gbs": round(w_bytes / t / 1e9, 1),
                           "frac_on_weights": round(w_bytes / t / 1e9 / PEAK_HBM_GBS, 4),
                           "traffic": measured_traffic(name, datagen.FMT_NAMES[fmt])}
    del Ws, As, Os, x
    torch.cuda.empty_cache()
    return out


def calibrate(kq, stream):
    """Calibration kernels of the library, each timed with HIP events on the
    stream it runs on (one warm-up launch, then the best of three)."""
    import torch

    def rate(kind, param=0, buf=None, nbytes=0):
        kq.kq_calib_launch(kind, param, buf, nbytes, stream.cuda_stream)
        best = None
        for _ in range(3):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            work = kq.kq_calib_launch(kind, param, buf, nbytes, stream.cuda_stream)
            e1.record(stream)
            torch.cuda.synchronize()
            r = work / (e0.elapsed_time(e1) * 1e-3)
            best = r if best is None else max(best, r)
        return best

    nbytes = CALIB_READ_BYTES
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    buf.fill_(3)
    cal = {
        "mfma_i8_tops": round(rate(kq.KQ_CALIB_MFMA_I8) / 1e12, 1),
        "mfma_i8_toggle_tops": round(rate(kq.KQ_CALIB_MFMA_I8_TOGGLE) / 1e12, 1),
        "mfma_i8_tops_with_valu_per_mfma": {
            str(p + 2): round(rate(kq.KQ_CALIB_MFMA_I8_VALU, p) / 1e12, 1) for p in (2, 4, 6, 8)},
        "valu_f32_tflops": round(rate(kq.KQ_CALIB_VALU_F32) / 1e12, 2),
        "hbm_read_gbs": round(rate(kq.KQ_CALIB_HBM_READ, 0, buf, nbytes) / 1e9, 1),
        "hbm_read_bytes": nbytes,
    }
    del buf
    log(f"[bench] calibration: {cal}")
    return cal


def cpu_baseline(wl, W_np, x_np, out_dev, target_s):
    import datagen
    if wl.experts:
        # expert-indexed: the sample is expert 0 (its tokens and its weights),
        # against the GPU's routed rows of expert 0
        off, toks = datagen.draw_routing(wl.M, wl.experts, wl.topk, wl.seed)
        t0 = toks[off[0]:off[1]]
        return _cpu_baseline(wl, wl.name + " expert 0", W_np[:wl.N], x_np[t0],
                             out_dev[int(off[0]):int(off[1])], target_s)
    return _cpu_baseline(wl, wl.name, W_np, x_np, out_dev, target_s)


def _cpu_baseline(wl, label, W_np, x_np, out_dev, target_s):
    """The plain CPU oracle (fp32 Q8 quantize, fp64 dequantize-and-multiply) on
    a bounded sample of the workload: all tokens against a random subset of
    weight rows, sized to about target_s seconds of CPU time.  The quantize
    cost is charged to the sample in proportion to its share of the rows.  The
    GPU output of the last step is re-checked on a few of those rows."""
    import numpy as np

    from oracle import kqref

    act_fmt = kqref.ACT_FOR[wl.fmt]
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    t = time.perf_counter()
    qs, d, _ = kqref.quantize_act(act_fmt, x_np)
    tq = time.perf_counter() - t
    rng = np.random.default_rng(5)
    # calibrate: double the sample until one run takes >= 1 s, then scale
    n, per_row = 16, None
    while n <= wl.N:
        rows = np.sort(rng.choice(wl.N, n, replace=False))
        t = time.perf_counter()
        kqref.gemm(wl.fmt, W_np, qs, d, wl.K, rows=rows, want_tol=False)
        dt = time.perf_counter() - t
        per_row = dt / n
        if dt >= 1.0:
            break
        n *= 2
    nrows = int(min(wl.N, max(16, (target_s - tq) / per_row)))
    rows = np.sort(rng.choice(wl.N, nrows, replace=False))
    log(f"[bench] cpu baseline: {nrows} weight rows (~{nrows * per_row:.1f} s)")
    t = time.perf_counter()
    kqref.gemm(wl.fmt, W_np, qs, d, wl.K, rows=rows, want_tol=False)
    tg = time.perf_counter() - t
    Mx = x_np.shape[0]
    ops = 2.0 * Mx * nrows * wl.K
    t_sample = tg + tq * nrows / wl.N
    check = rows[:: max(1, nrows // 8)][:8]
    ref, tol = kqref.gemm(wl.fmt, W_np, qs, d, wl.K, rows=check)
    import torch
    got = out_dev[:, torch.from_numpy(check)].numpy()
    ratio = float((np.abs(got.astype(np.float64) - ref) / tol).max())
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            m = re.search(r"^model name\s*:\s*(.+)$", f.read(), re.M)
            model = m.group(1).strip() if m else None
    except OSError:
        pass
    return {"value": round(ops / t_sample / 1e12, 6), "unit": "TOPS", "cores": cores,
            "cpu_model": model, "kind": "oracle",
            "sample": f"{label}: all {Mx} tokens x {nrows} of {wl.N} weight rows (random), "
                      f"K={wl.K}; plain C oracle (fp32 Q8 quantize + fp64 "
                      f"dequantize-and-multiply), gcc -O2 -fopenmp; quantize {tq:.2f} s for all "
                      f"rows (charged pro rata), multiply {tg:.2f} s",
            "gpu_vs_oracle_max_err_over_tol": round(ratio, 4)}


if __name__ == "__main__":
    main()
