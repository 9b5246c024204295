#!/usr/bin/env python3
"""Benchmark of the FlashAttention forward pass (libfa355) on one MI355X.

One step = one fa_fwd call over one batch of the workload (the whole hot path: a single fused
kernel). Default workload: causal attention, B=4, Hq=Hkv=32, Nq=Nk=4096, D=64, fp16, scale 1/8 —
the pages' benchmark shape ("Flash Attention - Fast Memory-Efficient Attention", skill page,
Workflow 2 Step 4, [4, 4096, 32, 64] fp16, 10 warm-up and 100 timed iterations), run causal.

Metric: attention forward TFLOP/s with FLOPs = 4 * B * Hq * Nq * Nk * D, halved for causal; for
a sliding window the admitted-pair count replaces Nq * Nk (4 * B * Hq * D * pairs). Inputs are
resident in device memory before the timed region. Prints one JSON line.

``--workload varlen_...`` times fa_fwd_varlen on a packed batch of sequences of seeded lengths
(no padding); its FLOPs are the sum of the sequences' own (causal halved).

``--workload decode_*`` times fa_fwd_kvcache: a few new queries per sequence against a dense or
paged KV cache of seeded lengths. That path is bound by HBM bandwidth, so its line reports GB/s of
algorithmic traffic (each sequence's keys and values read once, q read, out and lse written)
against the 8 TB/s peak, with the TFLOP/s alongside.

``--workload blocksparse_*`` times fa_fwd_blocksparse on a long causal sequence with a local +
sink + random block mask; its FLOPs are 4 * D per admitted (query, key) pair, and the dense
causal forward on the same inputs is timed beside it (speedup).

``--pass bwd`` times the backward pass (fa_bwd: dq, dk, dv for a seeded N(0, 1) upstream gradient,
after one forward pass that provides out and lse) on the same workload; its FLOPs are counted as
2.5 times the forward's (the five products of the method's backward pass).

Also reported:
  * roofline — against the roof that binds the workload: the MFMA peak for its dtype (TFLOP/s),
    or HBM bandwidth (GB/s of algorithmic bytes) when those bytes take longer at 8 TB/s than the
    FLOPs at the MFMA peak (the window workloads; the TFLOP/s figures stay beside it); the mean
    launch from two HIP events on the launch stream around the K timed launches (the median
    comes from K further launches each between two events); HBM traffic from the committed
    rocprofv3 counter summary when it was taken on the current kernel source;
  * timing — the protocol (see `timed`): W warm-up steps, K steps as a run from an idle GPU sees
    them (`unheated_ms_per_step`), the step repeated for a quarter of a second (the engine clock
    rises over the first tenths of a second under load), then the K timed steps;
  * cold_cache — the median launch after 512 MiB of writes have evicted L2 and the MALL;
  * cpu_baseline — the fp64 CPU oracle timed on this host on a bounded sample of the same
    workload (whole heads), scaled to the same metric.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"f16": 2516.6, "bf16": 2516.6, "e4m3": 5033.2}   # 256 CU x 2.4 GHz x dense MFMA rate
HBM_PEAK_GBS = 8000.0
DEFAULT_WORKLOAD = "causal_b4_h32_n4096_d64_f16"
METRIC = "attention fwd TFLOP/s (4·B·H·Nq·Nk·D, causal halved) and % of MFMA peak"
METRIC_BWD = "attention bwd TFLOP/s (2.5 x the forward FLOPs: five products of the forward's size)"
BWD_FLOP_FACTOR = 2.5
_CSRC = "exact_attention_09_amd/csrc/"
_SHARED = ["fa_f16_common.hpp", "fa_device.hpp", "fa_mask.hpp", "fa_kernels.hpp", "fa_schedule.hpp", "fa355_api.hip"]
# sources whose change makes a committed counter summary stale, per pass
KERNEL_SOURCES = {
    "fwd": [_CSRC + f for f in ["fa_fwd_f16.hip", "fa_fwd_fp8.hip"] + _SHARED],
    "bwd": [_CSRC + f for f in ["fa_fwd_f16.hip", "fa_bwd_f16.hip", "fa_tile.hpp"] + _SHARED],
    "decode": [_CSRC + f for f in ["fa_decode.hip", "fa_tile.hpp"] + _SHARED],
}


def admitted_pairs(Nq, Nk, causal, window):
    """Number of admitted (query, key) pairs, by rows (closed-form interval per row)."""
    off = Nk - Nq
    wl, wr = window
    right = 0 if causal else wr
    total = 0
    for i in range(Nq):
        lo = 0 if wl < 0 else max(0, i + off - wl)
        hi = Nk - 1 if right < 0 else min(Nk - 1, i + off + right)
        total += max(0, hi - lo + 1)
    return total


def metric_flops(w):
    """Metric FLOPs of one forward pass of workload w."""
    if w.window == (-1, -1):
        f = 4.0 * w.B * w.Hq * w.Nq * w.Nk * w.D
        return f / 2 if w.causal else f
    return 4.0 * w.B * w.Hq * w.D * admitted_pairs(w.Nq, w.Nk, w.causal, w.window)


def varlen_flops(w, lengths):
    """Metric FLOPs of one fa_fwd_varlen call: the sum over the sequences (queries = keys)."""
    total = 0.0
    for n in lengths:
        if w.window == (-1, -1):
            f = 4.0 * w.Hq * n * n * w.D
            total += f / 2 if w.causal else f
        else:
            total += 4.0 * w.Hq * w.D * admitted_pairs(n, n, w.causal, w.window)
    return total


def roofline_bound(flops, alg_bytes, peak_tflops):
    """The roof that binds: "hbm" when the algorithmic bytes take longer at the HBM peak than the
    FLOPs at the MFMA peak, else "mfma"."""
    return "hbm" if alg_bytes / (HBM_PEAK_GBS * 1e9) > flops / (peak_tflops * 1e12) else "mfma"


def algorithmic_bytes(w):
    """Bytes the pass must move at least: q, k, v read once, out and lse written once."""
    es = 1 if w.dtype == "e4m3" else 2
    return (w.B * w.Nq * w.Hq * w.D * es + 2 * w.B * w.Nk * w.Hkv * w.D * es + w.B * w.Nq * w.Hq * w.D * 2
            + w.B * w.Hq * w.Nq * 4)


def algorithmic_bytes_bwd(w):
    """Bytes the backward pass must move at least: q, k, v, out, dout, lse read once; dq, dk, dv
    written once; the workspace (row sums dout . out and lse in base 2) written and read once."""
    es = 2
    rows_q = w.B * w.Nq * w.Hq
    return (4 * rows_q * w.D * es + 4 * w.B * w.Nk * w.Hkv * w.D * es + rows_q * 4 + 4 * rows_q * 4)


def kernel_source_hash(pass_="fwd"):
    h = hashlib.sha256()
    for p in KERNEL_SOURCES[pass_]:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def committed_counters(workload, pass_="fwd"):
    """The committed counter summary of the workload (profiles/traffic_<workload>.txt) if it was
    taken on the current kernel source, else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != kernel_source_hash(pass_):
        return None
    return t


def committed_traffic(workload, pass_="fwd"):
    """HBM bytes per launch from the committed counter summary, if taken on this kernel source."""
    t = committed_counters(workload, pass_)
    return t.get("hbm_bytes_per_launch") if t else None


def committed_clock(workload, pass_="fwd"):
    """The engine clock under this workload's kernel, from the same committed counter run: GPU
    busy cycles per XCD (GRBM_GUI_ACTIVE / 8) over the dispatch's duration. The SMU's own clock
    reports are not live on every host, so the clock is taken from the counters."""
    t = committed_counters(workload, pass_)
    mhz = t.get("gfx_clock_MHz") if t else None
    return {"MHz": mhz, "source": "GRBM_GUI_ACTIVE / 8 XCDs / dispatch duration, committed counter run of this "
                                  f"kernel source (profiles/traffic_{workload}.txt)" if mhz else
            "no counter run of this kernel source is committed"}


def blas_threads():
    """(threads, name) of the BLAS the oracle's matrix products run on."""
    try:
        from threadpoolctl import threadpool_info
        blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        threads = max((i.get("num_threads", 1) for i in blas), default=1)
        name = ",".join(sorted({i.get("internal_api", "?") for i in blas})) or "unknown"
        return int(threads), name
    except Exception:  # pragma: no cover
        return 1, "unknown"


def host_cpu_info():
    """(model name, physical cores, logical CPUs this process may run on) of the host, from
    /proc/cpuinfo (physical cores = distinct (physical id, core id) pairs)."""
    model, cores = "unknown", set()
    phys = core = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                key, _, val = line.partition(":")
                key, val = key.strip(), val.strip()
                if key == "model name" and model == "unknown":
                    model = val
                elif key == "physical id":
                    phys = val
                elif key == "core id":
                    core = val
                elif not key and phys is not None and core is not None:
                    cores.add((phys, core))
                    phys = core = None
        if phys is not None and core is not None:
            cores.add((phys, core))
    except OSError:
        pass
    try:
        logical = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        logical = os.cpu_count()
    return model, (len(cores) or None), logical


def host_note():
    model, phys, logical = host_cpu_info()
    return f"host CPU {model}, {phys} physical cores, {logical} logical CPUs available"


def cpu_baseline(w, q, k, v, descale, budget_s, dout=None):
    """Time the fp64 oracle on whole heads of the same inputs until budget_s has passed (the
    gradient oracle when dout is given)."""
    import numpy as np

    from oracle import attention_bwd_fp64, attention_fp64, decode_bf16_bits, decode_e4m3_codes, decode_f16_bits

    def dec(x, s):
        import torch
        x = x.contiguous()
        if x.dtype == torch.float16:
            return decode_f16_bits(x.view(torch.int16).numpy().view(np.uint16))
        if x.dtype == torch.bfloat16:
            return decode_bf16_bits(x.view(torch.int16).numpy().view(np.uint16))
        return decode_e4m3_codes(x.view(torch.uint8).numpy(), s)

    threads, blas_name = blas_threads()
    dq, dk, dv = descale if descale is not None else (1.0, 1.0, 1.0)
    G = w.Hq // w.Hkv
    heads = 0
    t0 = time.perf_counter()
    elapsed = 0.0
    for b in range(w.B):
        for h in range(w.Hq):
            g = h // G
            qh = dec(q[b:b + 1, :, h:h + 1, :], dq)
            kh = dec(k[b:b + 1, :, g:g + 1, :], dk)
            vh = dec(v[b:b + 1, :, g:g + 1, :], dv)
            if dout is None:
                attention_fp64(qh, kh, vh, w.softmax_scale(), w.causal, w.window)
            else:
                attention_bwd_fp64(qh, kh, vh, dec(dout[b:b + 1, :, h:h + 1, :], 1.0), w.softmax_scale(), w.causal,
                                   w.window)
            heads += 1
            elapsed = time.perf_counter() - t0
            if elapsed >= budget_s:
                break
        if elapsed >= budget_s:
            break
    per_head_flops = metric_flops(w) * (1.0 if dout is None else BWD_FLOP_FACTOR) / (w.B * w.Hq)
    model, phys, logical = host_cpu_info()
    return {
        "value": heads * per_head_flops / elapsed / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "host": {"cpu_model": model, "physical_cores": phys, "logical_cpus": logical, "blas": blas_name,
                 "blas_threads": int(threads)},
        "sample": f"{heads} of {w.B * w.Hq} (batch, head) pairs of the same inputs{' (gradients)' if dout is not None else ''}, full fp64 score matrix per "
                  f"head, {elapsed:.1f} s wall; metric FLOPs of those heads / wall time; BLAS={blas_name} "
                  f"threads={threads}, {host_note()}",
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--pass", dest="pass_", choices=("fwd", "bwd"), default="fwd",
                    help="time the forward pass (default, the headline metric) or the backward pass")
    ap.add_argument("--cpu-baseline-seconds", type=float, default=15.0,
                    help="oracle time budget on the host; 0 skips the CPU baseline")
    ap.add_argument("--no-bars", dest="bars", action="store_false",
                    help="with the default workload, skip the other bar configurations (bf16, fp8, long GQA)")
    ap.add_argument("--cold-launches", type=int, default=10,
                    help="launches timed after writing 512 MiB (cold L2/MALL); 0 skips them")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead of attention, run a plain device copy of MIB MiB (counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; multi-GPU runs are not part of this "
                                   "build (the forward pass shards by (batch, head) with no exchange)",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch

    import exact_attention_09_amd as fa
    from exact_attention_09_amd.inputs import (KVCACHE_WORKLOADS, SPARSE_WORKLOADS, VARLEN_WORKLOADS, WORKLOADS,
                                               make_inputs)

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        x = torch.ones(n, dtype=torch.float32, device=dev)
        y = torch.empty_like(x)
        for _ in range(args.warmup + args.steps):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n * 4, "copy_calibration_bytes_written": n * 4,
                          "launches": args.warmup + args.steps}))
        return

    if args.workload in SPARSE_WORKLOADS:
        if args.pass_ == "bwd":
            print(json.dumps({"error": "the block-sparse path is a forward pass"}))
            sys.exit(2)
        return bench_sparse(args, SPARSE_WORKLOADS[args.workload], dev)
    if args.workload in KVCACHE_WORKLOADS:
        if args.pass_ == "bwd":
            print(json.dumps({"error": "the KV-cache path is a forward pass"}))
            sys.exit(2)
        return bench_kvcache(args, KVCACHE_WORKLOADS[args.workload], dev)
    if args.workload in VARLEN_WORKLOADS:
        if args.pass_ == "bwd":
            print(json.dumps({"error": "the backward pass takes dense [B, N, H, D] batches"}))
            sys.exit(2)
        return bench_varlen(args, VARLEN_WORKLOADS[args.workload], dev)
    w = WORKLOADS[args.workload]
    bwd = args.pass_ == "bwd"
    if bwd and w.dtype == "e4m3":
        print(json.dumps({"error": "the backward pass takes fp16 or bf16 inputs"}))
        sys.exit(2)
    rec = bench_dense(args, w, dev, bwd, cold_launches=args.cold_launches, cpu_seconds=args.cpu_baseline_seconds)
    if not bwd and args.workload == DEFAULT_WORKLOAD and args.bars:
        # the other configurations the throughput bars are stated on, measured in the same run
        rec["bars"] = {}
        for name, bar_bwd in BAR_WORKLOADS:
            r = bench_dense(args, WORKLOADS[name], dev, bar_bwd, cold_launches=0, cpu_seconds=0)
            rf = r["roofline"]
            rec["bars"][name + ("_bwd" if bar_bwd else "")] = {
                "dtype": r["dtype"], "ms_per_step": r["ms_per_step"], "TFLOPs": r["value"],
                "pct_of_mfma_peak": r["pct_of_mfma_peak"], "kernel_avg_us": rf["kernel_avg_us"],
                "roofline": {key: rf[key] for key in ("bound", "achieved", "peak", "unit", "frac", "traffic")},
                "clock": r["clock"]}
    print(json.dumps(rec), flush=True)


# Configurations measured beside the default workload, as (workload, backward?): the same shape in
# bf16, the fp8 workload, the long GQA and MQA workloads (causal, and with the (256, 256) window),
# and the backward pass of the default workload (keyed with a "_bwd" suffix).
BAR_WORKLOADS = [("causal_b4_h32_n4096_d64_bf16", False), ("causal_fp8_b2_h32_n4096_d64_e4m3", False),
                 ("gqa_b1_hq32_hkv8_n16384_d128_bf16", False), ("gqa_win256_b1_hq32_hkv8_n16384_d128_bf16", False),
                 ("mqa_b1_hq32_hkv1_n16384_d128_bf16", False), ("mqa_win256_b1_hq32_hkv1_n16384_d128_bf16", False),
                 ("causal_b4_h32_n4096_d64_f16", True)]


def bench_dense(args, w, dev, bwd, cold_launches=0, cpu_seconds=0.0):
    """One fa_fwd (or fa_bwd) workload in the timing protocol; returns its JSON record."""
    import torch

    import exact_attention_09_amd as fa
    from exact_attention_09_amd.inputs import make_inputs

    seed = w.seeds[0]
    q, k, v, descale = make_inputs(w, seed)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    out = torch.empty(w.B, w.Nq, w.Hq, w.D, dtype=torch.float16 if w.dtype == "f16" else torch.bfloat16,
                      device=dev)
    lse = torch.empty(w.B, w.Hq, w.Nq, dtype=torch.float32, device=dev)
    scale = w.softmax_scale()

    def fwd_step():
        st = fa.fwd_raw(qd, kd, vd, out, lse, w.causal, w.window, scale, descale)
        if st != 0:
            raise fa.FaError(st, fa.status_str(st))

    step = fwd_step
    if bwd:
        # upstream gradient: seeded N(0, 1) in the storage type; out and lse from one forward pass
        g = torch.Generator().manual_seed(seed + 1)
        dout = torch.randn(w.B, w.Nq, w.Hq, w.D, generator=g).to(q.dtype)
        dod = dout.to(dev)
        fwd_step()
        dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
        ws = fa.bwd_workspace(qd, kd)

        def step():
            st = fa.bwd_raw(qd, kd, vd, out, dod, lse, dq, dk, dv, ws, w.causal, w.window, scale)
            if st != 0:
                raise fa.FaError(st, fa.status_str(st))

    stream = torch.cuda.current_stream(dev)     # fa_fwd launches on this stream
    ms_per_step, avg_kernel_s, med_kernel_s, tinfo = timed(step, args, stream)

    # Cold-cache variant: 512 MiB written between launches evicts L2 and the MALL.
    cold = None
    if cold_launches > 0:
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        cold_ms = []
        for i in range(cold_launches):
            flush.fill_(i & 0xFF)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            step()
            e1.record(stream)
            e1.synchronize()
            cold_ms.append(e0.elapsed_time(e1))
        del flush
        cold_med = sorted(cold_ms)[len(cold_ms) // 2] / 1e3
        cold = {"launches": cold_launches, "kernel_median_us": round(cold_med * 1e6, 3),
                "TFLOPs": round(metric_flops(w) * (BWD_FLOP_FACTOR if bwd else 1.0) / cold_med / 1e12, 2)}

    flops = metric_flops(w) * (BWD_FLOP_FACTOR if bwd else 1.0)
    value = flops / (ms_per_step / 1e3) / 1e12
    achieved = flops / avg_kernel_s / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    traffic = committed_traffic(("bwd_" if bwd else "") + w.name, "bwd" if bwd else "fwd")
    alg_bytes = algorithmic_bytes_bwd(w) if bwd else algorithmic_bytes(w)

    rec = {
        "metric": METRIC_BWD if bwd else METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "Nq": w.Nq, "Nk": w.Nk, "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D,
                   "causal": w.causal, "window": list(w.window), "softmax_scale": scale, "seed": seed,
                   "metric_flops": flops},
        "pct_of_mfma_peak": round(100.0 * value / peak, 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4), "traffic": traffic,
                     "kernel_avg_us": round(avg_kernel_s * 1e6, 3),
                     "kernel_median_us": round(med_kernel_s * 1e6, 3),
                     "algorithmic_bytes": alg_bytes,
                     "algorithmic_GBps": round(alg_bytes / avg_kernel_s / 1e9, 1)},
    }
    if roofline_bound(flops, alg_bytes, peak) == "hbm":
        gbs = alg_bytes / avg_kernel_s / 1e9
        rec["roofline"].update({"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                "frac": round(gbs / HBM_PEAK_GBS, 4), "achieved_TFLOPs": round(achieved, 2),
                                "frac_of_mfma_peak": round(achieved / peak, 4)})
    rec["timing"] = tinfo
    rec["clock"] = committed_clock(("bwd_" if bwd else "") + w.name, "bwd" if bwd else "fwd")
    if cold is not None:
        rec["cold_cache"] = cold
    if bwd:
        rec["config"]["pass"] = "bwd"
    if cpu_seconds > 0:
        rec["cpu_baseline"] = cpu_baseline(w, q, k, v, descale, cpu_seconds, dout if bwd else None)
    return rec



PREHEAT_S = 0.25   # seconds of the step run before the timed region (engine clock ramp)


def timed(step, args, stream):
    """The timing protocol of every bench line. W warm-up steps; K steps as a run that starts on an
    idle GPU sees them (reported as `unheated_ms_per_step`, not the value); the step repeated for
    PREHEAT_S seconds, because the engine clock rises over the first few tenths of a second under
    load (measured: c3 366-372 us per launch right after 10 warm-ups, 346 after a pre-heat; c5
    160 vs 137); then the K timed steps, back to back between a synchronize on each side (wall
    clock: `ms_per_step`, the value) with two HIP events on the launch stream around them (the mean
    launch); then K more launches, each between two events (the median launch). Returns
    (ms_per_step, mean launch s, median launch s, info)."""
    import torch

    def back_to_back(n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(stream)
        for _ in range(n):
            step()
        e1.record(stream)
        torch.cuda.synchronize()
        return time.perf_counter() - t0, e0.elapsed_time(e1) / 1e3

    for _ in range(args.warmup):
        step()
    _, unheated_s = back_to_back(args.steps)
    pre = 0
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < PREHEAT_S:
        for _ in range(4):
            step()
        pre += 4
        torch.cuda.synchronize()
    wall, events_s = back_to_back(args.steps)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    for i in range(args.steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    ms = sorted(s.elapsed_time(e) for s, e in zip(starts, ends))
    info = {"preheat_s": PREHEAT_S, "preheat_launches": pre,
            "unheated_ms_per_step": round(unheated_s / args.steps * 1e3, 5),
            "order": "warmup, unheated steps, preheat, timed steps, per-launch steps"}
    return wall / args.steps * 1e3, events_s / args.steps, ms[len(ms) // 2] / 1e3, info


def bench_varlen(args, w, dev):
    """fa_fwd_varlen on the packed workload w (queries = keys per sequence)."""
    import torch

    import exact_attention_09_amd as fa
    from exact_attention_09_amd.inputs import make_varlen_inputs

    lengths = w.lengths(0)
    q, k, v, cu_q, cu_k, descale = make_varlen_inputs(lengths, lengths, w.Hq, w.Hkv, w.D, w.dtype, seed=0)
    qd, kd, vd, cqd, ckd = q.to(dev), k.to(dev), v.to(dev), cu_q.to(dev), cu_k.to(dev)
    total = int(cu_q[-1])
    out = torch.empty(total, w.Hq, w.D, dtype=torch.float16 if w.dtype == "f16" else torch.bfloat16, device=dev)
    lse = torch.empty(w.Hq, total, dtype=torch.float32, device=dev)
    scale = w.softmax_scale()

    def step():
        st = fa.fwd_varlen_raw(qd, kd, vd, out, lse, cqd, ckd, max(lengths), w.causal, w.window, scale, descale)
        if st != 0:
            raise fa.FaError(st, fa.status_str(st))

    ms_per_step, avg_s, med_s, tinfo = timed(step, args, torch.cuda.current_stream(dev))
    flops = varlen_flops(w, lengths)
    peak = PEAK_TFLOPS[w.dtype]
    es = 1 if w.dtype == "e4m3" else 2
    alg_bytes = total * w.Hq * w.D * es + 2 * total * w.Hkv * w.D * es + total * w.Hq * w.D * 2 + total * w.Hq * 4
    rec = {
        "metric": METRIC, "value": round(flops / (ms_per_step / 1e3) / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "sequences": w.B, "lengths": lengths, "total_tokens": total, "Hq": w.Hq,
                   "Hkv": w.Hkv, "D": w.D, "causal": w.causal, "window": list(w.window), "softmax_scale": scale,
                   "metric_flops": flops},
        "pct_of_mfma_peak": round(100.0 * flops / (ms_per_step / 1e3) / 1e12 / peak, 2),
        "roofline": {"bound": "mfma", "achieved": round(flops / avg_s / 1e12, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(flops / avg_s / 1e12 / peak, 4), "traffic": committed_traffic(w.name),
                     "kernel_avg_us": round(avg_s * 1e6, 3), "kernel_median_us": round(med_s * 1e6, 3),
                     "algorithmic_bytes": alg_bytes, "algorithmic_GBps": round(alg_bytes / avg_s / 1e9, 1)},
        "timing": tinfo,
    }
    if args.cpu_baseline_seconds > 0:
        rec["cpu_baseline"] = cpu_baseline_varlen(w, lengths, q, k, v, cu_q, descale, args.cpu_baseline_seconds)
    print(json.dumps(rec), flush=True)


def sparse_pairs(w, mask_heads_mask):
    """Admitted (query, key) pairs per head of a block mask [hm, nqb, nkb] under w's causal mask."""
    import numpy as np
    m = mask_heads_mask.numpy() != 0
    N = w.N
    per_head = []
    r = np.arange(N)
    for hm in range(m.shape[0]):
        total = 0
        for qb in range(m.shape[1]):
            rows = r[qb * 128:(qb + 1) * 128]
            for kb in np.nonzero(m[hm, qb])[0]:
                j0, j1 = kb * 64, min(N, kb * 64 + 64)
                hi = np.minimum(rows, j1 - 1) if w.causal else np.full(len(rows), j1 - 1)
                total += int(np.maximum(0, hi - j0 + 1).sum())
        per_head.append(total)
    return per_head


def bench_sparse(args, w, dev):
    """fa_fwd_blocksparse on the sparse workload w, with the dense causal forward timed beside it."""
    import torch

    import exact_attention_09_amd as fa
    from exact_attention_09_amd.inputs import draw_qkv, to_storage

    q, k, v = draw_qkv(w.B, w.N, w.N, w.Hq, w.Hkv, w.D, seed=0)
    q, k, v, _ = to_storage(q, k, v, w.dtype)
    mask = w.mask(0)
    qd, kd, vd, md = q.to(dev), k.to(dev), v.to(dev), mask.to(dev)
    out = torch.empty_like(qd)
    lse = torch.empty(w.B, w.Hq, w.N, dtype=torch.float32, device=dev)
    scale = w.softmax_scale()

    def step():
        st = fa.fwd_blocksparse_raw(qd, kd, vd, out, lse, md, w.causal, (-1, -1), scale)
        if st != 0:
            raise fa.FaError(st, fa.status_str(st))

    def dense_step():
        st = fa.fwd_raw(qd, kd, vd, out, lse, w.causal, (-1, -1), scale)
        if st != 0:
            raise fa.FaError(st, fa.status_str(st))

    stream = torch.cuda.current_stream(dev)
    ms_per_step, avg_s, med_s, tinfo = timed(step, args, stream)
    dense_ms, dense_avg, _, dinfo = timed(dense_step, args, stream)
    pairs = sparse_pairs(w, mask)
    pairs_total = sum(pairs[0 if len(pairs) == 1 else h] for h in range(w.Hq)) * w.B
    flops = 4.0 * w.D * pairs_total
    peak = PEAK_TFLOPS[w.dtype]
    dense_flops = 4.0 * w.B * w.Hq * w.N * w.N * w.D / (2 if w.causal else 1)
    rec = {
        "metric": "block-sparse attention fwd TFLOP/s (4·D per admitted pair) and speedup over the dense causal pass",
        "value": round(flops / (ms_per_step / 1e3) / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "N": w.N, "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D, "causal": w.causal,
                   "mask_heads": w.mask_heads, "band_blocks": w.band, "sink_blocks": w.sinks, "p_random": w.p_random,
                   "block_density": round(float(mask.float().mean()), 5), "admitted_pairs": pairs_total,
                   "softmax_scale": scale, "metric_flops": flops},
        "pct_of_mfma_peak": round(100.0 * flops / (ms_per_step / 1e3) / 1e12 / peak, 2),
        "dense_causal": {"ms_per_step": round(dense_ms, 5), "TFLOPs": round(dense_flops / (dense_ms / 1e3) / 1e12, 2),
                         "speedup_of_sparse": round(dense_ms / ms_per_step, 2), "timing": dinfo},
        "roofline": {"bound": "mfma", "achieved": round(flops / avg_s / 1e12, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(flops / avg_s / 1e12 / peak, 4), "traffic": committed_traffic(w.name),
                     "kernel_avg_us": round(avg_s * 1e6, 3), "kernel_median_us": round(med_s * 1e6, 3)},
        "timing": tinfo,
    }
    if args.cpu_baseline_seconds > 0:
        rec["cpu_baseline"] = cpu_baseline_sparse(w, q, k, v, mask, args.cpu_baseline_seconds)
    print(json.dumps(rec), flush=True)


def cpu_baseline_sparse(w, q, k, v, mask, budget_s):
    """The block-sparse oracle on the last rows of the sequence (whole heads of those rows), growing
    the sample while it stays within budget_s; TFLOP/s on the admitted pairs it processed."""
    import numpy as np
    import torch

    from oracle import admitted, attention_blocksparse_fp64, block_admitted, decode_bf16_bits, decode_f16_bits

    def dec(x):
        x = x.contiguous()
        if x.dtype == torch.float16:
            return decode_f16_bits(x.view(torch.int16).numpy().view(np.uint16))
        return decode_bf16_bits(x.view(torch.int16).numpy().view(np.uint16))

    G = w.Hq // w.Hkv
    R = 128
    done_flops, elapsed, heads = 0.0, 0.0, 0
    t0 = time.perf_counter()
    rows = np.arange(w.N - R, w.N)
    for h in range(w.Hq):
        g = h // G
        bm = mask[0 if mask.shape[0] == 1 else h].numpy()
        # the last R rows as a problem of Nq = R against all N keys (bottom-right alignment keeps the
        # causal mask); their mask rows are the last R / 128 block rows
        attention_blocksparse_fp64(dec(q[:, -R:, h:h + 1]), dec(k[:, :, g:g + 1]), dec(v[:, :, g:g + 1]),
                                   bm[None, -(R // 128):], 128, 64, w.softmax_scale(), w.causal)
        pairs = int((block_admitted(bm, w.N, w.N, 128, 64, rows=rows) & admitted(w.N, w.N, w.causal, rows=rows)).sum())
        done_flops += 4.0 * w.D * pairs * w.B
        heads += 1
        elapsed = time.perf_counter() - t0
        if elapsed >= budget_s:
            break
    threads, blas_name = blas_threads()
    return {"value": done_flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"the last {R} rows of {heads} of {w.Hq} heads (all their keys), fp64, {elapsed:.1f} s wall; "
                      f"admitted-pair FLOPs of those rows / wall time; BLAS={blas_name} threads={threads}, "
                      f"{host_note()}"}


def kvcache_flops(w, lengths):
    """Metric FLOPs of one fa_fwd_kvcache call: 4 * Hq * D per admitted (query, key) pair."""
    pairs = 0
    for n in lengths:
        pairs += admitted_pairs(w.Nq, n, w.causal, (-1, -1)) if n > 0 else 0
    return 4.0 * w.Hq * w.D * pairs


def bench_kvcache(args, w, dev):
    """fa_fwd_kvcache on the cache workload w."""
    import torch

    import exact_attention_09_amd as fa
    from exact_attention_09_amd.inputs import make_kvcache_inputs

    lengths = w.lengths(0)
    q, k, v, seqlens, table = make_kvcache_inputs(w.B, w.Nq, w.Hq, w.Hkv, w.D, w.dtype, lengths, w.page_size, seed=0)
    qd, kd, vd, sd = q.to(dev), k.to(dev), v.to(dev), seqlens.to(dev)
    td = table.to(dev) if table is not None else None
    out = torch.empty_like(qd)
    lse = torch.empty(w.B, w.Hq, w.Nq, dtype=torch.float32, device=dev)
    max_k = max(lengths)
    ws = fa.kvcache_workspace(qd, w.Hkv, max_k)
    scale = w.softmax_scale()

    def step():
        st = fa.fwd_kvcache_raw(qd, kd, vd, out, lse, sd, td, max_k, causal=w.causal, softmax_scale=scale,
                                workspace=ws)
        if st != 0:
            raise fa.FaError(st, fa.status_str(st))

    ms_per_step, avg_s, med_s, tinfo = timed(step, args, torch.cuda.current_stream(dev))
    flops = kvcache_flops(w, lengths)
    es = 2
    kv_bytes = 2 * sum(lengths) * w.Hkv * w.D * es
    alg_bytes = kv_bytes + 2 * w.B * w.Nq * w.Hq * w.D * es + w.B * w.Hq * w.Nq * 4
    value = alg_bytes / (ms_per_step / 1e3) / 1e9
    achieved = alg_bytes / avg_s / 1e9
    rec = {
        "metric": "decode attention against a KV cache: algorithmic HBM GB/s (K/V read once)", "value": round(value, 1),
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "sequences": w.B, "Nq": w.Nq, "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D,
                   "page_size": w.page_size, "causal": w.causal, "total_keys": sum(lengths),
                   "min_len": min(lengths), "max_len": max_k, "softmax_scale": scale, "metric_flops": flops},
        "tflops": round(flops / (ms_per_step / 1e3) / 1e12, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": committed_traffic(w.name, "decode"),
                     "kernel_avg_us": round(avg_s * 1e6, 3), "kernel_median_us": round(med_s * 1e6, 3),
                     "algorithmic_bytes": alg_bytes},
        "timing": tinfo,
    }
    if args.cpu_baseline_seconds > 0:
        rec["cpu_baseline"] = cpu_baseline_kvcache(w, lengths, q, k, v, table, args.cpu_baseline_seconds, alg_bytes)
    print(json.dumps(rec), flush=True)


def cpu_baseline_kvcache(w, lengths, q, k, v, table, budget_s, alg_bytes):
    """The KV-cache oracle on whole sequences until budget_s has passed, in the same GB/s metric."""
    import numpy as np
    import torch

    from oracle import attention_kvcache_fp64, decode_bf16_bits, decode_f16_bits

    def dec(x):
        x = x.contiguous()
        if x.dtype == torch.float16:
            return decode_f16_bits(x.view(torch.int16).numpy().view(np.uint16))
        return decode_bf16_bits(x.view(torch.int16).numpy().view(np.uint16))

    done_bytes, n_seq = 0.0, 0
    t0 = time.perf_counter()
    elapsed = 0.0
    for b, n in enumerate(lengths):
        if table is not None:
            npg = (n + w.page_size - 1) // w.page_size
            pages = table[b, :npg].long()
            kb, vb, tb = dec(k[pages]), dec(v[pages]), np.arange(npg)[None]
        else:
            kb, vb, tb = dec(k[b:b + 1, :n]), dec(v[b:b + 1, :n]), None
        attention_kvcache_fp64(dec(q[b:b + 1]), kb, vb, [n], tb, w.page_size, w.softmax_scale(), w.causal)
        done_bytes += alg_bytes * n / sum(lengths)
        n_seq += 1
        elapsed = time.perf_counter() - t0
        if elapsed >= budget_s:
            break
    threads, blas_name = blas_threads()
    return {"value": done_bytes / elapsed / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{n_seq} of {len(lengths)} sequences of the same inputs (all heads), fp64, {elapsed:.1f} s wall; "
                      f"their share of the algorithmic bytes / wall time; BLAS={blas_name} threads={threads}, "
                      f"{host_note()}"}


def cpu_baseline_varlen(w, lengths, q, k, v, cu_q, descale, budget_s):
    """The varlen oracle on whole (sequence, head) pairs until budget_s has passed."""
    import numpy as np
    import torch

    from oracle import attention_varlen_fp64, decode_bf16_bits, decode_f16_bits

    def dec(x):
        x = x.contiguous()
        if x.dtype == torch.float16:
            return decode_f16_bits(x.view(torch.int16).numpy().view(np.uint16))
        return decode_bf16_bits(x.view(torch.int16).numpy().view(np.uint16))

    G = w.Hq // w.Hkv
    done_flops, n_pairs = 0.0, 0
    t0 = time.perf_counter()
    elapsed = 0.0
    for b, n in enumerate(lengths):
        s = int(cu_q[b])
        for h in range(w.Hq):
            g = h // G
            attention_varlen_fp64(dec(q[s:s + n, h:h + 1]), dec(k[s:s + n, g:g + 1]), dec(v[s:s + n, g:g + 1]),
                                  [0, n], [0, n], w.softmax_scale(), w.causal, w.window)
            done_flops += varlen_flops(w, [n]) / w.Hq
            n_pairs += 1
            elapsed = time.perf_counter() - t0
            if elapsed >= budget_s:
                break
        if elapsed >= budget_s:
            break
    threads, blas_name = blas_threads()
    return {"value": done_flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{n_pairs} of {len(lengths) * w.Hq} (sequence, head) pairs of the same inputs, full fp64 "
                      f"score matrix per pair, {elapsed:.1f} s wall; metric FLOPs of those pairs / wall time; "
                      f"BLAS={blas_name} threads={threads}, {host_note()}"}


if __name__ == "__main__":
    main()
