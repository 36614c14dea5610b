#!/usr/bin/env python3
"""Benchmark of the fused W4 base + sparse 4-bit residual linear on one MI355X.

One step = the decode hot path on the Llama-7B-shaped MLP up-projection
(W 11008x4096, group 128, residual density 0.5 %): one fused linear at each
of M = 1, 4 and 16 tokens. The packed layer is built on the GPU by mq_pack
before the timed region (packing is timed separately), inputs are resident
in HBM, and every launch reads a different packed copy so the 256 MB
Infinity Cache cannot serve the weights.

Timing: the warm-up steps and the timed steps are each captured once as a
HIP graph and replayed between device synchronisations, so the figures are
GPU time and not the Python launch rate (a decode launch is shorter than one
ctypes call through torch).

Printed: one JSON line with the decode GB/s (algorithmic bytes of the
canonical packed format + X + Y over kernel time), the roofline of the
dominant decode kernel against the 8 TB/s HBM peak (with the HBM bytes that
rocprofv3 counted for it, when those counters were taken on the current
kernel sources), the residual's cost t(rho) / t(rho = 0), the unfused
two-kernel comparison (dense kernel on a residual-free copy, then the
separate residual kernel), the prefill TFLOP/s on the 70B-shaped MLP
(28672x8192, M = 512 and 2048) against the 2.5 PFLOP/s dense fp16 MFMA
peak, and the CPU oracle timed on a bounded sample as a baseline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
FP16_PEAK_TFLOPS = 2516.6      # MI355X dense fp16 MFMA: 256 CU x 2.4 GHz x 4096 FLOP/clk
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense fp8 MFMA (5.0 PFLOP/s)
MALL_BYTES = 256 << 20
METRIC = "fused W4+sparse-residual linear: GB/s (decode) & TFLOP/s (prefill), % roofline"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--skip-prefill", action="store_true")
    ap.add_argument("--skip-cpu", action="store_true")
    ap.add_argument("--skip-extra", action="store_true",
                    help="skip the transformer-block, residual-sweep, block-residual, migration and W4A4 legs")
    ap.add_argument("--only", choices=["decode", "prefill", "copy", "stream", "mid", "tblock", "sweep", "blocks", "migration", "w4a4"],
                    default=None,
                    help="run one leg only (profiling runs); 'copy' runs the plain device copy that "
                         "calibrates the HBM byte counters; 'stream' times a plain streaming read of a "
                         "decode layer's size (the HBM read ceiling of the decode kernels)")
    ap.add_argument("--no-warm", action="store_true",
                    help="skip the warm single-copy decode leg (keeps per-kernel profiles all-cold)")
    return ap.parse_args()


def decode_bytes(p, M):
    """Algorithmic bytes of one decode launch: canonical packed layer + X + Y."""
    return p.canonical_bytes() + 2 * M * p.K + 2 * M * p.N


def attainable_tflops(flops, nbytes):
    """Roofline ceiling of a launch: min(dense fp16 MFMA peak, arithmetic
    intensity x HBM peak), in TFLOP/s (thin GEMMs at a few dozen tokens sit
    below the ridge, about 315 FLOP per byte)."""
    return min(FP16_PEAK_TFLOPS, flops / nbytes * HBM_PEAK_GBS / 1e3)


def time_events(fn, n):
    import torch
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(n):
        fn(i)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b)   # ms


def capture(torch, fn, n):
    """A HIP graph holding fn(0) .. fn(n-1) (fn launches on the current stream)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):      # first calls outside capture (one-time kernel attributes)
        for i in range(2):
            fn(i)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            fn(i)
    torch.cuda.synchronize()
    return g


def time_graphs(torch, fn, warmup, steps):
    """Replay a graph of `warmup` calls untimed, then time one replay of a
    graph of exactly `steps` calls between device synchronisations (ms)."""
    if warmup > 0:
        capture(torch, fn, warmup).replay()
    g = capture(torch, fn, steps)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b)


def replay_spread(torch, fn, warmup, steps, reps=9):
    """Per-launch time (ms) from `reps` timed replays of one graph of `steps`
    calls: (median, p10, p90) over the replays."""
    import numpy as np
    if warmup > 0:
        capture(torch, fn, warmup).replay()
    g = capture(torch, fn, steps)
    out = []
    for _ in range(reps):
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        out.append(a.elapsed_time(b) / steps)
    return float(np.median(out)), float(np.percentile(out, 10)), float(np.percentile(out, 90))


DECODE_SOURCES = ("gemv.hip", "gemv_group.h", "kernel_common.h", "mq_internal.h")
MID_SOURCES = ("gemm_mid.hip", "kernel_common.h", "mq_internal.h")
PREFILL_SOURCES = ("gemm.hip", "gemm_rw.hip", "kernel_common.h", "mq_internal.h")
STREAM_SOURCES = ("probe.hip",)


def source_digest(files=DECODE_SOURCES):
    """sha256 of kernel sources: a profile summary is only valid for these."""
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "bit_gemm_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def counted_traffic(kernel_tag):
    """HBM bytes per launch that rocprofv3 counted for `kernel_tag`, from the
    committed counter summary, or None when the summary is missing or was
    taken on other kernel sources."""
    v = profile_values("decode_hbm_counters.txt", DECODE_SOURCES).get(f"hbm_bytes_per_launch[{kernel_tag}]")
    return float(v) if v else None


def sha256_of(a) -> str:
    """SHA-256 of a generated host array's bytes (C order), so a run names
    the exact inputs it timed."""
    import numpy as np
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def host_cpu() -> dict:
    """The host CPU model and the cores this process may run on."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "affinity_cores": len(os.sched_getaffinity(0))}


def profile_values(name, sources):
    """key: value lines of a committed rocprofv3 summary under profiles/, or
    {} when the file is missing or its `source_sha256` differs from the
    current sources of the kernel it describes (then its figures are stale)."""
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return {}
    vals = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("source_sha256") != source_digest(sources):
        return {}
    return vals


class ClockSampler:
    """Samples the shader clock the driver reports (the active DPM level of
    pp_dpm_sclk) every few ms while a timed region runs; None where the
    file is not readable."""

    def __init__(self, period_s=0.002):
        import glob
        import threading
        self.paths = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.period, self.samples = period_s, []
        self._stop = threading.Event()
        self._thr = threading.Thread(target=self._run, daemon=True)

    def _read(self):
        for p in self.paths:
            try:
                with open(p) as fh:
                    for line in fh:
                        if line.rstrip().endswith("*"):
                            return float(line.split(":")[1].strip().rstrip("*").strip().lower().rstrip("mhz"))
            except (OSError, ValueError, IndexError):
                continue
        return None

    def _run(self):
        while not self._stop.is_set():
            v = self._read()
            if v is not None:
                self.samples.append(v)
            time.sleep(self.period)

    def __enter__(self):
        if self.paths:
            self._thr.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self.paths:
            self._thr.join()

    def summary(self):
        import numpy as np
        if not self.samples:
            return None
        a = np.array(self.samples)
        return {"samples": int(a.size), "median_MHz": float(np.median(a)), "max_MHz": float(a.max()),
                "min_MHz": float(a.min())}


def bench_decode(args, mq, synth, torch):
    wl = synth.WORKLOADS["decode-11008x4096"]
    layer = wl.layers[0]
    W_host = layer.W()
    shas = {"W": sha256_of(W_host)}
    W = torch.from_numpy(W_host).cuda()
    del W_host
    # packing, timed on its own (GPU events around mq_pack, which ends with a sync)
    t0 = time.perf_counter()
    first = mq.mq_pack(W, layer.group, layer.rho)
    pack_wall_ms = (time.perf_counter() - t0) * 1e3
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    again = mq.mq_pack(W, layer.group, layer.rho)
    ev1.record()
    torch.cuda.synchronize()
    pack_ms = ev0.elapsed_time(ev1)
    copies = [first, again]
    ncopy = max(2, math.ceil(2 * MALL_BYTES / first.device_bytes))
    while len(copies) < ncopy:
        copies.append(mq.mq_pack(W, layer.group, layer.rho))
    del W
    Ms = list(wl.batch)
    X_host = {M: layer.X(M) for M in Ms}
    shas.update({f"X[M={M}]": sha256_of(x) for M, x in X_host.items()})
    Xs = {M: torch.from_numpy(x).cuda() for M, x in X_host.items()}
    Ys = {M: torch.empty((M, layer.N), dtype=torch.float16, device="cuda") for M in Ms}

    def step(i):
        # every launch of the step reads its own packed copy (the copies are
        # dealt in launch order), so no launch finds the weights that the
        # launch before it pulled into the Infinity Cache
        for j, M in enumerate(Ms):
            mq.mq_linear_with(Xs[M], copies[(len(Ms) * i + j) % ncopy], mq.KERNEL_GEMV, Ys[M])

    ms = time_graphs(torch, step, args.warmup, args.steps)
    bytes_step = sum(decode_bytes(first, M) for M in Ms)
    per_m = {}
    for M in Ms:   # each M runs its own kernel: launch duration of each (median of 9 replays)
        def one(i, M=M):
            mq.mq_linear_with(Xs[M], copies[i % ncopy], mq.KERNEL_GEMV, Ys[M])
        mms, p10, p90 = replay_spread(torch, one, args.warmup, args.steps)
        per_m[str(M)] = {"us": round(mms * 1e3, 3), "p10_us": round(p10 * 1e3, 3), "p90_us": round(p90 * 1e3, 3),
                         "GBps": round(decode_bytes(first, M) / mms / 1e6, 1), "bytes": decode_bytes(first, M)}
    # the same layer packed without residual (rho = 0), rotated the same way:
    # t(rho) / t(0) is what the residual costs the fused kernel
    Wd = torch.from_numpy(layer.W()).cuda()
    plain = [mq.mq_pack(Wd, layer.group, 0.0)]
    nplain = max(2, math.ceil(2 * MALL_BYTES / plain[0].device_bytes))
    while len(plain) < nplain:
        plain.append(mq.mq_pack(Wd, layer.group, 0.0))
    del Wd
    overhead, unfused = {}, {}
    for M in Ms:
        def one0(i, M=M):
            mq.mq_linear_with(Xs[M], plain[i % nplain], mq.KERNEL_GEMV, Ys[M])
        m0 = replay_spread(torch, one0, args.warmup, args.steps)[0]
        overhead[str(M)] = round(per_m[str(M)]["us"] / (m0 * 1e3), 3)

        # unfused: the dense kernel on the residual-free copy, then the
        # separate residual kernel reading X again and merging into Y
        def two(i, M=M):
            mq.mq_linear_with(Xs[M], plain[i % nplain], mq.KERNEL_GEMV, Ys[M])
            mq.mq_residual_add(Xs[M], copies[i % ncopy], Ys[M])

        def res(i, M=M):
            mq.mq_residual_add(Xs[M], copies[i % ncopy], Ys[M])
        m2 = replay_spread(torch, two, args.warmup, args.steps)[0]
        mr = replay_spread(torch, res, args.warmup, args.steps)[0]
        unfused[str(M)] = {"us": round(m2 * 1e3, 3), "residual_kernel_us": round(mr * 1e3, 3),
                           "over_fused": round(m2 * 1e3 / per_m[str(M)]["us"], 3)}
    handle = {"plain_w4_bytes": plain[0].device_bytes, "elementwise_bytes": first.device_bytes,
              "over_plain_w4": round(first.device_bytes / plain[0].device_bytes, 4),
              "bits_per_weight": round(8.0 * first.device_bytes / (layer.N * layer.K), 4),
              "plain_w4_bits_per_weight": round(8.0 * plain[0].device_bytes / (layer.N * layer.K), 4)}
    for p in plain:
        p.free()
    # warm, single copy (weights can stay in the Infinity Cache): context only
    def warm(i):
        mq.mq_linear_with(Xs[1], first, mq.KERNEL_GEMV, Ys[1])
    warm_ms = float("nan") if args.no_warm else time_graphs(torch, warm, args.warmup, args.steps) / args.steps
    return {
        "layer": layer, "first": first, "ms_per_step": ms / args.steps, "bytes_step": bytes_step,
        "launches_per_step": len(Ms), "per_m": per_m, "pack_ms": pack_ms, "pack_wall_ms": pack_wall_ms,
        "copies": ncopy, "warm_us_m1": warm_ms * 1e3, "nnz": first.nnz, "overhead": overhead,
        "unfused": unfused, "handle": handle, "inputs_sha256": shas,
    }


def bench_prefill(args, mq, synth, torch):
    wl = synth.WORKLOADS["prefill-28672x8192"]
    layer = wl.layers[0]
    W_host = layer.W()
    shas = {"W": sha256_of(W_host)}
    W = torch.from_numpy(W_host).cuda()
    del W_host
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    p = mq.mq_pack(W, layer.group, layer.rho)
    ev1.record()
    torch.cuda.synchronize()
    pack_ms = ev0.elapsed_time(ev1)
    del W
    out = {"workload": wl.name, "N": layer.N, "K": layer.K, "rho": layer.rho, "nnz": p.nnz,
           "pack_ms": round(pack_ms, 3), "M": {}}
    out["inputs_sha256"] = shas
    for M in wl.batch:
        X_host = layer.X(M)
        shas[f"X[M={M}]"] = sha256_of(X_host)
        X = torch.from_numpy(X_host).cuda()
        Y = torch.empty((M, layer.N), dtype=torch.float16, device="cuda")
        n = max(3, min(args.steps, 50))

        def run(i):
            mq.mq_linear_with(X, p, mq.KERNEL_GEMM, Y)
        time_events(run, max(2, args.warmup // 4))
        with ClockSampler() as clk:
            ms = time_events(run, n) / n
        tflops = 2.0 * M * layer.N * layer.K / (ms * 1e-3) / 1e12
        out["M"][str(M)] = {"us": round(ms * 1e3, 2), "TFLOPs": round(tflops, 1),
                            "frac_mfma_peak": round(tflops / FP16_PEAK_TFLOPS, 4), "sclk": clk.summary(),
                            # the sparse residual's own multiply-adds, not in 2 M N K: the kernel
                            # folds the residual into the weight tile, so it issues no MFMA work for them
                            "residual_GFLOP": round(2.0 * M * p.nnz / 1e9, 4)}
    p.free()
    # roofline of the GEMM at the largest M: achieved TFLOP/s against the
    # dense fp16 MFMA peak, with the matrix-core busy fraction and the clock
    # that the committed rocprofv3 counter summary measured for this kernel
    mtop = str(max(wl.batch))
    cnt = profile_values("prefill_mfma_counters.txt", PREFILL_SOURCES)
    out["roofline"] = {"bound": "mfma", "achieved": out["M"][mtop]["TFLOPs"], "peak": FP16_PEAK_TFLOPS,
                       "unit": "TFLOP/s", "frac": out["M"][mtop]["frac_mfma_peak"], "M": int(mtop),
                       "flops_per_launch": 2 * int(mtop) * layer.N * layer.K,
                       "profile_mfma_busy": float(cnt[f"mfma_busy[M={mtop}]"]) if f"mfma_busy[M={mtop}]" in cnt else None,
                       "profile_clock_GHz": float(cnt[f"clock_GHz[M={mtop}]"]) if f"clock_GHz[M={mtop}]" in cnt else None,
                       "profile_kernel_avg_us": float(cnt[f"kernel_avg_us[M={mtop}]"]) if f"kernel_avg_us[M={mtop}]" in cnt else None,
                       "profile_mfma_busy_rho0": float(cnt[f"mfma_busy_rw[M={mtop}]"]) if f"mfma_busy_rw[M={mtop}]" in cnt else None}
    # the same layer without residual (rho = 0; the register-weight kernel):
    # its time and TFLOP/s, and t(rho) / t(0)
    W = torch.from_numpy(layer.W()).cuda()
    p0 = mq.mq_pack(W, layer.group, 0.0)
    del W
    out["residual_overhead_t_rho_over_t0"] = {}
    out["plain_w4"] = {}
    for M in wl.batch:
        X = torch.from_numpy(layer.X(M)).cuda()
        Y = torch.empty((M, layer.N), dtype=torch.float16, device="cuda")

        def run0(i):
            mq.mq_linear_with(X, p0, mq.KERNEL_GEMM, Y)
        time_events(run0, 3)
        n = max(3, min(args.steps, 50))
        ms0 = time_events(run0, n) / n
        out["residual_overhead_t_rho_over_t0"][str(M)] = round(out["M"][str(M)]["us"] / (ms0 * 1e3), 3)
        out["plain_w4"][str(M)] = {"us": round(ms0 * 1e3, 2),
                                   "TFLOPs": round(2.0 * M * layer.N * layer.K / (ms0 * 1e-3) / 1e12, 1)}
    p0.free()
    # Context only: a dense fp16 GEMM of the same shape through torch.matmul
    # (the vendor BLAS), random weights. It shows what the matrix cores give a
    # plain fp16 product of this shape on this chip; it is not part of the path.
    dense = {}
    Wd = torch.randn(layer.N, layer.K, dtype=torch.float16, device="cuda") * 0.02
    for M in wl.batch:
        Xd = torch.randn(M, layer.K, dtype=torch.float16, device="cuda")
        Yd = torch.empty((M, layer.N), dtype=torch.float16, device="cuda")

        def mm(i):
            torch.matmul(Xd, Wd.t(), out=Yd)
        time_events(mm, 3)
        n = max(3, min(args.steps, 20))
        ms = time_events(mm, n) / n
        dense[str(M)] = round(2.0 * M * layer.N * layer.K / (ms * 1e-3) / 1e12, 1)
    del Wd
    out["dense_fp16_matmul_TFLOPs"] = dense
    return out


def bench_block(args, mq, synth, torch):
    """The seven linears of one 4096-hidden block at M = 16, back to back on
    one stream (one step = 7 launches), rotated over enough packed copies
    that the Infinity Cache cannot hold them; then the same step with the
    layers of K = 4096 in one mq_linear_group launch, and with the layers
    that read one input joined by mq_concat (with and without the group)."""
    wl = synth.WORKLOADS["block-4096h"]
    M = wl.batch[0]
    first = []
    for layer in wl.layers:
        W = torch.from_numpy(layer.W()).cuda()
        first.append(mq.mq_pack(W, layer.group, layer.rho))
        del W
    ncopy = max(2, math.ceil(2 * MALL_BYTES / sum(p.device_bytes for p in first)))
    copies = [first]
    for _ in range(ncopy - 1):
        c = []
        for layer in wl.layers:
            W = torch.from_numpy(layer.W()).cuda()
            c.append(mq.mq_pack(W, layer.group, layer.rho))
            del W
        copies.append(c)
    Xs = [torch.from_numpy(layer.X(M)).cuda() for layer in wl.layers]
    Ys = [torch.empty((M, layer.N), dtype=torch.float16, device="cuda") for layer in wl.layers]

    def step(i):
        c = copies[i % ncopy]
        for x, p, y in zip(Xs, c, Ys):
            mq.mq_linear(x, p, y)
    med, p10, p90 = replay_spread(torch, step, max(2, args.warmup // 4), max(10, args.steps // 4))
    nbytes = sum(p.canonical_bytes() + 2 * M * p.K + 2 * M * p.N for p in first)
    # The same packed layers with the ones that read the same input joined
    # by mq_concat (q, k, v; and gate, up, or not): fewer launches per step,
    # each group reading its input once. Every layer keeps its own packing.
    names = [layer.name for layer in wl.layers]
    # The six layers of K = 4096, each with its own input and handle, in one
    # mq_linear_group launch; the down projection (K = 11008) on its own
    k4 = [i for i, layer in enumerate(wl.layers) if layer.K == 4096]
    kr = [i for i in range(len(wl.layers)) if i not in k4]

    def step_group(i):
        c = copies[i % ncopy]
        mq.mq_linear_group([Xs[j] for j in k4], [c[j] for j in k4], [Ys[j] for j in k4])
        for j in kr:
            mq.mq_linear(Xs[j], c[j], Ys[j])
    gmed, gp10, gp90 = replay_spread(torch, step_group, max(2, args.warmup // 4), max(10, args.steps // 4))
    grouped = {" ".join(names[j] for j in k4) + " grouped, down": {
        "launches_per_step": 1 + len(kr), "us": round(gmed * 1e3, 2), "p10_us": round(gp10 * 1e3, 2),
        "p90_us": round(gp90 * 1e3, 2), "GBps": round(nbytes / (gmed * 1e-3) / 1e9, 1),
        "frac_hbm": round(nbytes / (gmed * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "bytes": nbytes,
        "speedup_vs_separate": round(med / gmed, 3)}}
    # the same two steps with one token per linear (batch-1 decode)
    X1 = [torch.from_numpy(layer.X(1)).cuda() for layer in wl.layers]
    Y1 = [torch.empty((1, layer.N), dtype=torch.float16, device="cuda") for layer in wl.layers]

    def step_m1(i):
        c = copies[i % ncopy]
        for x, p, y in zip(X1, c, Y1):
            mq.mq_linear(x, p, y)

    def step_m1_group(i):
        c = copies[i % ncopy]
        mq.mq_linear_group([X1[j] for j in k4], [c[j] for j in k4], [Y1[j] for j in k4])
        for j in kr:
            mq.mq_linear(X1[j], c[j], Y1[j])
    # (calls, not launches: at one token a layer with a row block of more
    # than 16 residual chunks runs on its own inside mq_linear_group)
    m1 = {}
    for tag, fn, calls in (("7 launches", step_m1, len(wl.layers)),
                           (" ".join(names[j] for j in k4) + " grouped, down", step_m1_group, 1 + len(kr))):
        t1 = replay_spread(torch, fn, max(2, args.warmup // 4), max(10, args.steps // 4))
        m1[tag] = {"calls_per_step": calls, "us": round(t1[0] * 1e3, 2), "p10_us": round(t1[1] * 1e3, 2),
                   "p90_us": round(t1[2] * 1e3, 2)}
    joined = {}
    for groups in ([["q", "k", "v"], ["o"], ["gate", "up"], ["down"]],
                   [["q", "k", "v"], ["o"], ["gate"], ["up"], ["down"]]):
        fused = []
        for c in copies:
            fused.append([mq.mq_concat([c[names.index(n)] for n in g]) if len(g) > 1 else None for g in groups])
        Xg = [Xs[names.index(g[0])] for g in groups]
        Yg = [torch.empty((M, sum(wl.layers[names.index(n)].N for n in g)), dtype=torch.float16, device="cuda")
              for g in groups]

        def step_fused(i, groups=groups, fused=fused, Xg=Xg, Yg=Yg):
            c, fc = copies[i % ncopy], fused[i % ncopy]
            for gi, g in enumerate(groups):
                mq.mq_linear(Xg[gi], fc[gi] if fc[gi] is not None else c[names.index(g[0])], Yg[gi])
        fmed, fp10, fp90 = replay_spread(torch, step_fused, max(2, args.warmup // 4), max(10, args.steps // 4))
        fbytes = sum(p.canonical_bytes() + 2 * M * p.N for p in first) + sum(
            2 * M * wl.layers[names.index(g[0])].K for g in groups)
        if len(groups) == 4:
            # the joined K = 4096 layers in one mq_linear_group launch, the
            # down projection on its own
            gk = [gi for gi, g in enumerate(groups) if wl.layers[names.index(g[0])].K == 4096]
            go = [gi for gi in range(len(groups)) if gi not in gk]

            def step_fg(i, groups=groups, fused=fused, Xg=Xg, Yg=Yg):
                c, fc = copies[i % ncopy], fused[i % ncopy]
                hs = [fc[gi] if fc[gi] is not None else c[names.index(g[0])] for gi, g in enumerate(groups)]
                mq.mq_linear_group([Xg[gi] for gi in gk], [hs[gi] for gi in gk], [Yg[gi] for gi in gk])
                for gi in go:
                    mq.mq_linear(Xg[gi], hs[gi], Yg[gi])
            gmed, gp10, gp90 = replay_spread(torch, step_fg, max(2, args.warmup // 4), max(10, args.steps // 4))
            grouped[" ".join("+".join(groups[gi]) for gi in gk) + " grouped, down"] = {
                "launches_per_step": 1 + len(go), "us": round(gmed * 1e3, 2), "p10_us": round(gp10 * 1e3, 2),
                "p90_us": round(gp90 * 1e3, 2), "GBps": round(fbytes / (gmed * 1e-3) / 1e9, 1),
                "frac_hbm": round(fbytes / (gmed * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "bytes": fbytes,
                "speedup_vs_separate": round(med / gmed, 3)}
        for fc in fused:
            for p in fc:
                if p is not None:
                    p.free()
        joined[" ".join("+".join(g) for g in groups)] = {
            "launches_per_step": len(groups), "us": round(fmed * 1e3, 2), "p10_us": round(fp10 * 1e3, 2),
            "p90_us": round(fp90 * 1e3, 2), "GBps": round(fbytes / (fmed * 1e-3) / 1e9, 1),
            "frac_hbm": round(fbytes / (fmed * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "bytes": fbytes,
            "speedup_vs_separate": round(med / fmed, 3)}
    for c in copies:
        for p in c:
            p.free()
    return {"workload": wl.name, "M": M, "launches_per_step": len(wl.layers), "packed_copies": ncopy,
            "us": round(med * 1e3, 2), "p10_us": round(p10 * 1e3, 2), "p90_us": round(p90 * 1e3, 2),
            "GBps": round(nbytes / (med * 1e-3) / 1e9, 1), "frac_hbm": round(nbytes / (med * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "bytes": nbytes, "shared_input_joined": joined, "grouped_launch": grouped, "batch_1": m1}


def bench_sweep(args, mq, synth, torch):
    """The 14336x4096 residual sweep: for each outlier placement, the layer
    packed at rho = 0 and at each density; mq_pack timed on its own (GPU
    events) and the linear at M = 1, 64 and 512 (rotated copies, graph
    replay); t(rho) / t(0) per M."""
    out = {}
    for mode, _ in synth.SWEEP_MODES:
        layer0 = synth.sweep_layer(mode, 0.0)
        W = torch.from_numpy(layer0.W()).cuda()
        Xs = {M: torch.from_numpy(layer0.X(M)).cuda() for M in synth.SWEEP_BATCH}
        Ys = {M: torch.empty((M, layer0.N), dtype=torch.float16, device="cuda") for M in synth.SWEEP_BATCH}
        per = {}
        for rho in (0.0,) + tuple(synth.SWEEP_RHOS):
            ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ev0.record()
            p = mq.mq_pack(W, layer0.group, rho)
            ev1.record()
            torch.cuda.synchronize()
            entry = {"nnz": p.nnz, "pack_ms": round(ev0.elapsed_time(ev1), 3), "us": {}}
            ncopy = max(2, math.ceil(2 * MALL_BYTES / p.device_bytes))
            copies = [p] + [mq.mq_pack(W, layer0.group, rho) for _ in range(ncopy - 1)]
            for M in synth.SWEEP_BATCH:
                # graph replays over the rotated copies (cold weights); fewer
                # launches per graph at M = 512, where one takes ~0.1 ms
                def one(i, M=M):
                    mq.mq_linear(Xs[M], copies[i % ncopy], Ys[M])
                steps = max(20, args.steps // 4) if M <= 64 else 20
                us = replay_spread(torch, one, max(2, args.warmup // 4), steps, reps=5)[0] * 1e3
                entry["us"][str(M)] = round(us, 2)
                flops = 2.0 * M * layer0.N * layer0.K
                att = attainable_tflops(flops, p.canonical_bytes() + 2 * M * layer0.K + 2 * M * layer0.N)
                entry.setdefault("frac_attainable", {})[str(M)] = round(flops / (us * 1e-6) / 1e12 / att, 4)
            for c in copies:
                c.free()
            per[str(rho)] = entry
        base = per["0.0"]["us"]
        for rho, entry in per.items():
            entry["t_over_t0"] = {M: round(v / base[M], 3) for M, v in entry["us"].items()}
        out[mode] = per
        del W
    return {"workload": "sweep-14336x4096", "N": 14336, "K": 4096, "group": 128, "by_placement": out}


def bench_mid(args, mq, synth, torch):
    """Mid-size batches on the 14336x4096 sweep layer (columns placement):
    16, 32, 48 and 64 tokens through mq_linear (the mid-size kernel), at
    rho = 0 and 0.005, rotated copies, graph replay. Bytes: the packed layer
    as stored plus X and Y; FLOPs: 2 M N K; each against min(MFMA peak,
    intensity x HBM peak)."""
    layer = synth.sweep_layer("columns", 0.0)
    W = torch.from_numpy(layer.W()).cuda()
    Ms = (16, 32, 48, 64)
    Xs = {M: torch.from_numpy(layer.X(M)).cuda() for M in Ms}
    Ys = {M: torch.empty((M, layer.N), dtype=torch.float16, device="cuda") for M in Ms}
    out = {}
    for rho in (0.0, 0.005):
        p = mq.mq_pack(W, layer.group, rho)
        ncopy = max(2, math.ceil(2 * MALL_BYTES / p.device_bytes))
        copies = [p] + [mq.mq_pack(W, layer.group, rho) for _ in range(ncopy - 1)]
        per = {}
        for M in Ms:
            def one(i, M=M):
                mq.mq_linear(Xs[M], copies[i % ncopy], Ys[M])
            med, p10, p90 = replay_spread(torch, one, max(2, args.warmup // 4), max(20, args.steps // 2), reps=5)
            nbytes = p.canonical_bytes() + 2 * M * layer.K + 2 * M * layer.N
            flops = 2.0 * M * layer.N * layer.K
            tflops = flops / (med * 1e-3) / 1e12
            att = attainable_tflops(flops, nbytes)
            per[str(M)] = {"us": round(med * 1e3, 2), "p10_us": round(p10 * 1e3, 2), "p90_us": round(p90 * 1e3, 2),
                           "GBps": round(nbytes / (med * 1e-3) / 1e9, 1), "TFLOPs": round(tflops, 1),
                           "attainable_TFLOPs": round(att, 1), "frac_attainable": round(tflops / att, 4)}
        for c in copies:
            c.free()
        out[str(rho)] = {"nnz": p.nnz, "per_M": per}
    del W
    return {"workload": "sweep-14336x4096 (columns)", "N": layer.N, "K": layer.K, "group": layer.group,
            "kernel": "k_gemm_mid", "by_rho": out}


def bench_blocks(args, mq, synth, torch):
    """Block-wise residual (Hessian-guided top-K of 16x128 blocks) on the
    11008x4096 decode layer: for each block fraction, mq_pack_blocks time, the
    share of the output distortion of the plain W4 base it recovers on
    held-out activations (||Y - X W^T||^2 against an fp32 torch product, over
    256 tokens that share the calibration set's 4 hot channels), and the
    decode time at M = 1 and 16 (rotated copies, graph replay). Beside each,
    the element-wise residual with the same canonical residual bytes."""
    layer = synth.WORKLOADS["decode-11008x4096"].layers[0]
    N, K = layer.N, layer.K
    W = torch.from_numpy(layer.W()).cuda()
    Xcal = torch.from_numpy(layer.calibration(256, 4)).cuda()
    Xev = torch.from_numpy(layer.calibration(256, 4, held_out=True)).cuda()
    h = (Xcal.float() ** 2).sum(0)                       # diagonal Hessian estimate of the input channels
    Yref = Xev.float() @ W.float().t()
    Xs = {M: torch.from_numpy(layer.X(M)).cuda() for M in (1, 16)}

    def distortion(p):
        Y = mq.mq_linear(Xev, p).float()
        return float(((Y - Yref) ** 2).sum())

    def decode_us(make):
        p0 = make()
        ncopy = max(2, math.ceil(2 * MALL_BYTES / p0.device_bytes))
        copies = [p0] + [make() for _ in range(ncopy - 1)]
        out = {}
        for M, X in Xs.items():
            Y = torch.empty((M, N), dtype=torch.float16, device="cuda")

            def one(i, X=X, Y=Y):
                mq.mq_linear(X, copies[i % ncopy], Y)
            out[str(M)] = round(replay_spread(torch, one, 4, 40, reps=5)[0] * 1e3, 2)
        for c in copies:
            c.free()
        return out

    base = mq.mq_pack(W, layer.group, 0.0)
    D0 = distortion(base)
    plain_bytes = base.device_bytes
    res = {"workload": "decode-11008x4096", "block": "16x128", "calibration_tokens": 256,
           "D_base": D0, "base_us": decode_us(lambda: mq.mq_pack(W, layer.group, 0.0)),
           "plain_w4_device_bytes": plain_bytes, "by_fraction": {}}
    base.free()
    for beta in (0.01, 0.05, 0.1, 0.2):
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record()
        p = mq.mq_pack_blocks(W, layer.group, beta, h)
        ev1.record()
        torch.cuda.synchronize()
        rbytes = p.nblk * (16 * 64 + 16 * 4)             # 4-bit codes + fp32 scale per block row
        entry = {"nblk": p.nblk, "entries": p.nnz, "pack_ms": round(ev0.elapsed_time(ev1), 3),
                 "device_bytes": p.device_bytes, "over_plain_w4": round(p.device_bytes / plain_bytes, 4),
                 "bits_per_weight": round(8.0 * p.device_bytes / (N * K), 4),
                 "residual_bytes": rbytes, "recovered": round(1.0 - distortion(p) / D0, 4),
                 "us": decode_us(lambda: mq.mq_pack_blocks(W, layer.group, beta, h))}
        p.free()
        rho = rbytes / 2.5 / (N * K)                     # element-wise: 2 B column + 1/2 B code per entry
        pe = mq.mq_pack(W, layer.group, rho)
        entry["elementwise_same_bytes"] = {"rho": round(rho, 5), "recovered": round(1.0 - distortion(pe) / D0, 4),
                                           "us": decode_us(lambda: mq.mq_pack(W, layer.group, rho))}
        pe.free()
        res["by_fraction"][str(beta)] = entry
    # the prefill GEMM with 10 % of the blocks, against plain W4 and the
    # element-wise residual of that layer (rho 1 %), on the 28672x8192 layer
    pl = synth.WORKLOADS["prefill-28672x8192"].layers[0]
    Wp = torch.from_numpy(pl.W()).cuda()
    hp = (torch.from_numpy(pl.calibration(256, 4)).cuda().float() ** 2).sum(0)
    pre = {}
    for name, make in (("plain_w4", lambda: mq.mq_pack(Wp, pl.group, 0.0)),
                       ("elementwise_rho_0.01", lambda: mq.mq_pack(Wp, pl.group, 0.01)),
                       ("blocks_0.1", lambda: mq.mq_pack_blocks(Wp, pl.group, 0.1, hp))):
        p = make()
        pre[name] = {}
        for M in (512, 2048):
            X = torch.from_numpy(pl.X(M)).cuda()
            Y = torch.empty((M, pl.N), dtype=torch.float16, device="cuda")

            def run(i, X=X, Y=Y, p=p):
                mq.mq_linear(X, p, Y)
            time_events(run, 3)
            us = time_events(run, 10) / 10 * 1e3
            pre[name][str(M)] = {"us": round(us, 1), "TFLOPs": round(2.0 * M * pl.N * pl.K / us / 1e6, 1)}
        p.free()
    res["prefill_28672x8192"] = pre
    return res


def bench_migration(args, mq, synth, torch):
    """Outlier migration before packing on the 11008x4096 decode layer: the
    output distortion ||Y - X W^T||^2 on 256 held-out tokens (4 hot channels
    x50, the same channels as the 256 calibration tokens the migration and
    the block scores use) of plain W4, the element-wise residual (rho 0.5 %)
    and the block residual (10 % of the blocks), each without and with
    migration; and the time of mq_smooth_weights and of one
    mq_smooth_activations call at M = 16."""
    layer = synth.WORKLOADS["decode-11008x4096"].layers[0]
    W = torch.from_numpy(layer.W()).cuda()
    Xcal = torch.from_numpy(layer.calibration(256, 4)).cuda()
    Xev = torch.from_numpy(layer.calibration(256, 4, held_out=True)).cuda()
    Yref = Xev.float() @ W.float().t()
    amax = Xcal.float().abs().amax(0)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    Wm, e = mq.mq_smooth_weights(W, amax)
    ev1.record()
    torch.cuda.synchronize()
    smooth_ms = ev0.elapsed_time(ev1)
    Xev_m = mq.mq_smooth_activations(Xev, e)
    Xcal_m = mq.mq_smooth_activations(Xcal, e)

    def dist(p, X):
        Y = mq.mq_linear(X, p).float()
        return float(((Y - Yref) ** 2).sum())

    out = {"workload": "decode-11008x4096", "smooth_weights_ms": round(smooth_ms, 3),
           "channels_moved": int((e != 0).sum())}
    for tag, Wx, Xe, Xc in (("without", W, Xev, Xcal), ("with", Wm, Xev_m, Xcal_m)):
        h = (Xc.float() ** 2).sum(0)
        d = {}
        for name, make in (("plain_w4", lambda: mq.mq_pack(Wx, layer.group, 0.0)),
                           ("elementwise_rho_0.005", lambda: mq.mq_pack(Wx, layer.group, 0.005)),
                           ("blocks_0.1", lambda: mq.mq_pack_blocks(Wx, layer.group, 0.1, h))):
            p = make()
            d[name] = dist(p, Xe)
            p.free()
        out[tag + "_migration"] = d
    base = out["without_migration"]["plain_w4"]
    out["relative_to_plain_w4_without"] = {
        tag: {k: round(v / base, 4) for k, v in out[tag + "_migration"].items()} for tag in ("without", "with")}
    X16 = torch.from_numpy(layer.X(16)).cuda()
    Xo = torch.empty_like(X16)

    def smooth(i):
        mq.mq_smooth_activations(X16, e, Xo)
    out["smooth_activations_us_M16"] = round(replay_spread(torch, smooth, 4, 40, reps=5)[0] * 1e3, 2)
    return out


def bench_w4a4(args, mq, synth, torch):
    """4-bit activations. Prefill on the 28672x8192 layer at M = 512, 2048 and
    4096: mq_quantize_activations + mq_linear_a4 (the quantization stage is
    part of the step) and the W4A4 GEMM alone, against the fp16-activation
    GEMM (mq_linear) on the same handle; plain W4 and 10 % residual blocks.
    TFLOP/s count 2 M N K. Decode time at M = 1 and 16 on the 11008x4096
    layer (rotated copies, graph replay). Output distortion ||Y - X W^T||^2 on
    the held-out activations of that layer (4 hot channels x50): W4A16 and
    W4A4, plain and with blocks, without and with outlier migration."""
    import numpy as np
    res = {}
    pl = synth.WORKLOADS["prefill-28672x8192"].layers[0]
    Wp = torch.from_numpy(pl.W()).cuda()
    hp = (torch.from_numpy(pl.calibration(256, 4)).cuda().float() ** 2).sum(0)
    pre = {}
    for name, make in (("plain_w4", lambda: mq.mq_pack(Wp, pl.group, 0.0)),
                       ("blocks_0.1", lambda: mq.mq_pack_blocks(Wp, pl.group, 0.1, hp))):
        p = make()
        pre[name] = {}
        for M in (512, 2048, 4096):
            X = torch.from_numpy(pl.X(M)).cuda()
            Y = torch.empty((M, pl.N), dtype=torch.float16, device="cuda")
            xq, xm = mq.mq_quantize_activations(X, pl.group)

            def step(i, X=X, Y=Y, p=p, xq=xq, xm=xm):
                mq.mq_quantize_activations(X, pl.group, xq, xm)
                mq.mq_linear_a4(xq, xm, p, Y)

            def gemm(i, Y=Y, p=p, xq=xq, xm=xm):
                mq.mq_linear_a4(xq, xm, p, Y)

            def a16(i, X=X, Y=Y, p=p):
                mq.mq_linear(X, p, Y)
            # the three are timed in turn, round after round, and each keeps
            # its median: the shader clock drifts by several % over a leg of
            # this length, and timing one after the other would set it apart
            # from the others
            runs = {"w4a4_step": [], "w4a4_gemm": [], "w4a16_gemm": []}
            fns = (("w4a4_step", step), ("w4a4_gemm", gemm), ("w4a16_gemm", a16))
            for tag, fn in fns:
                time_events(fn, 2)
            for _ in range(5):
                for tag, fn in fns:
                    runs[tag].append(time_events(fn, 3) / 3 * 1e3)
            e = {}
            for tag, v in runs.items():
                us = float(np.median(v))
                e[tag] = {"us": round(us, 1), "TFLOPs": round(2.0 * M * pl.N * pl.K / us / 1e6, 1)}
            e["w4a4_gemm"]["frac_fp8_peak"] = round(e["w4a4_gemm"]["TFLOPs"] / FP8_PEAK_TFLOPS, 4)
            e["speedup_step_vs_w4a16"] = round(e["w4a16_gemm"]["us"] / e["w4a4_step"]["us"], 3)
            pre[name][str(M)] = e
        p.free()
    del Wp
    res["prefill_28672x8192"] = pre

    layer = synth.WORKLOADS["decode-11008x4096"].layers[0]
    N, K, G = layer.N, layer.K, layer.group
    W = torch.from_numpy(layer.W()).cuda()
    dec = {}
    for M in (1, 2, 16):
        X = torch.from_numpy(layer.X(M)).cuda()
        Y = torch.empty((M, N), dtype=torch.float16, device="cuda")
        p0 = mq.mq_pack(W, G, 0.0)
        ncopy = max(2, math.ceil(2 * MALL_BYTES / p0.device_bytes))
        copies = [p0] + [mq.mq_pack(W, G, 0.0) for _ in range(ncopy - 1)]
        xq, xm = mq.mq_quantize_activations(X, G)

        def a4(i, X=X, Y=Y, xq=xq, xm=xm):
            mq.mq_quantize_activations(X, G, xq, xm)
            mq.mq_linear_a4(xq, xm, copies[i % ncopy], Y)

        def a16(i, X=X, Y=Y):
            mq.mq_linear(X, copies[i % ncopy], Y)

        def a4f(i, X=X, Y=Y):   # the quantizer inside the decode kernel: one launch
            mq.mq_decode_a4(X, copies[i % ncopy], Y)
        dec[str(M)] = {"w4a4_step_us": round(replay_spread(torch, a4, 4, 40, reps=5)[0] * 1e3, 2),
                       "w4a16_us": round(replay_spread(torch, a16, 4, 40, reps=5)[0] * 1e3, 2)}
        if M <= 2:
            dec[str(M)]["w4a4_one_kernel_us"] = round(replay_spread(torch, a4f, 4, 40, reps=5)[0] * 1e3, 2)
        for c in copies:
            c.free()
    res["decode_11008x4096_plain"] = dec

    Xcal = torch.from_numpy(layer.calibration(256, 4)).cuda()
    Xev = torch.from_numpy(layer.calibration(256, 4, held_out=True)).cuda()
    Yref = Xev.float() @ W.float().t()
    amax = Xcal.float().abs().amax(0)
    Wm, e = mq.mq_smooth_weights(W, amax)
    dist = {}
    for tag, Wx, Xe, Xc in (("without_migration", W, Xev, Xcal),
                            ("with_migration", Wm, mq.mq_smooth_activations(Xev, e),
                             mq.mq_smooth_activations(Xcal, e))):
        h = (Xc.float() ** 2).sum(0)
        d = {}
        for name, make in (("plain_w4", lambda: mq.mq_pack(Wx, G, 0.0)),
                           ("blocks_0.1", lambda: mq.mq_pack_blocks(Wx, G, 0.1, h))):
            p = make()
            d[name + "_a16"] = float(((mq.mq_linear(Xe, p).float() - Yref) ** 2).sum())
            xq, xm = mq.mq_quantize_activations(Xe, G)
            d[name + "_a4"] = float(((mq.mq_linear_a4(xq, xm, p).float() - Yref) ** 2).sum())
            p.free()
        dist[tag] = d
    base = dist["without_migration"]["plain_w4_a16"]
    res["distortion_11008x4096"] = {
        "workload": "decode-11008x4096", "held_out_tokens": 256,
        "relative_to_w4a16_plain": {t: {k: round(v / base, 4) for k, v in d.items()} for t, d in dist.items()}}
    return res


def bench_stream(args, mq, torch, nbytes=24 << 20):
    """Read ceiling: mq_stream_read over `nbytes` (the decode layer's packed
    size), every launch on another buffer (rotated over more than twice the
    Infinity Cache), back-to-back launches in a graph, at several grid sizes.
    Per-launch period from HIP events, as for the decode kernels."""
    nbuf = max(2, math.ceil(2 * MALL_BYTES / nbytes))
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device="cuda").random_(0, 255) for _ in range(nbuf)]
    out = {"bytes": nbytes, "buffers": nbuf, "by_workgroups": {}}
    for wg in (384, 768, 1536, 3072, 6144):   # 16, 8, 4, 2, 1 loads per thread
        sink = torch.empty(wg, dtype=torch.int32, device="cuda")

        def rd(i, wg=wg, sink=sink):
            mq.mq_stream_read(bufs[i % nbuf], wg, sink)
        med, p10, p90 = replay_spread(torch, rd, max(2, args.warmup // 4), max(20, args.steps // 2), reps=5)
        out["by_workgroups"][str(wg)] = {"us": round(med * 1e3, 3), "p10_us": round(p10 * 1e3, 3),
                                         "p90_us": round(p90 * 1e3, 3),
                                         "GBps": round(nbytes / (med * 1e-3) / 1e9, 1)}
    best = min(out["by_workgroups"].values(), key=lambda v: v["us"])
    out["best"] = best
    return out


def cpu_baseline(layer, Ms, min_seconds=10.0, max_steps=60):
    """The oracle, as it stands, on the same decode layer: one step is its
    dequantisation plus the float64 linear for M = 1, 4, 16 (packing by the
    oracle is done first and reported apart). Steps repeat until about
    `min_seconds` of CPU work (at most `max_steps`), so the sample is long
    enough to time and the default run still ends within minutes."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    W = layer.W()
    t0 = time.perf_counter()
    packed = oracle.pack(W, layer.group, layer.rho)
    t_pack = time.perf_counter() - t0
    Xs = {M: layer.X(M) for M in Ms}
    t0 = time.perf_counter()
    steps = 0
    while True:
        Wt = oracle.dequant(packed)
        for M in Ms:
            oracle.linear(Xs[M], Wt)
        steps += 1
        t_lin = time.perf_counter() - t0
        if t_lin >= min_seconds or steps >= max_steps:
            break
    canon = (layer.N * layer.K // 2 + 2 * layer.N * (layer.K // layer.group) + 4 * (layer.N + 1)
             + 2 * packed["nnz"] + (packed["nnz"] + 1) // 2 + 4 * layer.N)
    nbytes = steps * sum(canon + 2 * M * layer.K + 2 * M * layer.N for M in Ms)
    return {"value": round(nbytes / t_lin / 1e9, 3), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            **host_cpu(),
            "sample": f"{steps} steps of the oracle's dequant + float64 linear of the full {layer.N}x{layer.K} "
                      f"layer at M={Ms}; the oracle's pack of the layer ({t_pack:.1f} s) is not included",
            "seconds": round(t_lin, 3), "steps": steps, "pack_seconds": round(t_pack, 2)}


def cpu_baseline_configs(synth):
    """The oracle, as it stands, on the other configurations, pack and
    linear timed apart (one run each; a baseline, not a target):
      * block-4096h: the seven linears of the 4096-hidden block, packed, then
        dequantised and multiplied at M = 16;
      * prefill-28672x8192: packed, dequantised, multiplied at M = 512 and
        2048 (float64);
      * sweep-14336x4096 (columns placement): packed at each density, and at
        0.5 % dequantised and multiplied at M = 1, 64 and 512."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))

    def timed(fn):
        t0 = time.perf_counter()
        r = fn()
        return r, time.perf_counter() - t0

    out = {"cores": int(threads), "kind": "oracle", **host_cpu()}
    # block-4096h at M = 16
    wl = synth.WORKLOADS["block-4096h"]
    M = wl.batch[0]
    t_pack = t_deq = t_lin = 0.0
    flops = 0
    for layer in wl.layers:
        W = layer.W()
        pk, dt = timed(lambda: oracle.pack(W, layer.group, layer.rho))
        t_pack += dt
        Wt, dt = timed(lambda: oracle.dequant(pk))
        t_deq += dt
        _, dt = timed(lambda: oracle.linear(layer.X(M), Wt))
        t_lin += dt
        flops += 2 * M * layer.N * layer.K
    out["block_4096h_m16"] = {"pack_seconds": round(t_pack, 2), "dequant_seconds": round(t_deq, 2),
                              "linear_seconds": round(t_lin, 3), "linear_GFLOPs": round(flops / t_lin / 1e9, 2),
                              "sample": "the 7 layers once each"}
    # prefill at M = 512, 2048
    layer = synth.WORKLOADS["prefill-28672x8192"].layers[0]
    W = layer.W()
    pk, t_pack = timed(lambda: oracle.pack(W, layer.group, layer.rho))
    Wt, t_deq = timed(lambda: oracle.dequant(pk))
    lin = {}
    for M in (512, 2048):
        X = layer.X(M)
        _, dt = timed(lambda: oracle.linear(X, Wt))
        lin[str(M)] = {"seconds": round(dt, 3), "TFLOPs": round(2.0 * M * layer.N * layer.K / dt / 1e12, 4)}
    out["prefill_28672x8192"] = {"pack_seconds": round(t_pack, 2), "dequant_seconds": round(t_deq, 2),
                                 "linear": lin, "sample": "one pack, one dequant, one linear per M"}
    del Wt, pk, W
    # residual sweep, columns placement
    packs = {}
    for rho in synth.SWEEP_RHOS:
        sl = synth.sweep_layer("columns", rho)
        W = sl.W()
        pk, dt = timed(lambda: oracle.pack(W, sl.group, rho))
        packs[str(rho)] = round(dt, 2)
        if rho == 0.005:
            Wt, t_deq = timed(lambda: oracle.dequant(pk))
            lin = {}
            for M in synth.SWEEP_BATCH:
                X = sl.X(M)
                _, dt = timed(lambda: oracle.linear(X, Wt))
                lin[str(M)] = round(dt, 4)
            del Wt
    out["sweep_14336x4096_columns"] = {"pack_seconds_by_rho": packs, "dequant_seconds_rho_0.005": round(t_deq, 2),
                                       "linear_seconds_rho_0.005": lin,
                                       "sample": "one pack per density; one dequant and linear per M at 0.5 %"}
    return out


def progress(leg):
    """One line on stderr per finished leg (the JSON line stays alone on stdout)."""
    print(f"[bench] {leg} done at {time.strftime('%H:%M:%S')}", file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)
    import torch
    from bit_gemm_amd import mosaicq as mq
    from bit_gemm_amd import synth
    assert torch.cuda.is_available(), "bench.py needs the GPU"
    torch.cuda.set_device(0)

    if args.only == "copy":
        # a plain device copy of known size: reference for the HBM byte counters
        nbytes = 1 << 30
        src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").random_(0, 255)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "launches": 3}), flush=True)
        return
    if args.only == "stream":
        print(json.dumps({"stream_read": bench_stream(args, mq, torch)}), flush=True)
        return
    if args.only == "prefill":
        print(json.dumps({"prefill": bench_prefill(args, mq, synth, torch)}), flush=True)
        return
    if args.only == "mid":
        print(json.dumps({"mid_batch": bench_mid(args, mq, synth, torch)}), flush=True)
        return
    if args.only == "tblock":
        print(json.dumps({"block_4096h_m16": bench_block(args, mq, synth, torch)}), flush=True)
        return
    if args.only == "sweep":
        print(json.dumps({"residual_sweep": bench_sweep(args, mq, synth, torch)}), flush=True)
        return
    if args.only == "blocks":
        print(json.dumps({"block_residual": bench_blocks(args, mq, synth, torch)}), flush=True)
        return
    if args.only == "migration":
        print(json.dumps({"migration": bench_migration(args, mq, synth, torch)}), flush=True)
        return
    if args.only == "w4a4":
        print(json.dumps({"w4a4": bench_w4a4(args, mq, synth, torch)}), flush=True)
        return
    d = bench_decode(args, mq, synth, torch)
    value = d["bytes_step"] / (d["ms_per_step"] * 1e-3) / 1e9
    # dominant kernel: the decode launch with the longest average duration
    mdom = max(d["per_m"], key=lambda m: d["per_m"][m]["us"])
    dom = d["per_m"][mdom]
    achieved = dom["bytes"] / (dom["us"] * 1e-6) / 1e9
    tag = ("k_gemv_x" if int(mdom) <= 4 else "k_gemv_r") + f"@M={mdom}"
    traffic = counted_traffic(tag)
    # the same kernel's average duration in the committed rocprofv3 kernel
    # trace of `bench.py --only decode` (kernel time alone, without the
    # dispatch gap that a graph replay's per-launch period includes)
    trace = profile_values("decode_kernel_stats.txt", DECODE_SOURCES)
    trace_us = float(trace[f"kernel_avg_us[{tag}]"]) if f"kernel_avg_us[{tag}]" in trace else None
    period_us = float(trace[f"launch_period_us[{tag}]"]) if f"launch_period_us[{tag}]" in trace else None
    # the committed streaming-read ceiling for a buffer of this size (a plain
    # read kernel): the kernel's rate on kernel time as a fraction of it
    ceil = profile_values("stream_read_ceiling.txt", STREAM_SOURCES)
    ceil_gbs = float(ceil["ceiling_GBps"]) if "ceiling_GBps" in ceil else None
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(d["ms_per_step"], 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp16",
        "data": "synthetic",
        "config": {"workload": "decode-11008x4096", "N": 11008, "K": 4096, "group": 128, "rho": 0.005,
                   "nnz": d["nnz"], "M": [1, 4, 16], "packed_copies": d["copies"],
                   "timing": "hip graph replay; every launch reads another packed copy"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": tag,
                     "algorithmic_bytes_per_launch": dom["bytes"], "avg_launch_us": dom["us"],
                     "time_basis": "live: HIP events around a graph of back-to-back launches of this kernel "
                                   "(each on another packed copy) / launches = launch period, kernel + dispatch gap",
                     "profile_launch_period_us": period_us, "profile_kernel_avg_us": trace_us,
                     "frac_kernel_time": (round(dom["bytes"] / (trace_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
                                          if trace_us else None),
                     "streaming_ceiling_GBps": ceil_gbs,
                     "frac_of_streaming_ceiling": (round(dom["bytes"] / (trace_us * 1e-6) / 1e9 / ceil_gbs, 4)
                                                   if trace_us and ceil_gbs else None)},
        "decode_per_M": d["per_m"],
        "decode_residual_overhead_t_rho_over_t0": d["overhead"],
        "decode_unfused_two_kernels": d["unfused"],
        "decode_warm_single_copy_us_M1": None if args.no_warm else round(d["warm_us_m1"], 3),
        "handle_device_bytes": d["handle"],
        "inputs_sha256": d["inputs_sha256"],
        "pack": {"workload": "decode-11008x4096", "gpu_ms": round(d["pack_ms"], 3),
                 "wall_ms_first_call": round(d["pack_wall_ms"], 3)},
    }
    legs = []
    if args.only != "decode":
        if not args.skip_prefill:
            legs.append(("prefill", bench_prefill))
        if not args.skip_extra:
            legs += [("mid_batch", bench_mid), ("block_4096h_m16", bench_block), ("residual_sweep", bench_sweep),
                     ("block_residual", bench_blocks), ("migration", bench_migration), ("w4a4", bench_w4a4)]
    progress("decode")
    for name, fn in legs:
        line[name] = fn(args, mq, synth, torch)
        progress(name)
    if args.only != "decode" and not args.skip_cpu:
        line["cpu_baseline"] = cpu_baseline(d["layer"], [1, 4, 16])
        progress("cpu_baseline")
        line["cpu_baseline_configs"] = cpu_baseline_configs(synth)
        progress("cpu_baseline_configs")
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
