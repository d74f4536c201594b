#!/usr/bin/env python3
"""Benchmark of the NVFP4 W4A4 linear layer on one MI355X.

Headline (the `value`): NVFP4 W4A4 GEMM TFLOP/s on the prefill workload
X[4096x5120] bf16 (quantized on the fly) x W[17408x5120] NVFP4 -> Y bf16.
One step = one full serving-time pass: activation absmax, activation encode
and the block-scaled GEMM with its epilogue (nvfp4_gemm_prepare followed by
nvfp4_gemm_run, which together are nvfp4_gemm).  Weight quantization and
the fused-group repair are checkpoint-side steps and are timed separately.

The same JSON line carries, under "also", the decode GEMV (M = 1, 4, 16,
fused gate/up W[34816x5120], GB/s with 4 rotated weight copies so that the
last-level cache cannot hold them), the standalone activation quantize at
long prefill (X[32768x5120], GB/s on the two-pass byte count), the fused
q/k/v repair + GEMM and the offline weight quantize.  The decode and quantize
lines also time the calibrated-scale form (the activation tensor scale given,
no absmax pass) under "calibrated_scale", and the decode lines the W4A16 form
(bf16 activations as given, one GEMV launch) under "w4a16"; a separate line
times W4A16 at the prefill shape.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

Defaults: 100 warm-up steps, then 100 timed steps.  From idle the GPU clock
takes a few tens of milliseconds of sustained load to settle (the first 20
prefill steps run about a quarter slower than the settled rate), so the
warm-up is long enough to time the settled, sustained rate.
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

METRIC = "NVFP4 W4A4 GEMM TFLOP/s at M=4096 and GB/s at M=1; quantize GB/s"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, published
PEAK_FP16_TFLOPS = 2500.0      # MI355X dense fp16/bf16 MFMA, published
PROFILE_DIR = os.path.join(ROOT, "profiles")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--headline-only", action="store_true",
                    help="skip the secondary workloads (profiling runs)")
    ap.add_argument("--only", choices=["prefill", "decode", "qkv", "quantize", "fp8", "weight"],
                    help="run one workload group alone and print its lines (profiling runs); prefill: the "
                         "headline, its settled rerun and W4A16, without the secondary lines and box peaks")
    ap.add_argument("--no-numerics", action="store_true",
                    help="skip the input statistics and fake-quantization errors")
    ap.add_argument("--no-box-peaks", action="store_true",
                    help="skip the box-measured reference rates (device copy, torch fp16 GEMM)")
    ap.add_argument("--copy-ref", action="store_true",
                    help="first run one plain 1 GiB device copy, the reference kernel for HBM counters")
    return ap.parse_args()


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def source_sha():
    """Hash of every source the library is built from (kernels, launchers,
    the ABI layer and its header): counters taken on other sources are not
    reported as the current kernels' traffic."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "nvfp4_w4a4_quantized_02_amd", "csrc")
    for path in [os.path.join(csrc, n) for n in sorted(os.listdir(csrc))] + \
            [os.path.join(ROOT, "include", "nvfp4.h")]:
        if os.path.isfile(path):
            with open(path, "rb") as f:
                h.update(os.path.basename(path).encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def traffic_for(kernel_key, sha):
    """HBM bytes per launch from committed rocprofv3 PMC summaries, if they
    were taken on the current kernel source; otherwise None."""
    path = os.path.join(PROFILE_DIR, "pmc_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(kernel_key)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha") != sha:
        return None
    return rec.get("hbm_bytes_per_launch")


class Timer:
    """Per-step CUDA events on the current stream (the stream the library
    launches on), split into named phases."""

    def __init__(self, torch, steps, phases):
        self.torch = torch
        self.ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(phases) + 1)]
                   for _ in range(steps)]
        self.phases = phases

    def mark(self, step, i):
        self.ev[step][i].record()

    def phase_ms(self, i):
        return [e[i].elapsed_time(e[i + 1]) for e in self.ev]


def time_steps(torch, steps, warmup, body, nphase):
    """Run `body(step, mark)` warmup+steps times; returns (ms/step, per-phase
    ms lists).  The timed region is bracketed by device synchronizations."""
    for i in range(warmup):
        body(i, lambda j: None)
    torch.cuda.synchronize()
    tm = Timer(torch, steps, list(range(nphase)))
    t0 = time.perf_counter()
    for i in range(steps):
        body(i, lambda j, i=i: tm.mark(i, j))
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    return wall, [tm.phase_ms(j) for j in range(nphase)]


def graph_step_ms(torch, fn, nsteps, out, reps=20, batches=5, warm_ms=30.0):
    """GPU ms per step of fn(i), i = 0..nsteps-1, captured as one graph:
    replayed for at least warm_ms first (the clock settles under sustained
    load), then `batches` batches of `reps` replays between events; the
    median batch is returned.  The replay's `out` must equal the eager result
    bit for bit (the kernels are deterministic)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(nsteps):
            fn(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(nsteps):
            fn(i)
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    if not torch.equal(out, eager):
        raise RuntimeError("graph replay differs from the eager result")
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < warm_ms:
        for _ in range(reps):
            g.replay()
        torch.cuda.synchronize()
    times = []
    for _ in range(batches):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) / (reps * nsteps))
    return sorted(times)[len(times) // 2]


def mean(v):
    return sum(v) / len(v)


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import workloads
    import nvfp4_w4a4_quantized_02_amd as nv

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_ref:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    def to_gpu(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    # ------------------------------------------------------------ headline workload
    log("generating prefill workload X[4096x5120] bf16, W[17408x5120]")
    p = workloads.prefill()
    M, K, N = p.M, p.K, p.N
    w32 = torch.from_numpy(p.w_parts[0]).to(dev)
    wc, ws, wg = nv.nvfp4_quantize(w32)
    del w32
    x = to_gpu(p.x)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    ws_buf = torch.empty(nv.lib.nvfp4_gemm_workspace_size(M, N, K), dtype=torch.uint8, device=dev)
    flops = 2.0 * M * N * K
    sha = source_sha()

    if args.only and args.only != "prefill":
        print(json.dumps({"only": args.only, "also": secondary(torch, np, nv, workloads, to_gpu, dev, args)}),
              flush=True)
        return

    # The secondary lines and the machine's reference rates run first, so the
    # headline's warm-up starts on a GPU that is already under load (from
    # idle, the clock takes tens of milliseconds of sustained load to settle).
    also = []
    bp = None
    if not args.headline_only and args.only != "prefill":
        also += secondary(torch, np, nv, workloads, to_gpu, dev, args)
        if not args.no_box_peaks:
            bp = box_peaks(torch, dev, M, N, K)

    def step(i, mark):
        mark(0)
        prep = nv.nvfp4_gemm_prepare(x, ws=ws_buf)
        mark(1)
        nv.nvfp4_gemm_run(prep, wc, ws, wg, out=y)
        mark(2)

    log("timing prefill GEMM: %d warmup, %d steps" % (args.warmup, args.steps))
    wall_ms, (prep_ms, run_ms) = time_steps(torch, args.steps, args.warmup, step, 2)
    step_ms = wall_ms                      # timed region / steps, synchronized on both sides
    value = flops / (step_ms * 1e-3) / 1e12
    gemm_tflops = flops / (mean(run_ms) * 1e-3) / 1e12
    traffic = traffic_for("gemm_prefill", sha)
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "device_ms_per_step": round(mean(prep_ms) + mean(run_ms), 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "arith": "NVFP4 (E2M1 x E4M3) operands expanded exactly to fp16; MFMA fp16 with fp32 accumulate",
        "data": "synthetic (seeded; shapes and distributions of the prefill workload)",
        "config": {"workload": "prefill W4A4 linear: X[4096x5120] bf16 Student-t(3) quantized on the fly "
                               "x W[17408x5120] NVFP4 from N(0,0.02) -> Y bf16",
                   "M": M, "N": N, "K": K, "x_dtype": "bf16", "y_dtype": "bf16"},
        "timed_after": ("the secondary lines and the box peaks (the GPU is under load when the warm-up starts)"
                        if not args.headline_only else "nothing (headline only)"),
        "phases_ms": {"activation_quantize": round(mean(prep_ms), 4), "gemm": round(mean(run_ms), 4)},
        "roofline": {"bound": "mfma", "kernel": "nvfp4_gemm_run: gemm_kernel (fp16 MFMA 32x32x16) + split-K reduce",
                     "achieved": round(gemm_tflops, 2), "peak": PEAK_FP16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(gemm_tflops / PEAK_FP16_TFLOPS, 4), "traffic": traffic,
                     "algorithmic": "2*M*N*K = %.4g flop per launch" % flops},
    }
    if not args.headline_only:
        # the same step again with 100 warm-up and 100 timed steps: the
        # sustained rate, whatever warm-up the headline was given
        wall2, (prep2, run2) = time_steps(torch, 100, 100, step, 2)
        out["settled"] = {"warmup": 100, "steps": 100, "ms_per_step": round(wall2, 4),
                          "TFLOPs": round(flops / (wall2 * 1e-3) / 1e12, 2),
                          "gemm_TFLOPs": round(flops / (mean(run2) * 1e-3) / 1e12, 2)}
        # W4A16: the same weights against the bf16 activations as given
        wsz16 = nv.lib.nvfp4_gemm_w4a16_workspace_size(M, N, K)
        ws16 = torch.empty(max(wsz16, 256), dtype=torch.uint8, device=dev)

        def step16(i, mark):
            mark(0)
            st = nv.lib.nvfp4_gemm_w4a16(x.data_ptr(), 1, M, K, K, wc.data_ptr(), ws.data_ptr(), wg.data_ptr(), N,
                                         y.data_ptr(), 1, N, ws16.data_ptr(), ws16.numel(),
                                         torch.cuda.current_stream().cuda_stream)
            assert st == 0
            mark(1)

        _, (w16_ms,) = time_steps(torch, args.steps, args.warmup, step16, 1)
        t16 = flops / (mean(w16_ms) * 1e-3) / 1e12
        also.insert(0, {"metric": "W4A16 GEMM TFLOP/s at M=4096", "value": round(t16, 2), "unit": "TFLOP/s",
                        "ms_per_step": round(mean(w16_ms), 4),
                        "config": {"workload": "prefill W4A16 linear: X[4096x5120] bf16 Student-t(3) as given x "
                                               "W[17408x5120] NVFP4 -> Y bf16"},
                        "roofline": {"bound": "mfma", "kernel": "nvfp4_gemm_w4a16: gemm_kernel (bf16 MFMA 32x32x16) "
                                                                 "+ split-K reduce",
                                     "achieved": round(t16, 2), "peak": PEAK_FP16_TFLOPS, "unit": "TFLOP/s",
                                     "frac": round(t16 / PEAK_FP16_TFLOPS, 4),
                                     "traffic": traffic_for("gemm_prefill_w4a16", sha)}})
        log("W4A16 prefill: %.1f TFLOP/s" % t16)
        del ws16
        if not args.no_numerics:
            out["numerics"] = numerics(torch, nv, workloads, to_gpu, dev, p, x, wc, ws, wg)
    del y, x

    # ------------------------------------------------------------ box-measured peaks
    if bp is not None:
        out["box_peaks"] = bp
        # the same achieved rates against what this machine sustains on plain work
        out["roofline"]["frac_of_box"] = round(out["roofline"]["achieved"] / bp["fp16_gemm_TFLOPs"], 4)
        for line in also:
            r = line.get("roofline")
            if not r or r.get("achieved") is None:
                continue
            if r.get("unit") == "GB/s":
                r["frac_of_box"] = round(r["achieved"] / bp["hbm_read_GBs"], 4)
            elif r.get("unit") == "TFLOP/s" and r.get("peak") == PEAK_FP16_TFLOPS:
                r["frac_of_box"] = round(r["achieved"] / bp["fp16_gemm_TFLOPs"], 4)

    # ------------------------------------------------------------ CPU oracle
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(np, p)
    out["also"] = also
    print(json.dumps(out), flush=True)


def secondary(torch, np, nv, workloads, to_gpu, dev, args):
    res = []
    steps, warmup = args.steps, args.warmup

    def want(group):
        return args.only is None or args.only == group

    # ------------------------------------------------ decode GEMV, M = 1/4/16
    if want("decode"):
        log("generating decode workload (fused gate/up W[34816x5120])")
        d = workloads.decode(M=1)
        q = [nv.nvfp4_quantize(torch.from_numpy(w).to(dev)) for w in d.w_parts]
        shared = nv.nvfp4_fuse_rescale([s for _, s, _ in q], [g for _, _, g in q])
        wc0 = torch.cat([c for c, _, _ in q])
        ws0 = torch.cat([s for _, s, _ in q])
        del q
        R = 4                                  # 4 x 100 MB > the 256 MB last-level cache
        copies = [(wc0.clone(), ws0.clone()) for _ in range(R)]
        del wc0, ws0
        N, K = d.N, d.K
        wbytes = copies[0][0].numel() + copies[0][1].numel()
        for M in (1, 4, 16):
            dm = workloads.decode(M=M, N_each=1)          # only X is used from it
            x = to_gpu(dm.x)
            y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            wsb = torch.empty(nv.lib.nvfp4_gemm_workspace_size(M, N, K), dtype=torch.uint8, device=dev)
            xgs = nv.nvfp4_quantize(x)[2]

            # Each form is captured as one graph of R steps (one per weight copy)
            # and replayed, so the time is the GPU's and not the launch overhead
            # of the Python binding; the replay's output is checked against the
            # eager call's.
            # the whole call (M = 1: quantize and GEMV in one launch)
            def w4a4(i, x=x, y=y, wsb=wsb):
                c, s = copies[i]
                nv.nvfp4_gemm(x, c, s, shared, out=y, ws=wsb)

            def w4a4_static(i, x=x, y=y, wsb=wsb, xgs=xgs):
                c, s = copies[i]
                nv.nvfp4_gemm(x, c, s, shared, out=y, x_gs=xgs, ws=wsb)

            # the same product as two launches (quantize, then the GEMV)
            def two_launch(i, x=x, y=y, wsb=wsb):
                c, s = copies[i]
                nv.nvfp4_gemm_run(nv.nvfp4_gemm_prepare(x, ws=wsb), c, s, shared, out=y)

            prep = nv.nvfp4_gemm_prepare(x, ws=wsb)

            def gemv_only(i, y=y, prep=prep):
                c, s = copies[i]
                nv.nvfp4_gemm_run(prep, c, s, shared, out=y)

            def prep_only(i, x=x, wsb=wsb):
                nv.nvfp4_gemm_prepare(x, ws=wsb)

            def w4a16(i, x=x, y=y):
                c, s = copies[i]
                nv.nvfp4_gemm_w4a16(x, c, s, shared, out=y)

            t = {}
            for name, fn in (("w4a4", w4a4), ("w4a4_static", w4a4_static), ("two_launch", two_launch),
                             ("gemv", gemv_only), ("prep", prep_only), ("w4a16", w4a16)):
                t[name] = graph_step_ms(torch, fn, R, y, reps=max(steps, 20))
            nbytes = wbytes + M * K * 2 + M * N * 2
            gbs = nbytes / (t["w4a4"] * 1e-3) / 1e9
            kgbs = nbytes / (t["gemv"] * 1e-3) / 1e9
            if M <= 4:   # one launch does the whole step: that kernel is the one on the roofline
                kname, kkey, kgbs = "nvfp4_gemm: gemv_fp4_kernel (quantize + FP4 GEMV)", "gemv_fp4_m%d" % M, gbs
            else:
                kname, kkey = "nvfp4_gemm_run: gemv kernel", "gemv_m%d" % M
            res.append({"metric": "decode GEMV GB/s at M=%d" % M, "value": round(gbs, 1), "unit": "GB/s",
                        "ms_per_step": round(t["w4a4"], 5),
                        "timing": "graph of %d steps (one per weight copy) replayed 30 ms to warm up, then the median of 5 "
                                  "batches of replays between events" % R,
                        "phases_ms": {"activation_quantize": round(t["prep"], 5), "gemv": round(t["gemv"], 5),
                                      "quantize_then_gemv": round(t["two_launch"], 5)},
                        "w4a16": {"ms_per_step": round(t["w4a16"], 5),
                                  "GBs": round(nbytes / (t["w4a16"] * 1e-3) / 1e9, 1),
                                  "frac": round(nbytes / (t["w4a16"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                                  "traffic": traffic_for("gemv_m%d_w4a16" % M, source_sha())},
                        "calibrated_scale": {"ms_per_step": round(t["w4a4_static"], 5),
                                             "GBs": round(nbytes / (t["w4a4_static"] * 1e-3) / 1e9, 1)},
                        "config": {"workload": "decode: X[%dx5120] bf16 x fused gate/up W[34816x5120] NVFP4 "
                                               "(4 rotated copies) -> Y bf16" % M},
                        "roofline": {"bound": "hbm", "kernel": kname, "achieved": round(kgbs, 1),
                                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(kgbs / PEAK_HBM_GBS, 4),
                                     "traffic": traffic_for(kkey, source_sha()),
                                     "algorithmic": "W codes+scales %d B + X + Y = %d B per launch" % (wbytes,
                                                                                                      nbytes)}})
            log("decode M=%d: step %.2f us (%.1f GB/s), two launches %.2f us, gemv %.2f us (%.1f GB/s), "
                "prep %.2f us, W4A16 %.2f us" % (M, t["w4a4"] * 1e3, gbs, t["two_launch"] * 1e3, t["gemv"] * 1e3,
                                                  kgbs, t["prep"] * 1e3, t["w4a16"] * 1e3))
        del copies

    # ------------------------------------------------ fused q/k/v repair + GEMM
    if want("qkv"):
        log("fused q/k/v workload")
        f = workloads.fused_qkv()
        parts = [torch.from_numpy(w).to(dev) for w in f.w_parts]
        qs = [nv.nvfp4_quantize(w) for w in parts]
        scales = [s for _, s, _ in qs]
        gss = [g for _, _, g in qs]
        sc_backup = [s.clone() for s in scales]

        def rstep(i, mark):
            for s, b in zip(scales, sc_backup):
                s.copy_(b)
            mark(0)
            nv.nvfp4_fuse_rescale(scales, gss)
            mark(1)

        _, (resc_ms,) = time_steps(torch, steps, warmup, rstep, 1)
        shared = nv.nvfp4_fuse_rescale([s.copy_(b) for s, b in zip(scales, sc_backup)], gss)
        fwc = torch.cat([c for c, _, _ in qs])
        fws = torch.cat(scales)
        x = to_gpu(f.x)
        M, N, K = f.M, f.N, f.K
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        wsb = torch.empty(nv.lib.nvfp4_gemm_workspace_size(M, N, K), dtype=torch.uint8, device=dev)

        def fstep(i, mark):
            mark(0)
            prep = nv.nvfp4_gemm_prepare(x, ws=wsb)
            mark(1)
            nv.nvfp4_gemm_run(prep, fwc, fws, shared, out=y)
            mark(2)

        _, (prep_ms, run_ms) = time_steps(torch, steps, warmup, fstep, 2)
        flops = 2.0 * M * N * K
        step_ms = mean(prep_ms) + mean(run_ms)
        rbytes = 2 * sum(s.numel() for s in scales)
        res.append({"metric": "fused q/k/v W4A4 GEMM TFLOP/s at M=2048", "value": round(flops / step_ms / 1e9, 2),
                    "unit": "TFLOP/s", "ms_per_step": round(step_ms, 4),
                    "phases_ms": {"activation_quantize": round(mean(prep_ms), 4), "gemm": round(mean(run_ms), 4),
                                  "fuse_rescale_offline": round(mean(resc_ms), 5)},
                    "config": {"workload": "fused q/k/v: X[2048x5120] bf16 x [q 6144; k 1024; v 1024]x5120 NVFP4, "
                                           "block scales repaired onto the shared tensor scale"},
                    "roofline": {"bound": "mfma", "kernel": "gemm_kernel",
                                 "achieved": round(flops / mean(run_ms) / 1e9, 2), "peak": PEAK_FP16_TFLOPS,
                                 "unit": "TFLOP/s", "frac": round(flops / mean(run_ms) / 1e9 / PEAK_FP16_TFLOPS, 4),
                                 "traffic": traffic_for("gemm_qkv", source_sha())},
                    "fuse_rescale_GBs": round(rbytes / mean(resc_ms) / 1e6, 1)})
        del parts, qs, x, y, wsb, fwc, fws

    # ------------------------------------------------ standalone quantize, long prefill
    if want("quantize"):
        log("generating long-prefill activations X[32768x5120] bf16")
        xl = to_gpu(workloads.long_prefill_activations())
        rows, K = xl.shape
        codes = torch.empty((rows, K // 2), dtype=torch.uint8, device=dev)
        scl = torch.empty((rows, K // 16), dtype=torch.uint8, device=dev)
        gs = torch.empty(1, dtype=torch.float32, device=dev)
        qws = nv.workspace(nv.lib.nvfp4_quantize_workspace_size(rows, K), dev)

        def qstep(i, mark):
            mark(0)
            st = nv.lib.nvfp4_quantize(xl.data_ptr(), 1, rows, K, K, codes.data_ptr(), scl.data_ptr(), gs.data_ptr(),
                                       qws.data_ptr(), qws.numel(), torch.cuda.current_stream().cuda_stream)
            assert st == 0
            mark(1)

        _, (q_ms,) = time_steps(torch, steps, warmup, qstep, 1)
        gcal = gs.clone()

        def sqstep(i, mark):
            mark(0)
            st = nv.lib.nvfp4_quantize_static(xl.data_ptr(), 1, rows, K, K, gcal.data_ptr(), codes.data_ptr(),
                                              scl.data_ptr(), torch.cuda.current_stream().cuda_stream)
            assert st == 0
            mark(1)

        _, (sq_ms,) = time_steps(torch, steps, warmup, sqstep, 1)
        xbytes = rows * K * 2
        two_pass = 2 * xbytes + rows * K // 2 + rows * K // 16
        single = xbytes + rows * K // 2 + rows * K // 16
        qgbs = two_pass / (mean(q_ms) * 1e-3) / 1e9
        res.append({"metric": "activation quantize GB/s (two-pass bytes)", "value": round(qgbs, 1), "unit": "GB/s",
                    "ms_per_step": round(mean(q_ms), 4),
                    "single_read_GBs": round(single / (mean(q_ms) * 1e-3) / 1e9, 1),
                    "calibrated_scale": {"ms_per_step": round(mean(sq_ms), 4),
                                         "GBs": round(single / (mean(sq_ms) * 1e-3) / 1e9, 1),
                                         "frac": round(single / (mean(sq_ms) * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                                         "algorithmic": "1 read of X + codes + scales = %d B per call" % single,
                                         "traffic": traffic_for("quantize_long_static", source_sha())},
                    "config": {"workload": "long-prefill quantize: X[32768x5120] bf16 Student-t(2.5), 16 hot "
                                           "channels x200 -> packed E2M1 + E4M3 scales + FP32 scale"},
                    "roofline": {"bound": "hbm", "kernel": "nvfp4_quantize: amax_partials_kernel + quantize_kernel",
                                 "achieved": round(qgbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                 "frac": round(qgbs / PEAK_HBM_GBS, 4),
                                 "traffic": traffic_for("quantize_long", source_sha()),
                                 "algorithmic": "2 reads of X + codes + scales = %d B per call" % two_pass}})
        log("quantize: %.1f GB/s (two-pass count); calibrated scale %.1f GB/s (one read)"
            % (qgbs, single / (mean(sq_ms) * 1e-3) / 1e9))
        if not args.no_numerics:
            from nvfp4_w4a4_quantized_02_amd import stats
            res[-1]["input_stats"] = {**stats.tensor_stats(xl), "a4": stats.fake_quant_error(xl)}
        del xl, codes, scl

    # ------------------------------------------------ FP8-weight linears (W8A16, W8A8)
    if want("fp8"):
        res += fp8_lines(torch, nv, workloads, to_gpu, dev, args)

    # ------------------------------------------------ offline weight quantize (fp32 in)
    if want("weight"):
        w = torch.from_numpy(workloads.gaussian(3, 1, 17408, 5120, 0.02)).to(dev)

        def wstep(i, mark):
            mark(0)
            nv.nvfp4_quantize(w)
            mark(1)

        _, (w_ms,) = time_steps(torch, max(4, steps // 4), 2, wstep, 1)
        wb = 2 * w.numel() * 4 + w.numel() // 2 + w.numel() // 16
        res.append({"metric": "weight quantize GB/s (fp32 in, two-pass bytes)",
                    "value": round(wb / (mean(w_ms) * 1e-3) / 1e9, 1), "unit": "GB/s",
                    "ms_per_step": round(mean(w_ms), 4),
                    "config": {"workload": "offline weight quantize W[17408x5120] fp32 N(0,0.02)"}})
    return res


PEAK_FP8_TFLOPS = 5000.0       # MI355X dense fp8 MFMA, published


def fp8_lines(torch, nv, workloads, to_gpu, dev, args):
    """W8A16 / W8A8 on FP8 E4M3 weights: decode GB/s (M = 1, 16, weights of the
    fused gate/up shape, 4 rotated copies) and prefill TFLOP/s (M = 4096)."""
    res = []
    steps, warmup = args.steps, args.warmup
    log("FP8 linears: quantizing weights to E4M3")
    d = workloads.decode(M=1)
    w32 = torch.cat([torch.from_numpy(w).to(dev) for w in d.w_parts])
    wq0, sw = nv.nvfp4_fp8_quantize(w32)
    del w32
    R = 4
    copies = [wq0.clone() for _ in range(R)]
    del wq0
    N, K = d.N, d.K
    for M in (1, 16):
        x = to_gpu(workloads.decode(M=M, N_each=1).x)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        nbytes = N * K + M * K * 2 + M * N * 2
        line = {"metric": "FP8-weight decode GB/s at M=%d" % M, "unit": "GB/s",
                "config": {"workload": "decode: X[%dx5120] bf16 x W[34816x5120] E4M3 per-tensor scale "
                                       "(4 rotated copies) -> Y bf16" % M},
                "algorithmic": "W %d B + X + Y = %d B per call" % (N * K, nbytes)}
        for name, fn in (("w8a16", nv.nvfp4_gemm_w8a16), ("w8a8", nv.nvfp4_gemm_w8a8)):
            def st(i, fn=fn, x=x, y=y):
                fn(x, copies[i], sw, out=y)
            ms = graph_step_ms(torch, st, R, y, reps=max(steps, 20))
            gbs = nbytes / (ms * 1e-3) / 1e9
            line[name] = {"ms_per_call": round(ms, 5), "GBs": round(gbs, 1), "frac": round(gbs / PEAK_HBM_GBS, 4),
                          "timing": "graph replay"}
        line["value"] = line["w8a16"]["GBs"]
        res.append(line)
        log("FP8 decode M=%d: W8A16 %.1f GB/s, W8A8 %.1f GB/s" % (M, line["w8a16"]["GBs"], line["w8a8"]["GBs"]))
    del copies
    p = workloads.prefill()
    M, N, K = p.M, p.N, p.K
    w32 = torch.from_numpy(p.w_parts[0]).to(dev)
    wq, sw = nv.nvfp4_fp8_quantize(w32)
    del w32
    x = to_gpu(p.x)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    flops = 2.0 * M * N * K
    line = {"metric": "FP8-weight GEMM TFLOP/s at M=4096", "unit": "TFLOP/s",
            "config": {"workload": "prefill: X[4096x5120] bf16 x W[17408x5120] E4M3 per-tensor scale -> Y bf16; "
                                   "W8A8 includes the dynamic activation quantize"}}
    for name, fn, peak in (("w8a16", nv.nvfp4_gemm_w8a16, PEAK_FP16_TFLOPS),
                           ("w8a8", nv.nvfp4_gemm_w8a8, PEAK_FP8_TFLOPS)):
        def st(i, mark, fn=fn):
            mark(0)
            fn(x, wq, sw, out=y)
            mark(1)
        _, (ms,) = time_steps(torch, steps, warmup, st, 1)
        tf = flops / (mean(ms) * 1e-3) / 1e12
        line[name] = {"ms_per_call": round(mean(ms), 4), "TFLOPs": round(tf, 2), "peak": peak,
                      "frac": round(tf / peak, 4)}
    line["value"] = line["w8a8"]["TFLOPs"]
    res.append(line)
    log("FP8 prefill: W8A16 %.1f TFLOP/s, W8A8 %.1f TFLOP/s" % (line["w8a16"]["TFLOPs"], line["w8a8"]["TFLOPs"]))
    return res


# Paper "Why Gated DeltaNet Survives 4-Bit Quantization", section 5.1, Table 2
# (medians over layers of captured activations; weights near-Gaussian).
PAPER_MEDIANS = {"max_over_rms": 63.5, "kurtosis": 1560, "hot_channel_ratio": 100,
                 "one_hot_block_share": [0.10, 0.32], "a4_rel_error": [0.075, 0.092],
                 "w4_rel_error": [0.105, 0.119]}


def numerics(torch, nv, workloads, to_gpu, dev, p, x, wc, ws, wg):
    """Where the synthetic inputs sit against the paper's statistics, and
    the fake-quantization and GEMM errors they give."""
    from nvfp4_w4a4_quantized_02_amd import stats
    log("numerics: input statistics and fake-quantization errors")
    res = {"paper_medians": PAPER_MEDIANS}
    w32 = torch.from_numpy(p.w_parts[0]).to(dev)
    res["prefill_x"] = {**stats.tensor_stats(x), "a4": stats.fake_quant_error(x)}
    res["prefill_w"] = {**stats.tensor_stats(w32), "w4": stats.fake_quant_error(w32)}
    yref = x.float() @ w32.t()
    y44 = nv.nvfp4_gemm(x, wc, ws, wg, out_dtype=torch.float32)
    y416 = nv.nvfp4_gemm_w4a16(x, wc, ws, wg, out_dtype=torch.float32)
    res["prefill_gemm_rel_error"] = {"w4a4": stats.gemm_error(y44, yref), "w4a16": stats.gemm_error(y416, yref),
                                     "reference": "fp32 X.W^T of the unquantized bf16 X and fp32 W"}
    del yref, y44, y416, w32
    xd = to_gpu(workloads.decode(M=16, N_each=1).x)
    res["decode_x_m16"] = {**stats.tensor_stats(xd), "a4": stats.fake_quant_error(xd)}
    return res


def _read_probe():
    import ctypes
    path = os.path.join(ROOT, "nvfp4_w4a4_quantized_02_amd", "libnvfp4_probe.so")
    if not os.path.exists(path):
        return None
    L = ctypes.CDLL(path)
    L.nvfp4_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_uint32,
                                   ctypes.c_int, ctypes.c_void_p]
    L.nvfp4_probe_read.restype = ctypes.c_int
    return L


def read_rate(torch, dev, nbytes, copies, reps=20):
    """GB/s of a plain streaming read (the reference kernel of
    libnvfp4_probe.so) over `copies` buffers of nbytes read in turn, best of
    five timed rounds; None when the probe library is not built."""
    L = _read_probe()
    if L is None:
        return None, None
    bufs = [torch.full((nbytes // 4,), i + 1, dtype=torch.int32, device=dev) for i in range(copies)]
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    best = {}
    for grid in (1024, 2048, 4096):
        ms = []
        for r in range(6):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for i in range(reps):
                assert L.nvfp4_probe_read(bufs[i % copies].data_ptr(), nbytes, sink.data_ptr(), 0x9E3779B9,
                                          grid, stream) == 0
            e1.record()
            torch.cuda.synchronize()
            if r:
                ms.append(e0.elapsed_time(e1) / reps)
        best[grid] = min(ms)
    del bufs
    grid = min(best, key=best.get)
    return nbytes / (best[grid] * 1e-3) / 1e9, grid


def box_peaks(torch, dev, M, N, K):
    """What this machine sustains on plain work, measured beside the
    nominal peaks: a streaming read of 100 MB (the decode weight size, four
    buffers read in turn so the 256 MB last-level cache cannot hold them) and
    of 1 GiB, a 1 GiB device-to-device copy (HBM read + write) and torch's own
    fp16 GEMM (hipBLASLt) at the prefill shape with fp32 accumulation, the
    same MFMA arithmetic the W4A4 GEMM runs after its exact expansion.
    Context for the roofline fractions, not part of any step."""
    log("box peaks: streaming read 100 MB and 1 GiB, 1 GiB copy, fp16 GEMM %dx%dx%d" % (M, N, K))
    read100, g100 = read_rate(torch, dev, 100 << 20, 4)
    read1g, g1g = read_rate(torch, dev, 1 << 30, 2, reps=5)
    a = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
    b = torch.empty_like(a)
    ms = []
    for i in range(8):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        b.copy_(a)
        e1.record()
        torch.cuda.synchronize()
        if i >= 3:
            ms.append(e0.elapsed_time(e1))
    copy_gbs = 2 * (1 << 30) / (min(ms) * 1e-3) / 1e9
    del a, b
    x = torch.randn(M, K, device=dev, dtype=torch.float16)
    w = torch.randn(N, K, device=dev, dtype=torch.float16)
    ms = []
    for i in range(8):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        torch.mm(x, w.t())
        e1.record()
        torch.cuda.synchronize()
        if i >= 3:
            ms.append(e0.elapsed_time(e1))
    gemm_tf = 2.0 * M * N * K / (min(ms) * 1e-3) / 1e12
    del x, w
    res = {"hbm_copy_GBs": round(copy_gbs, 1),
           "fp16_gemm_TFLOPs": round(gemm_tf, 1),
           "note": "best of 5 timed runs; copy counts read + write bytes; torch fp16 GEMM at the prefill shape; "
                   "reads: a plain streaming-read kernel (libnvfp4_probe.so), best grid of 1024/2048/4096 "
                   "workgroups"}
    if read100 is not None:
        res["hbm_read_GBs"] = round(read100, 1)
        res["hbm_read_100MB_grid"] = g100
        res["hbm_read_1GiB_GBs"] = round(read1g, 1)
    else:
        res["hbm_read_GBs"] = res["hbm_copy_GBs"]
        res["note"] += "; the read probe library is not built, hbm_read_GBs repeats the copy rate"
    log("box peaks: read %s GB/s (100 MB), %s GB/s (1 GiB), copy %.0f GB/s, fp16 GEMM %.0f TFLOP/s" % (
        res.get("hbm_read_GBs"), res.get("hbm_read_1GiB_GBs"), copy_gbs, gemm_tf))
    return res


def _cpu_info():
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    return {"cpu_model": model, "nproc": usable, "os_cpu_count": os.cpu_count()}


def cpu_baseline(np, p):
    """The oracle, untuned, on bounded samples of the benchmark workloads, on
    the host cores: the headline W4A4 linear for the first m rows of X
    against the whole weight (weights quantized beforehand, untimed, as on
    the GPU); the decode GEMV at M = 1 (the oracle spreads rows over its
    threads, so one row runs on one thread); and the long-prefill activation
    quantize on its first rows (the two-pass byte count, as on the GPU)."""
    import oracle
    import workloads
    info = _cpu_info()
    nt = oracle.num_threads()
    log("cpu baseline on %s (%d usable CPUs, %d oracle threads)" % (info["cpu_model"], info["nproc"], nt))
    log("cpu baseline: oracle weight quantize (untimed)")
    wc, ws, wg = oracle.quantize(p.w_parts[0])
    N, K = p.N, p.K
    t0 = time.perf_counter()
    oracle.linear(np.ascontiguousarray(p.x[:1]), wc, ws, wg)
    t1 = time.perf_counter() - t0
    # The oracle spreads rows over its threads, one row per thread at a time:
    # a whole number of rows per thread keeps every thread busy for ~15 s.
    rounds = int(max(1, round(15.0 / max(t1, 1e-3))))
    m = int(min(p.M, nt * rounds))
    log("cpu baseline: 1 row took %.2f s, timing %d rows on %d threads" % (t1, m, nt))
    t0 = time.perf_counter()
    oracle.linear(np.ascontiguousarray(p.x[:m]), wc, ws, wg)
    dt = time.perf_counter() - t0
    flops = 2.0 * m * N * K
    del wc, ws
    res = {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": min(nt, m),
           "kind": "oracle", "seconds": round(dt, 2), **info,
           "sample": "W4A4 linear of the first %d of 4096 activation rows (on-the-fly quantize of those rows "
                     "+ exact int64 GEMM) against the full W[17408x5120]" % m}

    # decode GEMV, M = 1: one row against the fused gate/up weight
    d = workloads.decode(M=1)
    gss = [oracle.tensor_scale(w) for w in d.w_parts]
    q = [oracle.quantize(w, gs=g) for w, g in zip(d.w_parts, gss)]
    scales, S = oracle.fuse_rescale([s for _, s, _ in q], gss)
    dwc = np.concatenate([c for c, _, _ in q])
    dws = np.concatenate(scales)
    del q
    t0 = time.perf_counter()
    oracle.linear(d.x, dwc, dws, S)
    dt = time.perf_counter() - t0
    nbytes = dwc.nbytes + dws.nbytes + d.x.nbytes + dwc.shape[0] * 2
    res["decode_gemv_m1"] = {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1,
                             "seconds": round(dt, 2),
                             "sample": "decode W4A4 linear X[1x5120] x fused W[34816x5120] (whole call)"}
    del dwc, dws

    # long-prefill quantize on the first rows, sized for ~5 s
    # (the generator gives the same first rows whatever the row count)
    rows = 256
    t0 = time.perf_counter()
    oracle.quantize(workloads.long_prefill_activations(M=rows))
    t1 = time.perf_counter() - t0
    rows = int(min(32768, max(rows, rows * 5.0 / max(t1, 1e-3))))
    xs = workloads.long_prefill_activations(M=rows)
    t0 = time.perf_counter()
    oracle.quantize(xs)
    dt = time.perf_counter() - t0
    two_pass = 2 * xs.nbytes + xs.size // 2 + xs.size // 16
    res["quantize_long_prefill"] = {"value": round(two_pass / dt / 1e9, 4), "unit": "GB/s",
                                    "cores": min(nt, rows), "seconds": round(dt, 2),
                                    "sample": "NVFP4 quantize of the first %d of 32768 long-prefill rows "
                                              "(two-pass byte count)" % rows}
    log("cpu baseline: GEMM %.2e TFLOP/s, decode GEMV %.3f GB/s, quantize %.3f GB/s" % (
        res["value"], res["decode_gemv_m1"]["value"], res["quantize_long_prefill"]["value"]))
    return res


if __name__ == "__main__":
    main()
