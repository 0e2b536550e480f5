#!/usr/bin/env python3
"""Benchmark of the block-scaled FP8 hot path on one MI355X.

Default (the one JSON line on stdout):
    python bench.py [--steps K] [--warmup W]
A step is one pass of the FP8 block_scaled_mm path at m = n = k = 4096,
group_n = group_k = 128: quantize the float32 activations (1 x 128 blocks,
E4M3 + float32 scales), quantize the float32 weights (128 x 128 tiles), then
the block-scaled GEMM with its fused float32 epilogue.  Inputs are resident
in HBM before timing; four input sets are rotated so that the 256 MB
last-level cache cannot serve the quantizers' reads.  After settling steps
(the clocks of an idle GPU ramp up over the first ~150 steps) and the W
warm-up steps, K plain steps give `value`: the GEMM's algorithmic 2 m n k
FLOPs per step time (TFLOP/s).  The GEMM kernel's roofline comes from K
back-to-back launches of it on the step's inputs, bracketed by HIP events
on the launch stream; a second pass of K steps whose GEMM launches carry
attached HIP events is reported beside it (those events also hold the
dispatch of the GEMM's workgroups).  The JSON line also carries the CPU
oracle timed on a bounded sample on this host.

    python bench.py --suite [--out FILE]
times every kernel of the path at its own workload (quantizers, FP8 GEMM
sweep, INT8 per-channel, MXFP8 batched, MXFP8 backward) and writes one JSON
object per kernel to FILE (default bench_out/suite.jsonl).

    python bench.py --sweep [--out FILE]
runs the GEMM on every row of the block_scaled_mm page's shape table.

    python bench.py --operand-sweep [--steps K] [--warmup W] [--out FILE]
times the 4096^3 GEMM on operands of different value patterns (the recipe's
codes, uniform random codes, zeros, a constant, mostly zeros): same
instructions, different clock.

One GPU only: --gpus N with N > 1 exits with a message.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "TFLOP/s & % of FP8 MFMA peak, block-scaled GEMM m=n=k=4096 group 128"
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense FP8 MFMA
SETTLE_STEPS = 400            # untimed steps before the warm-up (clock ramp of an idle GPU)
PEAK_INT8_TOPS = 5000.0       # MI355X dense INT8 MFMA
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense BF16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
# block_scaled_mm row 14 (m = n = k = 4096): T_Prod = 1.06 ms on unstated
# hardware, i.e. 2 * 4096^3 / 1.06 ms = 129.66 TFLOP/s (GEMM only).
PAGE_T_PROD_TFLOPS_4096 = 2 * 4096 ** 3 / 1.06e-3 / 1e12
GEMM_SRC = os.path.join(ROOT, "block_scaled_precision_blockwise_amd", "csrc", "gemm.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_fp8_4096_traffic.json")
DEFAULT_SUITE_OUT = os.path.join(ROOT, "bench_out", "suite.jsonl")


def _log(*a):
    print(*a, file=sys.stderr, flush=True)


def _code_text(src: str) -> str:
    """C++ source without its comments, whitespace runs collapsed to one
    space: what the compiler reads, so that editing a comment does not
    change it.  String and character literals are kept as they are."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c == "/" and src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif c == "/" and src.startswith("/*", i):
            j = src.find("*/", i + 2)
            out.append(" ")
            i = n if j < 0 else j + 2
        elif c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def _code_hash(path):
    """sha256 (first 16 hex digits) of a source file's code without comments."""
    with open(path, encoding="utf-8") as f:
        return hashlib.sha256(_code_text(f.read()).encode()).hexdigest()[:16]


def _gpu_setup():
    import torch
    import block_scaled_precision_blockwise_amd as bsq

    if not bsq.is_built():
        import __graft_entry__
        __graft_entry__.build()
    torch.cuda.set_device(0)
    bsq.bsq_device_check()
    return torch, bsq


def _hip_runtime():
    """The HIP runtime this process already uses (torch's copy, which libbsq
    shares through the same soname), opened by its path so that no second
    copy is loaded."""
    import ctypes
    path = None
    with open("/proc/self/maps") as f:
        for line in f:
            if "libamdhip64" in line:
                path = line.split()[-1]
                break
    if path is None:
        raise RuntimeError("the HIP runtime is not loaded in this process")
    hip = ctypes.CDLL(path)
    hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
    hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return hip


class KernelTimer:
    """Per-launch HIP events for the GEMM kernel, recorded by the kernel's
    own dispatch: before each timed GEMM call the library is asked
    (bsq_time_next_gemm) to launch its next GEMM kernel with
    hipExtLaunchKernel and these two events, which then hold that kernel's
    start and end on the stream it runs on.  No marker packet sits between
    the kernels.  The pair starts when the GEMM's dispatch begins, after
    the quantizer before it has finished, so it also covers the launch of
    the GEMM's workgroups: it reads about 5 us (7 %) above the kernel
    trace's duration of the same launches, and a step whose GEMM carries
    the events takes about 5 us longer than one without.  (Events recorded
    around the call with hipEventRecord added a marker packet and a
    dispatch gap of their own to every step.)"""

    def __init__(self, torch, launches):
        import ctypes
        self.ct = ctypes
        self.hip = _hip_runtime()
        self.events = []
        for _ in range(2 * launches):
            ev = ctypes.c_void_p()
            rc = self.hip.hipEventCreateWithFlags(ctypes.byref(ev), 0)
            if rc != 0:
                raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
            self.events.append(ev)
        self.used = 0

    def around(self, fn):
        import block_scaled_precision_blockwise_amd as bsq
        s, e = self.events[self.used], self.events[self.used + 1]
        self.used += 2
        bsq.bsq_time_next_gemm(s.value, e.value)
        fn()

    def mean_ms(self):
        total = 0.0
        n = self.used // 2
        for i in range(n):
            s, e = self.events[2 * i], self.events[2 * i + 1]
            if self.hip.hipEventSynchronize(e) != 0:
                raise RuntimeError("hipEventSynchronize failed")
            ms = self.ct.c_float()
            if self.hip.hipEventElapsedTime(self.ct.byref(ms), s, e) != 0:
                raise RuntimeError("hipEventElapsedTime failed")
            total += ms.value
        for ev in self.events:
            self.hip.hipEventDestroy(ev)
        self.events = []
        return total / max(n, 1)


def _queue_ahead(torch):
    """Occupy the stream with torch's spin kernel (a few milliseconds) so
    that the host has queued every launch of a timed batch before the GPU
    reaches the batch: the events then see the kernels back to back, not
    the host's per-call cost (about 8 us per binding call, more than a
    short quantizer takes)."""
    torch.cuda._sleep(10_000_000)


# --------------------------------------------------------------- main ----

def run_main(args):
    torch, bsq = _gpu_setup()
    import numpy as np
    import synth

    M = N = K = 4096
    dev = torch.device("cuda:0")
    _log(f"[bench] main step: quant 1x128 + quant 128x128 + GEMM at {M}x{N}x{K}")
    sets = []
    for i in range(4):
        a32, b32 = synth.fp8_blockwise_raw(M, N, K, 204 + 2 * i, 205 + 2 * i)
        sets.append((torch.from_numpy(a32).to(dev), torch.from_numpy(b32).to(dev)))
    aq = torch.empty(M, K, dtype=torch.uint8, device=dev)
    bq = torch.empty(N, K, dtype=torch.uint8, device=dev)
    sa = torch.empty(M, K // 128, dtype=torch.float32, device=dev)
    sb = torch.empty(N // 128, K // 128, dtype=torch.float32, device=dev)
    y = torch.empty(M, N, dtype=torch.float32, device=dev)
    gemm_t = KernelTimer(torch, args.steps)

    def step(i, timed):
        a, b = sets[i % len(sets)]
        bsq.bsq_quant_fp8_rowblock(a, aq, sa, 128)
        bsq.bsq_quant_fp8_tile(b, bq, sb, 128, 128)
        if timed:
            gemm_t.around(lambda: bsq.bsq_blockwise_fp8_matmul(aq, bq, sa, sb, y))
        else:
            bsq.bsq_blockwise_fp8_matmul(aq, bq, sa, sb, y)

    def timed_steps(with_events):
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for i in range(args.steps):
            step(i, with_events)
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / args.steps

    # A GPU that has been idle runs its first ~150 steps about 10 % slower
    # while its clocks rise; SETTLE_STEPS untimed steps come before the W
    # warm-up steps so that neither timed pass sees that ramp.
    for i in range(SETTLE_STEPS):
        step(i, False)
    for i in range(args.warmup):
        step(i, False)
    # value: K steps exactly as a caller runs them.  The GEMM's attached
    # events add about 5 us per step (the dispatch that records them waits
    # longer to start), so the per-launch GEMM duration comes from a second
    # pass of K steps whose GEMM launches carry them.
    ms = timed_steps(False)
    ms_events = timed_steps(True)
    flops = 2.0 * M * N * K
    value = flops / (ms * 1e-3) / 1e12
    attached_ms = gemm_t.mean_ms()

    # The GEMM kernel's own launch duration: K launches back to back on the
    # step's last inputs, bracketed by two events on the launch stream (the
    # binding launches on torch's current stream).  Back to back, each
    # dispatch starts as the previous kernel ends, so the mean is the
    # kernel's duration (the pair attached to each in-step launch above also
    # holds the dispatch of the GEMM's workgroups after the quantizer).
    def gemm_back_to_back():
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            bsq.bsq_blockwise_fp8_matmul(aq, bq, sa, sb, y)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    gemm_ms = gemm_back_to_back()
    gemm_tflops = flops / (gemm_ms * 1e-3) / 1e12
    _log(f"[bench] step {ms * 1e3:.1f} us -> {value:.1f} TFLOP/s (with attached GEMM events {ms_events * 1e3:.1f} us); "
         f"GEMM {gemm_ms * 1e3:.1f} us back to back -> {gemm_tflops:.1f} TFLOP/s "
         f"({100 * gemm_tflops / PEAK_FP8_TFLOPS:.1f}% of FP8 peak); attached in-step events {attached_ms * 1e3:.1f} us")

    traffic = None
    try:
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if tr.get("gemm_code_sha256_16") == _code_hash(GEMM_SRC):
            traffic = tr.get("bytes_per_launch")
    except (OSError, ValueError):
        traffic = None

    if args.calibrate_copy:
        # a plain device copy of known size, for scaling the HBM byte counters
        nbytes = 512 << 20
        src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        _log(f"[bench] calibration copy: 5 x {nbytes} bytes read and written")
    cpu = None if args.no_cpu_baseline else cpu_baseline()
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_steps": SETTLE_STEPS,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(value / PAGE_T_PROD_TFLOPS_4096, 3),
        "vs_baseline_ref": "block_scaled_mm row 14 T_Prod 1.06 ms (GEMM only, unstated hardware) = "
                           f"{PAGE_T_PROD_TFLOPS_4096:.1f} TFLOP/s; our value includes both quantizers",
        "dtype": "e4m3",
        "data": "synthetic",
        "pct_of_fp8_peak": round(100 * value / PEAK_FP8_TFLOPS, 2),
        "config": {
            "workload": "block_scaled_mm FP8 e4m3, m=n=k=4096, group_n=group_k=128, fp32 out; "
                        "step = 1x128 activation quant + 128x128 weight quant + GEMM",
            "m": M, "n": N, "k": K, "group_n": 128, "group_k": 128,
            "inputs": "randn float32 (PCG64 seeds 204..211), 4 rotating sets",
        },
        "roofline": {
            "kernel": "k_gemm<FP8G> (block-scaled GEMM, fused fp32 epilogue)",
            "bound": "mfma",
            "achieved": round(gemm_tflops, 2),
            "peak": PEAK_FP8_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(gemm_tflops / PEAK_FP8_TFLOPS, 4),
            "traffic": traffic,
            "avg_launch_us": round(gemm_ms * 1e3, 2),
            "timed_by": "HIP events on the launch stream around K back-to-back GEMM launches on the "
                        "step's inputs",
            "in_step_attached_event_us": round(attached_ms * 1e3, 2),
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(runs: int = 3):
    """The oracle as written, on one whole step of the same workload: both
    quantizers, then the oracle GEMM (its float64 product and its
    error-bound product), with the BLAS thread pool set to the cores this
    process may run on (its affinity mask, capped by OMP_NUM_THREADS).  The median of `runs` runs (about 4 s each on 16
    cores) is reported as TFLOP/s on the GEMM's 2 m n k."""
    import numpy as np
    import synth
    from oracle import matmul as OM
    from oracle import quantize as OQ

    affinity = len(os.sched_getaffinity(0))
    # the host's share for this process: its affinity mask, capped by the
    # thread count the environment grants (a shared GPU host may show more
    # CPUs than one job may use)
    want = affinity
    try:
        want = min(want, int(os.environ.get("OMP_NUM_THREADS", affinity)))
    except ValueError:
        pass
    limit = None
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        limit = threadpool_limits(limits=want, user_api="blas")
        threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"]
                      or [want])
    except Exception:
        threads = want
    M = N = K = 4096
    rows = 4096
    a32, b32 = synth.fp8_blockwise_raw(M, N, K, 204, 205)
    _log(f"[bench] cpu baseline: oracle on {rows} of {M} rows, {runs} runs, {threads} BLAS threads ...")
    times = []
    try:
        for r in range(runs):
            t0 = time.perf_counter()
            a, sa = OQ.fp8_rowblock(a32[:rows])
            b, sb = OQ.fp8_tile(b32)
            y, T = OM.blockwise_fp8(a, b, sa, sb)
            times.append(time.perf_counter() - t0)
            _log(f"[bench] cpu baseline run {r}: {times[-1]:.2f} s")
    finally:
        if limit is not None:
            limit.restore_original_limits()
    dt = sorted(times)[len(times) // 2]
    flops = 2.0 * rows * N * K
    _log(f"[bench] cpu baseline: median {dt:.2f} s -> {flops / dt / 1e12:.5f} TFLOP/s")
    return {
        "value": round(flops / dt / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"one full step ({rows}x4096x4096): oracle 1x128 and 128x128 quantizers + float64 "
                  f"blockwise GEMM with its error-bound GEMM; median of {runs} runs",
        "seconds": round(dt, 3),
        "runs_s": [round(t, 3) for t in times],
        "affinity_cpus": affinity,
        "cpu_model": _cpu_model(),
    }


# --------------------------------------------------------------- suite ---

def run_suite(args):
    torch, bsq = _gpu_setup()
    import numpy as np
    import synth

    dev = torch.device("cuda:0")
    out_path = args.out
    os.makedirs(os.path.dirname(os.path.abspath(out_path)), exist_ok=True)
    rows = []

    last = {}

    def time_launches(fn, n_iter, rotate=1, reps=20):
        """Median over `reps` batches of the per-launch time of a batch of
        n_iter back-to-back launches (the minimum is kept for the row)."""
        for i in range(3):
            fn(i % rotate)
        torch.cuda.synchronize()
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        per = []
        for r in range(reps):
            _queue_ahead(torch)
            s.record()
            for i in range(n_iter):
                fn((r * n_iter + i) % rotate)
            e.record()
            torch.cuda.synchronize()
            per.append(s.elapsed_time(e) / n_iter)
        per.sort()
        last["min_ms"] = per[0]
        last["launches"] = reps * n_iter
        return per[len(per) // 2]  # ms

    def emit(row):
        rows.append(row)
        _log("[suite] " + json.dumps(row))
        with open(out_path, "a") as f:
            f.write(json.dumps(row) + "\n")

    def hbm_row(name, workload, ms, nbytes):
        gbs = nbytes / (ms * 1e-3) / 1e9
        emit({"kernel": name, "workload": workload, "us": round(ms * 1e3, 2),
              "us_min": round(last["min_ms"] * 1e3, 2), "launches": last["launches"], "bytes": int(nbytes),
              "GB/s": round(gbs, 1), "pct_hbm": round(100 * gbs / PEAK_HBM_GBS, 1)})

    def mfma_row(name, workload, ms, flops, peak, nbytes=None):
        tf = flops / (ms * 1e-3) / 1e12
        row = {"kernel": name, "workload": workload, "us": round(ms * 1e3, 2),
               "us_min": round(last["min_ms"] * 1e3, 2), "launches": last["launches"], "flops": flops,
               "TFLOP/s": round(tf, 1), "pct_peak": round(100 * tf / peak, 1)}
        if nbytes is not None:
            # roofline of the shape: the MFMA peak or HBM at its arithmetic intensity
            roof = min(peak, flops / nbytes * PEAK_HBM_GBS / 1e3)
            row["bound"] = "mfma" if roof >= peak else "hbm"
            row["pct_roofline"] = round(100 * tf / roof, 1)
        emit(row)

    open(out_path, "w").close()
    # ---- FP8 quantizers (rotating 8 input sets of 64 MB so the 256 MB cache cannot serve them)
    for (R, C) in [(4096, 4096)]:
        xs = [torch.randn(R, C, device=dev) for _ in range(8)]
        codes = torch.empty(R, C, dtype=torch.uint8, device=dev)
        sc = torch.empty(R, C // 128, dtype=torch.float32, device=dev)
        ms = time_launches(lambda i: bsq.bsq_quant_fp8_rowblock(xs[i], codes, sc, 128), 40, 8)
        hbm_row("quant_fp8_rowblock 1x128", f"{R}x{C} f32", ms, R * C * 5 + R * C // 128 * 4)
        st = torch.empty(R // 128, C // 128, dtype=torch.float32, device=dev)
        ms = time_launches(lambda i: bsq.bsq_quant_fp8_tile(xs[i], codes, st, 128, 128), 40, 8)
        hbm_row("quant_fp8_tile 128x128", f"{R}x{C} f32", ms, R * C * 5 + st.numel() * 4)
        del codes, sc, st, xs
    # the large forward's activation (1 GiB of fp32: larger than the cache by itself)
    for (R, C) in [(65536, 4096)]:
        xl = torch.randn(R, C, device=dev)
        codes = torch.empty(R, C, dtype=torch.uint8, device=dev)
        sc = torch.empty(R, C // 128, dtype=torch.float32, device=dev)
        ms = time_launches(lambda i: bsq.bsq_quant_fp8_rowblock(xl, codes, sc, 128), 10)
        hbm_row("quant_fp8_rowblock 1x128", f"{R}x{C} f32 (large forward activation)", ms, R * C * 5 + R * C // 128 * 4)
        del xl, codes, sc
    # ---- FP8 GEMM sweep
    for (M, N, K) in [(256, 512, 512)] + list(synth.FP8_SWEEP) + [(65536, 4096, 4096)]:
        a = torch.randint(0, 126, (M, K), dtype=torch.uint8, device=dev)
        b = torch.randint(0, 126, (N, K), dtype=torch.uint8, device=dev)
        sa = torch.rand(M, K // 128, device=dev)
        sb = torch.rand(N // 128, K // 128, device=dev)
        y = torch.empty(M, N, dtype=torch.float32, device=dev)
        n_it = 20 if M * N * K < 2 ** 38 else 5
        ms = time_launches(lambda i: bsq.bsq_blockwise_fp8_matmul(a, b, sa, sb, y), n_it)
        mfma_row("gemm_fp8_blockwise", f"{M}x{N}x{K} g128 f32 out", ms, 2 * M * N * K, PEAK_FP8_TFLOPS,
                 M * K + N * K + (M + N // 128) * (K // 128) * 4 + M * N * 4)
        del a, b, sa, sb, y
    # ---- the other sweep shapes cold: as many operand sets as exceed
    # 540 MB (more than twice the 256 MB cache), rotated, so no launch finds
    # its operands cached
    for (M, N, K) in synth.FP8_SWEEP:
        if (M, N, K) == (4096, 4096, 4096):
            continue  # its own cold row follows
        per_set = M * K + N * K + (M + N // 128) * (K // 128) * 4
        n_sets = min(128, -(-540_000_000 // per_set))
        ops = [(torch.randint(0, 126, (M, K), dtype=torch.uint8, device=dev),
                torch.randint(0, 126, (N, K), dtype=torch.uint8, device=dev),
                torch.rand(M, K // 128, device=dev), torch.rand(N // 128, K // 128, device=dev))
               for _ in range(n_sets)]
        y = torch.empty(M, N, dtype=torch.float32, device=dev)
        ms = time_launches(lambda i: bsq.bsq_blockwise_fp8_matmul(*ops[i], y), n_sets, n_sets)
        mfma_row("gemm_fp8_blockwise (cold operands)", f"{M}x{N}x{K} g128 f32 out, {n_sets} rotating operand sets",
                 ms, 2 * M * N * K, PEAK_FP8_TFLOPS, per_set + M * N * 4)
        del ops, y
    # ---- the same GEMM cold: 16 operand sets (512 MiB of codes) rotated, so
    # the 256 MB cache cannot hold the operands between launches
    M = N = K = 4096
    ops = [(torch.randint(0, 126, (M, K), dtype=torch.uint8, device=dev),
            torch.randint(0, 126, (N, K), dtype=torch.uint8, device=dev),
            torch.rand(M, K // 128, device=dev), torch.rand(N // 128, K // 128, device=dev)) for _ in range(16)]
    y = torch.empty(M, N, dtype=torch.float32, device=dev)
    ms = time_launches(lambda i: bsq.bsq_blockwise_fp8_matmul(*ops[i], y), 16, 16)
    mfma_row("gemm_fp8_blockwise (cold operands)", f"{M}x{N}x{K} g128 f32 out, 16 rotating operand sets", ms,
             2 * M * N * K, PEAK_FP8_TFLOPS)
    del ops, y
    # ---- general groups (the same kernel, general scale indexing)
    M = N = K = 4096
    a = torch.randint(0, 126, (M, K), dtype=torch.uint8, device=dev)
    b = torch.randint(0, 126, (N, K), dtype=torch.uint8, device=dev)
    y = torch.empty(M, N, dtype=torch.float32, device=dev)
    for gn, gk in ((128, 256), (64, 128), (128, 64)):
        sa = torch.rand(M, K // gk, device=dev)
        sb = torch.rand(N // gn, K // gk, device=dev)
        ms = time_launches(lambda i: bsq.bsq_blockwise_fp8_matmul(a, b, sa, sb, y, group_n=gn, group_k=gk), 20)
        mfma_row("gemm_fp8_blockwise", f"{M}x{N}x{K} group_n {gn} group_k {gk} f32 out", ms, 2 * M * N * K,
                 PEAK_FP8_TFLOPS)
    del a, b, sa, sb, y
    # ---- nvfp4 scaled_matmul (dequantize to bf16 + bf16 matrix core)
    Bt, M, N, K = 1, 4096, 4096, 4096
    a = torch.randint(0, 256, (Bt, M, K // 2), dtype=torch.uint8, device=dev)
    b = torch.randint(0, 256, (Bt, N, K // 2), dtype=torch.uint8, device=dev)
    sa = torch.randint(0x20, 0x50, (Bt, M, K // 16), dtype=torch.uint8, device=dev)
    sb = torch.randint(0x20, 0x50, (Bt, N, K // 16), dtype=torch.uint8, device=dev)
    y = torch.empty(Bt, M, N, dtype=torch.float32, device=dev)
    wsn = torch.empty(bsq.bsq_nvfp4_workspace_bytes(Bt, M, N, K), dtype=torch.uint8, device=dev)
    ms = time_launches(lambda i: bsq.bsq_scaled_matmul_nvfp4(a, b, sa, sb, y, wsn), 20)
    mfma_row("scaled_matmul_nvfp4 (dequantize + bf16 GEMM)", f"{M}x{N}x{K} e2m1 e4m3/16 f32 out", ms,
             2 * M * N * K, PEAK_BF16_TFLOPS)
    del a, b, sa, sb, y, wsn
    # ---- INT8 per-channel
    B, Din, Dout = 2048, 4096, 4096
    # input sets rotated through more than 512 MB, as for the fp8 quantizers
    xsets = [torch.randn(B, Din, device=dev) for _ in range(16)]
    wsets = [0.02 * torch.randn(Din, Dout, device=dev) for _ in range(8)]
    xq = torch.empty(B, Din, dtype=torch.int8, device=dev)
    xsc = torch.empty(B, device=dev)
    wq = torch.empty(Din, Dout, dtype=torch.int8, device=dev)
    wsc = torch.empty(Dout, device=dev)
    wqT = torch.empty(Dout, Din, dtype=torch.int8, device=dev)
    yi = torch.empty(B, Dout, device=dev)
    ms = time_launches(lambda i: bsq.bsq_int8_quant_rows(xsets[i], xq, xsc), 48, 16)
    hbm_row("int8_quant_rows", f"{B}x{Din} f32", ms, B * Din * 5 + B * 4)
    ms = time_launches(lambda i: bsq.bsq_int8_quant_cols(wsets[i], wq, wsc, None), 40, 8)
    hbm_row("int8_quant_cols", f"{Din}x{Dout} f32 (w_q only)", ms, Din * Dout * 5 + Dout * 4)
    ms = time_launches(lambda i: bsq.bsq_int8_quant_cols(wsets[i], wq, wsc, wqT), 40, 8)
    hbm_row("int8_quant_cols+T", f"{Din}x{Dout} f32 (w_q and w_qT)", ms, Din * Dout * 6 + Dout * 4)
    ms = time_launches(lambda i: bsq.bsq_int8_matmul(xq, wqT, xsc, wsc, yi), 20)
    mfma_row("gemm_int8", f"{B}x{Dout}x{Din} i32 acc, f32 epilogue", ms, 2 * B * Din * Dout, PEAK_INT8_TOPS)
    # the whole problem: both quantizers and the GEMM
    wk = torch.empty(max(bsq.bsq_int8_workspace_bytes(Din, Dout), 16), dtype=torch.uint8, device=dev)
    ms = time_launches(lambda i: bsq.bsq_int8_per_channel_matmul(xsets[i], wsets[i % 8], wq, wsc, xq, xsc, yi, wk),
                       32, 16)
    mfma_row("int8_per_channel (quantize x and w, GEMM)", f"{B}x{Dout}x{Din}", ms, 2 * B * Din * Dout,
             PEAK_INT8_TOPS)
    del wk
    del xsets, wsets, xq, wq, wqT, yi
    # ---- MXFP8 batched scaled_matmul
    Bt, M, N, K = 8, 2048, 2048, 4096
    lhs32 = torch.randn(Bt * M, K, device=dev)
    lq = torch.empty(Bt * M, K, dtype=torch.uint8, device=dev)
    ls = torch.empty(Bt * M, K // 32, dtype=torch.uint8, device=dev)
    ms = time_launches(lambda i: bsq.bsq_quant_mx(lhs32, lq, ls, axis=1, code_dtype=bsq.BSQ_E4M3), 20)
    hbm_row("quant_mx rows e4m3", f"{Bt * M}x{K} f32", ms, Bt * M * K * 5 + Bt * M * K // 32)
    rq = lq.clone()
    sa = torch.randint(124, 131, (Bt, M, K // 32), dtype=torch.uint8, device=dev)
    sb = torch.randint(124, 131, (Bt, N, K // 32), dtype=torch.uint8, device=dev)
    ym = torch.empty(Bt, M, N, device=dev)
    ms = time_launches(lambda i: bsq.bsq_scaled_matmul(lq.view(Bt, M, K), rq.view(Bt, N, K), sa, sb, ym,
                                                       lhs_dtype=bsq.BSQ_E4M3, rhs_dtype=bsq.BSQ_E4M3,
                                                       scale_dtype=bsq.BSQ_E8M0), 10)
    mfma_row("gemm_mx_batched", f"B={Bt} {M}x{N}x{K} e4m3 e8m0/32 f32 out", ms, 2 * Bt * M * N * K,
             PEAK_FP8_TFLOPS)
    sa64 = torch.randint(124, 131, (Bt, M, K // 64), dtype=torch.uint8, device=dev)
    sb64 = torch.randint(124, 131, (Bt, N, K // 64), dtype=torch.uint8, device=dev)
    ms = time_launches(lambda i: bsq.bsq_scaled_matmul(lq.view(Bt, M, K), rq.view(Bt, N, K), sa64, sb64, ym,
                                                       lhs_dtype=bsq.BSQ_E4M3, rhs_dtype=bsq.BSQ_E4M3,
                                                       scale_dtype=bsq.BSQ_E8M0), 10)
    mfma_row("gemm_mx_batched", f"B={Bt} {M}x{N}x{K} e4m3 e8m0/64 f32 out", ms, 2 * Bt * M * N * K,
             PEAK_FP8_TFLOPS)
    sa16 = torch.randint(124, 131, (Bt, M, K // 16), dtype=torch.uint8, device=dev)
    sb16 = torch.randint(124, 131, (Bt, N, K // 16), dtype=torch.uint8, device=dev)
    ms = time_launches(lambda i: bsq.bsq_scaled_matmul(lq.view(Bt, M, K), rq.view(Bt, N, K), sa16, sb16, ym,
                                                       lhs_dtype=bsq.BSQ_E4M3, rhs_dtype=bsq.BSQ_E4M3,
                                                       scale_dtype=bsq.BSQ_E8M0), 10)
    mfma_row("gemm_mx_batched", f"B={Bt} {M}x{N}x{K} e4m3 e8m0/16 f32 out (two products per step)", ms,
             2 * Bt * M * N * K, PEAK_FP8_TFLOPS)
    del sa16, sb16
    del lhs32, ls
    # cold: 4 operand sets (512 MiB of codes) rotated
    mops = [(lq.view(Bt, M, K), rq.view(Bt, N, K))] + [
        (torch.randint(0, 126, (Bt, M, K), dtype=torch.uint8, device=dev),
         torch.randint(0, 126, (Bt, N, K), dtype=torch.uint8, device=dev)) for _ in range(3)]
    ms = time_launches(lambda i: bsq.bsq_scaled_matmul(mops[i][0], mops[i][1], sa, sb, ym,
                                                       lhs_dtype=bsq.BSQ_E4M3, rhs_dtype=bsq.BSQ_E4M3,
                                                       scale_dtype=bsq.BSQ_E8M0), 8, 4)
    mfma_row("gemm_mx_batched (cold operands)", f"B={Bt} {M}x{N}x{K} e4m3 e8m0/32 f32 out, 4 rotating operand sets",
             ms, 2 * Bt * M * N * K, PEAK_FP8_TFLOPS)
    del mops, lq, rq, ym
    # ---- MXFP8 backward
    M, N, K = 8192, 4096, 4096
    dY = torch.randn(M, N, device=dev).to(torch.bfloat16)
    W = torch.randn(N, K, device=dev).to(torch.bfloat16)
    X = torch.randn(M, K, device=dev).to(torch.bfloat16)
    dX = torch.empty(M, K, dtype=torch.bfloat16, device=dev)
    dW = torch.empty(N, K, dtype=torch.bfloat16, device=dev)
    wsb = torch.empty(bsq.bsq_mxfp8_backward_workspace_bytes(M, N, K), dtype=torch.uint8, device=dev)
    ms = time_launches(lambda i: bsq.bsq_mxfp8_backward(dY, W, X, dX, dW, wsb), 10)
    mfma_row("mxfp8_backward (4 quant + 2 GEMM)", f"dY {M}x{N}, W {N}x{K}, X {M}x{K} e5m2 bf16 out", ms,
             2 * 2 * M * N * K, PEAK_FP8_TFLOPS)
    # the same backward with its four operands already quantized (the page's
    # pre-computed scales): only the two products
    shp = bsq.mxfp8_backward_operand_shapes(M, N, K)
    ops = {n: (torch.empty(c, dtype=torch.uint8, device=dev), torch.empty(sc, dtype=torch.uint8, device=dev))
           for n, (c, sc) in shp.items()}
    bsq.bsq_mxfp8_backward_quantize(M, N, K, dY=dY, W=W, X=X, **ops)
    ms = time_launches(lambda i: bsq.bsq_mxfp8_backward_gemms(M, N, K, dX=dX, dW=dW, **ops), 10)
    mfma_row("mxfp8_backward, pre-quantized (2 GEMM)", f"dY {M}x{N}, W {N}x{K}, X {M}x{K} e5m2 bf16 out", ms,
             2 * 2 * M * N * K, PEAK_FP8_TFLOPS)
    del ops
    codes = torch.empty(N, M, dtype=torch.uint8, device=dev)
    scs = torch.empty(N, M // 32, dtype=torch.uint8, device=dev)
    # 8 rotating dY of 67 MB: more than 512 MB, so the cache cannot serve them
    dys = [dY] + [torch.randn(M, N, device=dev).to(torch.bfloat16) for _ in range(7)]
    ms = time_launches(lambda i: bsq.bsq_quant_mx(dys[i], codes, scs, axis=0, code_dtype=bsq.BSQ_E5M2), 24, 8)
    hbm_row("quant_mx cols^T e5m2", f"{M}x{N} bf16", ms, M * N * 3 + M * N // 32)
    # dY in both orientations (the backward's dX and dW operands) in one pass
    codes_n = torch.empty(M, N, dtype=torch.uint8, device=dev)
    scs_n = torch.empty(M, N // 32, dtype=torch.uint8, device=dev)
    ms = time_launches(lambda i: bsq.bsq_mxfp8_backward_quantize(M, N, K, dY=dys[i], dyn=(codes_n, scs_n),
                                                                 dyt=(codes, scs)), 24, 8)
    hbm_row("quant_mx dY rows + cols^T, one pass, e5m2", f"{M}x{N} bf16", ms, M * N * 4 + M * N // 16)
    _log(f"[suite] wrote {len(rows)} rows to {out_path}")


# The block_scaled_mm page's shape table ("Shapes"): m, n, k (group 128 x
# 128), and its T_SOL (XPU-A) and T_Prod in microseconds - another
# machine's figures, quoted beside ours as context.
PAGE_SWEEP = [
    (349, 2048, 2048, 6.36, 61.80), (1024, 2048, 2048, 18.67, 73.90),
    (4533, 2048, 2048, 82.66, 300.00), (6918, 2048, 2048, 126.15, 440.40),
    (20480, 2048, 2048, 373.46, 1240.0), (51200, 2048, 2048, 933.65, 3100.0),
    (65536, 2048, 2048, 1200.0, 3970.0), (98304, 2048, 2048, 1790.0, 5930.0),
    (118784, 2048, 2048, 2170.0, 7180.0), (250880, 2048, 2048, 4570.0, 15130.0),
    (516096, 2048, 2048, 9410.0, 31140.0), (704512, 2048, 2048, 12850.0, 42520.0),
    (237, 4096, 4096, 17.29, 118.30), (3072, 4096, 4096, 224.10, 801.90),
    (4096, 4096, 4096, 298.80, 1060.0), (8192, 4096, 4096, 597.60, 2090.0),
    (16384, 4096, 4096, 1200.0, 4190.0), (24576, 4096, 4096, 1790.0, 6240.0),
    (49152, 4096, 4096, 3590.0, 12430.0), (65536, 4096, 4096, 4780.0, 16550.0),
    (98304, 4096, 4096, 7170.0, 24810.0), (131072, 4096, 4096, 9560.0, 33050.0),
    (258048, 4096, 4096, 18820.0, 65100.0), (299520, 4096, 4096, 21850.0, 75570.0),
]


def run_sweep(args):
    """Every row of the page's shape table: operands randn (torch's seeded
    generator on the device) quantized by the library's own 1 x 128 and
    128 x 128 quantizers (not timed), then the GEMM timed with HIP events
    around back-to-back launches, fp32 and bf16 output."""
    torch, bsq = _gpu_setup()
    dev = torch.device("cuda:0")
    out_path = args.out
    os.makedirs(os.path.dirname(os.path.abspath(out_path)), exist_ok=True)
    open(out_path, "w").close()
    gen = torch.Generator(device=dev)

    def time_gemm(fn, n_iter):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        _queue_ahead(torch)
        s.record()
        for _ in range(n_iter):
            fn()
        e.record()
        torch.cuda.synchronize()
        return s.elapsed_time(e) / n_iter  # ms

    for idx, (M, N, K, t_sol, t_prod) in enumerate(PAGE_SWEEP):
        gen.manual_seed(1000 + idx)
        a32 = torch.randn(M, K, device=dev, generator=gen)
        b32 = torch.randn(N, K, device=dev, generator=gen)
        aq = torch.empty(M, K, dtype=torch.uint8, device=dev)
        bq = torch.empty(N, K, dtype=torch.uint8, device=dev)
        sa = torch.empty(M, K // 128, dtype=torch.float32, device=dev)
        sb = torch.empty(N // 128, K // 128, dtype=torch.float32, device=dev)
        bsq.bsq_quant_fp8_rowblock(a32, aq, sa, 128)
        bsq.bsq_quant_fp8_tile(b32, bq, sb, 128, 128)
        del a32, b32
        flops = 2.0 * M * N * K
        n_it = max(3, min(50, int(2e13 / flops)))
        row = {"row": idx, "m": M, "n": N, "k": K, "page_T_SOL_us": t_sol, "page_T_Prod_us": t_prod}
        for name, dt in (("f32", torch.float32), ("bf16", torch.bfloat16)):
            y = torch.empty(M, N, dtype=dt, device=dev)
            ms = time_gemm(lambda: bsq.bsq_blockwise_fp8_matmul(aq, bq, sa, sb, y), n_it)
            tf = flops / (ms * 1e-3) / 1e12
            row[f"us_{name}"] = round(ms * 1e3, 2)
            row[f"TFLOP/s_{name}"] = round(tf, 1)
            row[f"pct_peak_{name}"] = round(100 * tf / PEAK_FP8_TFLOPS, 1)
            # roofline of this shape: algorithmic bytes (codes, scales, output)
            nbytes = M * K + N * K + (M + N // 128) * (K // 128) * 4 + M * N * (4 if name == "f32" else 2)
            roof = min(PEAK_FP8_TFLOPS, flops / nbytes * PEAK_HBM_GBS / 1e3)
            row[f"bound_{name}"] = "mfma" if roof >= PEAK_FP8_TFLOPS else "hbm"
            row[f"pct_roofline_{name}"] = round(100 * tf / roof, 1)
            del y
        _log("[sweep] " + json.dumps(row))
        with open(out_path, "a") as f:
            f.write(json.dumps(row) + "\n")
        del aq, bq, sa, sb
        torch.cuda.empty_cache()


# ------------------------------------------------------- operand sweep ---

OPERAND_SETS = ("recipe", "uniform", "zero", "constant", "sparse")


def run_operand_sweep(args):
    """The 4096^3 group-128 GEMM on operands of different value patterns,
    with the same scales: the recipe's (randn quantized 1 x 128 and
    128 x 128, as in the main step), uniform random e4m3 codes, all-zero
    codes, one constant code (1.0), and random codes of which 7 in 8 are
    zero.  The kernel's instruction stream does not depend on the values,
    so a difference in time is a difference in clock: under a counter pass
    (GRBM_GUI_ACTIVE) every set takes the same cycles.  Sets are separated
    by a fill of a 7-element tensor so that a trace can be split."""
    torch, bsq = _gpu_setup()
    import synth

    M = N = K = 4096
    dev = torch.device("cuda:0")
    out_path = args.out
    os.makedirs(os.path.dirname(os.path.abspath(out_path)), exist_ok=True)
    open(out_path, "w").close()
    a32, b32 = synth.fp8_blockwise_raw(M, N, K, 204, 205)
    a32 = torch.from_numpy(a32).to(dev)
    b32 = torch.from_numpy(b32).to(dev)
    rq = torch.empty(M, K, dtype=torch.uint8, device=dev)
    wq = torch.empty(N, K, dtype=torch.uint8, device=dev)
    sa = torch.empty(M, K // 128, dtype=torch.float32, device=dev)
    sb = torch.empty(N // 128, K // 128, dtype=torch.float32, device=dev)
    bsq.bsq_quant_fp8_rowblock(a32, rq, sa, 128)
    bsq.bsq_quant_fp8_tile(b32, wq, sb, 128, 128)
    del a32, b32
    gen = torch.Generator(device=dev)
    gen.manual_seed(77)
    aq = torch.empty_like(rq)
    bq = torch.empty_like(wq)
    y = torch.empty(M, N, dtype=torch.float32, device=dev)
    marker = torch.empty(7, device=dev)
    flops = 2.0 * M * N * K
    for name in OPERAND_SETS:
        if name == "recipe":
            aq.copy_(rq)
            bq.copy_(wq)
        elif name == "zero":
            aq.zero_()
            bq.zero_()
        elif name == "constant":
            aq.fill_(0x38)  # e4m3 1.0
            bq.fill_(0x38)
        else:
            # e4m3 codes 0x00..0x7D and their negatives (no NaN)
            for t in (aq, bq):
                c = torch.randint(0, 126, t.shape, dtype=torch.uint8, device=dev, generator=gen)
                c |= (torch.randint(0, 2, t.shape, dtype=torch.uint8, device=dev, generator=gen) << 7)
                if name == "sparse":
                    c *= (torch.rand(t.shape, device=dev, generator=gen) < 0.125).to(torch.uint8)
                t.copy_(c)
        marker.fill_(0.0)
        for _ in range(args.warmup):
            bsq.bsq_blockwise_fp8_matmul(aq, bq, sa, sb, y)
        per = []
        for _ in range(5):
            torch.cuda.synchronize()
            s = torch.cuda.Event(enable_timing=True)
            e = torch.cuda.Event(enable_timing=True)
            s.record()
            for _ in range(args.steps):
                bsq.bsq_blockwise_fp8_matmul(aq, bq, sa, sb, y)
            e.record()
            torch.cuda.synchronize()
            per.append(s.elapsed_time(e) / args.steps)
        per.sort()
        ms = per[2]
        row = {"operands": name, "m": M, "n": N, "k": K, "launches": args.warmup + 5 * args.steps,
               "us": round(ms * 1e3, 2), "us_min": round(per[0] * 1e3, 2),
               "TFLOP/s": round(flops / (ms * 1e-3) / 1e12, 1)}
        _log("[operands] " + json.dumps(row))
        with open(out_path, "a") as f:
            f.write(json.dumps(row) + "\n")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--suite", action="store_true")
    ap.add_argument("--sweep", action="store_true",
                    help="every row of the block_scaled_mm page's shape table (fp32 and bf16 output)")
    ap.add_argument("--operand-sweep", action="store_true",
                    help="the 4096^3 GEMM on operands of different value patterns (clock versus data)")
    ap.add_argument("--out", default=DEFAULT_SUITE_OUT)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after the timed steps, copy 512 MiB five times (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this library's path runs on a single MI355X and has no "
              "multi-GPU mode; run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.suite:
        run_suite(args)
    elif args.operand_sweep:
        if args.out == DEFAULT_SUITE_OUT:
            args.out = os.path.join(ROOT, "bench_out", "operands.jsonl")
        run_operand_sweep(args)
    elif args.sweep:
        if args.out == DEFAULT_SUITE_OUT:
            args.out = os.path.join(ROOT, "bench_out", "sweep.jsonl")
        run_sweep(args)
    else:
        run_main(args)


if __name__ == "__main__":
    main()
