"""Benchmark: Q4_K GEMV weight-stream GB/s on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 3]

A step is one q4k_gemv launch (validation, x staging, superblock stream,
decode, dot, reduction and store all happen inside it) over one copy of the
weights.  To measure HBM and not the 256 MB last-level cache, the weights are
replicated into >= 1 GiB of distinct copies and the steps cycle through them.
Inputs are resident in HBM before timing starts.  W untimed warm-up steps,
then exactly K steps between HIP events on the launch stream (seven batches,
events between them), bracketed by device synchronisation.  The defaults (20000 and 20000, about 0.3 s each
on the LM head) let the GPU's clocks settle before the timed region: a few
hundred warm-up steps leave the first milliseconds of the timed region 2-5 %
slower on MI355X.

Printed as one JSON line (rank 0):
  value        weight bytes streamed per second over the timed region (GB/s)
  roofline     algorithmic bytes per launch (weights + x + y) / average launch
               time, against the 8 TB/s HBM3E peak; `traffic` is the measured
               HBM bytes per launch from the committed rocprofv3 counter
               summary when it was taken on the current kernel source
  cpu_baseline the CPU oracle (f32 dequant + f64 dot, OpenMP) on the same
               workload; its sampled rows are also compared with the GPU y
  calibration  a plain 16-byte-load streaming read (the whole grid sweeping
               the bytes in address order) over the rotation buffer and over
               one weight copy per launch: the achievable read rate on this
               part, and the one-launch read time of the workload's bytes
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "Q4_K GEMV weight-stream GB/s and % of HBM peak (n×k, m=1)"
HBM_PEAK_GBPS = 8000.0
FP16_PEAK_TFLOPS = 2500.0       # dense fp16 matrix-core peak of MI355X
DEFAULT_WORKLOAD = 3


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "block_quantized_decode_q4_amd", "csrc", "*"))):
        with open(f, "rb") as fh:
            h.update(os.path.basename(f).encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def committed_traffic(workload_name: str):
    """HBM bytes per launch from profiles/<workload>_counters.md, if it was
    measured on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "%s_counters.md" % workload_name)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    src = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    tb = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not src or not tb or src.group(1) != kernel_source_hash():
        return None
    return float(tb.group(1))


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, x, n, k, m, weight_bytes, y_gpu, target_s=12.0):
    """Time the CPU oracle on the whole workload, repeated for about
    `target_s` seconds of CPU work after one warm-up run (median run), on
    all the threads OpenMP takes, then once more on one thread; check the
    GPU output against it."""
    import numpy as np
    import oracle

    threads = oracle.num_threads()
    y_ref, bound = oracle.gemv(w, x, n)           # warm-up
    times = []
    t_total = time.time()
    while True:
        t0 = time.perf_counter()
        y_ref, bound = oracle.gemv(w, x, n)
        times.append(time.perf_counter() - t0)
        if len(times) >= 3 and time.time() - t_total > target_s:
            break
        if len(times) >= 5000:
            break
    t_med = sorted(times)[len(times) // 2]
    # one thread: the same workload, median of three runs
    oracle.set_num_threads(1)
    try:
        t1 = []
        for _ in range(3):
            t0 = time.perf_counter()
            oracle.gemv(w, x, n)
            t1.append(time.perf_counter() - t0)
    finally:
        oracle.set_num_threads(threads)
    t1_med = sorted(t1)[1]
    err = np.abs(y_gpu.astype(np.float64) - y_ref) / np.maximum(bound, 1e-300)
    return {
        "value": weight_bytes / t_med / 1e9,
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": "whole workload (%d x %d, m=%d) repeated for %.1f s after one warm-up run, "
                  "median of %d runs, f32 dequant + f64 dot, OpenMP over rows"
                  % (n, k, m, sum(times), len(times)),
        "cpu_model": cpu_model(),
        "gemv_per_s": 1.0 / t_med,
        "one_thread": {"value": weight_bytes / t1_med / 1e9, "unit": "GB/s",
                       "gemv_per_s": 1.0 / t1_med, "sample": "the same workload, median of 3 runs"},
        "gpu_max_err_over_bound": float(err.max()),
    }


KERNEL_NAMES = {1: "gemv_kernel", 2: "gemv_stream_kernel", 3: "gemv_dot4_lines_kernel",
                4: "gemv_i8_lines_kernel", 5: "gemv_i8_sub_kernel (x staged)",
                6: "gemv_i8_sub_kernel (x per wave)", 7: "gemv_i8_sub_kernel (x window)"}

# The arithmetic each kernel computes in (the plan's kernel number)
KERNEL_DTYPE = {
    1: ("f32-x/f64", "x f32; each weight fl32(d sc q - dmin m) as the format defines it; "
                     "products exact and sums in f64; y rounded once to f32"),
    2: ("f32-x/f64", "as kernel 1 (streaming kernel)"),
    3: ("i8x4-x/i32/f64", "x as four int8 digits of a per-32-element integer grid (values far "
                          "below their sub-block's largest, inf and NaN added exactly); int32 "
                          "dot4 sums; per sub-block D T - M XI rounded once in f64; y rounded "
                          "once to f32"),
    4: ("i8x4-x/i32/f64", "as kernel 3, digit sums on int8 matrix cores (16x16x64)"),
    5: ("i8x4-x/i32/f64", "as kernel 3, digit sums on int8 matrix cores (16x16x32), x staged whole"),
    6: ("i8x4-x/i32/f64", "as kernel 5, x converted per column by each wave"),
    7: ("i8x4-x/i32/f64", "as kernel 5, x converted once per workgroup into a two-column "
                          "window of every slab"),
}


def time_q6k(q4k, synth, torch, lib, n, k, x_d, y_d, sp, stream, args):
    """Time q6k_gemv on seeded Q6_K weights of shape n x k (the same x):
    dense rows (when their bytes are a multiple of 16) and rows padded to
    whole lines.  Returns a list of results, one per layout."""
    dense = q4k.q6k_row_bytes(k)
    layouts = [s for s in (0 if dense % 16 == 0 else None, -(-dense // 128) * 128)
               if s is not None]
    res = []
    for stride in dict.fromkeys(layouts):
        st = stride or dense
        w6, _ = synth.make_q6k_inputs(n, k, 1, seed=2000 + n + k, row_stride=stride)
        nbytes = w6.size                              # n * st
        copies = max(4, math.ceil(args.rotate_gib * (1 << 30) / nbytes))
        pool = torch.empty((copies, nbytes + 128), dtype=torch.uint8, device="cuda")
        base = pool.data_ptr()
        # every copy at a 128-byte-aligned address (the row pitch is nbytes + 128)
        offs = [(-(base + c * (nbytes + 128))) % 128 for c in range(copies)]
        src = torch.from_numpy(w6).cuda()
        for c in range(copies):
            pool[c, offs[c]:offs[c] + nbytes].copy_(src)
        del src
        ptrs = [base + c * (nbytes + 128) + offs[c] for c in range(copies)]
        xp, yp = x_d.data_ptr(), y_d.data_ptr()

        def step6(i):
            rc = lib.q6k_gemv(ptrs[i % copies], xp, yp, n, k, stride, sp)
            if rc != 0:
                raise q4k.Q4KError(rc, "q6k_gemv")
        steps = max(100, min(args.steps, 5000))
        for i in range(min(args.warmup, 5000)):
            step6(i)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(steps):
            step6(i)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / steps
        wbytes = n * dense
        plan = q4k.q6k_plan(n, k, stride, True)
        res.append({"entry": "q6k_gemv",
                    "workload": "q6k_gemv_n%d_k%d_m1" % (n, k),
                    "row_stride": st, "unit_bytes": plan.unit_bytes,
                    "column_groups": plan.column_groups,
                    "us_per_step": round(us, 3), "steps": steps,
                    "value": round(wbytes / us / 1e3, 2), "unit": "GB/s",
                    "frac_of_hbm_peak": round((wbytes + 4 * k + 4 * n) / us / 1e3
                                              / HBM_PEAK_GBPS, 4)})
        log("bench: q6k_gemv n=%d k=%d stride=%d: %.3f us" % (n, k, st, us))
        del pool
        torch.cuda.empty_cache()
    return res


def time_wide_batches(q4k, synth, torch, lib, sp, stream, args, n=14336, k=4096, ms=(16, 32)):
    """Time q4k_gemv with more vectors than the pages' batch of eight (one
    pass over the weights on the sub-block matrix-core kernels) on seeded
    Q4_K weights of n x k, cycling through >= rotate-gib of copies."""
    w, x = synth.make_inputs(n, k, max(ms), seed=3000 + n + k)
    nbytes = w.size
    copies = max(4, math.ceil(args.rotate_gib * (1 << 30) / nbytes))
    pool = torch.empty((copies, nbytes), dtype=torch.uint8, device="cuda")
    src = torch.from_numpy(w).cuda()
    for c in range(copies):
        pool[c].copy_(src)
    del src
    ptrs = [pool[c].data_ptr() for c in range(copies)]
    x_d = torch.from_numpy(x).cuda()
    y_d = torch.empty((max(ms), n), dtype=torch.float32, device="cuda")
    res = []
    for m in ms:
        def stepm(i):
            rc = lib.q4k_gemv(ptrs[i % copies], x_d.data_ptr(), y_d.data_ptr(), n, k, m, sp)
            if rc != 0:
                raise q4k.Q4KError(rc, "q4k_gemv")
        steps = max(100, min(args.steps, 2000))
        for i in range(min(args.warmup, 500)):
            stepm(i)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(steps):
            stepm(i)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / steps
        plan = q4k.q4k_plan(n, k, m)
        res.append({"entry": "q4k_gemv", "workload": "q4k_gemv_n%d_k%d_m%d" % (n, k, m),
                    "kernel": KERNEL_NAMES.get(plan.kernel, str(plan.kernel)),
                    "us_per_step": round(us, 3), "us_per_vector": round(us / m, 3),
                    "steps": steps, "value": round(nbytes / us / 1e3, 2), "unit": "GB/s"})
        log("bench: q4k_gemv n=%d k=%d m=%d: %.3f us" % (n, k, m, us))
    del pool, x_d, y_d
    torch.cuda.empty_cache()
    return res


def time_prefill(q4k, torch, sp, stream, args, m=512, shapes=((14336, 4096), (4096, 14336))):
    """Time q4k_f16_gemm (fp16 mirror x fp16 activations, f32 accumulation)
    at the prefill batch m on mirrors of the given (n, k) shapes (random
    fp16 values; the time does not depend on them).  TFLOP/s against the
    dense fp16 matrix-core peak."""
    res = []
    for n, k in shapes:
        g = torch.Generator(device="cuda").manual_seed(n + k)
        w16 = (torch.randn((n, k), device="cuda", generator=g) * 0.05).to(torch.float16)
        x16 = torch.randn((m, k), device="cuda", generator=g).to(torch.float16)
        y = torch.empty((m, n), dtype=torch.float32, device="cuda")
        lib = q4k.load_library()

        def step():
            rc = lib.q4k_f16_gemm(w16.data_ptr(), x16.data_ptr(), y.data_ptr(), m, n, k, sp)
            if rc != 0:
                raise q4k.Q4KError(rc, "q4k_f16_gemm")
        reps = max(20, min(args.steps // 20, 500))
        for _ in range(min(reps, 50)):
            step()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            step()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        tflops = 2.0 * m * n * k / us / 1e6
        res.append({"entry": "q4k_f16_gemm", "m": m, "n": n, "k": k, "us_per_gemm": round(us, 2),
                    "reps": reps, "value": round(tflops, 1), "unit": "TFLOP/s",
                    "frac_of_fp16_peak": round(tflops / FP16_PEAK_TFLOPS, 4)})
        log("bench: q4k_f16_gemm m=%d n=%d k=%d: %.2f us, %.1f TFLOP/s" % (m, n, k, us, tflops))
        del w16, x16, y
    torch.cuda.empty_cache()
    return res


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20000)
    ap.add_argument("--warmup", type=int, default=20000)
    ap.add_argument("--workload", type=int, default=DEFAULT_WORKLOAD)
    ap.add_argument("--shape", default=None, metavar="N:K:M",
                    help="time this shape (seeded synthetic inputs) instead of --workload")
    ap.add_argument("--rotate-gib", type=float, default=1.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: measures one GPU only (the GEMV runs on one MI355X; "
              "--gpus %d is not supported)" % args.gpus, file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from block_quantized_decode_q4_amd import q4k, synth

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    q4k.load_library()           # raises if libq4k.so is missing: no fallback
    torch.cuda.set_device(0)

    if args.shape:
        n_, k_, m_ = (int(t) for t in args.shape.split(":"))
        wl = synth.Workload(-1, "q4k_gemv_n%d_k%d_m%d" % (n_, k_, m_), n_, k_, m_)
        w, x = synth.make_inputs(n_, k_, m_, seed=n_ + k_ + m_)
    else:
        wl, w, x = synth.workload_inputs(args.workload)
    n, k, m = wl.n, wl.k, wl.m
    wb = wl.weight_bytes
    copies = max(4, math.ceil(args.rotate_gib * (1 << 30) / wb))
    log("bench: %s n=%d k=%d m=%d weight_bytes=%d copies=%d" % (wl.name, n, k, m, wb, copies))

    w_one = torch.from_numpy(w).cuda()
    pool = torch.empty((copies, wb), dtype=torch.uint8, device="cuda")
    for c in range(copies):
        pool[c].copy_(w_one)
    del w_one
    x_d = torch.from_numpy(x).cuda()
    y_d = torch.empty((m, n), dtype=torch.float32, device="cuda")
    ptrs = [pool[c].data_ptr() for c in range(copies)]
    xp, yp = x_d.data_ptr(), y_d.data_ptr()
    lib = q4k.load_library()
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    def step(i):
        rc = lib.q4k_gemv(ptrs[i % copies], xp, yp, n, k, m, sp)
        if rc != 0:
            raise q4k.Q4KError(rc, "q4k_gemv")

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # the K timed steps in 7 batches: events between the batches, so that the
    # median batch is reported beside the mean over the whole region
    nb = 7 if args.steps >= 7 else 1
    bounds = [round(i * args.steps / nb) for i in range(nb + 1)]
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(nb + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for b in range(nb):
        for i in range(bounds[b], bounds[b + 1]):
            step(args.warmup + i)
        ev[b + 1].record(stream)
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[nb])
    t_launch = ms / 1e3 / args.steps
    batch_us = sorted(ev[b].elapsed_time(ev[b + 1]) * 1e3 / (bounds[b + 1] - bounds[b])
                      for b in range(nb))
    t_median = batch_us[nb // 2] / 1e6
    y_last = y_d.cpu().numpy()
    log("bench: %.3f us per GEMV over %d steps" % (t_launch * 1e6, args.steps))

    # calibration: plain streaming read of the whole rotation buffer
    nblk = q4k.q4k_read_calibrate_blocks()
    cal_out = torch.empty(nblk, dtype=torch.float32, device="cuda")
    total = pool.numel()
    for _ in range(2):
        q4k.q4k_read_calibrate(pool, total, cal_out, stream=sp)
    c0 = torch.cuda.Event(enable_timing=True)
    c1 = torch.cuda.Event(enable_timing=True)
    reps = 5
    torch.cuda.synchronize()
    c0.record(stream)
    for _ in range(reps):
        q4k.q4k_read_calibrate(pool, total, cal_out, stream=sp)
    c1.record(stream)
    torch.cuda.synchronize()
    read_gbps = total * reps / (c0.elapsed_time(c1) / 1e3) / 1e9
    # the same read at the GEMV's size: one weight copy per launch, cycling
    # through the copies as the steps do (the ceiling a launch of this size
    # reaches with plain loads)
    # (the library call itself, as the timed steps make theirs, so that host
    # overhead per call stays below a launch of this size)
    wbr = wb - wb % 16
    one_reps = max(50, min(2000, args.steps))
    cp = cal_out.data_ptr()

    def read_one(i):
        rc = lib.q4k_read_calibrate(ptrs[i % copies], wbr, cp, sp)
        if rc != 0:
            raise q4k.Q4KError(rc, "q4k_read_calibrate")
    for i in range(200):
        read_one(i)
    torch.cuda.synchronize()
    c0.record(stream)
    for i in range(one_reps):
        read_one(i)
    c1.record(stream)
    torch.cuda.synchronize()
    one_us = c0.elapsed_time(c1) * 1e3 / one_reps

    # the integer-dot variant with Q8 activations (m = 1 only; its own
    # tolerance): the same rotation, after the headline measurement
    q8 = None
    if m == 1 and (ptrs[0] % 128) == 0:
        def step_q8(i):
            rc = lib.q4k_gemv_q8(ptrs[i % copies], xp, yp, n, k, 1, sp)
            if rc != 0:
                raise q4k.Q4KError(rc, "q4k_gemv_q8")
        q8_steps = max(100, min(args.steps, 5000))
        for i in range(min(args.warmup, 5000)):
            step_q8(i)
        torch.cuda.synchronize()
        c0.record(stream)
        for i in range(q8_steps):
            step_q8(i)
        c1.record(stream)
        torch.cuda.synchronize()
        q8_us = c0.elapsed_time(c1) * 1e3 / q8_steps
        q8 = {"entry": "q4k_gemv_q8", "us_per_step": round(q8_us, 3), "steps": q8_steps,
              "value": round(wb / q8_us / 1e3, 2), "unit": "GB/s",
              "frac_of_hbm_peak": round((wb + 4 * k + 4 * n) / q8_us / 1e3 / HBM_PEAK_GBPS, 4),
              "numerics": "x as Q8 (int8 codes, one f32 scale per 32 elements), int32 dot4, "
                          "f64 scaling; its own tolerance sum|w|(d/2(1+2^-19) + 2^-20|x|) + "
                          "2^-23|y_ref|"}

    # the Q6_K GEMV over a Q6_K matrix of the same shape (m = 1; the pages'
    # Q6_K LM head): dense rows and rows padded to whole 128-byte lines, each
    # cycling through >= rotate-gib of copies
    q6 = None
    if m == 1 and k % 256 == 0 and q4k.q6k_row_bytes(k) * n > 0:
        del pool
        torch.cuda.empty_cache()
        q6 = time_q6k(q4k, synth, torch, lib, n, k, x_d, y_d, sp, stream, args)

    # the prefill GEMM beside the decode path (fp16 mirror, m = 512)
    prefill = time_prefill(q4k, torch, sp, stream, args)

    # batches beyond eight vectors (one pass over the weights)
    wide = None
    if m == 1:
        if q6 is None:
            del pool
            torch.cuda.empty_cache()
        wide = time_wide_batches(q4k, synth, torch, lib, sp, stream, args)

    alg_bytes = wb + 4 * k * m + 4 * n * m
    achieved = alg_bytes / t_launch / 1e9
    traffic = committed_traffic(wl.name)
    plan = q4k.q4k_plan(n, k, m)
    dtype, numerics = KERNEL_DTYPE[plan.kernel]
    out = {
        "metric": METRIC,
        "value": round(wb / t_launch / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": t_launch * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "numerics": numerics,
        "data": "synthetic",
        "config": {
            "workload": wl.name,
            "n": n,
            "k": k,
            "m": m,
            "weight_format": "GGUF Q4_K (144 B / 256 weights)",
            "weight_bytes": wb,
            "rotation_copies": copies,
        },
        "pct_of_hbm_peak": round(100.0 * wb / t_launch / 1e9 / HBM_PEAK_GBPS, 2),
        "gemv_per_s": 1.0 / t_launch,
        "median_batch": {"us_per_step": round(t_median * 1e6, 3), "batches": nb,
                         "value": round(wb / t_median / 1e9, 2)},
        "roofline": {
            "kernel": KERNEL_NAMES.get(plan.kernel, str(plan.kernel)),
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
        },
        "calibration": {"read_gbps": round(read_gbps, 2),
                        "frac_of_peak": round(read_gbps / HBM_PEAK_GBPS, 4),
                        "read_one_copy_us": round(one_us, 3),
                        "read_one_copy_gbps": round(wbr / one_us / 1e3, 2)},
    }
    if q8 is not None:
        out["q8_variant"] = q8
    if q6:
        out["q6k"] = q6
    out["prefill_f16"] = prefill
    if wide:
        out["wide_batches"] = wide
    if not args.no_cpu_baseline:
        log("bench: timing the CPU oracle")
        out["cpu_baseline"] = cpu_baseline(w, x, n, k, m, wb, y_last)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
