"""Benchmark: Q4_K GEMV weight-stream GB/s on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 3]

A step is one q4k_gemv launch (validation, x staging, superblock stream,
decode, dot, reduction and store all happen inside it) over one copy of the
weights.  To measure HBM and not the 256 MB last-level cache, the weights are
replicated into >= 1 GiB of distinct copies and the steps cycle through them.
Inputs are resident in HBM before timing starts.  W untimed warm-up steps,
then exactly K steps between two HIP events on the launch stream, bracketed
by device synchronisation.  The defaults (20000 and 20000, about 0.3 s each
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
  calibration  a plain 16-byte-load streaming read over the rotation buffer:
               the achievable read rate on this part
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


def cpu_baseline(w, x, n, k, m, weight_bytes, y_gpu, target_s=12.0):
    """Time the CPU oracle on the whole workload, repeated for about
    `target_s` seconds of CPU work (median run), and check the GPU output
    against it."""
    import numpy as np
    import oracle

    threads = oracle.num_threads()
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
    err = np.abs(y_gpu.astype(np.float64) - y_ref) / np.maximum(bound, 1e-300)
    return {
        "value": weight_bytes / t_med / 1e9,
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": "whole workload (%d x %d, m=%d) repeated for %.1f s, median of %d runs, "
                  "f32 dequant + f64 dot, OpenMP over rows" % (n, k, m, sum(times), len(times)),
        "gemv_per_s": 1.0 / t_med,
        "gpu_max_err_over_bound": float(err.max()),
    }


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

    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end)
    t_launch = ms / 1e3 / args.steps
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

    alg_bytes = wb + 4 * k * m + 4 * n * m
    achieved = alg_bytes / t_launch / 1e9
    traffic = committed_traffic(wl.name)
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
        "dtype": "f32",
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
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
        },
        "calibration": {"read_gbps": round(read_gbps, 2),
                        "frac_of_peak": round(read_gbps / HBM_PEAK_GBPS, 4)},
    }
    if not args.no_cpu_baseline:
        log("bench: timing the CPU oracle")
        out["cpu_baseline"] = cpu_baseline(w, x, n, k, m, wb, y_last)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
