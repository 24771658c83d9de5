#!/usr/bin/env python3
"""Benchmark of the TQ1_0 x Q8_1 decode mat-vec on one MI355X.

A step is one pass of the hot path for one decode token on the 4096 x 4096
workload: Q8_1-quantize the fp32 activation column, then the TQ1_0 mat-vec.
Inputs are synthetic (seeded), resident in HBM before timing starts. Each
step reads a different copy of the packed weights from a rotation of at
least 1 GiB, so every mat-vec streams its weights from HBM rather than from
the 256 MB last-level cache.

Timed region: K steps captured once in a HIP graph and replayed, bracketed by
device synchronizations (the eager, launch-by-launch rate is reported beside
it). The dominant kernel's duration is measured separately with HIP events
around each launch on its stream; the roofline fraction divides its
algorithmic bytes by that duration. The CPU oracle is timed on a bounded
sample as a reported baseline.

Prints ONE JSON line on stdout; details go to stderr.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "µs/call and achieved HBM GB/s (% peak), TQ1_0 mat-vec N=4096 K=4096 T=1"
HBM_PEAK_GBS = 8000.0
COUNTERS_FILE = os.path.join(ROOT, "profiles", "counters_mmvq_tq1_0_decode_4096x4096.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash():
    """Hash of the HIP sources; counter readings are only valid for this hash."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "bit_quantized_mat_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".hpp")):
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(N, K, T):
    """Bytes a mat-vec call must move at minimum: packed weights once, the
    Q8_1 activations once, the fp32 outputs once."""
    return N * (K // 256) * 54 + T * (K // 32) * 36 + T * N * 4


def quantize_bytes(T, K):
    return T * K * 4 + T * (K // 32) * 36


def traffic_from_counters(N, K, T):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel sources; else None."""
    try:
        with open(COUNTERS_FILE) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("kernel_source_hash") != kernel_source_hash() or c.get("shape") != [N, K, T]:
        return None
    return c.get("hbm_bytes_per_launch")


def lanes_per_row_log2(nb):
    """Lanes per output row in the one-column kernel (largest power of two
    dividing the row's block count, at most 64)."""
    lr = 0
    while lr < 6 and nb % (2 << lr) == 0:
        lr += 1
    return lr


def cpu_baseline(inp, N, K, T, step_bytes, seconds):
    import oracle
    threads = max(1, min(16, os.cpu_count() or 1))
    oracle.set_threads(threads)
    w_ref = oracle.tq1_pack(inp.trits, inp.d16)
    x = inp.x[:T]
    n = 0
    t0 = time.perf_counter()
    while True:
        a = oracle.q8_1_quantize(x)
        oracle.mmvq(w_ref, a, N, K, T)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": round(step_bytes * n / el / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": "%d full decode steps (Q8_1 quantize + %dx%d mat-vec, T=%d) in %.1f s; "
                      "%.1f ms per step" % (n, N, K, T, el, 1e3 * el / n)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--rotation-gib", type=float, default=1.0,
                    help="total size of the rotated weight copies")
    ap.add_argument("--kernel-launches", type=int, default=400,
                    help="individually event-timed launches of the dominant kernel")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import bit_quantized_mat_amd as bqm
    from bit_quantized_mat_amd import synth

    wl = synth.WORKLOADS["decode"]
    N, K, T = wl.N, wl.K, 1
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = synth.make_inputs(wl)
    log("workload decode N=%d K=%d T=%d" % (N, K, T))

    w0 = bqm.tq1_pack(torch.from_numpy(inp.trits).to(dev),
                      torch.from_numpy(inp.d16.view(np.int16)).to(dev))
    wbytes = w0.numel()
    R = max(2, int(np.ceil(args.rotation_gib * (1 << 30) / wbytes)))
    wrot = torch.empty((R, wbytes), dtype=torch.uint8, device=dev)
    wrot.copy_(w0.view(1, -1).expand(R, wbytes))
    x = torch.from_numpy(inp.x[:T]).to(dev)
    a = torch.empty((T, (K // 32) * 36), dtype=torch.uint8, device=dev)
    y = torch.empty((T, N), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    log("rotation: %d copies of %d bytes (%.2f GiB)" % (R, wbytes, R * wbytes / 2**30))

    def step(i):
        bqm.q8_1_quantize(x, out=a)
        bqm.mmvq_tq1_0(wrot[i % R], a, N, K, T, out=y)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # eager rate (host launch cost included)
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) * 1e3 / args.steps

    # timed region: the K steps captured in one graph
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(args.steps):
            step(args.warmup + i)
    graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    graph.replay()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps

    # dominant kernel: per-launch HIP events on the launch stream
    stream = torch.cuda.current_stream(dev)
    M = args.kernel_launches

    def per_launch_us(launch, count):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(count)]
        for i, (s, e) in enumerate(evs):
            s.record(stream)
            launch(i)
            e.record(stream)
        torch.cuda.synchronize()
        return np.array([s.elapsed_time(e) * 1e3 for s, e in evs])

    def mmvq_launch(i):
        bqm.mmvq_tq1_0(wrot[(7 * i) % R], a, N, K, T, out=y, stream=stream)

    durs_us = per_launch_us(mmvq_launch, M)
    us_call = float(np.mean(durs_us))
    # back-to-back launches bracketed by one event pair (includes dispatch gaps)
    s0, e0 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s0.record(stream)
    for i in range(M):
        bqm.mmvq_tq1_0(wrot[(11 * i) % R], a, N, K, T, out=y, stream=stream)
    e0.record(stream)
    torch.cuda.synchronize()
    us_b2b = s0.elapsed_time(e0) * 1e3 / M

    # calibration: an empty dispatch, and a streaming read of the same weight
    # bytes with the mat-vec's grid and with a wider grid
    import ctypes
    probes = ctypes.CDLL(os.path.join(ROOT, "bit_quantized_mat_amd", "libbqm_probes.so"))
    probes.bqm_probe_empty.argtypes = [ctypes.c_int, ctypes.c_void_p]
    probes.bqm_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p,
                                      ctypes.c_int, ctypes.c_void_p]
    sptr = ctypes.c_void_p(stream.cuda_stream)
    pout = torch.empty(4096, dtype=torch.int32, device=dev)
    mm_grid = int(np.ceil(N / (4 * (64 >> lanes_per_row_log2(K // 256)))))
    rd_bytes = wbytes - wbytes % 16
    cal = {"empty_kernel_us": float(np.mean(per_launch_us(
        lambda i: probes.bqm_probe_empty(mm_grid, sptr), 200)))}
    for g in (mm_grid, 1024):
        d = per_launch_us(lambda i: probes.bqm_probe_read(
            ctypes.c_void_p(wrot[(13 * i + 1) % R].data_ptr()), rd_bytes,
            ctypes.c_void_p(pout.data_ptr()), g, sptr), 200)
        cal["read_%d_wg_us" % g] = float(np.mean(d))
        cal["read_%d_wg_gbs" % g] = round(rd_bytes / float(np.mean(d)) / 1e3, 1)
    cal["read_bytes"] = int(rd_bytes)
    cal["mmvq_grid_wg"] = mm_grid
    log("calibration:", cal)

    mm_bytes = algorithmic_bytes(N, K, T)
    step_bytes = mm_bytes + quantize_bytes(T, K)
    achieved = mm_bytes / (us_call * 1e-6) / 1e9
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    traffic = traffic_from_counters(N, K, T)
    log("mmvq: %.3f us/launch (events per launch, median %.3f, p10 %.3f, p90 %.3f), "
        "%.3f us back-to-back; %.1f GB/s = %.1f%% of %.0f GB/s"
        % (us_call, np.median(durs_us), np.percentile(durs_us, 10), np.percentile(durs_us, 90),
           us_b2b, achieved, 100 * achieved / HBM_PEAK_GBS, HBM_PEAK_GBS))
    log("step: %.3f us graph-replayed, %.3f us eager" % (ms_per_step * 1e3, eager_ms * 1e3))

    base = None
    if not args.no_cpu_baseline:
        base = cpu_baseline(inp, N, K, T, step_bytes, args.cpu_seconds)
        log("cpu baseline:", base)

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic",
        "config": {"workload": "decode mat-vec TQ1_0 N=4096 K=4096 T=1 (quantize + mmvq per step)",
                   "N": N, "K": K, "T": T, "weight_rotation_bytes": int(R * wbytes),
                   "timed": "HIP graph of all steps, replayed once"},
        "us_per_call": round(us_call, 4),
        "us_per_call_back_to_back": round(us_b2b, 4),
        "us_per_step_eager": round(eager_ms * 1e3, 4),
        "mmvq_gbs": round(achieved, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel": "mmvq_tq1_0",
                     "algorithmic_bytes_per_launch": mm_bytes},
        "calibration": {k: (round(v, 4) if isinstance(v, float) else v) for k, v in cal.items()},
        "cpu_baseline": base,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
