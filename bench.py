#!/usr/bin/env python3
"""Benchmark of the TQ1_0 x Q8_1 decode mat-vec on one MI355X.

A step is one pass of the hot path for one decode token on the 4096 x 4096
workload: Q8_1-quantize the fp32 activation column, then the TQ1_0 mat-vec.
Inputs are synthetic (seeded) and resident in HBM before timing starts. Each
step reads a different copy of the packed weights from a rotation of at
least 1 GiB, so every mat-vec streams its weights from HBM rather than from
the 256 MB last-level cache.

Timing: K steps are captured once in a HIP graph; one warm replay, then one
replay bracketed by HIP events on the launch stream (host launch cost is
not in the timed region; the eager rate is reported beside it). The dominant
kernel (the mat-vec) is timed the same way, as a graph of mat-vec launches
only; its algorithmic bytes divided by that time give the roofline figure.
The CPU oracle is timed on a bounded sample as a reported baseline.

--sweep PATH additionally measures every workload shape and column count
(the plain mat-vec and the expert-routed one) and writes a JSON table.

Prints ONE JSON line on stdout; details go to stderr.
"""
import argparse
import ctypes
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
# column counts of the prefill rows of the sweep (many-column product)
PREFILL_COLS = (64, 128, 512)
COUNTERS_FILE = os.path.join(ROOT, "profiles", "counters_mmvq_tq1_0_decode_4096x4096.json")
ROTATION_BYTES = 1 << 30


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# Sources the decode step's kernel (the staged kernel, fused with the Q8_1
# quantization) is compiled from: counter readings taken on other sources do
# not describe it.
DOMINANT_KERNEL_SOURCES = ("common.hpp", "q8_1.hpp", "tq1_decode.hpp", "mmvq_staged.hpp",
                           "mmvq_staged.hip", "launch.hpp", "bqm_api.hip")


def kernel_source_hash():
    """Hash of the dominant kernel's HIP sources; counter readings are only
    valid for this hash."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "bit_quantized_mat_amd", "csrc")
    for name in DOMINANT_KERNEL_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(N, K, T, block_bytes=54):
    """Bytes a mat-vec call must move at minimum: packed weights once (54-byte
    TQ1_0 or 66-byte TQ2_0 blocks), the Q8_1 activations once, the fp32
    outputs once."""
    return N * (K // 256) * block_bytes + T * (K // 32) * 36 + T * N * 4


def moe_algorithmic_bytes(ids, N, K, per_slot=False):
    """Expert-routed call: the matrices of the distinct experts routed to,
    once each; the Q8_1 activations (one column per token, or per pair with
    per_slot); fp32 outputs; the ids."""
    T, n_used = ids.shape
    distinct = len(set(ids.ravel().tolist()))
    cols = T * n_used if per_slot else T
    return (distinct * N * (K // 256) * 54 + cols * (K // 32) * 36 + T * n_used * N * 4
            + T * n_used * 4), distinct


def quantize_bytes(T, K):
    return T * K * 4 + T * (K // 32) * 36


def fused_bytes(N, K, T):
    """Bytes the fused quantize-and-multiply call must move at minimum: the
    packed weights, the fp32 activations and the fp32 outputs, once each
    (the Q8_1 blocks never leave the chip)."""
    return N * (K // 256) * 54 + T * K * 4 + T * N * 4


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
    """Lanes per output row in the staged kernels (log2): the smallest power
    of two, at most 64, not below the row's block count."""
    lr = 0
    while lr < 6 and (1 << lr) < nb:
        lr += 1
    return lr


def graph_us(torch, launch, count):
    """Average microseconds per launch: `count` launches captured in one HIP
    graph, one warm replay, then one replay timed with events on the stream."""
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(count):
            launch(i)
    graph.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record(stream)
    graph.replay()
    e.record(stream)
    torch.cuda.synchronize()
    del graph
    return s.elapsed_time(e) * 1e3 / count


def rotation(torch, w0, dev, extra=1):
    """Copies of the packed weights totalling at least ROTATION_BYTES."""
    nbytes = w0.numel()
    R = max(2, -(-ROTATION_BYTES // nbytes)) + extra
    wrot = torch.empty((R, nbytes), dtype=torch.uint8, device=dev)
    wrot.copy_(w0.reshape(1, -1).expand(R, nbytes))
    return wrot, R


def host_cpu_info():
    """What the oracle runs on: the CPU model, the logical CPUs the host
    reports, the CPUs this process may run on, and the OpenMP thread cap the
    job was given (the share of the host that goes with one GPU)."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = None
    return {"cpu_model": model, "nproc": os.cpu_count(), "affinity_cpus": affinity,
            "omp_num_threads_env": os.environ.get("OMP_NUM_THREADS")}


def oracle_threads_all():
    """Threads for the all-cores oracle run: every CPU this process may use,
    capped by OMP_NUM_THREADS when the job sets it (a GPU machine grants each GPU
    a fixed share of its host CPUs and sets OMP_NUM_THREADS to that share)."""
    info = host_cpu_info()
    n = info["affinity_cpus"] or info["nproc"] or 1
    env = info["omp_num_threads_env"]
    if env and env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, n)


def oracle_median_us(fn, runs=5):
    """Median wall time (us) of fn over `runs` calls after one warm-up call."""
    import statistics
    fn()
    ts = []
    for _ in range(runs):
        t0 = time.perf_counter()
        fn()
        ts.append((time.perf_counter() - t0) * 1e6)
    return statistics.median(ts)


def cpu_baseline(inp, N, K, T, seconds):
    """The oracle's mat-vec on the decode workload, timed apart from its
    quantization (median of 5 after 1 warm-up, more runs to fill about
    `seconds` of CPU work): on all the job's host CPUs and on one thread."""
    import oracle
    info = host_cpu_info()
    threads = oracle_threads_all()
    w_ref = oracle.tq1_pack(inp.trits, inp.d16)
    x = inp.x[:T]
    a = oracle.q8_1_quantize(x)
    out = {}
    for label, nt in (("all", threads), ("one", 1)):
        oracle.set_threads(nt)
        t0 = time.perf_counter()
        one = oracle_median_us(lambda: oracle.mmvq(w_ref, a, N, K, T), runs=1)
        runs = int(max(5, min(200, 0.5 * seconds * 1e6 / max(one, 1.0))))
        mm_us = oracle_median_us(lambda: oracle.mmvq(w_ref, a, N, K, T), runs=runs)
        q_us = oracle_median_us(lambda: oracle.q8_1_quantize(x), runs=runs)
        out[label] = {"threads": nt, "mmvq_us": round(mm_us, 1), "quantize_us": round(q_us, 1),
                      "runs": runs, "seconds": round(time.perf_counter() - t0, 1)}
    oracle.set_threads(threads)
    mm_bytes = algorithmic_bytes(N, K, T)
    base = {"value": round(mm_bytes / out["all"]["mmvq_us"] / 1e3, 4), "unit": "GB/s",
            "cores": threads, "kind": "oracle",
            "sample": "the oracle's %dx%d T=%d mat-vec alone (its Q8_1 quantization timed "
                      "apart), median of %d runs after one warm-up on %d threads: %.1f us; on "
                      "one thread %.1f us; quantize %.1f us (%d threads), %.1f us (one)"
                      % (N, K, T, out["all"]["runs"], threads, out["all"]["mmvq_us"],
                         out["one"]["mmvq_us"], out["all"]["quantize_us"], threads,
                         out["one"]["quantize_us"]),
            "single_thread_gbs": round(mm_bytes / out["one"]["mmvq_us"] / 1e3, 4),
            "runs": out}
    base.update(info)
    return base


def cpu_table(path):
    """The oracle on every workload shape and column count (no GPU): median
    of 3 runs after one warm-up, on one thread and on all the job's CPUs;
    mat-vec and expert-routed product timed apart from quantization."""
    import numpy as np
    import oracle
    from bit_quantized_mat_amd import synth
    info = host_cpu_info()
    threads = oracle_threads_all()
    rows = []
    for name in ("tiny", "decode", "multicol", "ffn", "moe"):
        wl = synth.WORKLOADS[name]
        inp = synth.make_inputs(wl)
        w_ref = oracle.tq1_pack(inp.trits, inp.d16)
        a_all = oracle.q8_1_quantize(inp.x)
        for T in wl.Ts:
            a = np.ascontiguousarray(a_all[:T])
            row = {"workload": name, "T": T, "N": wl.N, "K": wl.K}
            for label, nt in (("one", 1), ("all", threads)):
                oracle.set_threads(nt)
                if wl.experts:
                    ids = np.ascontiguousarray(inp.ids[:T])
                    fn = lambda: oracle.mmvq_id(w_ref, a, ids, wl.experts, wl.N, wl.K, T,
                                                wl.n_used)
                else:
                    fn = lambda: oracle.mmvq(w_ref, a, wl.N, wl.K, T)
                row["oracle_us_" + label] = round(oracle_median_us(fn, runs=3), 1)
                row["quantize_us_" + label] = round(oracle_median_us(
                    lambda: oracle.q8_1_quantize(inp.x[:T]), runs=3), 1)
            row["threads_all"] = threads
            rows.append(row)
            log("cpu", row)
        if name in ("decode", "multicol", "ffn"):
            # the same matrices packed as TQ2_0
            w2 = oracle.tq2_pack(inp.trits, inp.d16)
            for T in wl.Ts:
                a = np.ascontiguousarray(a_all[:T])
                row = {"workload": name, "op": "mmvq_tq2_0", "T": T, "N": wl.N, "K": wl.K}
                for label, nt in (("one", 1), ("all", threads)):
                    oracle.set_threads(nt)
                    row["oracle_us_" + label] = round(oracle_median_us(
                        lambda: oracle.tq2_mmvq(w2, a, wl.N, wl.K, T), runs=3), 1)
                row["threads_all"] = threads
                rows.append(row)
                log("cpu", row)
    oracle.set_threads(threads)
    with open(path, "w") as f:
        json.dump({"host": info, "rows": rows}, f, indent=1)
    return rows


def calibrate(torch, np, wrot, R, nbytes, grid_wg):
    """Empty dispatch and plain streaming reads of the same weight bytes."""
    probes = ctypes.CDLL(os.path.join(ROOT, "bit_quantized_mat_amd", "libbqm_probes.so"))
    probes.bqm_probe_empty.argtypes = [ctypes.c_int, ctypes.c_void_p]
    probes.bqm_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p,
                                      ctypes.c_int, ctypes.c_void_p]
    pout = torch.empty(4096, dtype=torch.int32, device=wrot.device)
    rd = nbytes - nbytes % 16
    cur = lambda: ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    cal = {"empty_kernel_us": graph_us(torch, lambda i: probes.bqm_probe_empty(grid_wg, cur()), 200)}
    for g in (grid_wg, 1024):
        us = graph_us(torch, lambda i: probes.bqm_probe_read(
            ctypes.c_void_p(wrot[(13 * i + 1) % R].data_ptr()), rd,
            ctypes.c_void_p(pout.data_ptr()), g, cur()), 200)
        cal["read_%d_wg_us" % g] = us
        cal["read_%d_wg_gbs" % g] = round(rd / us / 1e3, 1)
    cal["read_bytes"] = int(rd)
    cal["mmvq_grid_wg"] = int(grid_wg)
    cal.update(valu_rates(torch, probes))
    return {k: (round(v, 4) if isinstance(v, float) else v) for k, v in cal.items()}


# 256 compute units x 4 SIMDs x 16 lanes x 2.4 GHz: one 32-bit vector
# instruction per lane per cycle at full rate (a wave of 64 lanes issues over
# four cycles on its 16-lane SIMD)
VALU_PEAK_LANE_OPS = 256 * 64 * 2.4e9


def valu_rates(torch, probes):
    """Vector-ALU issue rate of the instruction kinds the decode is made of:
    lane operations per second of long independent chains of one kind
    (8192 waves, 8 per SIMD), and the fraction of the 256 CU x 64 lanes x
    2.4 GHz figure."""
    probes.bqm_probe_valu.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
                                      ctypes.c_void_p]
    grid, iters = 2048, 2048
    out = torch.empty(grid * 256, dtype=torch.int32, device="cuda")
    cur = lambda: ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    res = {}
    for kind, name in enumerate(("dot4_i32_i8", "mad_u32_u24", "pk_mul_lo_u16", "perm_b32")):
        us = graph_us(torch, lambda i: probes.bqm_probe_valu(kind, iters, ctypes.c_void_p(
            out.data_ptr()), grid, cur()), 5)
        lane_ops = grid * 4 * 32 * iters * 64.0
        rate = lane_ops / (us * 1e-6)
        res["valu_%s_lane_ops_per_s" % name] = float("%.4g" % rate)
        res["valu_%s_frac" % name] = round(rate / VALU_PEAK_LANE_OPS, 4)
    return res


def read_probe_row(torch, wrot, R, nbytes, name, launches):
    """A plain streaming read of one weight copy (what any kernel reading
    the same bytes from HBM can reach), best of a few grid sizes."""
    probes = ctypes.CDLL(os.path.join(ROOT, "bit_quantized_mat_amd", "libbqm_probes.so"))
    probes.bqm_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p,
                                      ctypes.c_int, ctypes.c_void_p]
    pout = torch.empty(8192, dtype=torch.int32, device=wrot.device)
    rd = nbytes - nbytes % 16
    cur = lambda: ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    best = None
    for g in (1024, 2048, 4096, 8192):
        us = graph_us(torch, lambda i: probes.bqm_probe_read(
            ctypes.c_void_p(wrot[i % R].data_ptr()), rd, ctypes.c_void_p(pout.data_ptr()), g,
            cur()), launches)
        if best is None or us < best[0]:
            best = (us, g)
    return {"workload": name, "op": "read_probe", "bytes": int(rd), "grid_wg": best[1],
            "us": round(best[0], 3), "gbs": round(rd / best[0] / 1e3, 1),
            "frac_of_8tbs": round(rd / best[0] / 1e3 / HBM_PEAK_GBS, 4)}


def c_abi_eager(torch, bqm, wrot, R, x, y, N, K, T, iters):
    """Eager steps of mmvq_tq1_0_f32 called from C (the probe library's loop
    over the library's own entry point, rotating weight copies): host time
    per call to enqueue, and wall time per call until the stream drains."""
    probes = ctypes.CDLL(os.path.join(ROOT, "bit_quantized_mat_amd", "libbqm_probes.so"))
    probes.bqm_probe_eager.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64,
                                       ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                                       ctypes.c_int, ctypes.c_void_p,
                                       ctypes.POINTER(ctypes.c_double),
                                       ctypes.POINTER(ctypes.c_double)]
    fn = ctypes.cast(bqm.library().mmvq_tq1_0_f32, ctypes.c_void_p)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    enq, wall = ctypes.c_double(), ctypes.c_double()
    res = {}
    for rep in range(2):  # the first pass warms the host path
        rc = probes.bqm_probe_eager(fn, ctypes.c_void_p(wrot.data_ptr()), wrot.shape[1], R,
                                    ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(y.data_ptr()),
                                    N, K, T, iters, stream, ctypes.byref(enq), ctypes.byref(wall))
        if rc != 0:
            raise RuntimeError("bqm_probe_eager: status %d" % rc)
        res = {"enqueue_us": round(enq.value, 4), "wall_us": round(wall.value, 4),
               "calls": iters}
    return res


def dequant_rows(torch, bqm, wrot, R, wbytes, name, N, K, launches):
    """Dequantize the whole matrix (fp16, bf16, fp32) and gather 1024 rows
    (fp16); beside them a copy probe moving as many bytes, for scale."""
    rows_out = []
    for dt, size in ((torch.float16, 2), (torch.bfloat16, 2), (torch.float32, 4)):
        out = torch.empty((N, K), dtype=dt, device=wrot.device)
        us = graph_us(torch, lambda i: bqm.tq1_dequantize(wrot[i % R], N, K, dtype=dt, out=out),
                      launches)
        b = wbytes + N * K * size
        rows_out.append({"workload": name, "op": "tq1_dequantize", "dtype": str(dt).split(".")[1],
                         "N": N, "K": K, "us": round(us, 3), "algorithmic_bytes": b,
                         "gbs": round(b / us / 1e3, 1), "frac_of_8tbs": round(b / us / 1e3 / HBM_PEAK_GBS, 4)})
        log("sweep", rows_out[-1])
        del out
    g = min(1024, N)
    ids = torch.randint(0, N, (g,), dtype=torch.int32, device=wrot.device, generator=torch.Generator(
        device=wrot.device).manual_seed(7))
    out = torch.empty((g, K), dtype=torch.float16, device=wrot.device)
    us = graph_us(torch, lambda i: bqm.tq1_dequantize(wrot[i % R], N, K, rows=ids, out=out), launches)
    b = g * (K // 256) * 54 + g * 4 + g * K * 2
    rows_out.append({"workload": name, "op": "tq1_get_rows", "dtype": "float16", "N": N, "K": K,
                     "rows": g, "us": round(us, 3), "algorithmic_bytes": b,
                     "gbs": round(b / us / 1e3, 1), "frac_of_8tbs": round(b / us / 1e3 / HBM_PEAK_GBS, 4)})
    log("sweep", rows_out[-1])
    # the copy probe on a buffer as large as the fp16 output: read + write
    probes = ctypes.CDLL(os.path.join(ROOT, "bit_quantized_mat_amd", "libbqm_probes.so"))
    probes.bqm_probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64,
                                      ctypes.c_int, ctypes.c_void_p]
    nbytes = N * K * 2
    src = torch.empty(nbytes, dtype=torch.uint8, device=wrot.device)
    dst = torch.empty(nbytes, dtype=torch.uint8, device=wrot.device)
    cur = lambda: ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    best = None
    for grid in (1024, 4096, 16384):
        us = graph_us(torch, lambda i: probes.bqm_probe_copy(ctypes.c_void_p(src.data_ptr()),
                                                            ctypes.c_void_p(dst.data_ptr()),
                                                            nbytes, grid, cur()), launches)
        best = us if best is None else min(best, us)
    rows_out.append({"workload": name, "op": "copy_probe", "bytes_moved": 2 * nbytes,
                     "us": round(best, 3), "gbs": round(2 * nbytes / best / 1e3, 1),
                     "frac_of_8tbs": round(2 * nbytes / best / 1e3 / HBM_PEAK_GBS, 4)})
    log("sweep", rows_out[-1])
    del src, dst, out
    torch.cuda.empty_cache()
    return rows_out


class SweepTimer:
    """Times sweep rows and tags them for the kernel trace.

    Around each row's graph two marker dispatches (the empty probe kernel on
    MARKER_BASE + 2 row-index workgroups before, one more after) are
    launched, so that a rocprofv3 kernel trace of the sweep can be cut into
    rows (--trace-summary). After
    the timing the row records a position-weighted checksum of its output,
    sum over k of (k + 1) * y[k] in float64 over the flattened output, which
    moves when an output lands in the wrong place."""

    MARKER_BASE = 1000

    def __init__(self, torch, table):
        self.torch = torch
        self.table = table
        self.probes = ctypes.CDLL(os.path.join(ROOT, "bit_quantized_mat_amd",
                                               "libbqm_probes.so"))
        self.probes.bqm_probe_empty.argtypes = [ctypes.c_int, ctypes.c_void_p]

    def marker(self, tag, end):
        torch = self.torch
        self.probes.bqm_probe_empty(self.MARKER_BASE + 2 * tag + int(end),
                                    ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))

    def time(self, row, launch, count, out=None):
        torch = self.torch
        self.marker(len(self.table), False)
        us = graph_us(torch, launch, count)
        self.marker(len(self.table), True)
        row["us"] = round(us, 3)
        row["launches"] = count
        row["row_index"] = len(self.table)
        if out is not None:
            torch.cuda.synchronize()
            v = out.detach().reshape(-1).double()
            k = torch.arange(1, v.numel() + 1, dtype=torch.float64, device=v.device)
            row["checksum"] = float((k * v).sum().item())
        self.table.append(row)
        log("sweep", row)
        return us


def _rate_fields(row, b, us, read_gbs=None):
    row["algorithmic_bytes"] = b
    row["gbs"] = round(b / us / 1e3, 1)
    row["frac_of_8tbs"] = round(b / us / 1e3 / HBM_PEAK_GBS, 4)
    if read_gbs:
        # fraction of what a plain read of the same weight bytes reaches in one
        # dispatch (the read probe's rate on this workload's matrix)
        row["frac_of_read_probe"] = round(b / us / 1e3 / read_gbs, 4)


def sweep(path, torch, np, bqm, synth, dev, launches, only=None):
    """Every workload shape and column count, cold weights, graph-timed; an
    untouched control row (decode T = 1) first and last to bound drift.
    only: optional set of workload names to restrict the sweep to."""
    table = []
    timer = SweepTimer(torch, table)

    def control(label):
        wl = synth.WORKLOADS["decode"]
        inp = synth.make_inputs(wl)
        N, K = wl.N, wl.K
        w0 = bqm.tq1_pack(torch.from_numpy(inp.trits).to(dev),
                          torch.from_numpy(inp.d16.view(np.int16)).to(dev))
        wrot, R = rotation(torch, w0, dev)
        a = bqm.q8_1_quantize(torch.from_numpy(inp.x[:1]).to(dev))
        y = torch.empty((1, N), dtype=torch.float32, device=dev)
        row = {"workload": "control (decode, " + label + ")", "op": "mmvq_tq1_0", "N": N, "K": K,
               "T": 1}
        us = timer.time(row, lambda i: bqm.mmvq_tq1_0(wrot[i % R], a, N, K, 1, out=y), launches, y)
        _rate_fields(row, algorithmic_bytes(N, K, 1), us)
        del wrot, w0
        torch.cuda.empty_cache()

    control("session start")
    for name in ("tiny", "decode", "multicol", "ffn"):
        if only and name not in only:
            continue
        wl = synth.WORKLOADS[name]
        # at least two columns: the gate-up rows take one and two
        inp = synth.make_inputs(wl, T=max(max(wl.Ts), 2))
        N, K = wl.N, wl.K
        w0 = bqm.tq1_pack(torch.from_numpy(inp.trits).to(dev),
                          torch.from_numpy(inp.d16.view(np.int16)).to(dev))
        wrot, R = rotation(torch, w0, dev)
        a_all = bqm.q8_1_quantize(torch.from_numpy(inp.x).to(dev))
        table.append(read_probe_row(torch, wrot, R, w0.numel(), name, launches))
        read_gbs = table[-1]["gbs"]
        log("sweep", table[-1])
        if name in ("decode", "ffn"):
            table.extend(dequant_rows(torch, bqm, wrot, R, w0.numel(), name, N, K, launches))
        for T in wl.Ts:
            a = a_all[:T].contiguous()
            y = torch.empty((T, N), dtype=torch.float32, device=dev)
            row = {"workload": name, "op": "mmvq_tq1_0", "N": N, "K": K, "T": T}
            us = timer.time(row, lambda i: bqm.mmvq_tq1_0(wrot[i % R], a, N, K, T, out=y),
                            launches, y)
            _rate_fields(row, algorithmic_bytes(N, K, T), us, read_gbs)
        if name in ("decode", "ffn"):
            # the gate-up pair with its SiLU-gated epilogue: two matrices of
            # this shape (two rotation copies) against the same columns
            x_all = torch.from_numpy(inp.x).to(dev)
            for op, T in (("mmvq_tq1_0_glu", 1), ("mmvq_tq1_0_glu", 2), ("mmvq_tq1_0_f32_glu", 1)):
                src = (x_all if op == "mmvq_tq1_0_f32_glu" else a_all)[:T].contiguous()
                fn = getattr(bqm, op)
                y = torch.empty((T, N), dtype=torch.float32, device=dev)
                row = {"workload": name, "op": op, "N": N, "K": K, "T": T}
                us = timer.time(row, lambda i: fn(wrot[i % R], wrot[(i + 1) % R], src, N, K, T,
                                                  out=y), launches, y)
                xb = T * K * 4 - T * (K // 32) * 36 if op == "mmvq_tq1_0_f32_glu" else 0
                # no read-probe fraction: the probe reads one matrix, the call two
                _rate_fields(row, algorithmic_bytes(N, K, T) + w0.numel() + xb, us)
            del x_all
        del wrot, w0
        torch.cuda.empty_cache()
        if name != "tiny":
            # the same trits and scales packed as TQ2_0 (66-byte blocks)
            w2 = bqm.tq2_pack(torch.from_numpy(inp.trits).to(dev),
                              torch.from_numpy(inp.d16.view(np.int16)).to(dev))
            wrot, R = rotation(torch, w2, dev)
            table.append(read_probe_row(torch, wrot, R, w2.numel(), name + " tq2", launches))
            read_gbs = table[-1]["gbs"]
            log("sweep", table[-1])
            for T in wl.Ts:
                a = a_all[:T].contiguous()
                y = torch.empty((T, N), dtype=torch.float32, device=dev)
                row = {"workload": name, "op": "mmvq_tq2_0", "N": N, "K": K, "T": T}
                us = timer.time(row, lambda i: bqm.mmvq_tq2_0(wrot[i % R], a, N, K, T, out=y),
                                launches, y)
                _rate_fields(row, algorithmic_bytes(N, K, T, 66), us, read_gbs)
            del wrot, w2
        del a_all
        torch.cuda.empty_cache()
    # many-column product: prefill batches on the decode and ffn matrices
    for name in ("decode", "ffn"):
        if only and "prefill" not in only:
            break
        wl = synth.WORKLOADS[name]
        Tmax = max(PREFILL_COLS)
        inp = synth.make_inputs(wl, T=Tmax)
        N, K = wl.N, wl.K
        w0 = bqm.tq1_pack(torch.from_numpy(inp.trits).to(dev),
                          torch.from_numpy(inp.d16.view(np.int16)).to(dev))
        wrot, R = rotation(torch, w0, dev)
        a_all = bqm.q8_1_quantize(torch.from_numpy(inp.x).to(dev))
        for T in PREFILL_COLS:
            a = a_all[:T].contiguous()
            y = torch.empty((T, N), dtype=torch.float32, device=dev)
            row = {"workload": name + " prefill", "op": "mm_tq1_0", "N": N, "K": K, "T": T}
            us = timer.time(row, lambda i: bqm.mm_tq1_0(wrot[i % R], a, N, K, T, out=y),
                            max(10, launches // 4), y)
            _rate_fields(row, algorithmic_bytes(N, K, T), us)
            row["int8_tops"] = round(2.0 * N * K * T / us / 1e6, 1)
        del wrot, a_all, w0
        torch.cuda.empty_cache()
    if not only or "moe" in only:
        wl = synth.WORKLOADS["moe"]
        inp = synth.make_inputs(wl)
        E, N, K, n_used = wl.experts, wl.N, wl.K, wl.n_used
        w0 = bqm.tq1_pack(torch.from_numpy(inp.trits).to(dev),
                          torch.from_numpy(inp.d16.view(np.int16)).to(dev))
        wrot, R = rotation(torch, w0, dev)
        a_all = bqm.q8_1_quantize(torch.from_numpy(inp.x).to(dev))
        table.append(read_probe_row(torch, wrot, R, w0.numel(), "moe (all experts)", launches))
        read_gbs = table[-1]["gbs"]
        log("sweep", table[-1])
        a_slots = bqm.q8_1_quantize(torch.from_numpy(synth.slot_activations(wl)).to(dev))
        for op, per_slot in (("mmvq_id_tq1_0", False), ("mmvq_id_tq1_0_slots", True)):
            fn = getattr(bqm, op)
            for T in wl.Ts:
                ids_np = np.ascontiguousarray(inp.ids[:T])
                ids = torch.from_numpy(ids_np).to(dev)
                a = (a_slots[:T * n_used] if per_slot else a_all[:T]).contiguous()
                y = torch.empty((T, n_used, N), dtype=torch.float32, device=dev)
                ws = torch.empty(max(bqm.mmvq_id_tq1_0_workspace_bytes(E, T, n_used), 256),
                                 dtype=torch.uint8, device=dev)
                b, distinct = moe_algorithmic_bytes(ids_np, N, K, per_slot=per_slot)
                row = {"workload": "moe", "op": op, "E": E, "N": N, "K": K, "T": T,
                       "n_used": n_used, "distinct_experts": distinct}
                us = timer.time(row, lambda i: fn(wrot[i % R], a, ids, E, N, K, T, n_used, out=y,
                                                  workspace=ws), launches, y)
                _rate_fields(row, b, us, read_gbs)
        del wrot, a_all, a_slots, w0
        torch.cuda.empty_cache()
    control("session end")
    with open(path, "w") as f:
        json.dump(table, f, indent=1)
    return table


def trace_summary(trace_csv, sweep_json, out_md):
    """Per-row kernel durations of a sweep run under rocprofv3 --kernel-trace:
    the marker dispatches cut the trace into rows; within a row every call
    (its kernels: 1 for the products, up to 3 for the expert-routed one) is
    one unit, its duration the sum of its kernels' (end - start); median,
    p10 and p90 over all replayed calls. Writes them into the sweep JSON and
    a markdown table."""
    import csv
    with open(trace_csv) as f:
        recs = list(csv.DictReader(f))
    key = lambda r, *names: next(r[n] for n in names if n in r)
    recs.sort(key=lambda r: int(key(r, "Start_Timestamp", "start_timestamp")))
    with open(sweep_json) as f:
        table = json.load(f)
    rows = {r["row_index"]: r for r in table if "row_index" in r}
    seg, cur = {}, None
    for r in recs:
        name = key(r, "Kernel_Name", "kernel_name")
        grid = int(key(r, "Grid_Size_X", "Grid_Size", "grid_size_x"))
        wg = int(key(r, "Workgroup_Size_X", "Workgroup_Size", "workgroup_size_x"))
        if "empty_kernel" in name and grid // max(wg, 1) >= SweepTimer.MARKER_BASE:
            m = grid // wg - SweepTimer.MARKER_BASE
            cur = None if m & 1 else m // 2
            if cur is not None:
                seg[cur] = []
            continue
        if cur is not None and cur in rows and _kernel_family(name).startswith("bqm::"):
            # (torch's own small kernels of the graph capture are left out)
            d = (int(key(r, "End_Timestamp", "end_timestamp")) -
                 int(key(r, "Start_Timestamp", "start_timestamp"))) / 1e3
            seg[cur].append((name, d))
    lines = ["| row | workload | op | T | calls | kernels per call | median µs | p10 | p90 | "
             "replay corr. | event-timed µs |", "|---|---|---|---|---|---|---|---|---|---|---|"]
    for idx, row in sorted(rows.items()):
        ds = seg.get(idx, [])
        # each row's graph is replayed twice (warm, then timed)
        ncalls = 2 * row["launches"]
        if not ds or len(ds) % ncalls:
            row["trace"] = {"dispatches": len(ds), "note": "dispatch count not a multiple of calls"}
            continue
        kpc = len(ds) // ncalls
        calls = [sum(d for _, d in ds[c * kpc:(c + 1) * kpc]) for c in range(ncalls)]
        # the two replays run the same launches on the same weight copies in
        # the same order: a duration spread tied to the copy (where its pages
        # sit in HBM) repeats from one replay to the other, one that comes
        # from the moment does not
        half = ncalls // 2
        a, b = calls[:half], calls[half:]
        ma, mb = sum(a) / half, sum(b) / half
        cov = sum((x - ma) * (z - mb) for x, z in zip(a, b))
        va = sum((x - ma) ** 2 for x in a)
        vb = sum((z - mb) ** 2 for z in b)
        replay_corr = cov / (va * vb) ** 0.5 if va > 0 and vb > 0 else 0.0
        calls.sort()
        q = lambda p: calls[min(len(calls) - 1, int(p * len(calls)))]
        med = calls[len(calls) // 2]
        row["trace"] = {"calls": ncalls, "kernels_per_call": kpc, "median_us": round(med, 3),
                        "p10_us": round(q(0.10), 3), "p90_us": round(q(0.90), 3),
                        "replay_corr": round(replay_corr, 3),
                        "kernels": sorted(set(_kernel_family(n) for n, _ in ds))}
        if kpc > 1:
            # calls of several kernels (the expert-routed product: routing
            # pre-pass, narrow items, wide items): each kernel's own median
            sub = {}
            for c in range(ncalls):
                for n, d in ds[c * kpc:(c + 1) * kpc]:
                    sub.setdefault(_kernel_family(n), []).append(d)
            row["trace"]["per_kernel_median_us"] = {
                k: round(sorted(v)[len(v) // 2], 3) for k, v in sorted(sub.items())}
        if "algorithmic_bytes" in row:
            row["trace"]["gbs_at_median"] = round(row["algorithmic_bytes"] / med / 1e3, 1)
        lines.append("| %d | %s | %s | %s | %d | %d | %.3f | %.3f | %.3f | %.2f | %.3f |" % (
            idx, row["workload"], row["op"], row.get("T", ""), ncalls, kpc, med, q(0.10),
            q(0.90), replay_corr, row["us"]))
    subs = [(idx, row) for idx, row in sorted(rows.items())
            if "per_kernel_median_us" in row.get("trace", {})]
    if subs:
        lines += ["", "| row | workload | op | T | kernel | median µs |", "|---|---|---|---|---|---|"]
        for idx, row in subs:
            for k, v in row["trace"]["per_kernel_median_us"].items():
                lines.append("| %d | %s | %s | %s | `%s` | %.3f |" % (
                    idx, row["workload"], row["op"], row.get("T", ""), k, v))
    with open(sweep_json, "w") as f:
        json.dump(table, f, indent=1)
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def sweep_report(sweep_json, traced_json=None, cpu_json=None):
    """Markdown tables of a sweep (event-timed rows; with traced_json, the
    per-dispatch median, p10 and p90 of the same rows from a traced run after
    --trace-summary; with cpu_json, the oracle's times from --cpu-table)."""
    with open(sweep_json) as f:
        rows = json.load(f)
    tr = {}
    if traced_json:
        with open(traced_json) as f:
            tr = {(r["workload"], r["op"], r.get("T")): r.get("trace") for r in json.load(f)
                  if r.get("trace") and "median_us" in r.get("trace", {})}
    cpu = {}
    if cpu_json:
        with open(cpu_json) as f:
            c = json.load(f)
        cpu = {(r["workload"], r["T"], r.get("op", "")): r for r in c["rows"]}
    out = ["| workload | op | N x K | T | event µs | GB/s | % of 8 TB/s | % of read probe | "
           "trace median µs (p10, p90) | GB/s at median | oracle µs, 1 thread / all | "
           "checksum |", "|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for r in rows:
        if r["op"] in ("read_probe", "copy_probe", "tq1_dequantize", "tq1_get_rows"):
            continue
        t = tr.get((r["workload"], r["op"], r.get("T")))
        cp = (cpu.get((r["workload"], r.get("T"), "mmvq_tq2_0" if "tq2" in r["op"] else ""))
              if r["op"].startswith("mmvq") and "glu" not in r["op"] else None)
        nk = ("%d x %d x %d" % (r["E"], r["N"], r["K"])) if "E" in r else (
            "%d x %d" % (r["N"], r["K"]))
        out.append("| %s | %s | %s | %s | %.3f | %.1f | %.1f | %s | %s | %s | %s | %s |" % (
            r["workload"] + ((" (%d distinct)" % r["distinct_experts"]) if "distinct_experts" in r
                             else ""),
            r["op"], nk, r.get("T", ""), r["us"], r["gbs"], 100 * r["frac_of_8tbs"],
            ("%.1f" % (100 * r["frac_of_read_probe"])) if r.get("frac_of_read_probe") else "",
            ("%.3f (%.3f, %.3f)" % (t["median_us"], t["p10_us"], t["p90_us"])) if t else "",
            ("%.1f" % t["gbs_at_median"]) if t and "gbs_at_median" in t else "",
            ("%.0f / %.0f" % (cp["oracle_us_one"], cp["oracle_us_all"])) if cp else "",
            ("%.6g" % r["checksum"]) if "checksum" in r else ""))
    out.append("")
    out.append("| workload | op | bytes | µs | GB/s | % of 8 TB/s |")
    out.append("|---|---|---|---|---|---|")
    for r in rows:
        if r["op"] in ("read_probe", "copy_probe", "tq1_dequantize", "tq1_get_rows"):
            b = r.get("bytes") or r.get("bytes_moved") or r.get("algorithmic_bytes")
            out.append("| %s | %s%s | %d | %.3f | %.1f | %.1f |" % (
                r["workload"], r["op"], (" " + r["dtype"]) if "dtype" in r else "", b, r["us"],
                r["gbs"], 100 * r["frac_of_8tbs"]))
    text = "\n".join(out)
    print(text)
    return text


def profile_run(spec, torch, np, bqm, synth, dev):
    """A few launches of one workload shape for counter collection: `launches`
    mat-vec calls on cold weight copies (or, with a fourth field mm, calls of
    the many-column product; with dq_f16, dq_bf16 or dq_f32, dequantizations
    of the whole matrix to that type),
    then as many streaming reads of the same weight bytes by the probe kernel
    and copies of them (references of known size)."""
    parts = spec.split(":")
    name, T = parts[0], int(parts[1])
    launches = int(parts[2]) if len(parts) > 2 else 20
    op = parts[3] if len(parts) > 3 else "mmvq"
    wl = synth.WORKLOADS[name]
    inp = synth.make_inputs(wl, T=T)
    N, K = wl.N, wl.K
    w0 = bqm.tq1_pack(torch.from_numpy(inp.trits).to(dev),
                      torch.from_numpy(inp.d16.view(np.int16)).to(dev))
    wrot, R = rotation(torch, w0, dev)
    a = bqm.q8_1_quantize(torch.from_numpy(inp.x[:T]).to(dev))
    if op == "mm":
        y = torch.empty((T, N), dtype=torch.float32, device=dev)
        run = lambda i: bqm.mm_tq1_0(wrot[i % R], a, N, K, T, out=y)
    elif op != "mmvq":
        dt = {"dq_f16": torch.float16, "dq_bf16": torch.bfloat16, "dq_f32": torch.float32}[op]
        dq = torch.empty((N, K), dtype=dt, device=dev)
        run = lambda i: bqm.tq1_dequantize(wrot[i % R], N, K, dtype=dt, out=dq)
    elif wl.experts:
        ids = torch.from_numpy(np.ascontiguousarray(inp.ids[:T])).to(dev)
        y = torch.empty((T, wl.n_used, N), dtype=torch.float32, device=dev)
        ws = torch.empty(max(bqm.mmvq_id_tq1_0_workspace_bytes(wl.experts, T, wl.n_used), 256),
                         dtype=torch.uint8, device=dev)
        run = lambda i: bqm.mmvq_id_tq1_0(wrot[i % R], a, ids, wl.experts, N, K, T, wl.n_used,
                                          out=y, workspace=ws)
    else:
        y = torch.empty((T, N), dtype=torch.float32, device=dev)
        run = lambda i: bqm.mmvq_tq1_0(wrot[i % R], a, N, K, T, out=y)
    torch.cuda.synchronize()
    for i in range(launches):
        run(i)
    torch.cuda.synchronize()
    if op == "mmvq" and not wl.experts and T <= bqm.MMVQ_F32_MAX_COLS:
        # the fused quantize-and-multiply kernel on the same shapes
        x = torch.from_numpy(inp.x[:T]).to(dev)
        for i in range(launches):
            bqm.mmvq_tq1_0_f32(wrot[(i + 5) % R], x, N, K, T, out=y)
        torch.cuda.synchronize()
    probes = ctypes.CDLL(os.path.join(ROOT, "bit_quantized_mat_amd", "libbqm_probes.so"))
    probes.bqm_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p,
                                      ctypes.c_int, ctypes.c_void_p]
    probes.bqm_probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64,
                                      ctypes.c_int, ctypes.c_void_p]
    pout = torch.empty(4096, dtype=torch.int32, device=dev)
    nbytes = w0.numel() - w0.numel() % 16
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for i in range(launches):
        probes.bqm_probe_read(ctypes.c_void_p(wrot[(i + 1) % R].data_ptr()), nbytes,
                              ctypes.c_void_p(pout.data_ptr()), 1024, stream)
    torch.cuda.synchronize()
    # the copies are all equal, so copying one onto another changes nothing
    for i in range(launches):
        probes.bqm_probe_copy(ctypes.c_void_p(wrot[(i + 2) % R].data_ptr()),
                              ctypes.c_void_p(wrot[(i + 3) % R].data_ptr()), nbytes, 1024,
                              stream)
    torch.cuda.synchronize()
    print(json.dumps({"profile": name, "op": op, "N": N, "K": K, "T": T, "launches": launches,
                      "weight_bytes": int(w0.numel()), "probe_bytes": int(nbytes),
                      "kernel_source_hash": kernel_source_hash()}), flush=True)


SPREAD_PATTERNS = (("graph of 300 calls, replayed twice", 600),
                   ("eager, back to back", 300),
                   ("eager, a device sync after each call", 300),
                   ("one warm weight copy, a device sync after each call", 300))


def spread_run(torch, np, bqm, synth, dev):
    """The decode step's fused call launched in four patterns, for a kernel
    trace of how per-dispatch durations spread: back to back in a graph,
    eagerly back to back, eagerly with a device sync after each call (cold
    weight copies), and with a sync after each call on one warm copy."""
    wl = synth.WORKLOADS["decode"]
    inp = synth.make_inputs(wl)
    N, K = wl.N, wl.K
    w0 = bqm.tq1_pack(torch.from_numpy(inp.trits).to(dev),
                      torch.from_numpy(inp.d16.view(np.int16)).to(dev))
    wrot, R = rotation(torch, w0, dev)
    x = torch.from_numpy(inp.x[:1]).to(dev)
    y = torch.empty((1, N), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    graph_us(torch, lambda i: bqm.mmvq_tq1_0_f32(wrot[i % R], x, N, K, 1, out=y), 300)
    log("spread: graph done")
    for i in range(300):
        bqm.mmvq_tq1_0_f32(wrot[i % R], x, N, K, 1, out=y)
    torch.cuda.synchronize()
    for i in range(300):
        bqm.mmvq_tq1_0_f32(wrot[i % R], x, N, K, 1, out=y)
        torch.cuda.synchronize()
    for i in range(300):
        bqm.mmvq_tq1_0_f32(wrot[0], x, N, K, 1, out=y)
        torch.cuda.synchronize()
    log("spread: done")


def spread_summary(trace_csv):
    """Median, p10, p90 of the fused call's dispatch durations per pattern of
    --spread, and the median gap from the previous dispatch's end (µs)."""
    import csv
    import statistics
    with open(trace_csv) as f:
        rows = [r for r in csv.DictReader(f)
                if "mmvq_staged_kernel<1, false, true, 4>" in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    st = [int(r["Start_Timestamp"]) for r in rows]
    en = [int(r["End_Timestamp"]) for r in rows]
    lines = ["| pattern | dispatches | median | p10 | p90 | min | max | gap to the previous dispatch (median) |",
             "|---|---|---|---|---|---|---|---|"]
    i = 0
    for name, n in SPREAD_PATTERNS:
        d = sorted((en[k] - st[k]) / 1e3 for k in range(i, i + n))
        gaps = [(st[k] - en[k - 1]) / 1e3 for k in range(i + 1, i + n)]
        lines.append("| %s | %d | %.3f | %.3f | %.3f | %.3f | %.3f | %.2f |" % (
            name, n, statistics.median(d), d[int(0.1 * (n - 1))], d[int(0.9 * (n - 1))], d[0],
            d[-1], statistics.median(gaps)))
        i += n
    return "\n".join(lines)


def _counter_medians(csv_dir, counter):
    """Median per-dispatch value of one counter, by kernel family, from a
    rocprofv3 --pmc csv output directory."""
    import csv
    import glob
    import statistics
    vals = {}
    for path in glob.glob(os.path.join(csv_dir, "*counter_collection.csv")):
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                name = r["Kernel_Name"]
                fam = ("copy_probe" if "copy_kernel" in name else
                       "read_probe" if "read_kernel" in name else
                       "fused" if "mmvq_staged_kernel<1, false, true, 4>" in name else
                       "mmvq" if "mmvq" in name else None)
                if fam:
                    vals.setdefault(fam, []).append(float(r["Counter_Value"]))
    return {k: statistics.median(v) for k, v in vals.items()}


def _kernel_family(name):
    """A kernel's name without its parameter list."""
    import re
    name = name.replace("(anonymous namespace)::", "")
    name = re.sub(r"^void ", "", name)
    return name.split("(")[0]


def counter_table(dirs, probe_bytes=None):
    """Median per-dispatch counter values by kernel, from rocprofv3 --pmc csv
    output directories (one per counter pass), as a markdown table; with
    probe_bytes (the bytes the read and copy probes move, printed by
    --profile), FETCH_SIZE and WRITE_SIZE also as bytes, scaled by bytes
    moved / counter reading of the copy probe."""
    import csv
    import glob
    import statistics
    vals = {}
    for d in dirs:
        for path in glob.glob(os.path.join(d, "*counter_collection.csv")):
            with open(path) as f:
                for r in csv.DictReader(f):
                    fam = _kernel_family(r["Kernel_Name"])
                    if not (fam in ("read_kernel", "copy_kernel") or fam.startswith("bqm::")):
                        continue
                    vals.setdefault(fam, {}).setdefault(r["Counter_Name"], []).append(
                        float(r["Counter_Value"]))
    med = {k: {c: statistics.median(v) for c, v in cs.items()} for k, cs in vals.items()}
    scale = {}
    if probe_bytes:
        cp = med.get("copy_kernel", {})
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            if cp.get(c):
                scale[c] = probe_bytes / cp[c]
    lines = ["| kernel | counter | median per dispatch | derived |", "|---|---|---|---|"]
    for k in sorted(med):
        cs = med[k]
        waves = cs.get("SQ_WAVES")
        for c in sorted(cs):
            v = cs[c]
            d = ""
            if c in scale:
                d = "%.0f bytes" % (v * scale[c])
            elif c == "SQ_INSTS_VALU" and waves:
                d = "%.0f per wave, %.0f per SIMD (%.2f us of issue at 4 cycles, 2.4 GHz)" % (
                    v / waves, v / 1024, v / 1024 * 4 / 2400)
            elif c.startswith("SQ_INSTS_") and waves:
                d = "%.1f per wave" % (v / waves)
            lines.append("| `%s` | %s | %.6g | %s |" % (k, c, v, d))
    out = "\n".join(lines)
    print(out)
    return out


def write_counters(fetch_dir, write_dir, probe_bytes):
    """HBM bytes per launch of the decode step's kernel (the fused quantize
    and mat-vec) from two counter runs of `--profile decode:1`: FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch), each scaled by bytes moved / counter
    reading of the copy probe, which reads and writes probe_bytes bytes."""
    f = _counter_medians(fetch_dir, "FETCH_SIZE")
    w = _counter_medians(write_dir, "WRITE_SIZE")
    fetch_scale = probe_bytes / f["copy_probe"]
    write_scale = probe_bytes / w["copy_probe"]
    wl_N, wl_K = 4096, 4096
    out = {"kernel_source_hash": kernel_source_hash(), "shape": [wl_N, wl_K, 1],
           "kernel": "mmvq_staged_kernel<1, false, true, 4> (mmvq_tq1_0_f32)",
           "fetch_size_kib": f["fused"], "write_size_kib": w["fused"],
           "copy_probe_bytes": probe_bytes, "copy_probe_fetch_kib": f["copy_probe"],
           "copy_probe_write_kib": w["copy_probe"],
           "read_probe_fetch_kib": f.get("read_probe"),
           "plain_mmvq_fetch_kib": f.get("mmvq"), "plain_mmvq_write_kib": w.get("mmvq"),
           "fetch_bytes_per_kib": round(fetch_scale, 3), "write_bytes_per_kib": round(write_scale, 3),
           "hbm_fetch_bytes_per_launch": round(f["fused"] * fetch_scale),
           "hbm_write_bytes_per_launch": round(w["fused"] * write_scale)}
    out["hbm_bytes_per_launch"] = out["hbm_fetch_bytes_per_launch"] + out["hbm_write_bytes_per_launch"]
    out["algorithmic_bytes_per_launch"] = fused_bytes(wl_N, wl_K, 1)
    with open(COUNTERS_FILE, "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")
    print(json.dumps(out))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--kernel-launches", type=int, default=400,
                    help="graph-captured launches of the dominant kernel")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sweep", metavar="PATH", help="also measure every workload; JSON table")
    ap.add_argument("--sweep-launches", type=int, default=100)
    ap.add_argument("--sweep-only", default="", help="comma-separated workload names")
    ap.add_argument("--spread", action="store_true",
                    help="only launch the decode step's fused call in four patterns (for a kernel "
                         "trace of per-dispatch spread; --spread-summary reads the trace)")
    ap.add_argument("--spread-summary", metavar="TRACE_CSV",
                    help="no GPU: per-pattern duration spread from a kernel trace of --spread")
    ap.add_argument("--profile", metavar="WORKLOAD:T[:LAUNCHES[:OP]]",
                    help="only run a few launches of one shape (for counter collection)")
    ap.add_argument("--write-counters", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "PROBE_BYTES"),
                    help="no GPU: turn two rocprofv3 --pmc runs of --profile decode:1 "
                         "(FETCH_SIZE, then WRITE_SIZE) into the committed traffic figures")
    ap.add_argument("--trace-summary", nargs=3, metavar=("TRACE_CSV", "SWEEP_JSON", "OUT_MD"),
                    help="no GPU: per-row median/p10/p90 kernel durations of a sweep run "
                         "under rocprofv3 --kernel-trace")
    ap.add_argument("--counter-table", nargs="+", metavar="DIR",
                    help="no GPU: markdown table of median counter values per kernel from "
                         "rocprofv3 --pmc output directories (a leading number is the probe "
                         "bytes for the FETCH_SIZE / WRITE_SIZE scale)")
    ap.add_argument("--sweep-report", nargs="+", metavar="JSON",
                    help="no GPU: markdown tables of a sweep JSON [traced sweep JSON after "
                         "--trace-summary [--cpu-table JSON]]")
    ap.add_argument("--cpu-table", metavar="PATH",
                    help="no GPU: time the oracle on every workload (one thread and all the "
                         "job's CPUs) and write a JSON table")
    args = ap.parse_args()

    if args.cpu_table:
        cpu_table(args.cpu_table)
        return
    if args.spread_summary:
        print(spread_summary(args.spread_summary))
        return
    if args.trace_summary:
        trace_summary(*args.trace_summary)
        return
    if args.sweep_report:
        sweep_report(*args.sweep_report)
        return
    if args.counter_table:
        first = args.counter_table[0]
        if first.isdigit():
            counter_table(args.counter_table[1:], int(first))
        else:
            counter_table(args.counter_table)
        return

    if args.write_counters:
        write_counters(args.write_counters[0], args.write_counters[1],
                       int(args.write_counters[2]))
        return

    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import bit_quantized_mat_amd as bqm
    from bit_quantized_mat_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.profile:
        profile_run(args.profile, torch, np, bqm, synth, dev)
        return
    if args.spread:
        spread_run(torch, np, bqm, synth, dev)
        return
    wl = synth.WORKLOADS["decode"]
    N, K, T = wl.N, wl.K, 1
    inp = synth.make_inputs(wl)
    log("workload decode N=%d K=%d T=%d" % (N, K, T))

    w0 = bqm.tq1_pack(torch.from_numpy(inp.trits).to(dev),
                      torch.from_numpy(inp.d16.view(np.int16)).to(dev))
    wbytes = w0.numel()
    wrot, R = rotation(torch, w0, dev)
    x = torch.from_numpy(inp.x[:T]).to(dev)
    a = torch.empty((T, (K // 32) * 36), dtype=torch.uint8, device=dev)
    y = torch.empty((T, N), dtype=torch.float32, device=dev)
    a_y = torch.empty((T, N), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    log("rotation: %d copies of %d bytes (%.2f GiB)" % (R, wbytes, R * wbytes / 2**30))

    # one step of the hot path: quantize the fp32 column and multiply, fused
    # into one launch (bitwise the same result as the two calls)
    def step(i):
        bqm.mmvq_tq1_0_f32(wrot[i % R], x, N, K, T, out=y)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    eager_us = (time.perf_counter() - t0) * 1e6 / args.steps
    # the same eager steps through the C ABI with no Python in the loop
    c_eager = c_abi_eager(torch, bqm, wrot, R, x, y, N, K, T, max(args.steps, 200))

    # timed region: the K steps as one graph
    step_us = graph_us(torch, lambda i: step(args.warmup + i), args.steps)
    # dominant kernel (the fused one): a graph of launches on rotating weights
    us_call = graph_us(torch, lambda i: bqm.mmvq_tq1_0_f32(wrot[(7 * i) % R], x, N, K, T, out=y),
                       args.kernel_launches)
    # for comparison: the same step as two calls, and each call alone
    two_call_us = graph_us(torch, lambda i: (bqm.q8_1_quantize(x, out=a),
                                             bqm.mmvq_tq1_0(wrot[(7 * i) % R], a, N, K, T, out=y)),
                           args.kernel_launches)
    mmvq_us = graph_us(torch, lambda i: bqm.mmvq_tq1_0(wrot[(7 * i) % R], a, N, K, T, out=y),
                       args.kernel_launches)
    quant_us = graph_us(torch, lambda i: bqm.q8_1_quantize(x, out=a), 200)
    # the residual-block form of the step: quantize, multiply and add the
    # residual in one launch, against the same with the add as a second launch
    resid = torch.randn((T, N), dtype=torch.float32, device=dev)
    add_fused_us = graph_us(torch, lambda i: bqm.mmvq_tq1_0_f32_add(
        wrot[(7 * i) % R], x, resid, N, K, T, out=y), args.kernel_launches)
    add_two_us = graph_us(torch, lambda i: (bqm.mmvq_tq1_0_f32(wrot[(7 * i) % R], x, N, K, T,
                                                               out=a_y),
                                            torch.add(a_y, resid, out=y)),
                          args.kernel_launches)
    grid_wg = -(-N // (4 * (64 >> lanes_per_row_log2(K // 256))))
    cal = calibrate(torch, np, wrot, R, wbytes, grid_wg)
    log("calibration:", cal)

    step_bytes = fused_bytes(N, K, T)
    achieved = step_bytes / us_call / 1e3
    value = step_bytes / step_us / 1e3
    log("fused quantize + mat-vec: %.3f us per call (graph of %d), %.1f GB/s = %.2f%% of %.0f GB/s"
        % (us_call, args.kernel_launches, achieved, 100 * achieved / HBM_PEAK_GBS, HBM_PEAK_GBS))
    log("two calls: %.3f us (quantize %.3f us, mat-vec %.3f us = %.1f GB/s)"
        % (two_call_us, quant_us, mmvq_us, algorithmic_bytes(N, K, T) / mmvq_us / 1e3))
    log("step: %.3f us graph-replayed, %.3f us eager from Python, %.3f us eager from C "
        "(%.3f us of host time to enqueue each call)"
        % (step_us, eager_us, c_eager["wall_us"], c_eager["enqueue_us"]))
    log("with a residual: %.3f us fused (quantize + mat-vec + add, one launch), %.3f us as "
        "mat-vec then a separate add" % (add_fused_us, add_two_us))

    table = None
    if args.sweep:
        del wrot
        torch.cuda.empty_cache()
        only = set(filter(None, args.sweep_only.split(",")))
        table = sweep(args.sweep, torch, np, bqm, synth, dev, args.sweep_launches, only)

    base = None
    if not args.no_cpu_baseline:
        base = cpu_baseline(inp, N, K, T, args.cpu_seconds)
        log("cpu baseline:", base)

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_us / 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic",
        "config": {"workload": "decode mat-vec TQ1_0 N=4096 K=4096 T=1 (fp32 column quantized to "
                               "Q8_1 and multiplied, one fused launch per step)",
                   "N": N, "K": K, "T": T, "weight_rotation_bytes": int(R * wbytes),
                   "timed": "HIP graph of all steps, replayed once after a warm replay"},
        "us_per_call": round(us_call, 4),
        "two_call_step_us": round(two_call_us, 4),
        "mmvq_us": round(mmvq_us, 4),
        "mmvq_gbs": round(algorithmic_bytes(N, K, T) / mmvq_us / 1e3, 2),
        "quantize_us": round(quant_us, 4),
        "us_per_step_eager": round(eager_us, 4),
        "us_per_step_eager_c_abi": c_eager,
        "residual_add_fused_us": round(add_fused_us, 4),
        "residual_add_two_launch_us": round(add_two_us, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic_from_counters(N, K, T),
                     "kernel": "mmvq_tq1_0_f32 (mmvq_staged_kernel<1, false, true, 4>)",
                     "algorithmic_bytes_per_launch": step_bytes},
        "calibration": cal,
        "cpu_baseline": base,
    }
    if table is not None:
        line["sweep_file"] = args.sweep
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
