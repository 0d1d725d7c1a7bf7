"""Decode-attention benchmark on one MI355X.

One step = one pass of the whole decode hot path over one batch: the fused
prologue (QK-RMSNorm + NeoX RoPE + K/V append, when the workload has one),
the split-K attention pass and the log-sum-exp merge.  By default (--mode
fused) that is one C-ABI call, gqa_decode_step (gqa_decode_step_multi with
several query tokens per sequence), i.e. one kernel launch; --mode split
makes it three calls (prologue, split-K pass, merge).  Every launch goes to
torch's current stream and every input is already resident in HBM.  Before
each timed step, a read-only sweep of a 1 GiB buffer evicts the KV rows from
the L2s and the 256 MB Infinity Cache so they are read from HBM (outside the
timed region).  --graph captures one step in a HIP graph and times its
replays instead of eager launches.

The default workload is the largest single-GPU one: long-context
flash-decoding, L = 131072 rows, 64 partitions of 2048 rows merged by
log-sum-exp (537 MB of K/V per step).  Timing runs in --rounds independent
rounds of --steps steps each; ``ms_per_step`` is the mean of the round
medians.

Prints ONE JSON line.  ``value`` is the step's KV-read throughput: KV-cache
bytes the step must read (K and V rows of every attended window, bf16) per
second of whole-step time, in GB/s.  ``roofline`` rates the dominant kernel
(the fused step kernel, or the split-K pass with --mode split) against
MI355X's 8 TB/s HBM peak, with its duration from HIP events (created without
the system-scope fence) recorded on the launch stream around the kernel;
``traffic`` is the measured HBM bytes per launch from committed rocprofv3
counters when they were taken on the current kernel source.
``context.read_ceiling`` is a plain streaming read of exactly the step's KV
bytes (gqa_probe_stream_read, best of a few launch shapes) timed in the same
run after the same sweep: what the part streams for that many bytes.
``cpu_baseline`` times the fp64 CPU oracle on the same workload on this host,
with all the host's BLAS threads and with one.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--rounds R]
                       [--workload 4] [--mode fused|split] [--graph]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = ("decode-attention µs/step and achieved KV-read HBM GB/s "
          "(% of MI355X peak)")
HBM_PEAK_GBS = 8000.0
ATTN_SRC = os.path.join(ROOT, "gqa_attention_kv_amd", "csrc", "attn_decode_mfma.hip")
ATTN_KERNEL = "attn_decode_mfma_kernel"

WORKLOAD_NAMES = {
    "1": "tiny GQA decode step",
    "2a": "Qwen3-0.6B-shaped decode layer, L=512",
    "2b": "Qwen3-0.6B-shaped decode layer, L=2048",
    "3": "Llama-3-8B-shaped batched decode, ragged lengths",
    "4": "long-context flash-decoding, L=131072",
    "5": "70B-shaped sliding-window GQA decode (8:1)",
    "6": "draft-token verification: S=4 causal query tokens per sequence, Llama-3-8B shape",
    "7": "chunked prefill: the last 1024 tokens of four 8192-row sequences as causal "
         "queries, Llama-3-8B shape",
    "7f": "fresh-sequence causal prefill, S=1024, D=128, Llama-3-8B heads",
    "8": "packed QKV projection of the 70B-shaped decode batch (M=8, K=8192, N=10240)",
    "8a": "bf16 GEMV, one row, K=2048, N=8192",
    "8b": "bf16 GEMV, one row, K=4096, N=14336",
}
GEMV_WORKLOADS = ("8", "8a", "8b")
GEMV_KERNEL = "qkv_gemv_kernel"
PREFILL_WORKLOADS = ("7", "7f")
PREFILL_KERNEL = "attn_prefill_kernel"
PREFILL_SRC = os.path.join(ROOT, "gqa_attention_kv_amd", "csrc", "attn_prefill_mfma.hip")
GEMV_SRC = os.path.join(ROOT, "gqa_attention_kv_amd", "csrc", "qkv_gemv.hip")
MFMA_BF16_PEAK_TFLOPS = 2500.0


def _parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="4", choices=sorted(WORKLOAD_NAMES))
    ap.add_argument("--rounds", type=int, default=3,
                    help="independent timing rounds of --steps steps each")
    ap.add_argument("--graph", action="store_true",
                    help="capture one step in a HIP graph and time its replays")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the same-run streaming-read ceiling")
    ap.add_argument("--flush", default="read", choices=["read", "rmw", "none"],
                    help="cache sweep between steps: read a 1 GiB buffer (default), "
                         "read-modify-write it, or none (warm-cache figure)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-context", action="store_true",
                    help="skip the warm-cache figure (its extra launches would otherwise "
                         "appear in a kernel trace of this run)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="minimum CPU time spent timing the oracle")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also time a plain device copy of this many MiB")
    ap.add_argument("--part-tokens", type=int, default=0,
                    help="override the workload's split-K partition size")
    ap.add_argument("--mode", default="fused",
                    choices=["fused", "split", "prefill", "prefill_step"],
                    help="fused: the whole step as one launch (default); split: "
                         "prologue, split-K pass and merge as three launches; prefill: "
                         "prologue and the matrix-core prefill kernel; prefill_step: "
                         "the K/V append and the prefill kernel rotating q itself "
                         "(gqa_prefill_step, two launches timed together; the default "
                         "for the prefill workloads with a prologue)")
    ap.add_argument("--splits", type=int, default=0,
                    help="prefill: key splits per row block (0: the library's "
                         "suggestion for the device, gqa_attn_prefill_default_splits)")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU run: turn two rocprofv3 --pmc output directories "
                         "(FETCH_SIZE, WRITE_SIZE; each from a bench run with "
                         "--copy-probe-mib) into profiles/attn_traffic_workload<W>.json "
                         "(the attention kernel of the workload: decode or prefill)")
    return ap.parse_args()


def _src_sha(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def _kernel_of(workload: str):
    """(kernel name, kernel source) of the workload's dominant launch."""
    if workload in PREFILL_WORKLOADS:
        return PREFILL_KERNEL, PREFILL_SRC
    if workload in GEMV_WORKLOADS:
        return GEMV_KERNEL, GEMV_SRC
    return ATTN_KERNEL, ATTN_SRC


def _traffic(workload: str):
    """HBM bytes per attention launch from committed rocprofv3 counters, if
    they were taken on the current source of that kernel."""
    path = os.path.join(ROOT, "profiles", f"attn_traffic_workload{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    kernel, src = _kernel_of(workload)
    if rec.get("kernel") != kernel or rec.get("attn_src_sha") != _src_sha(src):
        return None
    return rec.get("bytes_per_launch")


def _pmc_rows(d: str):
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    with open(files[0]) as f:
        return list(csv.DictReader(f))


def _per_launch(rows, counter, kernel):
    """(mean KiB per attention dispatch, calibration factor from the copy
    probe: true bytes / counted bytes for a 256 MiB device copy)."""
    rows = [r for r in rows if r["Counter_Name"] == counter]
    attn = [float(r["Counter_Value"]) for r in rows if kernel in r["Kernel_Name"]]
    if not attn:
        raise SystemExit(f"{counter}: no {kernel} dispatches")
    last_attn = max(int(r["Dispatch_Id"]) for r in rows if kernel in r["Kernel_Name"])
    copies = [float(r["Counter_Value"]) for r in rows
              if "copyBuffer" in r["Kernel_Name"] and int(r["Dispatch_Id"]) > last_attn]
    # the probe's 256 MiB copies are the largest copy dispatches after the timed loop
    copies = [c for c in copies if copies and c >= 0.5 * max(copies)]
    if not attn or not copies:
        raise SystemExit(f"{counter}: attention or copy-probe dispatches missing")
    probe_kib = 256 * 1024     # the copy probe reads 256 MiB and writes 256 MiB
    factor = probe_kib / statistics.median(copies)
    return statistics.fmean(attn), factor


def _record_traffic(workload: str, fetch_dir: str, write_dir: str):
    kernel, src = _kernel_of(workload)
    f_kib, f_fac = _per_launch(_pmc_rows(fetch_dir), "FETCH_SIZE", kernel)
    w_kib, w_fac = _per_launch(_pmc_rows(write_dir), "WRITE_SIZE", kernel)
    rec = {
        "workload": workload,
        "kernel": kernel,
        "attn_src_sha": _src_sha(src),
        "fetch_kib_counted": round(f_kib, 1), "fetch_calibration": round(f_fac, 4),
        "write_kib_counted": round(w_kib, 1), "write_calibration": round(w_fac, 4),
        "bytes_per_launch": int(round((f_kib * f_fac + w_kib * w_fac) * 1024)),
        "read_bytes_per_launch": int(round(f_kib * f_fac * 1024)),
        "write_bytes_per_launch": int(round(w_kib * w_fac * 1024)),
    }
    out = os.path.join(ROOT, "profiles", f"attn_traffic_workload{workload}.json")
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec))


class _HipEvents:
    """Timing events of the HIP runtime torch has loaded, created without the
    system-scope release (hipEventDisableSystemFence), which costs several
    microseconds per record; recorded on the stream the kernels run on."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, count: int):
        import ctypes
        path = None
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    path = line.split()[-1]
                    break
        if path is None:
            raise RuntimeError("the HIP runtime is not loaded")
        self._c = ctypes
        self.hip = ctypes.CDLL(path)
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = []
        for _ in range(count):
            e = ctypes.c_void_p()
            if self.hip.hipEventCreateWithFlags(ctypes.byref(e), self.DISABLE_SYSTEM_FENCE) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            self.ev.append(e)

    def record(self, i: int, stream: int):
        if self.hip.hipEventRecord(self.ev[i], self._c.c_void_p(stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def ms(self, i: int, j: int) -> float:
        t = self._c.c_float()
        if self.hip.hipEventElapsedTime(self._c.byref(t), self.ev[i], self.ev[j]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return t.value

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(e)
        self.ev = []


def _timed_reps(fn, min_seconds: float):
    """(repetitions, seconds): call fn until min_seconds have passed (once at least)."""
    reps, t0 = 0, time.perf_counter()
    while True:
        fn()
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            return reps, el


def _cpu_baseline(w, min_seconds: float):
    """Time the fp64 oracle's decode step on this host (a baseline, not a
    target): with every BLAS thread numpy has, then with one thread."""
    import threadpoolctl
    import workloads
    from oracle import reference as oracle

    info = threadpoolctl.threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info] or [1])
    reps, el = _timed_reps(lambda: oracle.decode_step(w, split=False), min_seconds)
    with threadpoolctl.threadpool_limits(1):
        reps1, el1 = _timed_reps(lambda: oracle.decode_step(w, split=False), min_seconds)
    kvb = workloads.kv_bytes(w)
    return {
        "value": round(kvb * reps / el / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "cpu_model": _cpu_model(),
        "us_per_step": round(1e6 * el / reps),
        "single_thread": {"value": round(kvb * reps1 / el1 / 1e9, 4), "unit": "GB/s",
                          "cores": 1, "us_per_step": round(1e6 * el1 / reps1)},
        "sample": (f"{reps} full decode step(s) of the same workload (prologue + unsplit "
                   f"attention, float64 numpy) on {threads} threads, {el:.1f} s wall, "
                   f"{1e6 * el / reps:.0f} us/step; {reps1} on one thread, {el1:.1f} s, "
                   f"{1e6 * el1 / reps1:.0f} us/step"),
    }


# Launch shapes (workgroups, threads, loads in flight per thread) tried for
# the streaming-read ceiling; the best median is reported.
_CEILING_SHAPES = [(256, 256, 8), (256, 512, 8), (256, 1024, 4), (256, 256, 16),
                   (512, 256, 8), (512, 512, 4), (1024, 256, 4), (2048, 256, 4)]


def _read_ceiling(dev, nbytes: int, sweep, reps: int = 5):
    """A plain streaming read of exactly ``nbytes`` bytes (one contiguous
    buffer, each byte read once) after the same cache sweep as the timed
    steps: the median over ``reps`` launches for each launch shape, best
    shape reported."""
    import torch
    from gqa_attention_kv_amd import probe_stream_read

    nb = nbytes - nbytes % 16
    buf = torch.ones(nb // 4, dtype=torch.int32, device=dev)
    sink = torch.empty(max(wg * th for wg, th, _ in _CEILING_SHAPES), dtype=torch.int32,
                       device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    ev = _HipEvents(2 * reps)
    best = None
    every = {}
    for wg, th, un in _CEILING_SHAPES:
        probe_stream_read(buf, wg, th, un, sink=sink)       # warm the shape
        ts = []
        for i in range(reps):
            sweep()
            ev.record(2 * i, stream)
            probe_stream_read(buf, wg, th, un, sink=sink)
            ev.record(2 * i + 1, stream)
        torch.cuda.synchronize()
        ts = [ev.ms(2 * i, 2 * i + 1) for i in range(reps)]
        med = statistics.median(ts)
        every[f"{wg}x{th}x{un}"] = round(1e3 * med, 2)
        if best is None or med < best[0]:
            best = (med, wg, th, un)
    ev.close()
    med, wg, th, un = best
    gbps = nb / (med * 1e-3) / 1e9
    return {"bytes": nb, "us": round(1e3 * med, 2), "GBps": round(gbps, 1),
            "frac_of_peak": round(gbps / HBM_PEAK_GBS, 4),
            "shape": {"workgroups": wg, "threads": th, "loads_in_flight": un},
            "us_by_shape": every, "kernel": "stream_read_kernel"}


def _cpu_baseline_prefill(w, min_seconds: float):
    """Time the fp64 oracle on a bounded sample of a prefill step's tokens:
    each sampled token is single-token attention over its own rows (what the
    oracle's multi-token attention does per token), scaled to the whole step
    by its share of the step's attended rows."""
    import threadpoolctl
    import workloads
    from oracle import reference as oracle

    info = threadpoolctl.threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info] or [1])
    q = oracle.bf16_to_f64(w.q)
    rows = w.token_rows()                       # [B,S]
    order = np.random.default_rng(0).permutation(w.S)
    back = np.arange(w.S - 1, -1, -1) if w.causal else np.zeros(w.S, np.int64)
    done, toks, t0 = 0, 0, time.perf_counter()
    while True:
        s = int(order[toks % w.S])
        lens_s = w.lens.astype(np.int64) - back[s]
        oracle.attend(q[:, s], w.k_cache, w.v_cache, lens_s, w.window, 0.0)
        done += int(rows[:, s].sum())
        toks += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    est_step = el * float(rows.sum()) / max(done, 1)
    kvb = workloads.kv_bytes(w)
    return {
        "value": round(kvb / est_step / 1e9, 6),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "cpu_model": _cpu_model(),
        "sample": (f"{toks} of the step's {w.S} query tokens (all {w.B} sequences and "
                   f"{w.Hq} heads each; float64 numpy attention), {el:.1f} s wall, "
                   f"scaled by attended rows to {est_step:.1f} s per step; the prologue "
                   f"is not timed"),
    }


def _context(dev, run_once, warm_steps: int = 20, capture=None):
    """Context figures outside the timed rounds, all with warm caches (no
    sweep in between), HIP events on the launch stream:
    ``warm_us_per_step`` -- the mean of ``warm_steps`` event pairs, one
    around each step; ``warm_back_to_back_us_per_step`` -- ``warm_steps``
    steps between one event pair (the host enqueues ahead, unless its own
    per-call cost is the larger); with ``capture`` (a function returning a
    HIP graph of n consecutive steps), ``graph_of_steps_us_per_step`` -- one
    replay of a graph of ``warm_steps`` steps between one event pair."""
    import torch
    ev = _HipEvents(2 * warm_steps + 4)
    stream = torch.cuda.current_stream(dev).cuda_stream
    run_once()
    torch.cuda.synchronize()
    for i in range(warm_steps):
        ev.record(2 * i, stream)
        run_once()
        ev.record(2 * i + 1, stream)
    torch.cuda.synchronize()
    warm = statistics.fmean(ev.ms(2 * i, 2 * i + 1) for i in range(warm_steps))
    k = 2 * warm_steps
    ev.record(k, stream)
    for _ in range(warm_steps):
        run_once()
    ev.record(k + 1, stream)
    torch.cuda.synchronize()
    out = {"warm_us_per_step": round(1e3 * warm, 2),
           "warm_back_to_back_us_per_step": round(1e3 * ev.ms(k, k + 1) / warm_steps, 2)}
    if capture is not None:
        g = capture(warm_steps)
        g.replay()
        torch.cuda.synchronize()
        ev.record(k + 2, stream)
        g.replay()
        ev.record(k + 3, stream)
        torch.cuda.synchronize()
        out["graph_of_steps_us_per_step"] = round(1e3 * ev.ms(k + 2, k + 3) / warm_steps, 2)
        del g
    ev.close()
    return out


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _copy_probe(mib: int, dev, sweep):
    """Time a plain device copy of ``mib`` MiB (five runs, median) after the
    timed loop: its dispatches calibrate the FETCH_SIZE / WRITE_SIZE
    counters (--record-traffic)."""
    if not mib:
        return None
    import torch
    n = mib << 18
    src = torch.ones(n, dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    ts = []
    for _ in range(5):
        sweep()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b))
    t = statistics.median(ts)
    return {"bytes": 2 * n * 4, "ms": round(t, 4), "GBps": round(2 * n * 4 / (t * 1e-3) / 1e9, 1)}


def _bench_gemv(args, dev):
    """The packed QKV projection: one launch per step, weights read once."""
    import torch

    import workloads
    from gqa_attention_kv_amd.runner import DeviceGemv

    g = workloads.make_gemv(args.workload)
    nbytes = workloads.gemv_bytes(g)
    run = DeviceGemv(g, device=dev)
    # 1 GiB of int64, summed as int64: summing an int32 buffer into an int64
    # result made torch widen the whole buffer first (a 2 GiB temporary
    # written before every step, dirty lines included)
    flush = None if args.flush == "none" else torch.ones(1 << 27, dtype=torch.int64,
                                                          device=dev)
    flush_sink = torch.zeros((), dtype=torch.int64, device=dev)

    def sweep():
        if args.flush == "read":
            torch.sum(flush, dim=0, out=flush_sink)
        elif args.flush == "rmw":
            flush.add_(1)

    stream = torch.cuda.current_stream(dev).cuda_stream
    timer = _HipEvents(2 * args.steps)
    for _ in range(args.warmup):
        sweep()
        run.run()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for i in range(args.steps):
        sweep()
        timer.record(2 * i, stream)
        run.run()
        timer.record(2 * i + 1, stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = [timer.ms(2 * i, 2 * i + 1) for i in range(args.steps)]
    timer.close()
    mean = statistics.fmean(ms)
    gbps = nbytes / (mean * 1e-3) / 1e9
    context = {} if args.no_context else _context(dev, run.run)
    if not args.no_ceiling:
        context["read_ceiling"] = _read_ceiling(dev, nbytes, sweep)
        context["read_ceiling"]["step_frac_of_ceiling"] = round(
            gbps / context["read_ceiling"]["GBps"], 4)
    context = context or None
    copy_probe = _copy_probe(args.copy_probe_mib, dev, sweep)
    cpu = None
    if not args.no_cpu_baseline:
        import threadpoolctl
        from oracle import reference as oracle
        info = threadpoolctl.threadpool_info()
        threads = max([i.get("num_threads", 1) for i in info] or [1])
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle.linear(g.x, g.w)
            reps += 1
            el = time.perf_counter() - t0
            if el >= args.cpu_seconds:
                break
        cpu = {"value": round(nbytes * reps / el / 1e9, 4), "unit": "GB/s", "cores": threads,
               "kind": "oracle", "cpu_model": _cpu_model(),
               "sample": (f"{reps} full projection(s) of the same workload (bf16 widened to "
                          f"float64, numpy matrix product), {el:.1f} s wall, "
                          f"{1e6 * el / reps:.0f} us each")}
    line = {
        "metric": METRIC,
        "value": round(gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(mean, 5),
        "us_per_step": round(1e3 * mean, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": WORKLOAD_NAMES[args.workload],
            "M": g.M, "N": g.N, "K": g.K, "out_dtype": g.out_dtype, "path": "gemv",
            "bytes_per_step": nbytes,
            "cache_sweep_between_steps": args.flush,
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "hbm",
            "kernel": GEMV_KERNEL,
            "achieved": round(gbps, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(gbps / HBM_PEAK_GBS, 4),
            "traffic": _traffic(args.workload),
        },
        "kernels_us": {
            "mode": "gemv",
            "gemv": round(1e3 * mean, 2),
            "step_median": round(1e3 * statistics.median(ms), 2),
            "step_p10": round(1e3 * sorted(ms)[len(ms) // 10], 2),
            "step_p90": round(1e3 * sorted(ms)[(9 * len(ms)) // 10], 2),
        },
        "context": context,
        "wall_s_timed_loop": round(wall, 4),
        "output_finite": bool(torch.isfinite(run.y.float()).all().item()),
        "cpu_baseline": cpu,
    }
    if copy_probe:
        line["copy_probe"] = copy_probe
    print(json.dumps(line), flush=True)


def main():
    args = _parse()
    if args.record_traffic:
        _record_traffic(args.workload, *args.record_traffic)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    import workloads
    from gqa_attention_kv_amd import prefill_default_splits
    from gqa_attention_kv_amd.runner import DeviceStep

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.workload in GEMV_WORKLOADS:
        _bench_gemv(args, dev)
        return

    w = workloads.make(args.workload)
    if args.part_tokens:
        w.part_tokens = args.part_tokens
    kvb = workloads.kv_bytes(w)
    mode = args.mode
    splits = 1
    if args.workload in PREFILL_WORKLOADS:
        # with a prologue, the K/V append and the prefill kernel that rotates
        # q itself (two launches) unless --mode prefill asks for the
        # standalone prologue before it
        mode = "prefill" if args.mode == "prefill" or w.pos is None else "prefill_step"
        # key splits: the library's suggestion for this device unless given
        splits = args.splits or prefill_default_splits(w.B, w.S, w.Hq, w.Hkv)
    step = DeviceStep(w, device=dev, mode=mode, splits=splits)
    # 1 GiB of int64, summed as int64: summing an int32 buffer into an int64
    # result made torch widen the whole buffer first (a 2 GiB temporary
    # written before every step, dirty lines included)
    flush = None if args.flush == "none" else torch.ones(1 << 27, dtype=torch.int64,
                                                          device=dev)
    flush_sink = torch.zeros((), dtype=torch.int64, device=dev)

    def sweep():
        # A read-only sweep leaves the caches full of clean lines, so the timed
        # kernels pay no write-back of somebody else's dirty data.
        if args.flush == "read":
            torch.sum(flush, dim=0, out=flush_sink)
        elif args.flush == "rmw":
            flush.add_(1)

    one_call = mode in ("fused", "prefill_step") or args.graph

    def run_once():
        if mode in ("fused", "prefill_step"):
            step.run()
        else:
            step.prologue()
            step.attention()
            step.merge()

    def capture(nsteps: int):
        """A HIP graph of nsteps consecutive steps (all of their launches);
        warmed up on a side stream first, as capture requires."""
        side = torch.cuda.Stream(dev)
        side.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(side):
            for _ in range(2):
                run_once()
        torch.cuda.current_stream(dev).wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(nsteps):
                run_once()
        torch.cuda.synchronize()
        return g

    graph = capture(1) if args.graph else None

    stream = torch.cuda.current_stream(dev).cuda_stream   # every launch goes here
    timer = _HipEvents(4 * args.steps)

    def one_step(i=None):
        sweep()
        rec = (lambda k: timer.record(4 * i + k, stream)) if i is not None else (lambda k: None)
        rec(0)
        if graph is not None:
            graph.replay()
            rec(3)
            return
        if one_call:                           # one call: one event pair
            step.run()
            rec(3)
            return
        step.prologue()
        rec(1)
        step.attention()
        rec(2)
        step.merge()
        rec(3)

    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
    rounds, step_all, attn_all, pro_all, merge_all = [], [], [], [], []
    wall = 0.0
    for r in range(args.rounds):
        wall0 = time.perf_counter()
        for i in range(args.steps):
            one_step(i)
        torch.cuda.synchronize()
        wall += time.perf_counter() - wall0
        st = [timer.ms(4 * i, 4 * i + 3) for i in range(args.steps)]
        if one_call:
            at, pr, mg = st, [0.0], [0.0]
        else:
            pr = [timer.ms(4 * i, 4 * i + 1) for i in range(args.steps)]
            at = [timer.ms(4 * i + 1, 4 * i + 2) for i in range(args.steps)]
            mg = [timer.ms(4 * i + 2, 4 * i + 3) for i in range(args.steps)]
        ss = sorted(st)
        rounds.append({"median_us": round(1e3 * statistics.median(st), 2),
                       "mean_us": round(1e3 * statistics.fmean(st), 2),
                       "p10_us": round(1e3 * ss[len(ss) // 10], 2),
                       "p90_us": round(1e3 * ss[(9 * len(ss)) // 10], 2),
                       "attn_median_us": round(1e3 * statistics.median(at), 2)})
        step_all += st
        attn_all.append(statistics.median(at))
        pro_all += pr
        merge_all += mg
    timer.close()
    # the mean of the round medians
    mean_step = statistics.fmean(statistics.median(step_all[r * args.steps:(r + 1) * args.steps])
                                 for r in range(args.rounds))
    mean_attn = statistics.fmean(attn_all)

    context = {}
    if not args.no_context:
        context.update(_context(dev, graph.replay if graph is not None else run_once,
                                capture=capture if args.graph else None))
    ceiling = None
    if not args.no_ceiling and mode not in ("prefill", "prefill_step"):
        ceiling = _read_ceiling(dev, kvb, sweep)
        context["read_ceiling"] = ceiling
    value = kvb / (mean_step * 1e-3) / 1e9
    achieved = kvb / (mean_attn * 1e-3) / 1e9
    if ceiling:
        ceiling["step_frac_of_ceiling"] = round(achieved / ceiling["GBps"], 4)

    finite = bool(torch.isfinite(step.out.float()).all().item())

    copy_probe = _copy_probe(args.copy_probe_mib, dev, sweep)

    if args.no_cpu_baseline:
        cpu = None
    elif mode in ("prefill", "prefill_step"):
        cpu = _cpu_baseline_prefill(w, args.cpu_seconds)
    else:
        cpu = _cpu_baseline(w, args.cpu_seconds)

    traffic = _traffic(args.workload)
    if mode in ("prefill", "prefill_step"):
        flops = workloads.attention_flops(w)
        tflops = flops / (mean_attn * 1e-3) / 1e12
        roofline = {
            "bound": "mfma",
            "kernel": PREFILL_KERNEL + (" (with the K/V append launch)"
                                        if mode == "prefill_step" else ""),
            "achieved": round(tflops, 1),
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": traffic,
            "flops_per_launch": flops,
        }
        dtype = ("bf16 MFMA (bf16 q and P), fp32 accumulate and softmax"
                 if w.out_dtype == "bf16" else
                 "bf16 MFMA (P as a bf16 hi+lo pair), fp32 accumulate and softmax")
    else:
        roofline = {
            "bound": "hbm",
            "kernel": ATTN_KERNEL + (" (whole fused step)" if mode == "fused"
                                     else " (split-K partition pass)"),
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "bytes_per_launch": kvb,
        }
        dtype = ("bf16 K/V on bf16 MFMA with q and P as bf16 hi+lo pairs (~16 significant "
                 "bits), fp32 accumulate, softmax and merge")
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "rounds": args.rounds,
        "ms_per_step": round(mean_step, 5),
        "us_per_step": round(1e3 * mean_step, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {
            "workload": WORKLOAD_NAMES[args.workload],
            "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "head_dim": w.D, "T": w.T,
            "query_tokens": w.S,
            "window": w.window, "part_tokens": w.part_tokens, "out_dtype": w.out_dtype,
            "path": mode + (" (HIP graph replay)" if args.graph else ""),
            **({"key_splits": splits} if mode in ("prefill", "prefill_step") else {}),
            "prologue": ("qk_rmsnorm+rope+append" if w.w_q is not None else
                         "rope+append") if w.pos is not None else "none",
            "kv_bytes_per_step": kvb,
            "cache_sweep_between_steps": args.flush,
            "parallelism": "single GPU",
        },
        "roofline": roofline,
        "kernels_us": {
            "mode": mode,
            "graph": bool(args.graph),
            "prologue": round(1e3 * statistics.fmean(pro_all), 2),
            "attn": round(1e3 * mean_attn, 2),
            "merge": round(1e3 * statistics.fmean(merge_all), 2),
            "rounds": rounds,
        },
        "context": context or None,
        "wall_s_timed_loop": round(wall, 4),
        "output_finite": finite,
        "cpu_baseline": cpu,
    }
    if copy_probe:
        line["copy_probe"] = copy_probe
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
