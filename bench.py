#!/usr/bin/env python3
"""Throughput of the gfx950 dense GEMM on its headline workloads.

One step = one FP32 GEMM D = A*B at M=N=K=4096 followed by one BF16-input /
FP32-accumulate GEMM at M=N=K=8192 (row-major, no transpose, alpha=1,
beta=0), both through the library's C ABI with automatic kernel selection.
Inputs are seeded synthetic matrices (uniform[-1,1] fp32; normal(0,1) rounded
to bf16), generated on the host and resident in HBM before timing.  Two
buffer sets per workload are used in turn so that consecutive launches do not
find their inputs in cache.

Prints one JSON line: whole-job TFLOP/s (2*M*N*K summed over the step /
step time), per-workload rates and fractions of the MI355X dense peaks, a
roofline entry for the kernel that dominates the step, and the CPU oracle's
rate on a bounded sample of the same workloads (a reported baseline only).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

METRIC = ("GEMM TFLOPS (2MNK/s) FP32 4096³ & BF16→FP32 8192³; "
          "% of MI355X dense peak")
# MI355X published dense peaks (TFLOP/s) and HBM bandwidth (GB/s)
PEAK_TFLOPS = {"f32": 157.3, "bf16": 2516.6}
# fp32 vector ALU: 256 CUs x 256 FLOP per clock x 2.4 GHz = the published
# 157.3 TFLOP/s.  gfx950 reaches it without packed FP32 instructions (which
# this library does not emit): the two-operand v_fmac_f32 encoding issues at
# 2 FMAs per lane per clock (measured 222-226 FLOP/clock/CU), the
# three-operand v_fma_f32 at 1.
VALU_FP32_TFLOPS = 256 * 256 * 2.4e9 / 1e12
HBM_GBS = 8000.0
STEP_WORKLOADS = ("fp32_4096", "bf16_8192")
# the vector-FMA (no matrix cores) fp32 kernel reported beside the step
VECTOR_FMA_VARIANT = "f32_vfma_128x256x16_t8x16"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")


def compulsory_bytes(w: workloads.Workload, out_bytes: int = 4) -> int:
    """Read A and B once, read C once if beta != 0, write D once (C and D of
    out_bytes per element).

    The one-pass traffic of "Understanding Roofline and Tiling through Matrix
    Multiplication", section 8.5 (12 N^2 bytes for square fp32), generalized to
    M x N x K, bf16 operands and the beta*C read ("GEMM on NVIDIA GPUs",
    section 2, ideal traffic).
    """
    ea = 4 if w.dtype == "f32" else 2
    c = out_bytes * w.M * w.N if w.beta != 0.0 else 0
    return ea * (w.M * w.K + w.K * w.N) + c + out_bytes * w.M * w.N


# the sources that define the step's kernels (the direct-to-LDS template and
# the instantiation files of the selected variants)
STEP_KERNEL_SOURCES = ("common.hpp", "mfma_dma_gemm.hpp", "sk_ranges.hpp", "variants.hpp",
                       "selected_configs.hpp", "inst_bf16_dma.hip", "inst_f32_dma.hip")


def kernel_source_digest() -> str:
    """Digest of the device code of the step's kernels: a traffic record
    measured on other code is not reported."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "dense_gemm_11_amd", "csrc")
    for name in STEP_KERNEL_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


MFMA_KIND = {"mfma32x32x2": 0, "mfma16x16x4": 1, "mfma32x32x16": 2, "mfma16x16x32": 3}


def kernel_name_key(variant_name: str, tile) -> str:
    """Start of the template arguments, in the demangled kernel name, that
    identify a variant (the direct-to-LDS configuration continues with its
    pairing mode, register hint and pair-buffer count, which the selected
    variants' names do not spell out; they are one kernel each in a
    record)."""
    bm, bn, bk = tile
    for tag, kind in MFMA_KIND.items():
        if f"_{tag}_" in variant_name:
            return f"MfmaConfig<{kind}, {bm}, {bn}, {bk},"
        if f"_dma{tag[4:]}_" in variant_name:
            late = "_late" in variant_name
            stages = re.search(r"_s(\d+)(?:_|$)", variant_name).group(1)
            wm, wn = re.search(r"_w(\d+)x(\d+)_", variant_name).groups()
            return (f"DmaConfig<{kind}, {bm}, {bn}, {bk}, {wm}, {wn}, {stages}, "
                    f"{'true' if late else 'false'}")
    return f"FmaConfig<{bm}, {bn}, {bk}>"


def measured_traffic(variant_name: str, tile):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel sources; None otherwise."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_src_digest") != kernel_source_digest():
        return None
    key = kernel_name_key(variant_name, tile)
    hits = [v["hbm_bytes_per_launch"] for k, v in rec.get("kernels", {}).items()
            if key + ">" in k or key + ", " in k]
    return hits[0] if len(hits) == 1 else None


class Part:
    """One workload: buffer sets on the GPU and a launcher."""

    def __init__(self, g, h, name: str, nsets: int):
        self.g, self.h, self.name = g, h, name
        self.w = workloads.WORKLOADS[name]
        self.sets = []
        for s in range(nsets):
            w = self.w
            if s == 0:
                A, B, C = workloads.make_inputs(w)
            else:  # other sets: same recipe, shifted seeds
                ws = workloads.Workload(**{**w.__dict__, "index": w.index + 100 * s})
                A, B, C = workloads.make_inputs(ws)
            D = torch.empty(w.M, w.N, dtype=torch.float32, device="cuda")
            self.sets.append((A.cuda(), B.cuda(), None if C is None else C.cuda(), D))
        self.host_inputs = workloads.make_inputs(self.w)
        self.i = 0
        self.events = []

    def launch(self, stream_handle, record=False):
        A, B, C, D = self.sets[self.i % len(self.sets)]
        self.i += 1
        w = self.w
        if record:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
        self.g.run_tensors(self.h, A, B, D, C=C, transA=w.transA, transB=w.transB,
                           alpha=w.alpha, beta=w.beta, stream=stream_handle)
        if record:
            e1.record()
            self.events.append((e0, e1))

    def times_ms(self):
        return np.array([a.elapsed_time(b) for a, b in self.events])

    def kernel_ms(self):
        return float(np.mean(self.times_ms()))

    def hot_cache_ms(self, stream_handle, reps: int = 20):
        """Mean launch time on one buffer set (operands stay in L2/MALL as far
        as they fit): the secondary, hot-cache number."""
        A, B, C, D = self.sets[0]
        w = self.w
        run = lambda: self.g.run_tensors(self.h, A, B, D, C=C, transA=w.transA,
                                         transB=w.transB, alpha=w.alpha, beta=w.beta,
                                         stream=stream_handle)
        for _ in range(3):
            run()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            run()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps


MALL_BYTES = 256 << 20


def sets_needed(w: workloads.Workload) -> int:
    """Buffer sets whose total exceeds twice the 256 MiB MALL, so a launch
    finds none of its operands left in the cache by the previous one."""
    ea = 4 if w.dtype == "f32" else 2
    one = ea * (w.M * w.K + w.K * w.N) + 4 * w.M * w.N * (2 if w.beta != 0.0 else 1)
    return 2 * MALL_BYTES // one + 1


def roofline_tflops(w: workloads.Workload, out_bytes: int = 4) -> float:
    """min(compute peak, HBM bandwidth x compulsory intensity), in TFLOP/s
    ("GEMM on NVIDIA GPUs", section 2, roofline bound)."""
    return min(PEAK_TFLOPS[w.dtype],
               HBM_GBS * 1e9 * w.flops / compulsory_bytes(w, out_bytes) / 1e12)


def time_extra(g, h, name: str, variant_name, reps: int, warmup: int,
               out_dtype=torch.float32, activation=0):
    """Time one workload outside the step (own buffers, HIP events).

    out_dtype=torch.bfloat16 runs a bf16 workload with bf16 C and D; a nonzero
    activation (GEMM_ACT_*) runs the fused epilogue with a N(0, 0.02) bias."""
    w = workloads.WORKLOADS[name]
    A, B, C = workloads.make_inputs(w)
    A, B = A.cuda(), B.cuda()
    C = None if C is None else C.to("cuda", out_dtype)
    D = torch.empty(w.M, w.N, dtype=out_dtype, device="cuda")
    bias = None
    if activation:
        bias = workloads.draw_matrix((w.N,), "n002", w.seeds["sample"] + 1, "f32").to(
            "cuda", out_dtype)
    vid = -1
    if variant_name is not None:
        vid = [i for i, n, _, _ in g.variants() if n == variant_name][0]
    g.gemm_set_variant(h, vid)
    try:
        # the C call with its arguments marshalled once, so the loop times the
        # library and the kernel rather than Python's argument checks
        run = g.bind_tensors(h, A, B, D, C=C, transA=w.transA, transB=w.transB,
                             alpha=w.alpha, beta=w.beta, bias=bias, activation=activation)
        s0 = run()
        if s0 != g.GEMM_OK:
            raise g.GemmError(s0)
        # at least `warmup` calls and ~50 ms of them: clocks that dropped
        # while the GPU idled take tens of milliseconds to come back
        t0 = time.perf_counter()
        n = 0
        while n < warmup or time.perf_counter() - t0 < 0.05:
            run()
            n += 1
            if n % 8 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            run()
        e1.record()
        torch.cuda.synchronize()
        used = g.gemm_variant_name(g.gemm_last_variant(h))
        sk = g.gemm_last_stream_k(h)
    finally:
        g.gemm_set_variant(h, -1)
    ms = e0.elapsed_time(e1) / reps
    tf = w.flops / (ms * 1e-3) / 1e12
    roof = roofline_tflops(w, 2 if out_dtype == torch.bfloat16 else 4)
    del A, B, C, D
    return {"kernel_ms": round(ms, 4), "tflops": round(tf, 2), "variant": used,
            "stream_k_workgroups": sk,
            "peak_tflops": PEAK_TFLOPS[w.dtype], "frac_of_peak": round(tf / PEAK_TFLOPS[w.dtype], 4),
            "roofline_tflops": round(roof, 1), "frac_of_roofline": round(tf / roof, 4),
            "workload": (w.description.replace("FP32 accumulate/output", "FP32 accumulate, BF16 C/D")
                         if out_dtype == torch.bfloat16 else w.description)}


def store_only_call_ms(g, h, name: str, reps: int = 50) -> float:
    """Per-call time of the workload's call with alpha = beta = 0 (arguments
    marshalled once, as in time_extra): the library's launch path with one
    kernel writing D = 0, the floor under a small GEMM called one at a time."""
    w = workloads.WORKLOADS[name]
    A, B, _ = workloads.make_inputs(w)
    A, B = A.cuda(), B.cuda()
    D = torch.empty(w.M, w.N, dtype=torch.float32, device="cuda")
    run = g.bind_tensors(h, A, B, D, transA=w.transA, transB=w.transB, alpha=0.0, beta=0.0)
    if run() != g.GEMM_OK:
        raise RuntimeError("store-only call failed")
    # warm-up as in time_extra, synchronizing every 8 calls: a long unsynced
    # queue of these short calls left later calls issuing 2x slower
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < 0.05:
        run()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        run()
    e1.record()
    torch.cuda.synchronize()
    return round(e0.elapsed_time(e1) / reps, 4)


def graph_replay_ms(g, h, name: str, launches: int = 50, replays: int = 5,
                    store_only: bool = False) -> float:
    """Per-launch time with `launches` back-to-back calls captured in one HIP
    graph (through torch.cuda.graph) and replayed: the kernels without the
    host's per-call cost, which bounds a small GEMM called one at a time.
    store_only: the same call with alpha = beta = 0, which the library serves
    with one kernel writing D = 0 (no operand read, no matrix work)."""
    w = workloads.WORKLOADS[name]
    A, B, C = workloads.make_inputs(w)
    A, B = A.cuda(), B.cuda()
    C = None if C is None or store_only else C.cuda()
    D = torch.empty(w.M, w.N, dtype=torch.float32, device="cuda")
    alpha, beta = (0.0, 0.0) if store_only else (w.alpha, w.beta)
    run = lambda: g.run_tensors(h, A, B, D, C=C, transA=w.transA, transB=w.transB,
                                alpha=alpha, beta=beta)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(launches):
            run()
    graph.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    del graph
    return round(e0.elapsed_time(e1) / (replays * launches), 4)


def under_profiler() -> bool:
    """Whether a profiler's library is preloaded into this process (rocprofv3
    runs the program that way).  A child process started from here would
    inherit it and initialise the GPU before its own program starts, so
    under a profiler the benchmark starts no helper programs."""
    pre = os.environ.get("LD_PRELOAD", "")
    return "rocprof" in pre or any(k.startswith("ROCPROF") for k in os.environ)


def amd_smi_sample():
    """Socket power (W), mean graphics clock and memory clock (MHz) from
    `amd-smi metric -p -c --json`, or None where the tool is not there (or
    under a profiler, see under_profiler)."""
    import shutil
    import subprocess
    if under_profiler():
        return None
    exe = shutil.which("amd-smi")
    if not exe:
        return None
    try:
        out = subprocess.run([exe, "metric", "-p", "-c", "--json"], capture_output=True,
                             text=True, timeout=20)
        data = json.loads(out.stdout)
    except (OSError, ValueError, subprocess.SubprocessError):
        return None
    gpu = data["gpu_data"][0] if isinstance(data, dict) and "gpu_data" in data else data[0]

    def val(x):
        return x.get("value") if isinstance(x, dict) else None

    clocks = gpu.get("clock", {})
    gfx = [val(c.get("clk")) for k, c in clocks.items() if k.startswith("gfx_") and isinstance(c, dict)]
    gfx = [g for g in gfx if isinstance(g, (int, float))]
    mem = [val(c.get("clk")) for k, c in clocks.items() if k.startswith("mem") and isinstance(c, dict)]
    mem = [m for m in mem if isinstance(m, (int, float))]
    return {"socket_power_w": val(gpu.get("power", {}).get("socket_power")),
            "gfx_clock_mhz_mean": round(sum(gfx) / len(gfx), 1) if gfx else None,
            "mem_clock_mhz": mem[0] if mem else None}


def telemetry_under_load(part, stream_handle, seconds: float = 2.5, every: float = 0.25):
    """Clocks and power while part's kernel runs back to back (the bf16 matrix
    cores are power limited, so the clock under load belongs with the
    timing).  amd-smi's metrics refresh about once a second, so one sample
    taken right after the load starts still shows the idle state: a thread
    polls every `every` seconds through `seconds` of launches, and the
    samples from the last second of load are reported (the last one as
    under_load), beside one taken idle before."""
    import threading
    before = amd_smi_sample()
    if before is None:
        return None
    samples = []
    stop = threading.Event()
    t0 = time.perf_counter()

    def poll():
        while not stop.is_set():
            s = amd_smi_sample()
            samples.append((round(time.perf_counter() - t0, 2), s))
            time.sleep(every)

    th = threading.Thread(target=poll)
    th.start()
    launches = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(4):
            part.launch(stream_handle)
        launches += 4
        torch.cuda.synchronize()
    stop.set()
    th.join()
    late = [s for t, s in samples if t >= seconds - 1.0 and s]
    return {"workload": part.name, "before": before, "under_load": late[-1] if late else None,
            "samples_last_second_of_load": late, "load_seconds": seconds,
            "launches": launches}


def oracle_sample_rate(part: Part, cores: int, budget_s: float):
    """Time the CPU oracle on a sample of outputs of the part's workload."""
    import oracle
    w = part.w
    A, B, C = part.host_inputs
    A_np, B_np = workloads.as_numpy_operand(A), workloads.as_numpy_operand(B)
    C_np = None if C is None else C.numpy()
    rng = np.random.default_rng(w.seeds["sample"])

    def run(n):
        ii = rng.integers(0, w.M, size=n)
        jj = rng.integers(0, w.N, size=n)
        t0 = time.perf_counter()
        oracle.gemm_points(w.transA, w.transB, w.M, w.N, w.K, w.alpha, A_np, A.shape[1], B_np,
                           B.shape[1], w.beta, C_np, w.N, ii, jj, nthreads=cores)
        return time.perf_counter() - t0

    n = max(cores * 64, 256)             # calibrate: grow until a run takes budget/8
    t = run(n)
    while t < budget_s / 8 and n < 4_000_000:
        n *= 4
        t = run(n)
    n = int(min(n * budget_s / max(t, 1e-6), 16_000_000))
    t = run(n)
    per = t / n
    rec = {"outputs": n, "seconds": t, "tflops": 2.0 * w.K * n / t / 1e12,
           "us_per_output": per * 1e6, "extrapolated_full_gemm_s": per * w.M * w.N}
    # the same with one thread, on a smaller sample (about a second)
    n1 = max(64, min(n, int(1.0 / max(per * cores, 1e-9))))
    ii = rng.integers(0, w.M, size=n1)
    jj = rng.integers(0, w.N, size=n1)
    t0 = time.perf_counter()
    oracle.gemm_points(w.transA, w.transB, w.M, w.N, w.K, w.alpha, A_np, A.shape[1], B_np,
                       B.shape[1], w.beta, C_np, w.N, ii, jj, nthreads=1)
    t1 = time.perf_counter() - t0
    rec["one_thread"] = {"outputs": n1, "seconds": t1, "tflops": 2.0 * w.K * n1 / t1 / 1e12}
    return rec


def oracle_full_small(cores: int):
    """Whole-output oracle wall time on the 256^3 fp32 workload."""
    import oracle
    w = workloads.WORKLOADS["fp32_256"]
    A, B, C = workloads.make_inputs(w)
    A_np, B_np = workloads.as_numpy_operand(A), workloads.as_numpy_operand(B)
    out = {}
    for nt in (cores, 1):
        t0 = time.perf_counter()
        oracle.gemm_full(w.transA, w.transB, w.M, w.N, w.K, w.alpha, A_np, A.shape[1], B_np,
                         B.shape[1], w.beta, None, w.N, nthreads=nt)
        t = time.perf_counter() - t0
        out[f"threads_{nt}"] = {"seconds": t, "gflops": w.flops / t / 1e9}
    return out


# How the traffic record is made ($OUT: the directory the profiler writes to)
PMC_COMMANDS = {
    "fetch": "rocprofv3 --pmc FETCH_SIZE -d $OUT/pmc_fetch -o fetch --output-format csv "
             "-- python -u bench.py --steps 2 --warmup 1 --no-cpu-baseline --no-extras "
             "--copy-probe 512",
    "write": "rocprofv3 --pmc WRITE_SIZE -d $OUT/pmc_write -o write --output-format csv "
             "-- python -u bench.py --steps 2 --warmup 1 --no-cpu-baseline --no-extras "
             "--copy-probe 512",
    "ingest": "python bench.py --ingest-pmc $OUT/pmc_fetch/fetch_counter_collection.csv "
              "$OUT/pmc_write/write_counter_collection.csv > profiles/hbm_traffic.json",
}


def ingest_pmc(fetch_csv: str, write_csv: str) -> int:
    """Average FETCH_SIZE / WRITE_SIZE (KiB per dispatch) per kernel, scaled by
    the copy kernel's reading against its known byte count."""
    import csv
    import re

    def per_kernel(path, counter):
        acc = {}
        with open(path) as f:
            for row in csv.DictReader(f):
                if row.get("Counter_Name") != counter:
                    continue
                name = row.get("Kernel_Name", "")
                acc.setdefault(name, []).append(float(row["Counter_Value"]))
        return {k: float(np.mean(v)) for k, v in acc.items()}

    fetch = per_kernel(fetch_csv, "FETCH_SIZE")
    write = per_kernel(write_csv, "WRITE_SIZE")
    copy = [k for k in fetch if "copy" in k.lower() or "elementwise" in k.lower()]
    if not copy:
        print("no copy kernel found in the counter CSV", file=sys.stderr)
        return 1
    ck = max(copy, key=lambda k: fetch[k])
    copy_bytes = float(os.environ.get("COPY_PROBE_BYTES", 512 << 20))
    f_scale = copy_bytes / (fetch[ck] * 1024.0)
    w_scale = copy_bytes / (write.get(ck, fetch[ck]) * 1024.0)
    rec = {"kernel_src_digest": kernel_source_digest(), "copy_kernel": ck,
           "copy_bytes": copy_bytes, "fetch_scale": f_scale, "write_scale": w_scale,
           "kernels": {}, "commands": PMC_COMMANDS,
           "note": ("FETCH_SIZE/WRITE_SIZE are KiB per dispatch; each is scaled by "
                    "bytes/(counter*1024) of a 512 MiB device copy recorded in the same run.")}
    for k in fetch:
        m = re.search(r"gemm_kernel<", k)
        if not m:
            continue
        rec["kernels"][k] = {
            "fetch_kib_raw": fetch[k], "write_kib_raw": write.get(k),
            "hbm_bytes_per_launch": fetch[k] * 1024.0 * f_scale
            + (write.get(k, 0.0) * 1024.0 * w_scale)}
    print(json.dumps(rec, indent=1))
    return 0


def fit_pipeline_model(rows):
    """Fit the pipeline-depth model of "High-Performance FP16 GEMM on NVIDIA
    Ada Lovelace via CUTLASS and WMMA" (methodology: efficiency S/(S + kappa),
    extended by an occupancy cap gamma(S)) to measured rows.

    Each row: family (dtype, tile, BK), d = K-steps of lookahead (the depth
    that hides copy latency: S with a late barrier, S-1 with a half-way one),
    occ = resident workgroups per compute unit, tflops.  Model:
        T = T_inf(family) * d / (d + kappa) * gamma,
        gamma = (occ / occ_max(family)) ** eta   (1 at the family's best occupancy).
    kappa is shared by a dtype's families, fitted with gamma = 1 on the rows
    at their family's best occupancy (T_inf by least squares for each kappa
    on a grid); eta from the remaining rows.  Returns per-dtype parameters
    and per-row predictions of both the simple and the extended model."""
    out = {}
    for dt in sorted({r["dtype"] for r in rows}):
        rs = [r for r in rows if r["dtype"] == dt]
        fams = sorted({r["family"] for r in rs})
        occ_max = {f: max(r["occ"] for r in rs if r["family"] == f) for f in fams}
        full = [r for r in rs if r["occ"] == occ_max[r["family"]]]

        def tinf_for(kappa):
            t = {}
            for f in fams:
                xs = [r["d"] / (r["d"] + kappa) for r in full if r["family"] == f]
                ys = [r["tflops"] for r in full if r["family"] == f]
                t[f] = float(np.dot(xs, ys) / np.dot(xs, xs)) if xs else float("nan")
            return t

        best = None
        for kappa in np.linspace(0.0, 4.0, 401):
            t = tinf_for(kappa)
            err = sum((r["tflops"] - t[r["family"]] * r["d"] / (r["d"] + kappa)) ** 2
                      for r in full)
            if best is None or err < best[0]:
                best = (err, float(kappa), t)
        _, kappa, tinf = best
        capped = [r for r in rs if r["occ"] < occ_max[r["family"]]]
        eta = 0.0
        if capped:
            # least squares on log(T / simple) = eta * log(occ / occ_max)
            xs = [np.log(r["occ"] / occ_max[r["family"]]) for r in capped]
            ys = [np.log(r["tflops"] / (tinf[r["family"]] * r["d"] / (r["d"] + kappa)))
                  for r in capped]
            eta = float(np.dot(xs, ys) / np.dot(xs, xs))
        preds = []
        for r in rs:
            simple = tinf[r["family"]] * r["d"] / (r["d"] + kappa)
            ext = simple * (r["occ"] / occ_max[r["family"]]) ** eta
            preds.append({"variant": r["variant"], "d": r["d"], "occ": r["occ"],
                          "measured": round(r["tflops"], 1), "simple": round(simple, 1),
                          "simple_err": round(simple / r["tflops"] - 1.0, 4),
                          "extended": round(ext, 1),
                          "extended_err": round(ext / r["tflops"] - 1.0, 4)})
        out[dt] = {"kappa": round(kappa, 3), "eta": round(eta, 3),
                   "t_inf": {f: round(v, 1) for f, v in tinf.items()},
                   "occ_max": occ_max, "rows": preds}
    return out


def pipeline_sweep(g, h, reps: int = 10) -> dict:
    """Time every direct-to-LDS variant (forced) on the NN step shapes: bf16
    8192^3 and fp32 4096^3, one buffer set, after >= 50 ms of warm-up each.
    The model is fitted on the plain stage rings; variants that pair
    k-contiguous copies (`_pair`, `_pair3`) or cap registers for occupancy
    (`_o3`) change more than the depth and are timed beside it."""
    rows = []
    for i, name, dt, tile in g.variants():
        if "_dma" not in name:
            continue
        wname = "bf16_8192" if dt == g.GEMM_DTYPE_BF16_F32 else "fp32_4096"
        stages, ahead = g.gemm_variant_pipeline(i)
        occ = g.gemm_variant_occupancy(i)
        r = time_extra(g, h, wname, name, reps=reps, warmup=3)
        mech = "paired" if "_pair" in name else "capped registers" if "_o3" in name else "ring"
        # a family: one instruction, tile and wave grid; the depth is what varies
        instr = re.search(r"_dma(\d+x\d+x\d+)_", name).group(1)
        waves = re.search(r"_w(\d+x\d+)_", name).group(1)
        rows.append({"variant": name, "dtype": "bf16" if dt == g.GEMM_DTYPE_BF16_F32 else "f32",
                     "family": f"{'bf16' if dt else 'f32'}_{instr}_{tile[0]}x{tile[1]}x{tile[2]}"
                               f"_w{waves}",
                     "stages": stages, "d": ahead, "occ": occ, "kernel_ms": r["kernel_ms"],
                     "tflops": r["tflops"], "workload": wname, "mechanism": mech})
        print(f"[sweep] {name} S={stages} ahead={ahead} occ={occ} {r['kernel_ms']} ms "
              f"{r['tflops']} TFLOP/s", file=sys.stderr, flush=True)
    return {"rows": rows, "model": fit_pipeline_model([r for r in rows if r["mechanism"] == "ring"])}


POWER_SWEEP = [("auto", "NN"),
               ("bf16_dma32x32x16_256x256x32_w2x4_s3_late", "TT"),
               ("bf16_dma32x32x16_256x256x32_w4x2_s3_late", "TT"),
               ("bf16_dma32x32x16_256x256x32_w2x4_s4_late", "TT"),
               ("bf16_dma32x32x16_256x256x32_w2x4_s4_late_pair1", "TT"),
               ("bf16_dma32x32x16_256x256x32_w2x2_s3_late", "TT"),
               ("bf16_dma32x32x16_256x256x64_w2x4_s2_late", "TT"),
               ("bf16_dma32x32x16_256x256x32_w2x4_s3_late", "TN"),
               ("bf16_dma32x32x16_256x256x32_w2x2_s3_late", "TN"),
               ("bf16_dma32x32x16_128x256x32_w2x2_s3_late", "TT"),
               ("bf16_dma32x32x16_128x128x32_w2x2_s4_late", "TT")]


def power_sweep(g, h, seconds: float = 3.0) -> dict:
    """Clock, power and rate of bf16 8192^3 kernels run back to back.

    The bf16 matrix cores run at the board's power limit, so a kernel's rate
    is set by its energy per FLOP as much as by its efficiency per clock.
    Each (variant, layout) runs for `seconds` on N(0,1) operands (one buffer
    set); amd-smi is polled every 0.25 s and the samples of the last second
    are averaged.  A forced variant runs in the layout given (TT is the
    operand orientation of the NN-as-D^T launch the selector uses); "auto"
    is the selected path for NN."""
    import threading
    n = 8192
    gen = torch.Generator(device="cuda")
    gen.manual_seed(8192)
    X = torch.randn(n, n, device="cuda", generator=gen).to(torch.bfloat16)
    Y = torch.randn(n, n, device="cuda", generator=gen).to(torch.bfloat16)
    D = torch.empty(n, n, device="cuda")
    names = {name: i for i, name, _, _ in g.variants()}
    rows = []
    for vname, lay in POWER_SWEEP:
        if vname != "auto" and vname not in names:
            continue
        g.gemm_set_variant(h, -1 if vname == "auto" else names[vname])

        def run():
            st = g.run_tensors(h, X, Y, D, transA=lay[0], transB=lay[1], check=False)
            if st != g.GEMM_OK:
                raise RuntimeError(g.gemm_status_string(st))

        for _ in range(20):
            run()
        torch.cuda.synchronize()
        used = g.gemm_variant_name(g.gemm_last_variant(h))
        samples = []
        stop = threading.Event()
        t0 = time.perf_counter()

        def poll():
            while not stop.is_set():
                samples.append((time.perf_counter() - t0, amd_smi_sample()))
                time.sleep(0.25)

        th = threading.Thread(target=poll)
        th.start()
        launches = 0
        while time.perf_counter() - t0 < seconds:
            for _ in range(4):
                run()
            launches += 4
            torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        stop.set()
        th.join()
        late = [x for t, x in samples if t >= seconds - 1.0 and x]
        pw = sum(x["socket_power_w"] for x in late) / len(late) if late else None
        clk = sum(x["gfx_clock_mhz_mean"] for x in late) / len(late) if late else None
        tf = launches * 2.0 * n ** 3 / dt / 1e12
        row = {"variant": used, "layout": lay, "ms": round(dt * 1e3 / launches, 4),
               "tflops": round(tf, 1), "power_w": None if pw is None else round(pw),
               "clock_mhz": None if clk is None else round(clk),
               "tflops_per_ghz": None if clk is None else round(tf / clk * 1e3),
               "w_per_tflops": None if pw is None else round(pw / tf, 3)}
        rows.append(row)
        print(f"[power] {row}", file=sys.stderr, flush=True)
        time.sleep(1.0)
    g.gemm_set_variant(h, -1)
    return {"workload": "bf16 8192^3, N(0,1) operands, back to back", "seconds": seconds,
            "rows": rows}


SELECTOR_CANDIDATES = ["bf16_dma32x32x16_256x256x32_w2x4_s3_late",
                       "bf16_dma32x32x16_128x128x32_w2x2_s4_late",
                       "bf16_dma32x32x16_128x128x32_w2x2_s2_late",
                       "bf16_dma32x32x16_128x128x32_w2x2_s4_late_pair",
                       "bf16_dma32x32x16_128x256x32_w2x2_s3_late",
                       "bf16_dma32x32x16_256x128x32_w2x2_s3_late",
                       "bf16_dma32x32x16_192x256x32_w2x4_s3_late",
                       "bf16_dma32x32x16_256x192x32_w4x2_s3_late"]
SELECTOR_CANDIDATES_F32 = ["f32_dma32x32x2_256x256x32_w2x2_s2_late",
                           "f32_dma32x32x2_256x256x16_w2x2_s3_late",
                           "f32_dma32x32x2_256x256x16_w2x2_s4_late",
                           "f32_dma32x32x2_128x128x16_w2x2_s3_late"]


def selector_check(g, h, dims=(1024, 2048, 3072, 4096, 6144, 8192), ks=(1024, 4096),
                   layouts=("TN", "NT"), out_bf16: bool = False, f32: bool = False,
                   beta: float = 0.0) -> dict:
    """The automatic choice against every whole-tile bf16 candidate, forced,
    on a grid of shapes (fp32 output, N(0,1) operands).  TN and NT only: a
    forced variant runs as stored, while NN calls may run as D^T, so an NN
    comparison with forced variants would not be like for like.  Each
    candidate is timed, then the automatic choice, then the fastest candidate
    and the automatic choice again (best of the two each), so neither side
    pays the clock's warm-up.  With out_bf16, D is bf16 and the candidates
    are those that carry a bf16-output epilogue (a forced variant without
    one is refused as not supported and left out).  With f32, operands and D
    are fp32 and the candidates are the fp32 whole-tile variants.  A nonzero
    beta adds beta * C (C drawn U[-1, 1]) to every call."""
    candidates = SELECTOR_CANDIDATES_F32 if f32 else SELECTOR_CANDIDATES
    op_dtype = torch.float32 if f32 else torch.bfloat16
    names = {name: i for i, name, _, _ in g.variants()}

    def best_ms(run, reps=10):
        for _ in range(3):
            run()
        torch.cuda.synchronize()
        best = float("inf")
        for _ in range(3):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                run()
            e1.record()
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1) / reps)
        return best

    rows = []
    for lay in layouts:
        ta, tb = lay[0], lay[1]
        for M in dims:
            for N in dims:
                for K in ks:
                    A = torch.randn((M, K) if ta == "N" else (K, M), device="cuda").to(op_dtype)
                    B = torch.randn((K, N) if tb == "N" else (N, K), device="cuda").to(op_dtype)
                    D = torch.empty(M, N, device="cuda",
                                    dtype=torch.bfloat16 if out_bf16 else torch.float32)
                    C = (torch.rand(M, N, device="cuda") * 2 - 1).to(D.dtype) if beta else None

                    # arguments marshalled once: the handle's variant setting is
                    # read at each call, and calls of ~10 us are then not paced
                    # by Python's argument checks
                    bound = g.bind_tensors(h, A, B, D, C=C, transA=ta, transB=tb, beta=beta)

                    def run():
                        st = bound()
                        if st != g.GEMM_OK:
                            raise RuntimeError(g.gemm_status_string(st))

                    times = {}
                    for c in candidates:
                        g.gemm_set_variant(h, names[c])
                        g.gemm_set_stream_k(h, 0)
                        st = g.run_tensors(h, A, B, D, C=C, transA=ta, transB=tb, beta=beta,
                                           check=False)
                        if st == g.GEMM_ERR_NOT_SUPPORTED:
                            continue
                        times[c] = best_ms(run)
                    g.gemm_set_variant(h, -1)
                    g.gemm_set_stream_k(h, -1)
                    auto = best_ms(run)
                    chosen = g.gemm_variant_name(g.gemm_last_variant(h))
                    sk = g.gemm_last_stream_k(h)
                    b0 = min(times, key=times.get)
                    g.gemm_set_variant(h, names[b0])
                    g.gemm_set_stream_k(h, 0)
                    times[b0] = min(times[b0], best_ms(run))
                    g.gemm_set_variant(h, -1)
                    g.gemm_set_stream_k(h, -1)
                    auto = min(auto, best_ms(run))
                    best = min(times, key=times.get)
                    rows.append({"layout": lay, "M": M, "N": N, "K": K, "auto_ms": round(auto, 4),
                                 "auto_variant": chosen, "stream_k": sk,
                                 "best_ms": round(times[best], 4), "best_variant": best,
                                 "ratio": round(auto / times[best], 3),
                                 "times": {c.split("_", 2)[2]: round(t, 4) for c, t in times.items()}})
                    print(f"[select] {rows[-1]}", file=sys.stderr, flush=True)
                    del A, B, C, D
    torch.cuda.empty_cache()
    r = [x["ratio"] for x in rows]
    return {"rows": rows, "shapes": len(rows), "within_5pct": sum(1 for x in r if x <= 1.05),
            "worst_ratio": max(r) if r else None}


def trace_summary(trace_csv: str, stats_csv: str, warmup: int, steps: int) -> int:
    """Markdown summary of a rocprofv3 --kernel-trace --stats run of this
    benchmark: rocprofv3's own per-kernel statistics, and for each step kernel
    the mean over the timed steps' dispatches alone (the step runs every
    workload once per step, so a step kernel's dispatches warmup .. warmup +
    steps - 1 are the timed ones; later dispatches are the variant report and
    the hot-cache rows)."""
    import csv

    with open(stats_csv) as f:
        stats = list(csv.DictReader(f))
    with open(trace_csv) as f:
        trace = [r for r in csv.DictReader(f) if r.get("Kind") == "KERNEL_DISPATCH"]
    per = {}
    for r in sorted(trace, key=lambda r: int(r["Start_Timestamp"])):
        per.setdefault(r["Kernel_Name"], []).append(
            (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    print("| kernel (rocprofv3 --stats) | calls | average us | min us | max us | share % |")
    print("|---|---|---|---|---|---|")
    for r in stats[:12]:
        print(f"| `{r['Name'][:150]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
              f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
              f"{float(r['Percentage']):.2f} |")
    print()
    print("| step workload | kernel | timed dispatches | mean us | median us |")
    print("|---|---|---|---|---|")
    for name in STEP_WORKLOADS:
        w = workloads.WORKLOADS[name]
        # the step kernel: the one with exactly warmup + steps + 1 + 23 dispatches
        # whose name carries the workload's operand type
        ktype = "DmaConfig<0," if w.dtype == "f32" else "DmaConfig<2,"
        cands = [k for k, v in per.items() if ktype in k and len(v) >= warmup + steps]
        cands.sort(key=lambda k: -sum(per[k]))
        if not cands:
            continue
        k = cands[0]
        timed = per[k][warmup:warmup + steps]
        print(f"| {name} | `{k[:150]}` | {len(timed)} | {np.mean(timed):.1f} | "
              f"{np.median(timed):.1f} |")
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--sets", type=int, default=0,
                    help="buffer sets per workload (0: enough to exceed twice the MALL)")
    ap.add_argument("--cpu-budget", type=float, default=8.0,
                    help="seconds of oracle work per workload for the CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the untimed-for-value vector-FMA and edge-workload rows")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="also run one plain device copy of MIB MiB (a known-size kernel "
                         "for scaling HBM byte counters)")
    ap.add_argument("--ingest-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 --pmc counter CSVs (FETCH_SIZE, WRITE_SIZE) of "
                         "a --copy-probe run into the HBM-traffic record, then exit")
    ap.add_argument("--vector-fma-only", action="store_true",
                    help="time only the fp32 vector-FMA kernel at 4096^3 (for counter runs), "
                         "print one JSON object, then exit")
    ap.add_argument("--pipeline-sweep", action="store_true",
                    help="time every direct-to-LDS variant on the NN step shapes, fit the "
                         "pipeline-depth model, print one JSON object, then exit")
    ap.add_argument("--selector-check", action="store_true",
                    help="time the automatic choice against every whole-tile bf16 candidate "
                         "on a grid of TN and NT shapes, print one JSON object, then exit")
    ap.add_argument("--selector-ks", default="1024,4096",
                    help="comma-separated K values of the --selector-check grid")
    ap.add_argument("--selector-out", choices=("f32", "bf16"), default="f32",
                    help="output type of the --selector-check calls")
    ap.add_argument("--selector-f32", action="store_true",
                    help="fp32 operands and the fp32 candidates in --selector-check")
    ap.add_argument("--selector-dims", default="1024,2048,3072,4096,6144,8192",
                    help="comma-separated M and N values of the --selector-check grid")
    ap.add_argument("--selector-beta", type=float, default=0.0,
                    help="beta of the --selector-check calls (nonzero: C is read)")
    ap.add_argument("--selector-layouts", default="TN,NT",
                    help="comma-separated layouts of the --selector-check grid (an automatic "
                         "NN call may run as D^T while a forced candidate runs as stored)")
    ap.add_argument("--power-sweep", action="store_true",
                    help="run bf16 8192^3 kernels back to back and record clock, power and "
                         "rate for each, print one JSON object, then exit")
    ap.add_argument("--trace-summary", nargs=2, metavar=("TRACE_CSV", "STATS_CSV"),
                    help="summarize a rocprofv3 --kernel-trace --stats run of this benchmark "
                         "(its kernel_trace.csv and kernel_stats.csv; pass that run's --steps "
                         "and --warmup), then exit")
    args = ap.parse_args(argv)
    if args.trace_summary:
        return trace_summary(*args.trace_summary, args.warmup, args.steps)
    if args.ingest_pmc:
        return ingest_pmc(*args.ingest_pmc)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this library runs on one GPU; multi-GPU runs are not part of it "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        return 2
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 2

    import dense_gemm_11_amd as g
    torch.cuda.set_device(0)
    h = g.gemm_create()
    if args.pipeline_sweep:
        print(json.dumps(pipeline_sweep(g, h)), flush=True)
        g.gemm_destroy(h)
        return 0
    if args.power_sweep:
        print(json.dumps(power_sweep(g, h)), flush=True)
        g.gemm_destroy(h)
        return 0
    if args.selector_check:
        workspace = g.attach_workspace(h)
        ks = tuple(int(k) for k in args.selector_ks.split(","))
        dims = tuple(int(d) for d in args.selector_dims.split(","))
        print(json.dumps(selector_check(g, h, dims=dims, ks=ks,
                                        out_bf16=args.selector_out == "bf16",
                                        f32=args.selector_f32, beta=args.selector_beta,
                                        layouts=tuple(args.selector_layouts.split(",")))),
              flush=True)
        g.gemm_set_workspace(h, None, 0, None)
        del workspace
        g.gemm_destroy(h)
        return 0
    if args.vector_fma_only:
        print(json.dumps(time_extra(g, h, "fp32_4096", VECTOR_FMA_VARIANT, reps=args.steps,
                                    warmup=args.warmup)), flush=True)
        g.gemm_destroy(h)
        return 0
    # a stream-K workspace (the automatic policy keeps the two step workloads
    # on whole tiles; it splits the few-tile, long-K extra row)
    workspace = g.attach_workspace(h)
    parts = [Part(g, h, n, args.sets or sets_needed(workloads.WORKLOADS[n]))
             for n in STEP_WORKLOADS]
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    for _ in range(args.warmup):
        for p in parts:
            p.launch(sh)
    torch.cuda.synchronize()
    if args.copy_probe:
        n = args.copy_probe * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for _ in range(args.steps):
        for p in parts:
            p.launch(sh, record=True)
    t_end.record()
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps
    step_flops = sum(p.w.flops for p in parts)
    value = step_flops / (ms_per_step * 1e-3) / 1e12

    report_parts = {}
    for p in parts:
        kms = p.kernel_ms()
        tf = p.w.flops / (kms * 1e-3) / 1e12
        p10, p50, p90 = np.percentile(p.times_ms(), [10, 50, 90])
        report_parts[p.name] = {"kernel_ms": round(kms, 4), "tflops": round(tf, 2),
                                "frac_of_peak": round(tf / PEAK_TFLOPS[p.w.dtype], 4),
                                "peak_tflops": PEAK_TFLOPS[p.w.dtype],
                                "launch_ms_p10_p50_p90": [round(float(x), 4)
                                                          for x in (p10, p50, p90)],
                                "buffer_sets": len(p.sets)}
    for p in parts:
        hot = p.hot_cache_ms(sh)
        report_parts[p.name]["hot_cache_kernel_ms"] = round(hot, 4)
    telemetry = None
    if not args.no_extras:
        telemetry = [telemetry_under_load(p, sh) for p in parts]
    # which kernel each part used
    for p in parts:
        A, B, C, D = p.sets[0]
        w = p.w
        g.run_tensors(h, A, B, D, C=C, transA=w.transA, transB=w.transB, alpha=w.alpha,
                      beta=w.beta)
        vid = g.gemm_last_variant(h)
        report_parts[p.name]["variant"] = g.gemm_variant_name(vid)
        report_parts[p.name]["tile"] = list(g.gemm_variant_tile(vid))
    torch.cuda.synchronize()

    dom = max(parts, key=lambda p: report_parts[p.name]["kernel_ms"])
    drep = report_parts[dom.name]
    achieved = dom.w.flops / (drep["kernel_ms"] * 1e-3) / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 2),
                "peak": PEAK_TFLOPS[dom.w.dtype], "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_TFLOPS[dom.w.dtype], 4),
                "traffic": measured_traffic(drep["variant"], drep["tile"]),
                "kernel": drep["variant"], "workload": dom.name,
                "compulsory_bytes": compulsory_bytes(dom.w)}

    # the remaining hot-path rows, timed outside the step: the fp32 vector-FMA
    # mainloop at 4096^3, the full alpha/beta epilogue with ragged edges, the
    # bf16-output epilogue at 8192^3, the fused bias+GELU epilogue, the
    # transformer-layer sweep (and one GPU's share of it under an 8-way
    # split), and a few-tile long-K shape that the stream-K path takes
    extras = {}
    if not args.no_extras:
        vf = time_extra(g, h, "fp32_4096", VECTOR_FMA_VARIANT, reps=10, warmup=3)
        vf["roofline"] = {"bound": "alu", "peak": round(VALU_FP32_TFLOPS, 1),
                          "unit": "TFLOP/s", "frac": round(vf["tflops"] / VALU_FP32_TFLOPS, 4),
                          "note": "vector FP32 FMA rate, 2 v_fmac_f32 per lane per clock"}
        extras["fp32_4096_vector_fma"] = vf
        extras["fp32_256"] = time_extra(g, h, "fp32_256", None, reps=50, warmup=10)
        extras["fp32_256"]["graph_replay_kernel_ms"] = graph_replay_ms(g, h, "fp32_256")
        # the launch floor under it: the same call with alpha = beta = 0
        extras["fp32_256"]["store_only_call_ms"] = store_only_call_ms(g, h, "fp32_256")
        extras["fp32_256"]["store_only_graph_replay_ms"] = graph_replay_ms(
            g, h, "fp32_256", store_only=True)
        extras["bf16_tn_edge_alpha_beta"] = time_extra(g, h, "bf16_tn_edge", None, reps=20,
                                                       warmup=5)
        extras["bf16_8192_bf16_output"] = time_extra(g, h, "bf16_8192", None, reps=10, warmup=3,
                                                     out_dtype=torch.bfloat16)
        # the fused epilogue on the MLP-up shape: bias + GELU, bf16 output,
        # beside the same GEMM without them
        fused = time_extra(g, h, "bf16_mlp_up", None, reps=10, warmup=3,
                           out_dtype=torch.bfloat16, activation=g.GEMM_ACT_GELU)
        plain = time_extra(g, h, "bf16_mlp_up", None, reps=10, warmup=3,
                           out_dtype=torch.bfloat16)
        fused["plain_kernel_ms"] = plain["kernel_ms"]
        fused["epilogue"] = "bias (N(0,0.02), bf16) + GELU (erf form), bf16 C/D"
        extras["bf16_mlp_up_bias_gelu"] = fused
        for group, names in (("transformer_layer", ("bf16_qkv", "bf16_outproj", "bf16_mlp_up",
                                                    "bf16_mlp_down")),
                             ("transformer_layer_tp8_shard", ("bf16_qkv_tp8", "bf16_outproj_tp8",
                                                              "bf16_mlp_up_tp8",
                                                              "bf16_mlp_down_tp8"))):
            rows = {n: time_extra(g, h, n, None, reps=10, warmup=3) for n in names}
            fl = sum(workloads.WORKLOADS[n].flops for n in names)
            t = sum(rows[n]["kernel_ms"] for n in names)
            extras[group] = {"rows": rows, "aggregate_tflops": round(fl / (t * 1e-3) / 1e12, 2),
                             "aggregate": "sum of FLOPs / sum of kernel times"}
        extras["bf16_small_mn_long_k"] = time_extra(g, h, "bf16_small_mn_long_k", None, reps=10,
                                                    warmup=3)
        g.gemm_set_stream_k(h, 0)
        try:
            whole = time_extra(g, h, "bf16_small_mn_long_k", None, reps=5, warmup=2)
        finally:
            g.gemm_set_stream_k(h, -1)
        extras["bf16_small_mn_long_k"]["whole_tiles_kernel_ms"] = whole["kernel_ms"]
        # the MFMA instruction shape on the same kernel template, tile (128x128),
        # depth (64-deep steps, 2 stages) and problem
        extras["mfma_instruction_shape"] = {
            "workload": workloads.WORKLOADS["bf16_4096_tn"].description,
            "v_mfma_f32_32x32x16_bf16": time_extra(
                g, h, "bf16_4096_tn", "bf16_dma32x32x16_128x128x64_w2x2_s2_late", reps=10,
                warmup=3),
            "v_mfma_f32_16x16x32_bf16": time_extra(
                g, h, "bf16_4096_tn", "bf16_dma16x16x32_128x128x64_w2x2_s2_late", reps=10,
                warmup=3)}

    cpu = None
    if not args.no_cpu_baseline:
        cores = len(os.sched_getaffinity(0))
        samples = {p.name: oracle_sample_rate(p, cores, args.cpu_budget) for p in parts}
        secs = sum(s["seconds"] for s in samples.values())
        fl = sum(2.0 * p.w.K * samples[p.name]["outputs"] for p in parts)
        cpu = {"value": fl / secs / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
               "sample": "; ".join(f"{k}: {v['outputs']} random outputs, full K, "
                                    f"{v['seconds']:.1f} s" for k, v in samples.items()),
               "per_workload": samples, "fp32_256_full_output": oracle_full_small(cores)}

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp32 + bf16-in/fp32-acc", "data": "synthetic",
        "config": {"workload": "fp32 GEMM 4096^3 + bf16->fp32 GEMM 8192^3 (NN, alpha=1, beta=0)",
                   "parallelism": "single GPU",
                   "buffer_sets": {p.name: len(p.sets) for p in parts}},
        "parts": report_parts, "extra_rows": extras, "roofline": roofline, "cpu_baseline": cpu,
        "telemetry": telemetry,
    }
    print(json.dumps(out), flush=True)
    g.gemm_set_workspace(h, None, 0, None)
    g.gemm_destroy(h)
    del workspace
    return 0


if __name__ == "__main__":
    sys.exit(main())
