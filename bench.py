"""Benchmark of the fp8 hot path on one MI355X.

One step = the quantize of a bf16 8192x1536 activation in row, transposed and
dual layouts (E4M3, ring-mode delayed scaling with a 16-entry history, fold in
the last workgroup) followed by the per-tensor-scaled E4M3 GEMM at
4096x4096x4096 with a fused fp32 bias and bf16 output.  Inputs are resident
in HBM before timing starts and rotate over buffer sets larger than the
256 MB Infinity Cache, so every read is an HBM read.

Timing uses HIP events recorded on the stream the kernels run on, and a few
untimed GEMMs are queued before each timed region so that the host is ahead
of the GPU and no launch waits on Python:
  * the step time brackets K whole steps with one event pair;
  * each kernel's average launch duration comes from back-to-back launches
    of that kernel over rotating inputs between one event pair (an event
    between every pair of kernels costs ~5 us of GPU time on its own, which
    would inflate a 10 us kernel by a third); the kernels take turns in
    --rounds such windows and each reports its median window.

Prints one JSON line (value = GEMM TFLOP/s at 4096^3).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "mm_fp8 TFLOP/s @4096^3 + quantize GB/s @8192x1536 (% of MI355X peak)"
PEAK_FP8_TFLOPS = 5033.0        # 256 CU x 8192 flop/clk x 2.4 GHz, dense
PEAK_HBM_GBS = 8000.0           # HBM3E
MM = (4096, 4096, 4096)
QSHAPE = (8192, 1536)
HIST = 16
L20_4096_BIAS_TFLOPS = 191.1    # the pages' fused-bias figure at 4096^3 (NVIDIA L20), context only


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the other configs' shapes (profiling runs of the headline kernels)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 512 MiB device copy (counter calibration)")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip the clock-sampled run of the headline GEMM (counter-collection runs)")
    ap.add_argument("--rounds", type=int, default=5,
                    help="timing windows per kernel, interleaved across kernels; the median window counts")
    ap.add_argument("--launches", type=int, default=0,
                    help="back-to-back launches per headline kernel (default max(10, steps))")
    ap.add_argument("--trace-summary", metavar="CSV",
                    help="print per-kernel call counts, mean and median durations of a rocprofv3 "
                         "kernel-trace CSV and exit (no GPU use)")
    ap.add_argument("--mfma-summary", metavar="CSV",
                    help="print the GEMM launches' MFMA utilisation from a rocprofv3 --pmc CSV of the MFMA / LDS "
                         "counters and exit (no GPU use)")
    ap.add_argument("--traffic-summary", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "OUT_JSON"),
                    help="turn rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE counter CSVs of a --calibrate-copy "
                         "run into per-launch HBM bytes (OUT_JSON) and exit (no GPU use)")
    return ap.parse_args()


_POOL_X = None


def _pool_init():
    """Process-pool worker set-up: the same seeded bf16 tensor as the
    single-core leg, generated in the worker (nothing large is pickled)."""
    global _POOL_X
    import synth
    _POOL_X = synth.gaussian(QSHAPE, 1.0, "bf16", 90, 4)


def _quantize_block(bounds):
    """One process-pool task: the oracle's dual-layout quantize of a row block
    (row and transposed codes); returns the block's raw amax, whose maximum
    over the blocks the caller folds."""
    import oracle as O
    i0, i1 = bounds
    return O.quantize(_POOL_X[i0:i1], "bf16", O.E4M3, scale=1.0)["amax"]


def cpu_baseline(seconds_target=6.0):
    """The CPU oracle on a bounded sample of the same workload, timed on this
    host: the GEMM on a block of output rows of the 4096^3 problem (up to the
    whole problem; float64 BLAS on its own threads), and the dual-layout
    quantize of the 8192x1536 tensor, once on one core and once as a process
    pool over row blocks on every core this process may use.  Each leg repeats
    until about seconds_target of time so its rate is stable, and reports the
    cores it used."""
    import multiprocessing as mp

    import numpy as np
    import oracle as O
    import synth
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    M, N, K = MM
    rows = 64
    a = O.encode(synth.gaussian_f32((rows, K), 1.0, 90, 0) * np.float32(100.0), O.E4M3)
    b = O.encode(synth.gaussian_f32((N, K), 1.0, 90, 1) * np.float32(100.0), O.E4M3)
    bias = synth.gaussian_f32((N,), 1.0, 90, 2).astype(np.float64)
    t0 = time.perf_counter()
    O.mm(a, O.E4M3, b, O.E4M3, 0.5, 0.25, bias)
    t1 = time.perf_counter()
    # grow the sample toward the time target (one more timed run)
    scale = max(1, min(M // rows, int(seconds_target / max(t1 - t0, 1e-3))))
    if scale > 1:
        rows *= scale
        a = O.encode(synth.gaussian_f32((rows, K), 1.0, 90, 3) * np.float32(100.0), O.E4M3)
        t0 = time.perf_counter()
        O.mm(a, O.E4M3, b, O.E4M3, 0.5, 0.25, bias)
        t1 = time.perf_counter()
    mm_runs, mm_s = 1, t1 - t0
    while mm_s < seconds_target:
        t0 = time.perf_counter()
        O.mm(a, O.E4M3, b, O.E4M3, 0.5, 0.25, bias)
        mm_s += time.perf_counter() - t0
        mm_runs += 1
    mm_tflops = 2.0 * rows * N * K * mm_runs / mm_s / 1e12
    qrows, qcols = QSHAPE
    x = synth.gaussian((qrows, qcols), 1.0, "bf16", 90, 4)
    qbytes = qrows * qcols * (2 + 2)
    q_runs, q_s = 0, 0.0
    while q_s < seconds_target:
        t2 = time.perf_counter()
        O.quantize(x, "bf16", O.E4M3, ring=O.Ring.new(HIST, 1.0))
        q_s += time.perf_counter() - t2
        q_runs += 1
    # the same quantize over row blocks in a process pool: fresh interpreters
    # (spawn), one per usable core up to 16 (the host share of one GPU)
    pool_cores = max(1, min(16, len(os.sched_getaffinity(0))))
    step_rows = -(-qrows // pool_cores)
    blocks = [(i, min(i + step_rows, qrows)) for i in range(0, qrows, step_rows)]
    with mp.get_context("spawn").Pool(pool_cores, initializer=_pool_init) as pool:
        pool.map(_quantize_block, blocks)  # workers started and warm
        p_runs, p_s = 0, 0.0
        while p_s < seconds_target:
            t3 = time.perf_counter()
            amaxes = pool.map(_quantize_block, blocks)
            O.fold(O.Ring.new(HIST, 1.0), np.float32(max(amaxes)), O.E4M3)
            p_s += time.perf_counter() - t3
            p_runs += 1
    return {"value": round(mm_tflops, 6), "unit": "TFLOP/s", "cores": int(blas_threads), "kind": "oracle",
            "sample": f"GEMM: {rows} output rows of {M}x{N}x{K} (float64 BLAS on {blas_threads} threads + bf16 "
                      f"rounding), {mm_runs} runs, {mm_s:.1f} s; quantize dual {qrows}x{qcols} bf16: one core "
                      f"{q_runs} runs {q_s:.1f} s, process pool of {pool_cores} over {len(blocks)} row blocks "
                      f"{p_runs} runs {p_s:.1f} s",
            "quantize": {"GBps_1core": round(qbytes * q_runs / q_s / 1e9, 4), "cores_1core": 1,
                         "GBps_pool": round(qbytes * p_runs / p_s / 1e9, 4), "cores_pool": pool_cores,
                         "unit": "GB/s", "algorithmic_bytes": qbytes},
            "host_cpus": len(os.sched_getaffinity(0))}


def trace_summary(path):
    """Per (kernel, grid) call count, mean and median duration (us) from a
    rocprofv3 --kernel-trace CSV: the profiler's own clock, one row per
    launch.  Prints a table; kernels are named up to their template arguments."""
    import csv
    import re
    import statistics
    groups, lib_names = {}, set()
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            name = row.get("Kernel_Name", "")
            short = _short_kernel(name)
            grid = int(row.get("Grid_Size_X", row.get("Grid_Size", 0)) or 0) * \
                int(row.get("Grid_Size_Y", 1) or 1) * int(row.get("Grid_Size_Z", 1) or 1)
            dur = (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1e3
            groups.setdefault((short, grid), []).append(dur)
            if "fp8mi::" in name:
                lib_names.add(short)
    print(f"{'kernel':48s} {'grid':>8s} {'calls':>5s} {'mean':>8s} {'median':>8s} {'min':>8s} {'max':>8s}")
    # the library's kernels only (torch's input generation and copies are not part of the path)
    ours = {k: v for k, v in groups.items() if k[0] in lib_names}
    for (k, g), v in sorted(ours.items(), key=lambda kv: -sum(kv[1])):
        print(f"{k:48s} {g:8d} {len(v):5d} {statistics.fmean(v):8.2f} {statistics.median(v):8.2f} "
              f"{min(v):8.2f} {max(v):8.2f}")


# (kernel, grid threads) of the counted launches -> name in the bench line
TRAFFIC_KERNELS = {
    ("mm_fp8_dma<0, 0, 256, 256, 2, 4, 1, -1, 0, false, 0>", 131072): "mm_fp8",
    ("mm_fp8_dma<0, 0, 256, 256, 2, 4, 1, 0, 0, false, 0>", 131072): "mm_fp8_out_e4m3",
    ("mm_fp8_dma<0, 0, 256, 256, 2, 4, 1, -1, 3, false, 0>", 131072): "mm_fp8_kmajor",
    ("quantize_flat<2, 0, false, false>", 393216): "quantize_row",
    ("quantize_tiled<2, 0, 1, false, false, true>", 393216): "quantize_transposed",
    ("quantize_tiled<2, 0, 2, false, false, false>", 393216): "quantize_dual",
    ("quantize_flat<2, 0, false, true>", 393216): "quantize_dynamic_row_pass",
    ("quantize_tiled<2, 0, 2, false, true, true>", 393216): "quantize_dynamic_dual_pass",
    ("amax_partials<2>", 196864): "amax_pass_8192x1536",
    ("stream_kernel<true>", 393216): "stream_reference_row_bytes",
    ("stream_kernel<false>", 393216): "stream_reference_dual_bytes",
    ("mm_fp8_mixed<0, 0, -1, 0>", 491520): "training_forward_8192x6912x1536",
    ("mm_fp8_dma<1, 0, 256, 192, 2, 4, 1, -1, 0, false, 0>", 131072): "training_dx_8192x1536x6912",
    ("mm_fp8_dma<1, 0, 256, 192, 2, 4, 1, -1, 0, false, 0>", 110592): "training_dw_6912x1536x8192",
    ("quantize_tiled_pf<2, 1, 2, true, false>", 196608): "training_dy_dual_bias_grad_8192x6912",
}
CALIBRATION_KERNEL = ("stream_kernel<false>", 8388608)   # 512 MiB copy: 2^29 bytes read and written


def _short_kernel(name):
    import re
    m = re.search(r"(\w+<[^()]*>|\w+)\(", name)
    short = m.group(1) if m else name.split("(")[0]
    return re.sub(r"\(fp8mi::\w+\)", "", short).replace("fp8mi::", "")


def _counter_means(path, counter, lib_only=True):
    """Mean value per dispatch of one counter, per (kernel, grid threads);
    the library's kernels only unless lib_only is False."""
    import csv
    per_dispatch = {}
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            if row.get("Counter_Name") != counter or (lib_only and "fp8mi::" not in row["Kernel_Name"]):
                continue
            key = (_short_kernel(row["Kernel_Name"]), int(row.get("Grid_Size", 0) or 0))
            d = per_dispatch.setdefault(key, {})
            did = row.get("Dispatch_Id", row.get("Correlation_Id"))
            d[did] = d.get(did, 0.0) + float(row["Counter_Value"])
    return {k: sum(v.values()) / len(v) for k, v in per_dispatch.items()}


def traffic_summary(fetch_csv, write_csv, out_json):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) -> bytes per launch, scaled
    by what the same counters read for the 512 MiB calibration copy."""
    fetch, write = _counter_means(fetch_csv, "FETCH_SIZE"), _counter_means(write_csv, "WRITE_SIZE")
    nbytes = float(1 << 29)
    cal = {"fetch": fetch[CALIBRATION_KERNEL] * 1024 / nbytes, "write": write[CALIBRATION_KERNEL] * 1024 / nbytes}
    kernels = {}
    print(f"calibration (512 MiB copy): FETCH_SIZE reads {cal['fetch']:.4f} x, WRITE_SIZE {cal['write']:.4f} x its bytes")
    print(f"{'kernel':52s} {'grid':>8s} {'fetch MB':>9s} {'write MB':>9s}  name")
    for key in sorted(set(fetch) | set(write)):
        fb = fetch.get(key, 0.0) * 1024 / cal["fetch"]
        wb = write.get(key, 0.0) * 1024 / cal["write"]
        name = TRAFFIC_KERNELS.get(key, "")
        print(f"{key[0]:52s} {key[1]:8d} {fb / 1e6:9.2f} {wb / 1e6:9.2f}  {name}")
        if name:
            kernels[name] = {"fetch": fb, "write": wb, "grid": key[1]}
    rec = {"source_sha256": kernel_source_hash(), "calibration": cal, "kernels": kernels}
    with open(out_json, "w") as f:
        json.dump(rec, f, indent=1)


MFMA_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CU_CYCLES", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE",
                 "SQ_INSTS_LDS", "SQ_WAVE_CYCLES", "SQ_WAIT_INST_ANY", "GRBM_GUI_ACTIVE")


def mfma_summary(path, simds=1024, xcds=8):
    """MFMA utilisation of the GEMM launches from a rocprofv3 --pmc CSV of
    MFMA_COUNTERS: busy MFMA cycles per SIMD over the GPU-active cycles of one
    XCD (GRBM_GUI_ACTIVE sums the XCDs)."""
    vals = {c: _counter_means(path, c) for c in MFMA_COUNTERS}
    for key in sorted(vals["SQ_VALU_MFMA_BUSY_CYCLES"]):
        if not key[0].startswith("mm_fp8"):
            continue
        v = {c: vals[c].get(key, float("nan")) for c in MFMA_COUNTERS}
        util = v["SQ_VALU_MFMA_BUSY_CYCLES"] / simds / (v["GRBM_GUI_ACTIVE"] / xcds)
        print(f"{key[0]} grid {key[1]:8d}: mfma_util {util:.3f}  "
              f"lds_bank_conflict/lds_active {v['SQ_LDS_BANK_CONFLICT'] / v['SQ_LDS_IDX_ACTIVE']:.3f}  "
              f"wait_inst_any/wave_cycles {v['SQ_WAIT_INST_ANY'] / v['SQ_WAVE_CYCLES']:.3f}")
        print("    " + "  ".join(f"{c}={v[c]:.4g}" for c in sorted(MFMA_COUNTERS)))


class ClockSampler:
    """Samples the GPU's graphics clock (amdsmi, in-process) in a background
    thread while timed work runs: the MFMA peak assumes 2.4 GHz, and the
    chip lowers its clock under sustained load."""

    def __init__(self, period_s=0.005):
        import threading
        self.samples, self.avg_samples, self.error, self.period = [], [], None, period_s
        self._stop, self._ready = threading.Event(), threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    def _run(self):
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            try:
                h = amdsmi.amdsmi_get_processor_handles()[0]
                self._ready.set()
                while not self._stop.is_set():
                    # the driver's current graphics DPM level: its list holds the
                    # measured frequency at index `current` (Hz).  The SMU's
                    # gpu-metrics table, the other source, went stale on some hosts.
                    f = amdsmi.amdsmi_get_clk_freq(h, amdsmi.AmdSmiClkType.GFX)
                    cur, freqs = f.get("current"), f.get("frequency") or []
                    if isinstance(cur, int) and 0 <= cur < len(freqs) and freqs[cur]:
                        self.samples.append(freqs[cur] / 1e6)
                    m = amdsmi.amdsmi_get_gpu_metrics_info(h)
                    clks = [c for c in (m.get("current_gfxclks") or []) if isinstance(c, (int, float)) and c > 0]
                    if clks:
                        self.avg_samples.append(sum(clks) / len(clks))
                    time.sleep(self.period)
            finally:
                amdsmi.amdsmi_shut_down()
        except Exception as e:  # no SMI access on this host: report why
            self.error = f"{type(e).__name__}: {e}"[:200]
        finally:
            self._ready.set()

    def __enter__(self):
        self._thread.start()
        self._ready.wait(timeout=10)
        return self

    def __exit__(self, *exc):
        self._stop.set()
        self._thread.join(timeout=5)

    def summary(self):
        import statistics
        src = "amdsmi_get_clk_freq(GFX): frequency of the current DPM level, sampled every 5 ms"
        if not self.samples:
            return {"source": src, "error": self.error or "no samples"}
        out = {"source": src, "samples": len(self.samples), "median_MHz": statistics.median(self.samples),
               "min_MHz": min(self.samples), "max_MHz": max(self.samples)}
        if self.avg_samples:
            # the gpu-metrics table's per-XCD clocks, for comparison: a value
            # that never changes under load is a stale table, not the clock
            out["gpu_metrics_current_gfxclks_median_MHz"] = statistics.median(self.avg_samples)
            if max(self.avg_samples) == min(self.avg_samples):
                out["gpu_metrics_note"] = "constant over the run: stale table"
        return out


# host-only argument validation: no kernel code, so not part of the hash
HOST_ONLY_SOURCES = ("abi.hip",)


def code_tokens(src: str) -> str:
    """C++ source without comments and with whitespace runs collapsed, so
    that edits to comments or layout do not count as kernel changes."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c == '"' or c == "'":                      # string / char literal, kept verbatim
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            out.append(" ")
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash():
    """sha256 of the code (comments and layout ignored) of the HIP sources
    that hold or feed the kernels, and of the compiler flags they are built
    with: counters taken on other code are stale."""
    import hashlib
    from fp8_tensor_scaled_quantize_amd import build as _build
    csrc = os.path.join(ROOT, "fp8_tensor_scaled_quantize_amd", "csrc")
    h = hashlib.sha256()
    h.update(repr((_build.HIPCC_FLAGS[:-2], sorted(_build.EXTRA_FLAGS.items()))).encode())  # include path dropped
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".h")) and name not in HOST_ONLY_SOURCES:
            h.update(name.encode())
            h.update(code_tokens(open(os.path.join(csrc, name)).read()).encode())
    return h.hexdigest()


def counter_traffic():
    """Per-launch HBM bytes {kernel: {"fetch": B, "write": B}} from the
    committed rocprofv3 FETCH_SIZE / WRITE_SIZE summary, or None when it was
    taken on different kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != kernel_source_hash():
        return None
    return rec.get("kernels")


def time_training_step(torch, fp8mi, synth, steps, warmup):
    """The full fp8 linear training step at the 1.2B-model FFN shape: x bf16
    [4,2048,1536], W [6912,1536], bias, dY [8192,6912]; dual quantize x, W
    (E4M3) and dY (E5M2) with 16-entry rings, Y, dX, dW GEMMs, bias grad."""
    from fp8_tensor_scaled_quantize_amd.linear import Fp8Linear
    dev = torch.device("cuda:0")
    M, K, N = 8192, 1536, 6912
    w = synth.device_gaussian((N, K), 0.02, torch.bfloat16, 5000, dev)
    b = synth.device_gaussian((N,), 0.1, torch.bfloat16, 5001, dev)
    xs = [synth.device_gaussian((4, 2048, K), 1.0, torch.bfloat16, 5100 + i, dev) for i in range(3)]
    dys = [synth.device_gaussian((M, N), 1e-3, torch.bfloat16, 5200 + i, dev) for i in range(3)]
    layer = Fp8Linear(w, b, hist_len=HIST)
    layer.seed(xs[0], dys[0])
    for s in range(warmup):
        layer.forward(xs[s % 3])
        layer.backward(dys[s % 3])
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for s in range(steps):
        layer.forward(xs[s % 3])
        layer.backward(dys[s % 3])
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    # the same steps replayed from a HIP graph: three steps over the three
    # input sets captured once (the rings keep folding on every replay)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for s in range(3):
            layer.forward(xs[s])
            layer.backward(dys[s])
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    reps = max(1, steps // 3)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms_graph = e0.elapsed_time(e1) / (3 * reps)
    flops = 3 * 2.0 * M * N * K
    return {"workload": "fp8 linear fwd+bwd, x [4,2048,1536], W [6912,1536], dY [8192,6912], H=16",
            "ms_per_step": round(ms, 4), "gemm_TFLOPs_over_step": round(flops / (ms * 1e-3) / 1e12, 1),
            "launches_per_step": 9, "ms_per_step_graph_replay": round(ms_graph, 4)}


def sweep(torch, fp8mi, synth, dev, prime):
    """Throughput of every other config's GEMM and quantize shapes (back-to-back
    launches over two input sets, one untimed call first), with the pages'
    NVIDIA L20 figure where they give one (context, other hardware)."""
    def timed_us(fn, n):
        fn(0)
        torch.cuda.synchronize()
        prime()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(n):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n * 1e3

    def codes(shape, seed):
        x = synth.device_gaussian(shape, 1.0, torch.bfloat16, seed, dev)
        ring = fp8mi.new_ring(1, 1.0, dev)
        fp8mi.fp8_quantize(x.reshape(-1, shape[-1]), fp8mi.E4M3, ring=ring)
        return fp8mi.fp8_quantize(x.reshape(-1, shape[-1]), fp8mi.E4M3, ring=ring).reshape(shape)

    out = {}
    sa = torch.tensor([0.5], dtype=torch.float32, device=dev)
    sb = torch.tensor([0.25], dtype=torch.float32, device=dev)
    gemms = [  # name, batch, M, N, K, broadcast B, bias, L20 TF/s
        ("square 1024^3", 1, 1024, 1024, 1024, False, False, 106.3),
        ("square 2048^3", 1, 2048, 2048, 2048, False, False, 178.2),
        ("square 8192^3", 1, 8192, 8192, 8192, False, False, 200.0),
        ("skinny 64x8192x2048", 1, 64, 8192, 2048, False, False, 94.0),
        ("skinny 1024x1536x2048", 1, 1024, 1536, 2048, False, False, 108.0),
        ("odd N 1024x1537x2048 + bias", 1, 1024, 1537, 2048, False, True, None),
        ("bmm 64 x 512^3", 64, 512, 512, 512, False, False, 161.0),
        ("bmm 8 x 1024x2048x2048", 8, 1024, 2048, 2048, False, False, 186.0),
        ("bmm 8 x 1024x2048x2048, B stride 0", 8, 1024, 2048, 2048, True, False, None),
        ("linear 2048x1536x1536 + bias", 1, 2048, 1536, 1536, False, True, None),
        ("linear 2048x6912x1536 + bias", 1, 2048, 6912, 1536, False, True, None),
        ("linear 2048x1536x6912 + bias", 1, 2048, 1536, 6912, False, True, None),
    ]
    for gi, (name, batch, M, N, K, bcast, has_bias, l20) in enumerate(gemms):
        sets = []
        for r in range(2):
            a = codes((batch, M, K) if batch > 1 else (M, K), 7000 + 10 * gi + r)
            b = codes((N, K), 7100 + 10 * gi + r)
            if batch > 1:
                b = b.unsqueeze(0).expand(batch, N, K) if bcast else codes((batch, N, K), 7200 + 10 * gi + r)
            sets.append((a, b))
        bias = synth.device_gaussian((N,), 1.0, torch.float32, 7300 + gi, dev) if has_bias else None
        cbuf = torch.empty((batch, M, N) if batch > 1 else (M, N), dtype=torch.bfloat16, device=dev)
        flops = 2.0 * batch * M * N * K
        n = max(5, min(200, int(2e-3 / (flops / 2.0e15))))
        us = timed_us(lambda i: fp8mi.fp8_mm(sets[i % 2][0], sets[i % 2][1], fp8mi.E4M3, fp8mi.E4M3, sa, sb, bias,
                                             out=cbuf), n)
        tf = flops / (us * 1e-6) / 1e12
        out[name] = {"us": round(us, 2), "TFLOPs": round(tf, 1), "frac_fp8_peak": round(tf / PEAK_FP8_TFLOPS, 4),
                     "L20_TFLOPs": l20}
        del sets, cbuf
    quants = [  # name, rows, cols, layout, misaligned base, L20 GB/s
        ("transposed 2048x1536", 2048, 1536, "t", False, 294.0),
        ("dual 2048x1536", 2048, 1536, "dual", False, 329.0),
        ("row 8192x1535 (odd width)", 8192, 1535, "row", False, None),
        ("dual 8192x1536, base + 1 element", 8192, 1536, "dual", True, 384.0),
    ]
    ring = fp8mi.new_ring(16, 1.0, dev)
    for qi, (name, R, C, lay, mis, l20) in enumerate(quants):
        nset = 12 if R * C * 2 * 12 > 300e6 else 4
        bufs = [synth.device_gaussian((R * C + 8,), 1.0, torch.bfloat16, 7400 + 10 * qi + r, dev) for r in range(nset)]
        xs = [b[1:1 + R * C].view(R, C) if mis else b[:R * C].view(R, C) for b in bufs]
        o_r = torch.empty((R, C), dtype=torch.uint8, device=dev)
        o_t = torch.empty((C, R), dtype=torch.uint8, device=dev)
        if lay == "row":
            fn = lambda i: fp8mi.fp8_quantize(xs[i % nset], fp8mi.E4M3, False, out=o_r, ring=ring)
        elif lay == "t":
            fn = lambda i: fp8mi.fp8_quantize(xs[i % nset], fp8mi.E4M3, True, out=o_t, ring=ring)
        else:
            fn = lambda i: fp8mi.fp8_quantize_dual(xs[i % nset], fp8mi.E4M3, out_row=o_r, out_t=o_t, ring=ring)
        us = timed_us(fn, 50)
        by = R * C * (4 if lay == "dual" else 3)
        gbs = by / (us * 1e-6) / 1e9
        out["quantize " + name] = {"us": round(us, 2), "GBps": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
                                   "L20_GBps": l20}
        del bufs, xs
    return out


def main():
    args = parse()
    if args.trace_summary:
        trace_summary(args.trace_summary)
        return
    if args.traffic_summary:
        traffic_summary(*args.traffic_summary)
        return
    if args.mfma_summary:
        mfma_summary(args.mfma_summary)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (asked for --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import fp8_tensor_scaled_quantize_amd as fp8mi
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    M, N, K = MM
    R, C = QSHAPE

    # quantize inputs: 14 x 25 MB bf16 rotate through > 256 MB
    nq = 14
    xq = [synth.device_gaussian(QSHAPE, 1.0, torch.bfloat16, 1000 + i, dev) for i in range(nq)]
    out_row = torch.empty(QSHAPE, dtype=torch.uint8, device=dev)
    out_t = torch.empty((C, R), dtype=torch.uint8, device=dev)
    out_row2 = torch.empty(QSHAPE, dtype=torch.uint8, device=dev)
    out_t2 = torch.empty((C, R), dtype=torch.uint8, device=dev)
    rings = [fp8mi.new_ring(HIST, 100.0, dev) for _ in range(3)]
    sinv = torch.empty(3, dtype=torch.float32, device=dev)

    # GEMM inputs: quantized N(0,1) codes at 448/amax (made by the library itself), 9 pairs rotate (> 256 MB)
    nm = 9
    A, B = [], []
    for i in range(nm):
        for lst, seed in ((A, 2000 + i), (B, 3000 + i)):
            src = synth.device_gaussian((M, K), 1.0, torch.bfloat16, seed, dev)
            ring = fp8mi.new_ring(1, 1.0, dev)
            fp8mi.fp8_quantize(src, fp8mi.E4M3, ring=ring)            # publishes 448 / amax
            lst.append(fp8mi.fp8_quantize(src, fp8mi.E4M3, ring=ring))
            del src
    import numpy as np
    sa = torch.tensor([synth.loguniform_scale(-4, 4, 91, 0)], dtype=torch.float32, device=dev)
    sb = torch.tensor([synth.loguniform_scale(-4, 4, 91, 1)], dtype=torch.float32, device=dev)
    bias = synth.device_gaussian((N,), 1.0, torch.float32, 4000, dev)
    C_out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()

    def step(s):
        x = xq[s % nq]
        j = s % nm
        fp8mi.fp8_quantize(x, fp8mi.E4M3, False, out=out_row, ring=rings[0], scale_inv_out=sinv[0:1])
        fp8mi.fp8_quantize(x, fp8mi.E4M3, True, out=out_t, ring=rings[1], scale_inv_out=sinv[1:2])
        fp8mi.fp8_quantize_dual(x, fp8mi.E4M3, out_row=out_row2, out_t=out_t2, ring=rings[2],
                                scale_inv_out=sinv[2:3])
        fp8mi.fp8_mm(A[j], B[j], fp8mi.E4M3, fp8mi.E4M3, sa, sb, bias, out=C_out)

    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()

    def prime():
        # untimed GPU work queued ahead of a timed region: the host then runs
        # ahead of the GPU and no timed launch waits on the Python binding
        for i in range(3):
            fp8mi.fp8_mm(A[i], B[i], fp8mi.E4M3, fp8mi.E4M3, sa, sb, bias, out=C_out)

    def timed(fn, n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        fn(0)  # untimed first call: a kernel's first launch loads its code object (ms)
        torch.cuda.synchronize()
        prime()
        e0.record()
        for i in range(n):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n  # ms per call

    total_ms = timed(lambda i: step(args.warmup + i), args.steps) * args.steps
    nlaunch = args.launches if args.launches > 0 else max(10, args.steps)
    names = ["quantize_row", "quantize_transposed", "quantize_dual", "mm_fp8", "quantize_dynamic_row",
             "quantize_dynamic_dual", "mm_fp8_out_e4m3", "mm_fp8_kmajor"]
    C8_out = torch.empty((M, N), dtype=torch.uint8, device=dev)
    # K-major copies of the GEMM operands: [K, M] / [K, N] storage read through transposed views
    A_km = [a.t().contiguous() for a in A]
    B_km = [b.t().contiguous() for b in B]
    ring_c = fp8mi.new_ring(HIST, 1.0, dev)
    ws_dyn = torch.empty(fp8mi.DYNAMIC_WORKSPACE_BYTES, dtype=torch.uint8, device=dev)
    launches = {
        "quantize_row": lambda i: fp8mi.fp8_quantize(xq[i % nq], fp8mi.E4M3, False, out=out_row, ring=rings[0],
                                                      scale_inv_out=sinv[0:1]),
        "quantize_transposed": lambda i: fp8mi.fp8_quantize(xq[i % nq], fp8mi.E4M3, True, out=out_t, ring=rings[1],
                                                             scale_inv_out=sinv[1:2]),
        "quantize_dual": lambda i: fp8mi.fp8_quantize_dual(xq[i % nq], fp8mi.E4M3, out_row=out_row2, out_t=out_t2,
                                                           ring=rings[2], scale_inv_out=sinv[2:3]),
        "mm_fp8": lambda i: fp8mi.fp8_mm(A[i % nm], B[i % nm], fp8mi.E4M3, fp8mi.E4M3, sa, sb, bias, out=C_out),
        # current scaling: amax pass + quantize pass per call
        "quantize_dynamic_row": lambda i: fp8mi.fp8_quantize_dynamic(xq[i % nq], fp8mi.E4M3, 0, out_row=out_row,
                                                                     scale_inv_out=sinv[0:1], workspace=ws_dyn),
        "quantize_dynamic_dual": lambda i: fp8mi.fp8_quantize_dynamic(xq[i % nq], fp8mi.E4M3, 2, out_row=out_row2,
                                                                      out_t=out_t2, scale_inv_out=sinv[2:3],
                                                                      workspace=ws_dyn),
        # FP8-out GEMM: the quantizing epilogue with the output's ring fold
        "mm_fp8_out_e4m3": lambda i: fp8mi.fp8_mm_ex(A[i % nm], B[i % nm], fp8mi.E4M3, fp8mi.E4M3, sa, sb, bias,
                                                     out=C8_out, out_fmt=fp8mi.E4M3, out_ring=ring_c),
        # layout tags: both operands K-major (transposed views), bf16 out
        "mm_fp8_kmajor": lambda i: fp8mi.fp8_mm(A_km[i % nm].t(), B_km[i % nm].t(), fp8mi.E4M3, fp8mi.E4M3, sa, sb,
                                                bias, out=C_out),
    }
    # practical HBM ceiling: the streaming reference kernel moving the same
    # bytes as the row / transposed quantize (read 2 B, write 1 B per element)
    # and as the dual quantize (read 2 B, write 2 B), over the same inputs
    ref_row = torch.empty(R * C, dtype=torch.uint8, device=dev)
    ref_dual = torch.empty(R * C * 2, dtype=torch.uint8, device=dev)
    launches["stream_row"] = lambda i: fp8mi.stream_reference(xq[i % nq], ref_row)
    launches["stream_dual"] = lambda i: fp8mi.stream_reference(xq[i % nq], ref_dual)
    clock = None
    if not args.no_clock:
        # sample the graphics clock over a longer run of the headline GEMM
        with ClockSampler() as cs:
            timed(launches["mm_fp8"], 5000)
        clock = cs.summary()
    # every kernel is timed in `rounds` windows of nlaunch back-to-back
    # launches, the kernels taking turns window by window (so that no kernel
    # sees only the chip's state after one particular neighbour); the median
    # window counts
    import statistics
    windows = {nme: [] for nme in launches}
    for _ in range(args.rounds):
        for nme in launches:
            windows[nme].append(timed(launches[nme], nlaunch) * 1e3)
    us = [statistics.median(windows[nme]) for nme in names]
    ceil_us = {"row": statistics.median(windows["stream_row"]), "dual": statistics.median(windows["stream_dual"])}
    del ref_row, ref_dual
    qbytes = {"quantize_row": R * C * 3, "quantize_transposed": R * C * 3, "quantize_dual": R * C * 4,
              "quantize_dynamic_row": R * C * 3, "quantize_dynamic_dual": R * C * 4}
    flops = 2.0 * M * N * K
    mm_tflops = flops / (us[3] * 1e-6) / 1e12
    quant = {}
    for i, nme in enumerate(names):
        if nme.startswith("mm_fp8"):
            continue
        gbs = qbytes[nme] / (us[i] * 1e-6) / 1e9
        quant[nme] = {"us_per_launch": round(float(us[i]), 3), "GBps": round(gbs, 1),
                      "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4), "algorithmic_bytes": qbytes[nme]}
        if "dynamic" in nme:
            quant[nme]["note"] = "us per call = amax pass + quantize pass (two launches); bytes = one read + codes"
        else:
            c_us = ceil_us["dual" if nme.endswith("dual") else "row"]
            quant[nme]["frac_of_stream_reference"] = round(c_us / float(us[i]), 4)
    ceiling = {k: {"us_per_launch": round(v, 3), "GBps": round(R * C * (4 if k == "dual" else 3) / (v * 1e-6) / 1e9, 1),
                   "frac_hbm_peak": round(R * C * (4 if k == "dual" else 3) / (v * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
               for k, v in ceil_us.items()}

    if args.calibrate_copy:
        # counter calibration: the streaming reference copying 512 MiB (reads and writes 2^29 bytes)
        src = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            fp8mi.stream_reference(src, dst)
        torch.cuda.synchronize()
        del src, dst

    out = {
        "metric": METRIC,
        "value": round(mm_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(mm_tflops / L20_4096_BIAS_TFLOPS, 3),
        "vs_baseline_ref": "pages' NVIDIA L20 figure for 4096^3 E4M3 with fused bias, 191.1 TF/s (other hardware; context)",
        "dtype": "e4m3 (fp32 accumulate)",
        "data": "synthetic",
        "config": {"workload": "mm_fp8 E4M3 NT 4096x4096x4096 + fp32 bias -> bf16, per-tensor scales; "
                               "quantize bf16 8192x1536 -> E4M3 row / transposed / dual, ring fold H=16",
                   "M": M, "N": N, "K": K, "quantize_shape": list(QSHAPE), "hist_len": HIST},
        "roofline": {"bound": "mfma", "achieved": round(mm_tflops, 2), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(mm_tflops / PEAK_FP8_TFLOPS, 4), "traffic": None,
                     "kernel": "mm_fp8", "us_per_launch": round(float(us[3]), 3), "launches": nlaunch,
                     "timing": f"median of {args.rounds} windows of {nlaunch} back-to-back launches, "
                               "interleaved with the other kernels' windows (HIP events on the launch stream)",
                     "algorithmic_flops": flops},
        "roofline_quantize": {"bound": "hbm", "achieved": quant["quantize_dual"]["GBps"], "peak": PEAK_HBM_GBS,
                              "unit": "GB/s", "frac": quant["quantize_dual"]["frac_hbm_peak"], "traffic": None,
                              "kernel": "quantize_dual",
                              "stream_reference": dict(ceiling, note="fp8mi_stream_reference: the same bytes "
                                                       "with the row quantize's access shape and no arithmetic")},
        "gpu_clock_during_mm_fp8": clock,
        "quantize": quant,
        "mm_fp8_out_e4m3": {"us_per_launch": round(float(us[names.index("mm_fp8_out_e4m3")]), 3),
                            "TFLOPs": round(flops / (us[names.index("mm_fp8_out_e4m3")] * 1e-6) / 1e12, 1),
                            "workload": "4096^3 E4M3 + fp32 bias -> E4M3 codes, ring scale + amax fold (H=16)"},
        "mm_fp8_kmajor": {"us_per_launch": round(float(us[names.index("mm_fp8_kmajor")]), 3),
                          "TFLOPs": round(flops / (us[names.index("mm_fp8_kmajor")] * 1e-6) / 1e12, 1),
                          "workload": "4096^3 E4M3 + fp32 bias -> bf16, A and B given K-major (layout tags)"},
    }
    traffic = counter_traffic()
    if traffic:
        for name in ("mm_fp8_out_e4m3", "mm_fp8_kmajor"):
            t = traffic.get(name)
            if t:
                out[name]["traffic"] = int(t["fetch"] + t["write"])
        for key, name in (("roofline", "mm_fp8"), ("roofline_quantize", "quantize_dual")):
            t = traffic.get(name)
            if t:
                out[key]["traffic"] = int(t["fetch"] + t["write"])
                out[key]["traffic_fetch"] = int(t["fetch"])
                out[key]["traffic_write"] = int(t["write"])
    out["training_step"] = time_training_step(torch, fp8mi, synth, max(3, args.steps // 5), 2)
    del A_km, B_km, xq
    A[3:], B[3:] = [], []  # prime() keeps using the first three pairs
    if not args.no_sweep:
        out["sweep"] = sweep(torch, fp8mi, synth, dev, prime)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
