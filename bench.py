#!/usr/bin/env python3
"""Benchmark of the MI355X W4A4 MXFP4 linear (and the prefill / A16WFP4 BMM sweeps).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                    [--no-prefill] [--no-bmm]
    python bench.py --traffic-pass          (workload of the counter runs)
    python bench.py --prefill-pass [M]      (workload of the prefill counter runs; M = 8192 by default)
    python bench.py --hbm-pass              (workload of the quantisation / BMM counter runs)
    python bench.py --hbm-summary FETCH.csv WRITE.csv CMD...  (CPU only)
    python bench.py --traffic-summary FETCH.csv WRITE.csv CMD...   (CPU only)
    python bench.py --trace-summary STATS.csv TRACE.csv MARKER.csv BENCH.log CMD...  (CPU only)
    python bench.py --prefill-summary TRACE.csv COUNTERS.csv CMD...  (CPU only)
    python bench.py --prefill-stall-summary [--m M] PASS_A.csv PASS_B.csv PASS_C.csv CMD...  (CPU only)

Headline (the metric's M <= 16 decode regime): one step is one pass over the
decode sweep W4A4 MXFP4 linear at M in {1, 4, 16} x (N, K) in {(14336, 5120),
(5120, 14336), (34816, 5120)} -- for each shape, mxfp4_linear: per-1x32
quantisation of the bf16 activations and the block-scaled FP4 GEMM with a
bf16 bias and bf16 output (one launch with the quantisation fused into the
GEMM kernel at M = 1, and at M = 4 for N = 14336 and N = 34816; elsewhere
quantisation into a workspace, then the GEMM),
against weights quantised and preshuffled once at load time.  value = sum of the pipeline's algorithmic
bytes over the step / step time (GB/s).  Inputs are resident in HBM before the
timed region.  Each launch reads a different copy of its weights (>= 1 GiB of
copies per shape) so the 256 MB Infinity Cache and the L2s cannot serve them.
Steps are replayed from HIP graphs (one graph per step position in the copy
rotation), bracketed by HIP events on the capture/replay stream.

Also reported (same JSON line): the dominant kernel's roofline (the decode
GEMM on pre-quantised activations at the headline shapes, timed in its own
graph-replayed loop),
the full decode sweep (M up to 64: the whole call, the GEMM alone with quant
apart, the call on row-major prequantised activations, and the GEMM writing
MXFP4 for the next layer), the
prefill sweep (M in {512, 2048, 8192}: TFLOP/s and fraction of the 10.1
PFLOP/s dense FP4 peak), the A16WFP4 BMM sweep (MLA K-up / V-up on 16 heads),
and the CPU oracle timed on bounded samples of the headline workload, one
prefill shape and one BMM.

Timing: every row's value is the mean over its timed replays (each replay a
graph of >= 32 back-to-back launches, so graph-launch overhead is amortised),
with nothing recorded between the replays; a second pass of as many replays,
each between its own pair of events, gives the spread of the per-launch time
(p10 / p50 / p90, `*_spread_us`).  The headline's K steps run between two
events, replayed as graphs of 10 steps each (90 linear calls per graph, as a
captured decode pass over a model's layers; single-step graphs for a
remainder); a second pass of as many steps, an event after each 10-step
graph, gives its spread (`step_spread_us`, per step; its mean is the
headline's), and a third with one graph per step is reported beside it
(`one_step_per_graph`: each graph launch costs a few microseconds).  The
shader clock is sampled from sysfs (pp_dpm_sclk, current level) by a host
thread during the headline, the roofline loop and the prefill sweep
(`sclk`, `prefill.sclk`).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

PEAK_HBM = 8.0e12          # MI355X HBM3E, bytes/s
PEAK_FP4 = 10.1e15         # MI355X dense FP4 MFMA, flop/s
PEAK_BF16 = 2.5e15         # MI355X dense bf16 MFMA, flop/s

DECODE_NK = [(14336, 5120), (5120, 14336), (34816, 5120)]
HEADLINE_M = [1, 4, 16]
DECODE_M = [1, 4, 16, 32, 64]
PREFILL_M = [512, 2048, 8192]
BMM_CASES = [("K-up", 512, 192, False), ("V-up", 256, 512, True)]   # (name, N, K, batch_major)
BMM_M = [1, 64, 128, 256, 4096]
BMM_HEADS = 16
ROTATE_BYTES = 1 << 30
MIN_LAUNCHES = 32          # launches per timed graph (amortises graph-launch overhead)
HEADLINE_GRAPH_STEPS = 10  # headline steps per captured graph

METRIC = "W4A4 MXFP4 GEMM TFLOPS & % FP4 peak (M≥2048); GB/s & % HBM at M≤16"


def gemm_bytes(M, N, K, bias):
    """Algorithmic bytes of one GEMM launch: W + scales, A + scales, out, bias."""
    return N * K * 17 / 32 + M * K * 17 / 32 + 2 * M * N + (2 * N if bias else 0)


def pipeline_bytes(M, N, K, bias):
    """Algorithmic bytes of quant + GEMM: bf16 x replaces packed A + scales."""
    return N * K * 17 / 32 + 2 * M * K + 2 * M * N + (2 * N if bias else 0)


def quant_bytes(M, K):
    return 2 * M * K + 17 * M * K / 32


def bmm_bytes(B, M, N, K):
    return B * (2 * M * K + N * K * 17 / 32 + 2 * M * N)


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def copies_for(nbytes):
    return max(2, -(-ROTATE_BYTES // int(nbytes)))


def _stats(values):
    """mean, median, p10 and p90 of a list of per-launch (or per-step) times."""
    v = np.asarray(values, dtype=np.float64)
    return {"mean": float(v.mean()), "p10": float(np.percentile(v, 10)),
            "p50": float(np.percentile(v, 50)), "p90": float(np.percentile(v, 90)), "n": int(v.size)}


def _us(st):
    """A stats dict in seconds -> the same in microseconds, rounded, for the JSON line."""
    return {k: (round(v * 1e6, 3) if k != "n" else v) for k, v in st.items()}


class ClockSampler:
    """Samples the GPU's shader clock (the current level of the sysfs
    pp_dpm_sclk table, the line marked '*') from a host thread while a timed
    region runs; reports the median and p10 / p90 of the samples in MHz, or
    None where the file is not readable."""

    def __init__(self, period_s=0.002):
        import glob
        paths = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.path = paths[0] if paths else None
        self.period = period_s
        self.samples = []

    def _read(self):
        try:
            with open(self.path) as fh:
                for line in fh:
                    if line.rstrip().endswith("*"):
                        return float(line.split(":")[1].strip().split("Mhz")[0].split("MHz")[0])
        except (OSError, ValueError, IndexError):
            return None
        return None

    def __enter__(self):
        import threading
        self._stop = threading.Event()

        def run():
            while not self._stop.is_set():
                v = self._read() if self.path else None
                if v is not None:
                    self.samples.append(v)
                time.sleep(self.period)

        self._t = threading.Thread(target=run, daemon=True)
        self._t.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        self._t.join()

    def summary(self):
        if not self.samples:
            return None
        v = np.asarray(self.samples)
        return {"median_mhz": float(np.median(v)), "p10_mhz": float(np.percentile(v, 10)),
                "p90_mhz": float(np.percentile(v, 90)), "samples": int(v.size),
                "source": self.path}


class Timer:
    """HIP-event timing of graph replays on the current stream."""

    def __init__(self):
        self.stream = torch.cuda.current_stream()

    def capture(self, fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        return g

    def time_graphs(self, graphs, reps, warmup_s=0.025):
        """Seconds per replay: the mean from `reps` replays between two
        events, then the spread (p10 / p50 / p90) from `reps` more, each
        between its own pair of events.  An event recorded between replays
        costs a few microseconds of its own, so it stays out of the mean."""
        # Untimed replays of the same sequence for at least warmup_s first:
        # after a pause the GPU takes a few milliseconds of load to reach its
        # steady clocks (measured: a timed run right after two warm-up
        # replays came out 10-15% slower than the runs after it).
        t0 = time.perf_counter()
        i = 0
        while True:
            graphs[i % len(graphs)].replay()
            i += 1
            if i >= 2 and i % max(2, reps) == 0:
                torch.cuda.synchronize()
                if time.perf_counter() - t0 >= warmup_s:
                    break
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(reps):
            graphs[i % len(graphs)].replay()
        b.record()
        torch.cuda.synchronize()
        mean = a.elapsed_time(b) * 1e-3 / reps
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        ev[0].record()
        for i in range(reps):
            graphs[i % len(graphs)].replay()
            ev[i + 1].record()
        torch.cuda.synchronize()
        st = _stats([ev[i].elapsed_time(ev[i + 1]) * 1e-3 for i in range(reps)])
        st["mean"] = mean
        return st


TRAFFIC_MD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                          "gemm_decode_kernel__headline_traffic.md")
CALIB_BYTES = 256 << 20     # the calibration copy reads and writes this many bytes


def decode_source_digest():
    """sha256 over the sources the decode GEMM kernel is built from."""
    import hashlib
    csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                        "mxfp4_block_scaled_quant_amd", "csrc")
    h = hashlib.sha256()
    for f in ("gemm_decode.hip", "mxfp4_device.h", "mxfp4_launch.h"):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def read_traffic():
    """Measured HBM bytes per decode-GEMM launch (mean over the headline
    shapes) from the committed counter summary, or None when it is missing or
    was taken on other kernel sources."""
    try:
        text = open(TRAFFIC_MD).read()
    except OSError:
        return None
    import re
    m = re.search(r"```json\n(.*?)\n```", text, flags=re.S)
    if not m:
        return None
    d = json.loads(m.group(1))
    if d.get("source_sha256") != decode_source_digest():
        return None
    return d


def traffic_pass():
    """The workload of the FETCH_SIZE / WRITE_SIZE counter runs (run under
    rocprofv3 --pmc): a calibration copy of CALIB_BYTES (an elementwise
    int32 kernel reading and writing that many bytes), then the decode GEMM
    of every headline shape once on each of its rotated weight copies."""
    import mxfp4_block_scaled_quant_amd as mx
    from mxfp4_block_scaled_quant_amd import inputs
    mx.lib()
    dev = torch.device("cuda:0")
    src = torch.arange(CALIB_BYTES // 4, dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(4):
        torch.bitwise_not(src, out=dst)
    torch.cuda.synchronize()
    del src, dst
    plan = []
    for (N, K) in DECODE_NK:
        W = mx.quantize_weight(inputs.bits_to_torch_bf16(inputs.weights(N, K, 2)).to(dev))
        R = copies_for(W.w_pre.numel() + W.ws_pre.numel())
        copies = [W] + [mx.MXFP4Weight(W.w_pre.clone(), W.ws_pre.clone(), N, K) for _ in range(R - 1)]
        b = inputs.bits_to_torch_bf16(inputs.bias(N, 2)).to(dev)
        for M in HEADLINE_M:
            x = inputs.bits_to_torch_bf16(inputs.activations(M, K, 2)).to(dev)
            q, s = mx.mxfp4_quant_1x32(x, mx.MXFP4_LAYOUT_GEMM)
            out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            torch.cuda.synchronize()
            for cp in copies:
                mx.mxfp4_gemm_a4w4(q, s, cp.w_pre, cp.ws_pre, M, N, K, b, torch.bfloat16, out=out)
            torch.cuda.synchronize()
            plan.append((M, N, K, R))
        del copies, W
        torch.cuda.empty_cache()
    print(json.dumps({"traffic_pass": plan}), flush=True)


HBM_PASS_QUANT = [(8192, 5120, "gemm"), (8192, 14336, "gemm"), (8192, 5120, "rowmajor")]
HBM_PASS_BMM_M = 4096
HBM_PASS_REPS = 3


def _calibration_copy(dev):
    src = torch.arange(CALIB_BYTES // 4, dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(4):
        torch.bitwise_not(src, out=dst)
    torch.cuda.synchronize()


def hbm_pass():
    """The workload of the quantisation / BMM counter runs (FETCH_SIZE, then
    WRITE_SIZE, under rocprofv3 --pmc): inputs and weights prepared first,
    then the calibration copy, then HBM_PASS_REPS launches each of the
    activation quantisation at the prefill sweep's largest M (both scale
    layouts) and of the A16WFP4 BMM (K-up and V-up, 16 heads) at M = 4096,
    on the sweeps' inputs.  The summary reads only the launches after the
    calibration copy."""
    import mxfp4_block_scaled_quant_amd as mx
    from mxfp4_block_scaled_quant_amd import inputs
    mx.lib()
    dev = torch.device("cuda:0")
    quant = []
    for (M, K, layout) in HBM_PASS_QUANT:
        x = inputs.bits_to_torch_bf16(inputs.activations(M, K, 3, outliers=True)).to(dev)
        lay = mx.MXFP4_LAYOUT_GEMM if layout == "gemm" else mx.MXFP4_LAYOUT_ROWMAJOR
        q, sc = mx.mxfp4_quant_1x32(x, lay)
        quant.append((x, lay, q, sc))
    M = HBM_PASS_BMM_M
    bmm = []
    for name, N, K, bm in BMM_CASES:
        w = inputs.bits_to_torch_bf16(inputs.bmm_problem(BMM_HEADS, 1, N, K, 4)["w"].reshape(BMM_HEADS * N, K)).to(dev)
        W = mx.quantize_weight(w.reshape(BMM_HEADS, N, K))
        x = inputs.bits_to_torch_bf16(inputs.bmm_problem(BMM_HEADS, M, N, K, 4)["x"]).to(dev)
        out = (torch.empty((M, BMM_HEADS, N), dtype=torch.bfloat16, device=dev) if bm
               else torch.empty((BMM_HEADS, M, N), dtype=torch.bfloat16, device=dev))
        bmm.append((W, x, out, N, bm))
    torch.cuda.synchronize()
    _calibration_copy(dev)
    for (x, lay, q, sc) in quant:
        for _ in range(HBM_PASS_REPS):
            mx.mxfp4_quant_1x32(x, lay, q=q, scales=sc)
    for (W, x, out, N, bm) in bmm:
        for _ in range(HBM_PASS_REPS):
            mx.a16wfp4_bmm(x, W.w_pre, W.ws_pre, N, out=out, batch_major=bm)
    torch.cuda.synchronize()
    print(json.dumps({"hbm_pass": [list(c) for c in HBM_PASS_QUANT] + [c[0] for c in BMM_CASES]}), flush=True)


HBM_MD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                      "quant_and_bmm__hbm_traffic.md")


def hbm_summary(fetch_csv, write_csv, command):
    """The committed HBM-traffic summary of hbm_pass (HBM_MD): per launch,
    FETCH_SIZE and WRITE_SIZE scaled by the calibration copy, against the
    algorithmic bytes each kernel must read and write."""
    per = {}
    for name, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = [r for r in _counter_rows(path) if r[2] == name]
        calib = [v for _, k, _, v in rows if "bitwise_not" in k]
        last_calib = max(d for d, k, _, _ in rows if "bitwise_not" in k)
        work = [(k, v) for d, k, _, v in rows if d > last_calib]
        per[name] = (calib, work)
    f_cal, f_work = per["FETCH_SIZE"]
    w_cal, w_work = per["WRITE_SIZE"]
    ff = CALIB_BYTES / (np.mean(f_cal) * 1024)
    wf = CALIB_BYTES / (np.mean(w_cal) * 1024)
    n = HBM_PASS_REPS
    cases = []
    for (M, K, layout) in HBM_PASS_QUANT:
        cases.append((f"quant {layout} M={M} K={K}", 2 * M * K, 17 * M * K / 32))
    M = HBM_PASS_BMM_M
    for name, N, K, bm in BMM_CASES:
        cases.append((f"BMM {name} M={M} N={N} K={K} (16 heads)",
                      BMM_HEADS * (2 * M * K + N * K * 17 / 32), BMM_HEADS * 2 * M * N))
    assert len(f_work) == len(w_work) == n * len(cases), (len(f_work), len(w_work))
    rows = []
    for i, (label, alg_r, alg_w) in enumerate(cases):
        fk = float(np.mean([v for _, v in f_work[i * n:(i + 1) * n]]))
        wk = float(np.mean([v for _, v in w_work[i * n:(i + 1) * n]]))
        kern = f_work[i * n][0].split("(")[0].replace("void ", "")
        rows.append(dict(case=label, kernel=kern, fetch_bytes=round(fk * 1024 * ff),
                         write_bytes=round(wk * 1024 * wf), algorithmic_read=round(alg_r),
                         algorithmic_write=round(alg_w),
                         read_ratio=round(fk * 1024 * ff / alg_r, 4), write_ratio=round(wk * 1024 * wf / alg_w, 4)))
    lines = ["# Activation quantisation and A16WFP4 BMM — HBM traffic", "",
             "Two counter runs of the same workload (`python bench.py --hbm-pass`: a calibration",
             f"copy of {CALIB_BYTES >> 20} MiB, then {n} launches of each case on the sweeps' inputs):", "",
             "```", *command, "```", "",
             "Each counter is scaled by what it reads for the calibration copy (known bytes",
             "read and written) and averaged over the case's launches. Algorithmic bytes:",
             "quantisation reads 2MK (bf16) and writes 17MK/32 (codes and scales, before",
             "padding); the BMM reads its activations and the preshuffled weights",
             "(16 heads) and writes its bf16 output.", "",
             "| Case | Kernel | HBM read B | algorithmic | ratio | HBM write B | algorithmic | ratio |",
             "|---|---|---|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| {r['case']} | `{r['kernel']}` | {r['fetch_bytes']} | {r['algorithmic_read']} | "
                     f"{r['read_ratio']} | {r['write_bytes']} | {r['algorithmic_write']} | {r['write_ratio']} |")
    lines += ["", f"Calibration: FETCH_SIZE scale {ff:.4f}, WRITE_SIZE scale {wf:.4f}.", "",
              "```json", json.dumps(dict(cases=rows, fetch_scale=round(ff, 4), write_scale=round(wf, 4))), "```", ""]
    with open(HBM_MD, "w") as fh:
        fh.write("\n".join(lines))
    print(f"wrote {HBM_MD}")
    for r in rows:
        print(r)


PREFILL_PASS_M = 8192
PREFILL_PASS_REPS = 4   # launches per shape the summary reads, after one warm-up launch


def prefill_pass(M=PREFILL_PASS_M):
    """The workload of the prefill counter runs (run under rocprofv3): the
    prefill GEMM at M (8192 unless given) for each (N, K) of the sweep, one warm-up launch
    (its counters also catch the activity before it) then PREFILL_PASS_REPS
    launches, on the sweep's inputs (activations seed 3 with outliers,
    weights seed 2, no bias, bf16 out)."""
    import mxfp4_block_scaled_quant_amd as mx
    from mxfp4_block_scaled_quant_amd import inputs
    mx.lib()
    dev = torch.device("cuda:0")
    plan = []
    for (N, K) in DECODE_NK:
        W = mx.quantize_weight(inputs.bits_to_torch_bf16(inputs.weights(N, K, 2)).to(dev))
        x = inputs.bits_to_torch_bf16(inputs.activations(M, K, 3, outliers=True)).to(dev)
        q, s = mx.mxfp4_quant_1x32(x, mx.MXFP4_LAYOUT_GEMM)
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        torch.cuda.synchronize()
        for _ in range(1 + PREFILL_PASS_REPS):
            mx.mxfp4_gemm_a4w4(q, s, W.w_pre, W.ws_pre, M, N, K, None, torch.bfloat16, out=out)
        torch.cuda.synchronize()
        plan.append((M, N, K, PREFILL_PASS_REPS))
        del W, x, q, s, out
        torch.cuda.empty_cache()
    print(json.dumps({"prefill_pass": plan}), flush=True)


def _is_decode_gemm(kernel_name):
    """The decode GEMM's kernels: the streaming form and the persistent one."""
    return "gemm_decode_kernel" in kernel_name or "gemm_decode_persist_kernel" in kernel_name


def _counter_rows(csv_path):
    import csv
    rows = []
    with open(csv_path) as fh:
        for r in csv.DictReader(fh):
            rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], r["Counter_Name"],
                         float(r["Counter_Value"])))
    rows.sort()
    return rows


def traffic_summary(fetch_csv, write_csv, command):
    """Turn the two counter runs into the committed summary (TRAFFIC_MD)."""
    per = {}
    for name, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = [r for r in _counter_rows(path) if r[2] == name]
        calib = [v for _, k, _, v in rows if "bitwise_not" in k]
        gemm = [v for _, k, _, v in rows if _is_decode_gemm(k)]
        per[name] = (calib, gemm)
    f_cal, f_gemm = per["FETCH_SIZE"]
    w_cal, w_gemm = per["WRITE_SIZE"]
    ff = CALIB_BYTES / (np.mean(f_cal) * 1024)
    wf = CALIB_BYTES / (np.mean(w_cal) * 1024)
    shapes = []
    i = 0
    for (N, K) in DECODE_NK:
        for M in HEADLINE_M:
            R = copies_for(N * K * 17 // 32)   # traffic_pass's copies (data + scale bytes, unpadded here)
            fk = float(np.mean(f_gemm[i:i + R]))
            wk = float(np.mean(w_gemm[i:i + R]))
            i += R
            alg = gemm_bytes(M, N, K, True)
            tr = fk * 1024 * ff + wk * 1024 * wf
            shapes.append(dict(M=M, N=N, K=K, launches=R, fetch_kib=round(fk, 1), write_kib=round(wk, 1),
                               hbm_bytes=round(tr), algorithmic_bytes=round(alg),
                               ratio=round(tr / alg, 4)))
    assert i == len(f_gemm) == len(w_gemm), (i, len(f_gemm), len(w_gemm))
    traffic = float(np.mean([r["hbm_bytes"] for r in shapes]))
    summary = dict(kernel="gemm_decode_kernel / gemm_decode_persist_kernel", traffic_bytes_per_launch=round(traffic),
                   algorithmic_bytes_per_launch=round(float(np.mean([r["algorithmic_bytes"] for r in shapes]))),
                   fetch_scale=round(ff, 4), write_scale=round(wf, 4),
                   calibration=f"int32 bitwise_not (torch elementwise kernel) over {CALIB_BYTES} bytes: FETCH_SIZE "
                               f"{np.mean(f_cal):.0f} KiB, WRITE_SIZE {np.mean(w_cal):.0f} KiB per dispatch",
                   source_sha256=decode_source_digest(), shapes=shapes)
    lines = ["# gemm_decode_kernel — HBM traffic at the headline decode shapes", "",
             "Two counter runs of the same workload (`python bench.py --traffic-pass`: the",
             "decode GEMM of each headline shape once per rotated weight copy, after a",
             f"calibration copy of {CALIB_BYTES >> 20} MiB):", "", "```", *command, "```", "",
             "Each counter is scaled by what it reads for the calibration copy (known",
             "bytes read and written), then averaged per shape over its launches;",
             "`traffic_bytes_per_launch` is the mean over the 9 shapes, as `achieved`",
             "in the benchmark's roofline.  bench.py reports it only while",
             "`source_sha256` matches the decode kernel's sources.  The decode GEMM is",
             "`gemm_decode_kernel`, or its persistent form `gemm_decode_persist_kernel` where",
             "that is chosen (at these shapes: M = 16, N = 34816).", "",
             "| M | N | K | launches | FETCH KiB | WRITE KiB | HBM bytes | algorithmic | ratio |",
             "|---|---|---|---|---|---|---|---|---|"]
    for r in shapes:
        lines.append(f"| {r['M']} | {r['N']} | {r['K']} | {r['launches']} | {r['fetch_kib']} | "
                     f"{r['write_kib']} | {r['hbm_bytes']} | {r['algorithmic_bytes']} | {r['ratio']} |")
    lines += ["", "```json", json.dumps(summary), "```", ""]
    with open(TRAFFIC_MD, "w") as fh:
        fh.write("\n".join(lines))
    print(f"wrote {TRAFFIC_MD}: traffic {traffic:.0f} B/launch")


PROFILE_MD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                          "all_kernels__bench_default.md")


def trace_summary(stats_csv, trace_csv, marker_csv, bench_log, command):
    """The committed kernel-statistics summary of a traced default run
    (PROFILE_MD): rocprofv3's per-kernel statistics, and the roofline
    kernel's launches selected by the run's marker ranges next to the
    roofline.launch_us that run printed."""
    import csv
    import re
    stats = list(csv.DictReader(open(stats_csv)))
    trace = list(csv.DictReader(open(trace_csv)))
    marks = [r for r in csv.DictReader(open(marker_csv)) if "roofline" in json.dumps(r)]
    line = [l for l in open(bench_log) if l.startswith("{")][-1]
    bench = json.loads(line)
    per_shape = []
    for mk in marks:
        label = next(v for v in mk.values() if isinstance(v, str) and v.startswith("roofline"))
        t0, t1 = int(mk["Start_Timestamp"]), int(mk["End_Timestamp"])
        d = [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in trace
             if _is_decode_gemm(r["Kernel_Name"]) and t0 <= int(r["Start_Timestamp"]) <= t1]
        if d:
            per_shape.append((label, len(d), float(np.mean(d))))
    trace_us = float(np.mean([a for _, _, a in per_shape])) / 1e3 if per_shape else float("nan")
    lines = ["# rocprofv3 kernel statistics: `bench.py` default run (all kernels)", "",
             "Workload: the default `bench.py` run on one MI355X (headline step, roofline loop, "
             "decode sweep, prefill sweep, A16WFP4 BMM sweep, load-time weight quantisation).", "",
             "Command (from the repository root on the GPU host):", "", "```", *command, "```", "",
             "Durations in ns as written by rocprofv3 (`--stats`). Kernel-trace instrumentation",
             "lengthens short launches and slows graph replay, so the run's own event timings",
             "differ a little from untraced runs.", "",
             "| Kernel | Calls | Total ns | Average ns | % | Min ns | Max ns |",
             "|---|---|---|---|---|---|---|"]
    for r in stats:
        lines.append(f"| `{r['Name'][:100]}` | {r['Calls']} | {int(float(r['TotalDurationNs']))} | "
                     f"{int(float(r['AverageNs']))} | {float(r['Percentage']):.2f} | {r['MinNs']} | "
                     f"{r['MaxNs']} |")
    lines += ["", "## Roofline kernel: the decode GEMM at the 9 headline shapes", "",
              "Launches of the decode GEMM (`gemm_decode_kernel`, or `gemm_decode_persist_kernel`",
              "where that form is chosen) inside the run's `roofline M=.. N=.. K=..` marker",
              "ranges (kernel duration from the trace), averaged per shape, then over the shapes",
              "-- the same averaging as the benchmark's `roofline.launch_us`, which times the",
              "same graph replays with HIP events (dispatch gaps included).", "",
              "| Shape | Launches | Trace mean us |", "|---|---|---|"]
    for label, n, a in per_shape:
        lines.append(f"| {label[len('roofline '):]} | {n} | {a / 1e3:.3f} |")
    roof = bench.get("roofline", {})
    lines += ["", f"Trace mean over shapes: **{trace_us:.3f} us**; the same run's "
              f"`roofline.launch_us`: **{roof.get('launch_us')} us** (achieved "
              f"{roof.get('achieved')} GB/s, frac {roof.get('frac')}).", ""]
    with open(PROFILE_MD, "w") as fh:
        fh.write("\n".join(lines))
    print(f"wrote {PROFILE_MD}: trace {trace_us:.3f} us vs launch_us {roof.get('launch_us')}")


PREFILL_MD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                          "gemm_prefill_kernel__M8192_counters.md")


def prefill_counter_summary(trace_csv, pmc_csv, command):
    """The committed prefill counter summary (PREFILL_MD): per launch of
    prefill_pass, the kernel-trace duration, the shader clock the launch ran
    at (GRBM_GUI_ACTIVE summed over the 8 XCDs / 8 / the counter run's own
    duration) and the MFMA pipes' busy share (SQ_VALU_MFMA_BUSY_CYCLES summed
    over the 1024 SIMDs / (1024 x those cycles)).  A 16x16x128 FP4 MFMA keeps
    its pipe 16 cycles for 65536 FLOP, so the algorithmic MFMA cycles of a
    GEMM are 2MNK/65536 x 16 = MNK/2048."""
    import csv
    trace = [r for r in csv.DictReader(open(trace_csv)) if "gemm_prefill_kernel" in r["Kernel_Name"]]
    trace.sort(key=lambda r: int(r["Start_Timestamp"]))
    pmc = {}
    for r in csv.DictReader(open(pmc_csv)):
        if "gemm_prefill_kernel" not in r["Kernel_Name"]:
            continue
        d = pmc.setdefault(int(r["Dispatch_Id"]), {"us": (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3})
        d[r["Counter_Name"]] = float(r["Counter_Value"])
    pmc = [pmc[k] for k in sorted(pmc)]
    M = PREFILL_PASS_M
    per = 1 + PREFILL_PASS_REPS
    assert len(trace) == len(pmc) == per * len(DECODE_NK), (len(trace), len(pmc))
    keep = [i for i in range(len(trace)) if i % per]   # drop each shape's warm-up launch
    trace = [trace[i] for i in keep]
    pmc = [pmc[i] for i in keep]
    shapes = [(N, K) for (N, K) in DECODE_NK for _ in range(PREFILL_PASS_REPS)]
    rows = []
    for (N, K), t, c in zip(shapes, trace, pmc):
        us = (int(t["End_Timestamp"]) - int(t["Start_Timestamp"])) / 1e3
        cyc = c["GRBM_GUI_ACTIVE"] / 8
        ghz = cyc / (c["us"] * 1e3)
        alg = M * N * K / 2048
        busy = c["SQ_VALU_MFMA_BUSY_CYCLES"] / (1024 * cyc)
        pf = 2.0 * M * N * K / (us * 1e-6) / 1e15
        rows.append(dict(N=N, K=K, trace_us=round(us, 1), pflops=round(pf, 3), frac=round(pf / 10.1, 3),
                         counter_run_us=round(c["us"], 1), clock_ghz=round(ghz, 3),
                         mfma_cycles=int(c["SQ_VALU_MFMA_BUSY_CYCLES"]), algorithmic_mfma_cycles=int(alg),
                         mfma_busy=round(busy, 3), frac_at_clock=round(pf / (10.1 * ghz / 2.4), 3)))
    lines = ["# gemm_prefill_kernel — clock and MFMA occupancy at M = 8192", "",
             "Workload `python bench.py --prefill-pass`: the prefill GEMM (bf16 out, no bias) at",
             f"M = {M} for each (N, K), a warm-up launch (not listed) then {PREFILL_PASS_REPS} launches back to",
             "back, on the prefill sweep's inputs",
             "(activations seed 3 with outliers, weights seed 2). One kernel-trace run and one",
             "counter run (`GRBM_GUI_ACTIVE` and `SQ_VALU_MFMA_BUSY_CYCLES` in one pass):", "",
             "```", *command, "```", "",
             "- clock = GRBM_GUI_ACTIVE / 8 XCDs / the counter run's duration of that launch;",
             "- MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x those cycles);",
             "- algorithmic MFMA cycles = M N K / 2048 (16 cycles per 16x16x128 FP4 MFMA of",
             "  65536 FLOP): equal to the counter means no MFMA beyond the product's own;",
             "- frac = PFLOP/s (trace duration) / 10.1; frac at clock = the same against",
             "  10.1 PF x clock / 2.4 GHz.", "",
             "At N = 5120, K = 14336 the 640 tiles fill 2.5 rounds of the 256 workgroups: that",
             "launch takes the split schedule (the 128 leftover tiles in 2 K slices each,",
             "before 2 rounds of whole tiles); the other two shapes fill whole rounds.", "",
             "| N | K | trace us | PFLOP/s | frac | counter-run us | clock GHz | MFMA cycles | algorithmic | MFMA busy | frac at clock |",
             "|---|---|---|---|---|---|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| {r['N']} | {r['K']} | {r['trace_us']} | {r['pflops']} | {r['frac']} | {r['counter_run_us']} | "
                     f"{r['clock_ghz']} | {r['mfma_cycles']} | {r['algorithmic_mfma_cycles']} | {r['mfma_busy']} | "
                     f"{r['frac_at_clock']} |")
    lines += ["", "```json", json.dumps(dict(kernel="gemm_prefill_kernel", M=M, launches=rows)), "```", ""]
    with open(PREFILL_MD, "w") as fh:
        fh.write("\n".join(lines))
    print(f"wrote {PREFILL_MD}")
    for r in rows:
        print(r)


def prefill_stall_md(M):
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                        f"gemm_prefill_kernel__M{M}_stall_counters.md")
# the three counter passes of the stall summary (each well within one
# pass's limits: at most 8 SQ and 2 GRBM counters)
STALL_PASSES = [
    ["GRBM_GUI_ACTIVE", "SQ_WAVE_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_WAIT_INST_LDS",
     "SQ_VALU_MFMA_BUSY_CYCLES"],
    ["GRBM_GUI_ACTIVE", "SQ_WAVE_CYCLES", "SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS",
     "SQ_ACTIVE_INST_VMEM"],
    ["GRBM_GUI_ACTIVE", "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_ADDR_CONFLICT", "SQ_LDS_DATA_FIFO_FULL",
     "SQ_LDS_IDX_ACTIVE", "SQ_INSTS_MFMA"],
]


def prefill_stall_summary(pmc_a, pmc_b, pmc_c, command, M=PREFILL_PASS_M):
    """Where the prefill kernel's waves spend their time (prefill_stall_md(M)):
    three counter passes of prefill_pass(M) (STALL_PASSES), per (N, K) averaged over the measured
    launches (each shape's warm-up launch dropped).  SQ_WAVE_CYCLES and the
    SQ_WAIT_* counters count quad-cycles summed over waves; the SQ_ACTIVE_INST_*
    counters count cycles summed over waves; per-SE counters are summed over
    the 32 SEs (8 XCDs x 4)."""
    import csv

    def load(path):
        d = {}
        for r in csv.DictReader(open(path)):
            name = r["Kernel_Name"]
            if "gemm_prefill_kernel" not in name and "gemm_prefill_n128_kernel" not in name:
                continue
            e = d.setdefault(int(r["Dispatch_Id"]), {"us": (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3,
                                                       "bn": 128 if "n128" in name else 256})
            e[r["Counter_Name"]] = e.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        return [d[k] for k in sorted(d)]

    A, B, C = load(pmc_a), load(pmc_b), load(pmc_c)
    per = 1 + PREFILL_PASS_REPS
    assert len(A) == len(B) == len(C) == per * len(DECODE_NK), (len(A), len(B), len(C))
    rows = []
    for si, (N, K) in enumerate(DECODE_NK):
        ia = [A[si * per + k] for k in range(1, per)]
        ib = [B[si * per + k] for k in range(1, per)]
        ic = [C[si * per + k] for k in range(1, per)]

        def mean(lst, key):
            return float(np.mean([e[key] for e in lst]))
        cyc = mean(ia, "GRBM_GUI_ACTIVE") / 8                     # per XCD: the kernel's cycles
        wave_cyc = 4 * mean(ia, "SQ_WAVE_CYCLES")                  # summed over waves
        wave_cyc_b = 4 * mean(ib, "SQ_WAVE_CYCLES")
        pf = 2.0 * M * N * K / (mean(ia, "us") * 1e-6) / 1e15
        bn = ia[0]["bn"]
        tiles = -(-M // 256) * -(-N // bn)
        rows.append(dict(
            N=N, K=K, tile=f"256x{bn}", tiles=tiles,
            counter_run_us=round(mean(ia, "us"), 1), clock_ghz=round(cyc / (mean(ia, "us") * 1e3), 3),
            pflops_counter_run=round(pf, 3),
            mfma_busy=round(mean(ia, "SQ_VALU_MFMA_BUSY_CYCLES") / (1024 * cyc), 3),
            wave_wait_any=round(4 * mean(ia, "SQ_WAIT_ANY") / wave_cyc, 3),
            wave_wait_inst_any=round(4 * mean(ia, "SQ_WAIT_INST_ANY") / wave_cyc, 3),
            wave_wait_inst_lds=round(4 * mean(ia, "SQ_WAIT_INST_LDS") / wave_cyc, 3),
            wave_active_any=round(mean(ib, "SQ_ACTIVE_INST_ANY") / wave_cyc_b, 3),
            wave_active_valu=round(mean(ib, "SQ_ACTIVE_INST_VALU") / wave_cyc_b, 3),
            wave_active_lds=round(mean(ib, "SQ_ACTIVE_INST_LDS") / wave_cyc_b, 3),
            wave_active_vmem=round(mean(ib, "SQ_ACTIVE_INST_VMEM") / wave_cyc_b, 3),
            lds_insts_per_kstep_per_wave=round(mean(ic, "SQ_INSTS_LDS") / (tiles * (K / 128) * 8), 2),
            mfma_insts_per_kstep_per_wave=round(mean(ic, "SQ_INSTS_MFMA") / (tiles * (K / 128) * 8), 2),
            lds_active_per_cu=round(mean(ic, "SQ_LDS_IDX_ACTIVE") / (256 * mean(ic, "GRBM_GUI_ACTIVE") / 8), 3),
            lds_bank_conflict_per_cu=round(mean(ic, "SQ_LDS_BANK_CONFLICT") / (256 * mean(ic, "GRBM_GUI_ACTIVE") / 8), 4),
            lds_addr_conflict_per_cu=round(mean(ic, "SQ_LDS_ADDR_CONFLICT") / (256 * mean(ic, "GRBM_GUI_ACTIVE") / 8), 4),
            lds_data_fifo_full_per_cu=round(mean(ic, "SQ_LDS_DATA_FIFO_FULL") / (256 * mean(ic, "GRBM_GUI_ACTIVE") / 8), 4)))
    arg = "" if M == PREFILL_PASS_M else f" {M}"
    lines = [f"# gemm_prefill_kernel — where the waves spend their time at M = {M}", "",
             f"Workload `python bench.py --prefill-pass{arg}` (the prefill GEMM at M = {M} for each",
             f"(N, K), whole tiles, a warm-up launch then {PREFILL_PASS_REPS} launches, sweep inputs;",
             "the tile width is the one the launcher picks, 256 x 128 where 256-wide tiles would fill",
             "at most half a round of compute units). Three counter passes:", "",
             "```", *command, "```", "",
             "Per shape, the mean over the measured launches of:",
             "- clock = GRBM_GUI_ACTIVE / 8 XCDs / the launch's duration in the counter run;",
             "- MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x those cycles);",
             "- wave shares: each counter over the waves' total cycles (4 x SQ_WAVE_CYCLES):",
             "  waiting for anything (`s_waitcnt`, barrier: SQ_WAIT_ANY), waiting to issue",
             "  (SQ_WAIT_INST_ANY; its LDS part SQ_WAIT_INST_LDS), and executing any / VALU",
             "  (MFMA included) / LDS / VMEM instructions (SQ_ACTIVE_INST_*);",
             "- LDS and MFMA instructions per K-step per wave (SQ_INSTS_* over tiles x K-steps x 8",
             "  waves; per K-step and wave the 256-wide loop issues 12 fragment reads and 32 MFMAs,",
             "  the 128-wide one 10 and 16, each one scale read per 4 steps);",
             "- per-CU LDS shares: SQ_LDS_IDX_ACTIVE (LDS busy with indexed reads and writes), bank",
             "  and address conflict stalls, data-FIFO-full cycles, over 256 CUs x the cycles.", "",
             "| N | K | tile | tiles | us | GHz | PF | MFMA busy | wait any | wait issue | wait issue LDS | active any | active VALU | active LDS | active VMEM | LDS/step/wave | MFMA/step/wave | LDS busy/CU | bank confl/CU | addr confl/CU | LDS data FIFO full/CU |",
             "|---|---|---|---|---|---|---|---|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for r in rows:
        lines.append("| " + " | ".join(str(r[k]) for k in (
            "N", "K", "tile", "tiles", "counter_run_us", "clock_ghz", "pflops_counter_run", "mfma_busy", "wave_wait_any",
            "wave_wait_inst_any", "wave_wait_inst_lds", "wave_active_any", "wave_active_valu", "wave_active_lds",
            "wave_active_vmem", "lds_insts_per_kstep_per_wave", "mfma_insts_per_kstep_per_wave", "lds_active_per_cu",
            "lds_bank_conflict_per_cu", "lds_addr_conflict_per_cu", "lds_data_fifo_full_per_cu")) + " |")
    lines += ["", "```json", json.dumps(dict(kernel="gemm_prefill_kernel", M=M, shapes=rows)), "```", ""]
    with open(prefill_stall_md(M), "w") as fh:
        fh.write("\n".join(lines))
    print(f"wrote {prefill_stall_md(M)}")
    for r in rows:
        print(r)


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "--prefill-stall-summary":
        if sys.argv[2] == "--m":
            return prefill_stall_summary(sys.argv[4], sys.argv[5], sys.argv[6], sys.argv[7:], int(sys.argv[3]))
        return prefill_stall_summary(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5:])
    if len(sys.argv) > 1 and sys.argv[1] == "--hbm-pass":
        return hbm_pass()
    if len(sys.argv) > 1 and sys.argv[1] == "--hbm-summary":
        return hbm_summary(sys.argv[2], sys.argv[3], sys.argv[4:])
    if len(sys.argv) > 1 and sys.argv[1] == "--prefill-summary":
        return prefill_counter_summary(sys.argv[2], sys.argv[3], sys.argv[4:])
    if len(sys.argv) > 1 and sys.argv[1] == "--trace-summary":
        return trace_summary(*sys.argv[2:6], sys.argv[6:])
    if len(sys.argv) > 1 and sys.argv[1] == "--traffic-pass":
        return traffic_pass()
    if len(sys.argv) > 1 and sys.argv[1] == "--prefill-pass":
        return prefill_pass(int(sys.argv[2]) if len(sys.argv) > 2 else PREFILL_PASS_M)
    if len(sys.argv) > 1 and sys.argv[1] == "--traffic-summary":
        return traffic_summary(sys.argv[2], sys.argv[3], sys.argv[4:])
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-bmm", action="store_true")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the W4A4 linear and the BMM run on a single MI355X "
              "and the library has no multi-GPU path (--gpus must be 1).", file=sys.stderr)
        sys.exit(2)

    import mxfp4_block_scaled_quant_amd as mx
    from mxfp4_block_scaled_quant_amd import inputs

    mx.lib()   # fail loudly if the HIP library is missing
    if not torch.cuda.is_available():
        print("bench.py needs a gfx950 GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    T = Timer()

    def dev_bf16(bits):
        return inputs.bits_to_torch_bf16(bits).to(dev)

    # ---------------- load time: weights quantised + preshuffled, rotated copies
    t_load = time.time()
    weights = {}
    preshuffle_s = {}
    for (N, K) in DECODE_NK:
        w = dev_bf16(inputs.weights(N, K, 2))
        torch.cuda.synchronize()
        t0 = time.time()
        W = mx.quantize_weight(w)
        torch.cuda.synchronize()
        preshuffle_s[(N, K)] = time.time() - t0
        R = copies_for(W.w_pre.numel() + W.ws_pre.numel())
        copies = [W] + [mx.MXFP4Weight(W.w_pre.clone(), W.ws_pre.clone(), N, K) for _ in range(R - 1)]
        weights[(N, K)] = copies
        del w
    torch.cuda.synchronize()

    log(f"weights quantised + preshuffled, {sum(len(v) for v in weights.values())} rotation copies")
    # ---------------- headline: decode sweep M <= 16, quant + GEMM + bias
    cases = []
    for (N, K) in DECODE_NK:
        b = dev_bf16(inputs.bias(N, 2))
        for M in HEADLINE_M:
            x = dev_bf16(inputs.activations(M, K, 2))
            out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            need = mx.linear_workspace_bytes(M, N, K)
            work = torch.empty(need, dtype=torch.uint8, device=dev) if need else None
            cases.append(dict(M=M, N=N, K=K, x=x, out=out, bias=b, work=work))

    def launch_case(c, copy):
        mx.mxfp4_linear(c["x"], copy.w_pre, copy.ws_pre, c["N"], c["bias"], torch.bfloat16,
                        out=c["out"], workspace=c["work"])

    # Rotation: at position p of the cycle, the j-th launch of shape (N,K) in
    # the step uses copy (p * per_step + j) mod R; the cycle repeats after
    # lcm over shapes of R / gcd(R, per_step) steps.
    per_step = {nk: sum(1 for c in cases if (c["N"], c["K"]) == nk) for nk in DECODE_NK}
    cycle = 1
    for nk in DECODE_NK:
        R = len(weights[nk])
        k = R // np.gcd(R, per_step[nk])
        cycle = int(np.lcm(cycle, k))

    def capture_steps(pos, n):
        """A graph of n consecutive steps from rotation position pos."""
        counters = {nk: (pos * per_step[nk]) % len(weights[nk]) for nk in DECODE_NK}

        def body():
            for _ in range(n):
                for c in cases:
                    nk = (c["N"], c["K"])
                    launch_case(c, weights[nk][counters[nk] % len(weights[nk])])
                    counters[nk] += 1
        return T.capture(body)

    # Steps are replayed as graphs of HEADLINE_GRAPH_STEPS steps (each graph
    # holds 9 x that many linear calls, as a captured decode pass over a
    # model's layers would), single-step graphs for any remainder: each graph
    # launch costs ~4 us of its own before its first kernel (measured: 127.5
    # us per step with one step per graph, 123.2 with ten).
    step_graphs = [capture_steps(p, 1) for p in range(cycle)]
    multi = {}

    def run_steps(pos, n, events=None):
        """Replay n steps from position pos; returns the next position.  With
        `events`, one event after every full multi-step graph."""
        G = HEADLINE_GRAPH_STEPS
        for _ in range(n // G):
            if pos not in multi:
                multi[pos] = capture_steps(pos, G)
            multi[pos].replay()
            if events is not None:
                events.append(torch.cuda.Event(enable_timing=True))
                events[-1].record()
            pos = (pos + G) % cycle
        for _ in range(n % G):
            step_graphs[pos].replay()
            pos = (pos + 1) % cycle
        return pos

    # capture every multi-step graph the runs below replay, before any timing
    pos = args.warmup % cycle
    for _ in range(2 * (args.steps // HEADLINE_GRAPH_STEPS) + 1):
        if pos not in multi:
            multi[pos] = capture_steps(pos, HEADLINE_GRAPH_STEPS)
        pos = (pos + HEADLINE_GRAPH_STEPS) % cycle
    for i in range(args.warmup):
        step_graphs[i % cycle].replay()
    torch.cuda.synchronize()
    pos = args.warmup % cycle
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with ClockSampler() as clk_head:
        e0.record()
        pos = run_steps(pos, args.steps)
        e1.record()
        torch.cuda.synchronize()
    step_s = e0.elapsed_time(e1) * 1e-3 / args.steps
    # The spread: as many steps again, an event after every multi-step graph
    # (per step: the graph's time over its steps); an event between replays
    # costs a few microseconds of its own, so it stays out of the figure above.
    evs = [torch.cuda.Event(enable_timing=True)]
    evs[0].record()
    pos = run_steps(pos, args.steps - args.steps % HEADLINE_GRAPH_STEPS, evs)
    torch.cuda.synchronize()
    chunk = HEADLINE_GRAPH_STEPS
    step_stats = (_stats([evs[j].elapsed_time(evs[j + 1]) * 1e-3 / chunk for j in range(len(evs) - 1)])
                  if len(evs) > 1 else _stats([step_s]))
    # The same steps with one graph per step, for comparison with that form.
    torch.cuda.synchronize()
    e2, e3 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e2.record()
    for i in range(args.steps):
        step_graphs[(pos + i) % cycle].replay()
    e3.record()
    torch.cuda.synchronize()
    step_s_single = e2.elapsed_time(e3) * 1e-3 / args.steps
    step_bytes = sum(pipeline_bytes(c["M"], c["N"], c["K"], True) for c in cases)
    value_gbs = step_bytes / step_s / 1e9

    log(f"headline: {step_s * 1e6:.2f} us/step, {value_gbs:.1f} GB/s")
    # ---------------- dominant kernel: the decode GEMM alone, per shape
    def per_launch_time(launch, nvariants, reps_target):
        """Mean time of one launch: a graph of >= MIN_LAUNCHES back-to-back
        launches (cycling over `nvariants` input copies) replayed and timed
        with events, so graph-launch overhead is amortised."""
        n = nvariants * -(-MIN_LAUNCHES // nvariants)

        def body():
            for i in range(n):
                launch(i % nvariants)

        g = T.capture(body)
        reps = max(8, reps_target // n)
        st = T.time_graphs([g], reps)
        return {k: (v / n if k != "n" else v) for k, v in st.items()}

    def gemm_only_time(M, N, K, x_q, x_s, bias, out, copies, reps_target=400):
        def launch(i):
            cp = copies[i]
            mx.mxfp4_gemm_a4w4(x_q, x_s, cp.w_pre, cp.ws_pre, M, N, K, bias, torch.bfloat16, out=out)
        return per_launch_time(launch, len(copies), reps_target)

    def linear_time(M, N, K, x, bias, out, copies, reps_target=400):
        need = mx.linear_workspace_bytes(M, N, K)
        work = torch.empty(need, dtype=torch.uint8, device=dev) if need else None

        def launch(i):
            cp = copies[i]
            mx.mxfp4_linear(x, cp.w_pre, cp.ws_pre, N, bias, torch.bfloat16, out=out, workspace=work)
        return per_launch_time(launch, len(copies), reps_target)

    def quant_time(x, q, s, reps_target=400):
        return per_launch_time(lambda i: mx.mxfp4_quant_1x32(x, mx.MXFP4_LAYOUT_GEMM, q=q, scales=s),
                               1, reps_target)

    # The roofline kernel first, on its own: the decode GEMM at the headline
    # shapes, each shape inside a marker range so a kernel trace of this run
    # can select exactly these launches.
    roof_t = {}
    with ClockSampler() as clk_roof:
        for (N, K) in DECODE_NK:
            b = dev_bf16(inputs.bias(N, 2))
            for M in HEADLINE_M:
                x = dev_bf16(inputs.activations(M, K, 2))
                q, s = mx.mxfp4_quant_1x32(x, mx.MXFP4_LAYOUT_GEMM)
                out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
                torch.cuda.synchronize()
                torch.cuda.nvtx.range_push(f"roofline M={M} N={N} K={K}")
                roof_t[(M, N, K)] = gemm_only_time(M, N, K, q, s, b, out, weights[(N, K)])
                torch.cuda.synchronize()
                torch.cuda.nvtx.range_pop()

    decode_rows = []
    for (N, K) in DECODE_NK:
        b = dev_bf16(inputs.bias(N, 2))
        for M in DECODE_M:
            x = dev_bf16(inputs.activations(M, K, 2))
            q, s = mx.mxfp4_quant_1x32(x, mx.MXFP4_LAYOUT_GEMM)
            out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            ts = roof_t.get((M, N, K)) or gemm_only_time(M, N, K, q, s, b, out, weights[(N, K)])
            gb = gemm_bytes(M, N, K, True)
            tq = quant_time(x, q, s)
            tls = linear_time(M, N, K, x, b, out, weights[(N, K)])
            qr, sr = mx.mxfp4_quant_1x32(x, mx.MXFP4_LAYOUT_ROWMAJOR)
            sr = sr.reshape(M, K // 32)
            cps = weights[(N, K)]
            tp = per_launch_time(lambda i: mx.mxfp4_linear_prequantized(
                qr, sr, cps[i].w_pre, cps[i].ws_pre, N, b, torch.bfloat16, out=out), len(cps), 400)
            oq = torch.empty((M, N // 2), dtype=torch.uint8, device=dev)
            osc = torch.empty((M, N // 32), dtype=torch.uint8, device=dev)
            tf4 = per_launch_time(lambda i: mx.mxfp4_gemm_a4w4_mxfp4_out(
                q, s, cps[i].w_pre, cps[i].ws_pre, M, N, K, b, out_fp4=oq, out_scales=osc), len(cps), 400)
            pb = pipeline_bytes(M, N, K, True)
            t, tl = ts["mean"], tls["mean"]
            decode_rows.append(dict(M=M, N=N, K=K,
                                    linear_us=round(tl * 1e6, 3),
                                    linear_GBps=round(pb / tl / 1e9, 1),
                                    linear_hbm_frac=round(pb / tl / PEAK_HBM, 4),
                                    linear_spread_us=_us(tls),
                                    gemm_us=round(t * 1e6, 3),
                                    gemm_GBps=round(gb / t / 1e9, 1),
                                    hbm_frac=round(gb / t / PEAK_HBM, 4),
                                    gemm_spread_us=_us(ts),
                                    quant_us=round(tq["mean"] * 1e6, 3),
                                    prequantized_us=round(tp["mean"] * 1e6, 3),
                                    mxfp4_out_us=round(tf4["mean"] * 1e6, 3),
                                    tflops=round(2 * M * N * K / tl / 1e12, 2)))
    head_rows = [r for r in decode_rows if r["M"] in HEADLINE_M]
    dom_bytes = sum(gemm_bytes(r["M"], r["N"], r["K"], True) for r in head_rows)
    dom_time = sum(r["gemm_us"] for r in head_rows) * 1e-6
    achieved = dom_bytes / len(head_rows) / (dom_time / len(head_rows))
    # the spread of the roofline kernel's per-launch rate over the shapes'
    # replays: each shape's p10 / p50 / p90 launch time, averaged over shapes
    roof_spread = {q: round(dom_bytes / sum(roof_t[(r["M"], r["N"], r["K"])][q] for r in head_rows) / 1e9, 1)
                   for q in ("p10", "p50", "p90")}

    log("decode sweep done")
    # ---------------- prefill sweep (GEMM, TFLOP/s vs the FP4 peak)
    prefill_rows = []
    clk_prefill = None
    if not args.no_prefill:
        with ClockSampler() as clk:
            for (N, K) in DECODE_NK:
                for M in PREFILL_M:
                    x = dev_bf16(inputs.activations(M, K, 3, outliers=True))
                    q, s = mx.mxfp4_quant_1x32(x, mx.MXFP4_LAYOUT_GEMM)
                    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
                    cps = weights[(N, K)][:4]
                    ts = gemm_only_time(M, N, K, q, s, None, out, cps, reps_target=40)
                    oq = torch.empty((M, N // 2), dtype=torch.uint8, device=dev)
                    osc = torch.empty((M, N // 32), dtype=torch.uint8, device=dev)
                    tf4 = per_launch_time(lambda i: mx.mxfp4_gemm_a4w4_mxfp4_out(
                        q, s, cps[i].w_pre, cps[i].ws_pre, M, N, K, None, out_fp4=oq, out_scales=osc),
                        len(cps), 40)["mean"]
                    tq = quant_time(x, q, s, reps_target=64)["mean"]
                    fl = 2 * M * N * K
                    t = ts["mean"]
                    prefill_rows.append(dict(M=M, N=N, K=K, gemm_us=round(t * 1e6, 2),
                                             gemm_spread_us=_us(ts),
                                             # split-K of the leftover tiles (it needs a workspace)
                                             schedule="split" if mx.gemm_workspace_bytes(M, N, K) else "whole",
                                             tflops=round(fl / t / 1e12, 1),
                                             fp4_peak_frac=round(fl / t / PEAK_FP4, 4),
                                             quant_us=round(tq * 1e6, 2),
                                             mxfp4_out_us=round(tf4 * 1e6, 2),
                                             mxfp4_out_tflops=round(fl / tf4 / 1e12, 1),
                                             quant_GBps=round(quant_bytes(M, K) / tq / 1e9, 1)))
                    del x, q, s, out, oq, osc
            torch.cuda.empty_cache()
        clk_prefill = clk.summary()
    big = [r for r in prefill_rows if r["M"] >= 2048]
    prefill_summary = None
    if big:
        fl = sum(2 * r["M"] * r["N"] * r["K"] for r in big)
        tt = sum(r["gemm_us"] for r in big) * 1e-6
        prefill_summary = dict(tflops_M_ge_2048=round(fl / tt / 1e12, 1),
                               fp4_peak_frac=round(fl / tt / PEAK_FP4, 4), sclk=clk_prefill,
                               shapes=prefill_rows)

    log("prefill sweep done")
    # ---------------- A16WFP4 BMM sweep (MLA absorbed K-up / V-up, 16 heads)
    bmm_rows = []
    if not args.no_bmm:
        for name, N, K, bm in BMM_CASES:
            w = dev_bf16(inputs.bmm_problem(BMM_HEADS, 1, N, K, 4)["w"].reshape(BMM_HEADS * N, K))
            W = mx.quantize_weight(w.reshape(BMM_HEADS, N, K))
            for M in BMM_M:
                x = dev_bf16(inputs.bmm_problem(BMM_HEADS, M, N, K, 4)["x"])
                # rotate activation copies once they are large enough to matter
                R = 1 if x.numel() * 2 < (8 << 20) else min(48, copies_for(x.numel() * 2))
                xs = [x] + [x.clone() for _ in range(R - 1)]
                out = (torch.empty((M, BMM_HEADS, N), dtype=torch.bfloat16, device=dev) if bm
                       else torch.empty((BMM_HEADS, M, N), dtype=torch.bfloat16, device=dev))

                ts = per_launch_time(lambda i: mx.a16wfp4_bmm(xs[i], W.w_pre, W.ws_pre, N, out=out,
                                                              batch_major=bm), R, 400)
                t = ts["mean"]
                by = bmm_bytes(BMM_HEADS, M, N, K)
                fl = 2 * BMM_HEADS * M * N * K
                bmm_rows.append(dict(op=name, M=M, N=N, K=K, us=round(t * 1e6, 3), spread_us=_us(ts),
                                     GBps=round(by / t / 1e9, 1), hbm_frac=round(by / t / PEAK_HBM, 4),
                                     tflops=round(fl / t / 1e12, 2)))
                del xs, x, out
            torch.cuda.empty_cache()

    log("bmm sweep done")
    # ---------------- CPU oracle on a bounded sample of the headline workload
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(inputs)

    traffic = read_traffic()
    line = {
        "metric": METRIC,
        "value": round(value_gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4",
        "data": "synthetic",
        "config": {
            "workload": "decode-sweep W4A4 MXFP4 linear at M<=16: per-1x32 quant of bf16 "
                        "activations + block-scaled FP4 GEMM + bf16 bias, bf16 out",
            "M": HEADLINE_M, "NK": DECODE_NK,
            "step": "9 shapes x mxfp4_linear (M=1, and M=4 at N=14336 and N=34816: quant fused "
                    "into the GEMM; else quant then GEMM), weights preshuffled at load, rotated copies",
            "hbm_frac": round(value_gbs * 1e9 / PEAK_HBM, 4),
        },
        "step_spread_us": dict(_us(dict(step_stats, mean=step_s)), steps_per_sample=chunk),
        "graph_steps": HEADLINE_GRAPH_STEPS,
        "one_step_per_graph": {"ms_per_step": round(step_s_single * 1e3, 5),
                               "value": round(step_bytes / step_s_single / 1e9, 1)},
        "sclk": {"headline": clk_head.summary(), "roofline": clk_roof.summary()},
        "roofline": {
            "kernel": "decode W4A4 GEMM (gemm_decode_kernel; gemm_decode_persist_kernel at M=16, N=34816), "
                      "M<=16, mean over the 9 headline shapes",
            "bound": "hbm",
            "achieved": round(achieved / 1e9, 1),
            "peak": PEAK_HBM / 1e9,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM, 4),
            "traffic": traffic["traffic_bytes_per_launch"] if traffic else None,
            "launch_us": round(dom_time / len(head_rows) * 1e6, 3),
            "bytes_per_launch": round(dom_bytes / len(head_rows)),
            "achieved_at_p10_p50_p90_launch": roof_spread,
        },
        "cpu_baseline": cpu,
        "decode_sweep": decode_rows,
        "prefill": prefill_summary,
        "bmm": bmm_rows or None,
        "preshuffle_load_s": {f"{n}x{k}": round(v, 4) for (n, k), v in preshuffle_s.items()},
        "setup_s": round(time.time() - t_load, 1),
    }
    print(json.dumps(line), flush=True)


def _oracle_time(fn, budget_s):
    """Seconds per call of fn, repeated for about budget_s."""
    t0 = time.perf_counter()
    reps = 0
    while True:
        fn()
        reps += 1
        if time.perf_counter() - t0 > budget_s:
            break
    return (time.perf_counter() - t0) / reps


def cpu_baseline(inputs):
    """The oracle, as it stands, on bounded samples (about 20 s of CPU work in
    all).  Headline (the reported value, in the metric's GB/s): each headline
    shape with the first 256 output columns, repeated for about 1.5 s; weight
    quantisation is load time (untimed), as on the GPU; the timed work per
    shape is quant(x) + dequantise + fp64 matmul + bias.  Beside it, in their
    own units: one prefill shape (M = 2048, N = 14336, K = 5120) restricted to
    256 output columns (TFLOP/s over the sample's 2MNK) and one A16WFP4 BMM
    (MLA V-up, M = 256, 16 heads: GB/s over its algorithmic bytes)."""
    from oracle import linalg as OL
    from oracle import quant as OQ
    try:
        import threadpoolctl
        threads = max(i["num_threads"] for i in threadpoolctl.threadpool_info()
                      if i.get("user_api") == "blas")
    except Exception:
        threads = os.cpu_count()
    NS = 256
    total_bytes, total_s = 0.0, 0.0
    for (N, K) in DECODE_NK:
        w = inputs.weights(N, K, 2)[:NS]
        qw, sw = OQ.quant_1x32(w)
        b = inputs.bias(N, 2)[:NS]
        for M in HEADLINE_M:
            x = inputs.activations(M, K, 2)

            def step():
                qa, sa = OQ.quant_1x32(x)
                y, _ = OL.gemm_a4w4_from_quant(qa, sa, qw, sw, b)
                OL.to_bf16(y)
            total_s += _oracle_time(step, 1.5)
            total_bytes += pipeline_bytes(M, NS, K, True)
    # prefill sample
    Mp, Np, Kp = 2048, 14336, 5120
    xp = inputs.activations(Mp, Kp, 3, outliers=True)
    qwp, swp = OQ.quant_1x32(inputs.weights(Np, Kp, 2)[:NS])

    def pre():
        qa, sa = OQ.quant_1x32(xp)
        y, _ = OL.gemm_a4w4_from_quant(qa, sa, qwp, swp)
        OL.to_bf16(y)
    tp = _oracle_time(pre, 2.0)
    # BMM sample
    B, Mb, Nb, Kb = BMM_HEADS, 256, 256, 512
    pbm = inputs.bmm_problem(B, Mb, Nb, Kb, 4)
    qb, sb = OQ.quant_1x32(pbm["w"].reshape(B * Nb, Kb))
    qb, sb = qb.reshape(B, Nb, Kb // 2), sb.reshape(B, Nb, Kb // 32)

    def bmm():
        o, _ = OL.bmm_a16wfp4(pbm["x"], qb, sb)
        OL.to_bf16(o)
    tb = _oracle_time(bmm, 1.5)
    return {"value": round(total_bytes / total_s / 1e9, 4), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"headline shapes (M in {HEADLINE_M}, (N,K) in {DECODE_NK}) restricted to the "
                      f"first {NS} output columns; numpy fp64, BLAS threads {threads}; "
                      f"weight quantisation untimed (load time)",
            "prefill": {"value": round(2 * Mp * NS * Kp / tp / 1e12, 5), "unit": "TFLOP/s",
                        "sample": f"M={Mp}, N={Np} (first {NS} columns), K={Kp}: quant(x) + fp64 GEMM",
                        "seconds": round(tp, 3)},
            "bmm": {"value": round(bmm_bytes(B, Mb, Nb, Kb) / tb / 1e9, 4), "unit": "GB/s",
                    "sample": f"A16WFP4 V-up, {B} heads, M={Mb}, N={Nb}, K={Kb}: fp64 batched product",
                    "seconds": round(tb, 4)}}


if __name__ == "__main__":
    main()
