#!/usr/bin/env python3
"""W4A16 GEMM benchmark on one MI355X (gfx950).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extras] [--no-cpu-baseline] [--prefill-only]

A step is one pass of the decode workload through the C ABI: the symmetric
uint4b8 fp16 GEMMs with G = 128 for M in {1, 4, 8, 16} and (N, K) in
{(4096, 4096), (14336, 4096), (4096, 14336)}: twelve GEMMs, each dispatched on
M to the skinny kernel. Inputs are synthetic (seeded, w4a16_inputs) and
already repacked in HBM before timing (the repack is a one-time load step,
timed separately). Every launch reads a different copy of its weights from a
rotation pool larger than 1 GB, so neither L2 nor the 256 MB MALL can serve
them. Steps are captured into HIP graphs of eight steps each (step j of a
graph uses weight copy j mod 4), as a serving loop captures a forward pass,
plus one-step graphs for a remainder; W untimed steps, then exactly K timed
steps between a device synchronisation and HIP events on the launch stream.

Prints one JSON line: value = weight-stream GB/s of the whole step
(codes + scales [+ zeros] bytes per GEMM, summed, over the step time), the
roofline of the skinny kernel (algorithmic bytes incl. activations and
output per launch over its average duration, against 8 TB/s), the oracle's
CPU rate on a bounded sample, and extras: per-shape decode rates, the
skinny-vs-MFMA crossover and the prefill TFLOP/s of the MFMA kernel.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import mixed_precision_w4a16_repack_amd as w4  # noqa: E402
import w4a16_inputs as wi  # noqa: E402

METRIC = "W4A16 GEMM: weight-stream GB/s (M<=16) and TFLOP/s (M>=2048) vs peak, 1 GPU"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E
MFMA_PEAK_TFLOPS = 2516.6  # dense fp16/bf16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk
DEV = "cuda:0"
ROTATE_BYTES = 1 << 30
ROUND_STEPS = 8  # decode steps per captured graph
PREFILL_WARM_MS = 200.0  # GPU time of the same GEMM replayed before a prefill shape is timed


def weight_stream_bytes(N, K, G, qtype, with_zero_point):
    """Checkpoint bytes of one weight: codes + scales (+ packed zero points)."""
    Kg = K // wi.effective_group(K, G)
    b = N * K // 2 + N * Kg * 2
    if qtype == wi.UINT4 and with_zero_point:
        b += (N // 8) * Kg * 4
    return b


def algorithmic_bytes(M, N, K, G, qtype, with_zero_point):
    """Weight stream + activations read + output written (2-byte act)."""
    return weight_stream_bytes(N, K, G, qtype, with_zero_point) + M * K * 2 + M * N * 2


class Gemm:
    """One GEMM configuration with a rotation pool of packed weight copies."""

    def __init__(self, cfg_id, M, N, K, G, qtype, dtype, sigma, copies, path=w4.PATH_AUTO):
        case = wi.make_case(cfg_id, M, N, K, G, qtype, dtype, sigma=sigma)
        self.M, self.N, self.K, self.G, self.qtype, self.dtype = M, N, K, G, qtype, dtype
        self.path = path
        self.zp = case.weight_zero_point is not None
        wq = torch.from_numpy(case.weight_packed).to(DEV)
        ws = case.weight_scale.to(DEV)
        zp = None if case.weight_zero_point is None else torch.from_numpy(case.weight_zero_point).to(DEV)
        first = w4.repack(wq, ws, zp, G, qtype)
        self.packed = [first] + [first.clone() for _ in range(copies - 1)]
        self.A = case.A.to(DEV)
        self.C = torch.empty((M, N), dtype=case.torch_dtype, device=DEV)
        self.ws = w4.Workspace(DEV)
        self.ws.get(w4.workspace_size(M, N, K, G, path))
        self._repack_args = (wq, ws, zp)

    def launch(self, copy: int):
        w4.gemm(self.A, self.packed[copy % len(self.packed)], self.N, self.K, self.G, self.qtype,
                out=self.C, path=self.path, workspace=self.ws)

    @property
    def weight_bytes(self):
        return weight_stream_bytes(self.N, self.K, self.G, self.qtype, self.zp)

    @property
    def algo_bytes(self):
        return algorithmic_bytes(self.M, self.N, self.K, self.G, self.qtype, self.zp)

    @property
    def flops(self):
        return 2.0 * self.M * self.N * self.K

    def time_repack(self, reps=5):
        wq, ws, zp = self._repack_args
        out = torch.empty_like(self.packed[0])
        w4.repack(wq, ws, zp, self.G, self.qtype, out=out)
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(reps):
            w4.repack(wq, ws, zp, self.G, self.qtype, out=out)
        e.record()
        torch.cuda.synchronize()
        return s.elapsed_time(e) / reps * 1e3  # us


def capture_graphs(launch_fns_per_graph):
    """One HIP graph per list of launch callables (warmed up eagerly first)."""
    graphs = []
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for fns in launch_fns_per_graph:
            for f in fns:
                f()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for fns in launch_fns_per_graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for f in fns:
                f()
        graphs.append(g)
    torch.cuda.synchronize()
    return graphs


def time_graphs(graphs, reps, warmup):
    """Replays graphs round-robin; returns elapsed ms of `reps` replays."""
    for i in range(warmup):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for i in range(reps):
        graphs[i % len(graphs)].replay()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e)


def time_steps(round_graph, round_steps, step_graphs, steps, warmup):
    """Elapsed ms of exactly `steps` steps: whole rounds from round_graph,
    then the remainder from the one-step graphs (after `warmup` untimed
    steps the same way)."""
    def run(k):
        for _ in range(k // round_steps):
            round_graph.replay()
        for i in range(k % round_steps):
            step_graphs[i % len(step_graphs)].replay()

    run(warmup)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    run(steps)
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e)


def copies_for(total_bytes_per_round, minimum=2):
    return max(minimum, -(-ROTATE_BYTES // max(1, total_bytes_per_round)))


def decode_cases():
    wl = wi.WORKLOADS["decode_sym"]
    step_bytes = sum(weight_stream_bytes(N, K, wl["G"], wl["qtype"], False) for (_, N, K) in wl["shapes"])
    copies = copies_for(step_bytes)
    cases = [Gemm(wl["cfg_id"], M, N, K, wl["G"], wl["qtype"], wl["dtype"], wl["sigma"], copies)
             for (M, N, K) in wl["shapes"]]
    return cases, copies


def warm_up(graphs, warm_ms):
    """Replays graphs until about warm_ms of GPU time has passed, so that
    the clocks have left their idle state before anything is timed (a
    prefill GEMM follows seconds of host-side input generation)."""
    done, i = 0.0, 0
    while done < warm_ms:
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(4):
            graphs[i % len(graphs)].replay()
            i += 1
        e.record()
        torch.cuda.synchronize()
        done += s.elapsed_time(e)


def per_case_rate(g: Gemm, launches=None, reps=20, warm_ms=0.0):
    """Average duration of one launch of g, from graphs of back-to-back
    launches over its rotating copies (after warm_ms of the same work)."""
    n = launches or len(g.packed)
    graphs = capture_graphs([[(lambda c=c: g.launch(c)) for c in range(n)]])
    warm_up(graphs, warm_ms)
    ms = time_graphs(graphs, reps, 3)
    return ms * 1e3 / (reps * n)  # us per launch


def per_case_spread(g: Gemm, reps=30, min_launches=64):
    """p10 / p50 / p90 of the per-launch time over `reps` replays of one graph
    of back-to-back launches (cycling through the rotating copies, at least
    `min_launches` per graph so the replay's own overhead is spread thin), each
    replay bracketed by its own pair of events."""
    n = max(len(g.packed), min_launches)
    graph = capture_graphs([[(lambda c=c: g.launch(c)) for c in range(n)]])[0]
    for _ in range(3):
        graph.replay()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record()
    for i in range(reps):
        graph.replay()
        ev[i + 1].record()
    torch.cuda.synchronize()
    per = sorted(ev[i].elapsed_time(ev[i + 1]) * 1e3 / n for i in range(reps))
    pick = lambda q: per[min(reps - 1, int(round(q * (reps - 1))))]  # noqa: E731
    return {"p10_us": round(pick(0.1), 2), "p50_us": round(pick(0.5), 2), "p90_us": round(pick(0.9), 2)}


def cpu_model():
    """The host CPU's model name (first entry of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(budget_s=12.0):
    """The oracle (fp64, all host threads) on the decode workload's GEMMs,
    repeated until about budget_s seconds of CPU work."""
    import oracle

    wl = wi.WORKLOADS["decode_sym"]
    cases = [wi.make_case(wl["cfg_id"], M, N, K, wl["G"], wl["qtype"], wl["dtype"], sigma=wl["sigma"])
             for (M, N, K) in wl["shapes"]]
    done_bytes, done_gemms, used = 0, 0, 1
    t0 = time.perf_counter()
    while True:
        for c in cases:
            _, used = oracle.gemm(c.A, c.weight_packed, c.weight_scale, None, c.qtype, c.G)
            done_bytes += weight_stream_bytes(c.N, c.K, c.G, c.qtype, False)
            done_gemms += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {
        "value": round(done_bytes / dt / 1e9, 4),
        "unit": "GB/s",
        "cores": int(used),
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": f"{done_gemms} decode GEMMs (the step's 12 shapes in order, fp64 C oracle, all of each output) "
                  f"in {dt:.1f} s; weight-stream bytes / time",
    }


def kernel_source_hash():
    h = hashlib.sha256()
    for f in ("skinny.hip", "device_common.h", "exchange.h"):
        with open(os.path.join(ROOT, "mixed_precision_w4a16_repack_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM traffic per launch of the skinny kernel from the committed rocprofv3
    counter summary, if it was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", "skinny_decode_counters.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def _counter_rows(run_dir):
    """{dispatch id: (kernel name, {counter: value})} from a rocprofv3 --pmc
    csv directory (run_counter_collection.csv)."""
    import csv
    out = {}
    with open(os.path.join(run_dir, "run_counter_collection.csv")) as f:
        for r in csv.DictReader(f):
            d = out.setdefault(int(r["Dispatch_Id"]), (r["Kernel_Name"], {}))
            d[1][r["Counter_Name"]] = d[1].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return out


def summarize_counters(fetch_dir, write_dir, cal_fetch_dir, cal_write_dir, copy_mib, commands):
    """The HBM traffic of the skinny decode kernels from four rocprofv3 runs:
    FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of every skinny dispatch of
    the decode step, each scaled by what the same counter reads for a plain
    copy of known size (only the copy dispatches of the calibration run: those
    that read; the fill that creates the buffer reads nothing)."""
    copy_kib = copy_mib * 1024.0
    fetch = [v["FETCH_SIZE"] for k, v in _counter_rows(fetch_dir).values() if "skinny" in k]
    write = [v["WRITE_SIZE"] for k, v in _counter_rows(write_dir).values() if "skinny" in k]
    cal_f = [v["FETCH_SIZE"] for _, v in _counter_rows(cal_fetch_dir).values() if v["FETCH_SIZE"] > 0.25 * copy_kib]
    cal_w = [v["WRITE_SIZE"] for _, v in _counter_rows(cal_write_dir).values() if v["WRITE_SIZE"] > 0.25 * copy_kib]
    ff = copy_kib / (sum(cal_f) / len(cal_f))
    wf = copy_kib / (sum(cal_w) / len(cal_w))
    f_mean, w_mean = sum(fetch) / len(fetch), sum(write) / len(write)
    wl = wi.WORKLOADS["decode_sym"]
    algo = sum(algorithmic_bytes(M, N, K, wl["G"], wl["qtype"], False) for (M, N, K) in wl["shapes"]) / len(wl["shapes"])
    return {
        "kernel": "skinny decode kernels (all variants the 12-GEMM decode step launches)",
        "kernel_source_hash": kernel_source_hash(),
        "commands": commands,
        "calibration": {"copy_bytes": int(copy_kib * 1024), "copy_dispatches": len(cal_f),
                        "FETCH_SIZE_KB": sum(cal_f) / len(cal_f), "WRITE_SIZE_KB": sum(cal_w) / len(cal_w),
                        "fetch_factor": ff, "write_factor": wf},
        "dispatches": len(fetch),
        "FETCH_SIZE_KB_mean": f_mean,
        "WRITE_SIZE_KB_mean": w_mean,
        "hbm_bytes_per_launch": int(round((f_mean * ff + w_mean * wf) * 1024)),
        "algorithmic_bytes_per_launch": algo,
        "note": "mean over every skinny dispatch of the commands above (the step's 12 shapes in equal numbers); "
                "each counter scaled by its factor from the copy dispatches of the calibration run",
    }


def prefill_rates(quick=False):
    """Prefill workload on the MFMA kernel: TFLOP/s per shape and in total.
    quick: no warm-up and 3 replays (for counter runs under a profiler)."""
    wl = wi.WORKLOADS["prefill"]
    rows, tot_flop, tot_us = [], 0.0, 0.0
    for (G, qt) in wl["variants"]:
        for (M, N, K) in wl["shapes"]:
            g = Gemm(wl["cfg_id"], M, N, K, G, qt, wl["dtype"], wl["sigma"], 2)
            us = per_case_rate(g, launches=2, reps=3 if quick else 10, warm_ms=0.0 if quick else PREFILL_WARM_MS)
            tf = g.flops / us / 1e6
            rows.append({"M": M, "N": N, "K": K, "G": G, "qtype": qt, "us": round(us, 1), "tflops": round(tf, 1),
                         "frac_of_peak": round(tf / MFMA_PEAK_TFLOPS, 4)})
            tot_flop += g.flops
            tot_us += us
            del g
            torch.cuda.empty_cache()
    return {
        "workload": "M in {2048,8192} x (N,K) in {(14336,4096),(4096,14336)} x G in {-1,256} x {uint4b8, uint4+zp}, bf16",
        "tflops": round(tot_flop / tot_us / 1e6, 1),
        "frac_of_peak": round(tot_flop / tot_us / 1e6 / MFMA_PEAK_TFLOPS, 4),
        "peak_tflops": MFMA_PEAK_TFLOPS,
        "rows": rows,
    }


def row_stride_rates(pads=(0, 64, 256, 0)):
    """Prefill GEMMs (G = -1, uint4b8, bf16) with the activation and output
    row strides at their widths (8 KB to 28 KB rows, multiples of large powers
    of two) and padded by `pad` elements (64 = one 128-byte line): does a
    power-of-two row stride cost HBM channel balance on gfx950? Each stride
    is timed after the same warm-up, and the unpadded one again last, so an
    order effect would show as two different pad0 values."""
    rows = []
    for (M, N, K) in [(8192, 14336, 4096), (8192, 4096, 14336), (2048, 14336, 4096)]:
        g = Gemm(5, M, N, K, -1, wi.UINT4B8, "bf16", 1.0, 2)
        A0 = g.A
        row = {"M": M, "N": N, "K": K}
        for pad in pads:
            g.A = torch.empty((M, K + pad), dtype=A0.dtype, device=DEV)[:, :K]
            g.A.copy_(A0)
            g.C = torch.empty((M, N + pad), dtype=A0.dtype, device=DEV)[:, :N]
            us = per_case_rate(g, launches=2, reps=10, warm_ms=PREFILL_WARM_MS)
            key = f"pad{pad}_us" if f"pad{pad}_us" not in row else f"pad{pad}_again_us"
            row[key] = round(us, 1)
        rows.append(row)
        del g, A0
        torch.cuda.empty_cache()
    return {"workload": "lda = K + pad, ldc = N + pad (elements), G=-1 uint4b8 bf16, MFMA path", "rows": rows}


INT8_PEAK_TOPS = 5000.0  # dense int8 MFMA, MI355X


def w4a8_rates():
    """The W4A8 variant (w4a8_quantize + w4a8_gemm) on the decode shapes
    (fp16, G = 128, weight-stream GB/s of the GEMM) and the prefill shapes
    (bf16, G in {-1, 256}, symmetric weights; TOP/s against the int8 MFMA
    peak), after the same warm-up and weight rotation as the other paths."""
    out = {"int8_peak_tops": INT8_PEAK_TOPS}

    def timed(g, fn_of_copy, n, warm_ms, reps):
        graphs = capture_graphs([[(lambda c=c: fn_of_copy(c)) for c in range(n)]])
        warm_up(graphs, warm_ms)
        return time_graphs(graphs, reps, 3) * 1e3 / (reps * n)

    wl = wi.WORKLOADS["decode_sym"]
    dec = []
    for (M, N, K) in wl["shapes"]:
        g = Gemm(wl["cfg_id"], M, N, K, wl["G"], wl["qtype"], wl["dtype"], wl["sigma"],
                 copies_for(weight_stream_bytes(N, K, wl["G"], wl["qtype"], False)))
        qa, xs = w4.quantize_a8(g.A)
        C = torch.empty((M, N), dtype=g.A.dtype, device=DEV)
        ws = w4.Workspace(DEV)
        ws.get(w4.w4a8_workspace_size(M, N, K, wl["G"]))
        n = len(g.packed)
        gemm = lambda c: w4.gemm_w4a8(qa, xs, g.packed[c], N, K, wl["G"], g.A.dtype, out=C, workspace=ws)  # noqa: E731
        both = lambda c: (w4.quantize_a8(g.A, out=(qa, xs)), gemm(c))  # noqa: E731
        us = timed(g, gemm, n, 20.0, 5)
        us_both = timed(g, both, n, 20.0, 5)
        dec.append({"M": M, "N": N, "K": K, "gemm_us": round(us, 2), "with_quantize_us": round(us_both, 2),
                    "weight_GBps": round(g.weight_bytes / us / 1e3, 1)})
        del g
        torch.cuda.empty_cache()
    out["decode"] = {"workload": "decode shapes, G=128 symmetric weights, fp16 act", "rows": dec}

    wl = wi.WORKLOADS["prefill"]
    pre, tot_op, tot_us = [], 0.0, 0.0
    for G in (-1, 256):
        for (M, N, K) in wl["shapes"]:
            g = Gemm(wl["cfg_id"], M, N, K, G, wi.UINT4B8, wl["dtype"], wl["sigma"], 2)
            qa, xs = w4.quantize_a8(g.A)
            C = torch.empty((M, N), dtype=g.A.dtype, device=DEV)
            gemm = lambda c: w4.gemm_w4a8(qa, xs, g.packed[c], N, K, G, g.A.dtype, out=C)  # noqa: E731
            quant = lambda c: w4.quantize_a8(g.A, out=(qa, xs))  # noqa: E731
            us = timed(g, gemm, 2, PREFILL_WARM_MS, 10)
            us_q = timed(g, quant, 2, 20.0, 10)
            tops = g.flops / us / 1e6
            pre.append({"M": M, "N": N, "K": K, "G": G, "gemm_us": round(us, 1), "quantize_us": round(us_q, 1),
                        "tops": round(tops, 1), "frac_of_int8_peak": round(tops / INT8_PEAK_TOPS, 4)})
            tot_op += g.flops
            tot_us += us
            del g
            torch.cuda.empty_cache()
    out["prefill"] = {"workload": "prefill shapes, G in {-1, 256}, symmetric weights, bf16 act",
                      "tops": round(tot_op / tot_us / 1e6, 1),
                      "frac_of_int8_peak": round(tot_op / tot_us / 1e6 / INT8_PEAK_TOPS, 4), "rows": pre}
    return out


def prefill_dense_rates():
    """The dense prefill variant on the prefill workload: the dequantisation of
    each weight into a dense copy (w4a16_dequant) and hipBLASLt on that copy
    (w4a16_gemm_dense), timed separately; TFLOP/s of the GEMM alone (the
    cached-copy case of the pages) and of both together."""
    wl = wi.WORKLOADS["prefill"]
    rows, tot_flop, tot_gemm, tot_both = [], 0.0, 0.0, 0.0
    for (G, qt) in wl["variants"]:
        for (M, N, K) in wl["shapes"]:
            g = Gemm(wl["cfg_id"], M, N, K, G, qt, wl["dtype"], wl["sigma"], 2)
            dt = g.A.dtype
            dense = [torch.empty((N, K), dtype=dt, device=DEV) for _ in range(2)]
            deq = capture_graphs([[(lambda c=c: w4.dequant(g.packed[c], N, K, G, qt, dt, out=dense[c]))
                                   for c in range(2)]])
            warm_up(deq, 20.0)
            us_deq = time_graphs(deq, 5, 2) * 1e3 / 10
            mm = capture_graphs([[(lambda c=c: w4.gemm_dense(g.A, dense[c], out=g.C)) for c in range(2)]])
            warm_up(mm, PREFILL_WARM_MS)
            us_mm = time_graphs(mm, 10, 2) * 1e3 / 20
            rows.append({"M": M, "N": N, "K": K, "G": G, "qtype": qt, "dequant_us": round(us_deq, 1),
                         "gemm_us": round(us_mm, 1), "gemm_tflops": round(g.flops / us_mm / 1e6, 1),
                         "total_tflops": round(g.flops / (us_mm + us_deq) / 1e6, 1)})
            tot_flop += g.flops
            tot_gemm += us_mm
            tot_both += us_mm + us_deq
            del g, dense, deq, mm
            torch.cuda.empty_cache()
    return {
        "workload": "the prefill workload through w4a16_dequant + w4a16_gemm_dense (hipBLASLt), bf16",
        "gemm_tflops": round(tot_flop / tot_gemm / 1e6, 1),
        "total_tflops": round(tot_flop / tot_both / 1e6, 1),
        "rows": rows,
    }


def read_ceiling():
    """HBM read ceiling of one launch: a plain streaming-read kernel
    (libw4a16_ceiling.so) reads buffers of the decode weight sizes, replayed
    like the decode launches (graphs of >= 64 launches over >= 1 GB of
    rotating buffers), over a few launch shapes; the fastest per size."""
    import ctypes

    from mixed_precision_w4a16_repack_amd import build as lib_build

    lib = ctypes.CDLL(lib_build.CEILING_LIB)
    fn = lib.w4a16_ceiling_read
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                   ctypes.c_void_p]
    sink = torch.zeros(4096, dtype=torch.int32, device=DEV)
    shapes = [(256, 512, 8), (512, 512, 4), (1024, 256, 8), (2048, 256, 4)]
    rows = []
    sizes = {"empty": 16, "decode 4096x4096 G=128": weight_stream_bytes(4096, 4096, 128, wi.UINT4B8, False),
             "decode 14336x4096 G=128": weight_stream_bytes(14336, 4096, 128, wi.UINT4B8, False),
             "decode-asym 6144x4096 G=32": weight_stream_bytes(6144, 4096, 32, wi.UINT4, True)}
    for name, nbytes in sizes.items():
        copies = copies_for(nbytes) if nbytes > 16 else 2
        bufs = [torch.randint(-2**31, 2**31 - 1, (max(4, nbytes // 4),), dtype=torch.int32, device=DEV)
                for _ in range(copies)]
        n = max(64, copies)
        best = None
        for (grid, threads, unroll) in (shapes if nbytes > 16 else shapes[:1]):
            def launch(c, grid=grid, threads=threads, unroll=unroll):
                rc = fn(ctypes.c_void_p(bufs[c % copies].data_ptr()), nbytes, ctypes.c_void_p(sink.data_ptr()),
                        grid, threads, unroll, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
                if rc != 0:
                    raise RuntimeError(f"ceiling kernel launch failed: {rc}")
            graphs = capture_graphs([[(lambda c=c: launch(c)) for c in range(n)]])
            warm_up(graphs, 5.0)
            us = time_graphs(graphs, 10, 2) * 1e3 / (10 * n)
            if best is None or us < best["us"]:
                best = {"grid": grid, "threads": threads, "loads_per_thread": unroll, "us": round(us, 3)}
            del graphs
        rows.append({"size": name, "bytes": nbytes, **best,
                     "GBps": round(nbytes / best["us"] / 1e3, 1) if nbytes > 16 else None})
        del bufs
        torch.cuda.empty_cache()
    return {"kernel": "plain streaming read (16-byte nontemporal loads, XOR-folded)", "rows": rows}


def crossover_rates(paths=(("skinny_us", w4.PATH_SKINNY), ("mfma_us", w4.PATH_MFMA)), ms=None):
    """Crossover workload: skinny (16-row slices) vs MFMA at M = 32..256
    (or the rows ``ms`` of the same weight)."""
    wl = wi.WORKLOADS["crossover"]
    cross = []
    shapes = wl["shapes"] if ms is None else [(m, wl["shapes"][0][1], wl["shapes"][0][2]) for m in ms]
    for (M, N, K) in shapes:
        row = {"M": M}
        for name, path in paths:
            g = Gemm(wl["cfg_id"], M, N, K, wl["G"], wl["qtype"], wl["dtype"], wl["sigma"],
                     copies_for(weight_stream_bytes(N, K, wl["G"], wl["qtype"], False)), path=path)
            row[name] = round(per_case_rate(g, reps=10), 2)
            del g
        if "mfma_us" in row:
            row["mfma_tflops"] = round(2.0 * M * N * K / row["mfma_us"] / 1e6, 1)
        cross.append(row)
    out = {"workload": "N=14336, K=4096, G=64, uint4b8, fp16", "rows": cross}
    if all("skinny_us" in r and "mfma_us" in r for r in cross):
        out["crossover_M"] = next((r["M"] for r in cross if r["mfma_us"] < r["skinny_us"]), None)
    return out


def decode_asym_rates():
    """Decode asymmetric bf16 workload: N=6144, K=4096, G=32, uint4 + zero points."""
    wl = wi.WORKLOADS["decode_asym"]
    asym = []
    for (M, N, K) in wl["shapes"]:
        g = Gemm(wl["cfg_id"], M, N, K, wl["G"], wl["qtype"], wl["dtype"], wl["sigma"],
                 copies_for(weight_stream_bytes(N, K, wl["G"], wl["qtype"], True)))
        us = per_case_rate(g)
        asym.append({"M": M, "N": N, "K": K, "us": round(us, 2), "weight_GBps": round(g.weight_bytes / us / 1e3, 1)})
        del g
    return {"workload": "N=6144, K=4096, G=32, uint4 + zero points, bf16", "rows": asym}


def extras(warmup):
    out = {}
    out["read_ceiling"] = read_ceiling()
    out["crossover"] = crossover_rates()
    out["prefill"] = prefill_rates()
    out["prefill_dense"] = prefill_dense_rates()
    out["decode_asym"] = decode_asym_rates()
    wl = wi.WORKLOADS["tiny"]
    (M, N, K) = wl["shapes"][0]
    g = Gemm(wl["cfg_id"], M, N, K, wl["G"], wl["qtype"], wl["dtype"], wl["sigma"], 4)
    out["tiny_us"] = round(per_case_rate(g), 2)
    # One-time repack of the largest decode weight.
    g = Gemm(2, 1, 14336, 4096, 128, wi.UINT4B8, "f16", 1.0, 1)
    us = g.time_repack()
    out["repack"] = {"N": 14336, "K": 4096, "us": round(us, 1),
                     "GBps_read_plus_write": round(2 * g.weight_bytes / us / 1e3, 1)}
    out["repack_layout"] = time_repack_layouts(14336, 4096, 128)
    out["w4a8"] = w4a8_rates()
    return out


def time_repack_layouts(N, K, G, reps=5):
    """One-time repack from the AWQ (K, N/8) and AutoGPTQ (K/8, N) weight
    orientations, (K/G, N) scales and (K/G, N/8) zero points, uint4."""
    rows = []
    for name, od, pd in (("awq", 1, 1), ("autogptq", 1, 0)):
        L = wi.make_layout_weights(6, N, K, G, wi.UINT4, "bf16", od, pd, 1, 1)
        w = torch.from_numpy(L.weight).to(DEV)
        s_ = L.weight_scale.to(DEV)
        z = torch.from_numpy(L.weight_zero_point).to(DEV)
        out = w4.repack_layout(w, od, pd, s_, 1, z, 1, G, wi.UINT4)
        torch.cuda.synchronize()
        b, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        b.record()
        for _ in range(reps):
            w4.repack_layout(w, od, pd, s_, 1, z, 1, G, wi.UINT4, out=out)
        e.record()
        torch.cuda.synchronize()
        us = b.elapsed_time(e) / reps * 1e3
        moved = 2 * (w.numel() * 4 + s_.numel() * 2 + z.numel() * 4)
        rows.append({"orientation": name, "N": N, "K": K, "G": G, "us": round(us, 1),
                     "GBps_read_plus_write": round(moved / us / 1e3, 1)})
    return rows


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-breakdown", action="store_true", help="skip the per-shape decode timings")
    ap.add_argument("--w4a8-only", action="store_true",
                    help="only time the W4A8 variant (int8 activations) on the decode and prefill shapes")
    ap.add_argument("--strides-only", action="store_true",
                    help="only time prefill GEMMs with padded and unpadded activation/output row strides")
    ap.add_argument("--only", choices=["crossover", "crossover-mfma", "crossover-fine", "decode-asym", "read-ceiling",
                                       "prefill", "prefill-quick"],
                    help="only time one extra workload and print its JSON (the commands the profiles use)")
    ap.add_argument("--prefill-only", action="store_true",
                    help="only time the prefill workload (MFMA kernel, and the dense variant) and print its JSON")
    ap.add_argument("--summarize-counters", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "CAL_FETCH_DIR", "CAL_WRITE_DIR"),
                    help="write profiles/skinny_decode_counters.json from four rocprofv3 --pmc csv directories "
                         "(FETCH_SIZE and WRITE_SIZE of the decode step, then of --calibration-copy 256)")
    ap.add_argument("--calibration-copy", type=int, default=0, metavar="MIB",
                    help="only copy a MIB-sized buffer 10 times (a known-size workload that calibrates the "
                         "rocprofv3 FETCH_SIZE / WRITE_SIZE counters), then exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the W4A16 path here is a single-GPU kernel; across GPUs the weight would be split along N or K)",
              file=sys.stderr)
        sys.exit(2)
    if args.summarize_counters:
        fd, wd, cfd, cwd = args.summarize_counters
        cmds = [f"rocprofv3 --pmc FETCH_SIZE --kernel-include-regex skinny -f csv -d {fd} -o run -- python3 bench.py "
                "--no-extras --no-cpu-baseline --no-breakdown --steps 4 --warmup 1",
                f"rocprofv3 --pmc WRITE_SIZE --kernel-include-regex skinny -f csv -d {wd} -o run -- python3 bench.py "
                "--no-extras --no-cpu-baseline --no-breakdown --steps 4 --warmup 1",
                f"rocprofv3 --pmc FETCH_SIZE -f csv -d {cfd} -o run -- python3 bench.py --calibration-copy 256",
                f"rocprofv3 --pmc WRITE_SIZE -f csv -d {cwd} -o run -- python3 bench.py --calibration-copy 256"]
        rec = summarize_counters(fd, wd, cfd, cwd, 256, cmds)
        with open(os.path.join(ROOT, "profiles", "skinny_decode_counters.json"), "w") as f:
            json.dump(rec, f, indent=1)
        print(json.dumps(rec), flush=True)
        return
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    if args.calibration_copy:
        n = args.calibration_copy << 20
        src = torch.ones(n, dtype=torch.uint8, device=DEV)
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration_copy_bytes": n, "copies": 10}), flush=True)
        return
    w4.load_library()
    if args.w4a8_only:
        print(json.dumps({"w4a8": w4a8_rates()}), flush=True)
        return
    if args.strides_only:
        print(json.dumps({"row_strides": row_stride_rates()}), flush=True)
        return
    if args.only:
        fn = {"crossover": crossover_rates, "crossover-mfma": lambda: crossover_rates((("mfma_us", w4.PATH_MFMA),)),
              "crossover-fine": lambda: crossover_rates(ms=(16, 17, 20, 24, 28, 32, 48)),
              "decode-asym": decode_asym_rates, "read-ceiling": read_ceiling, "prefill": prefill_rates,
              "prefill-quick": lambda: prefill_rates(quick=True)}[args.only]
        print(json.dumps({args.only: fn()}), flush=True)
        return
    if args.prefill_only:
        print(json.dumps({"prefill": prefill_rates(), "prefill_dense": prefill_dense_rates()}), flush=True)
        return

    cases, copies = decode_cases()
    step_weight_bytes = sum(c.weight_bytes for c in cases)
    step_algo_bytes = sum(c.algo_bytes for c in cases)
    # Steps are replayed from graphs of ROUND_STEPS steps each (the 12 GEMMs
    # on copy j for step j of the round), as a serving loop captures a whole
    # forward pass; one-step graphs make up a remainder, so exactly
    # args.steps steps are timed.
    round_steps = ROUND_STEPS - ROUND_STEPS % copies if ROUND_STEPS >= copies else copies
    step_graphs = capture_graphs([[(lambda c=c, j=j: c.launch(j)) for c in cases] for j in range(copies)])
    round_graph = capture_graphs([[(lambda c=c, j=j: c.launch(j % copies)) for j in range(round_steps)
                                   for c in cases]])[0]
    torch.cuda.synchronize()
    ms = time_steps(round_graph, round_steps, step_graphs, args.steps, args.warmup)
    graphs = step_graphs + [round_graph]
    ms_per_step = ms / args.steps
    value = step_weight_bytes / (ms_per_step * 1e-3) / 1e9
    launches = len(cases)
    avg_launch_us = ms_per_step * 1e3 / launches
    achieved = (step_algo_bytes / launches) / (avg_launch_us * 1e-6) / 1e9

    breakdown = []
    for c in ([] if args.no_breakdown else cases):
        # Each shape alone, over its own rotation of at least ROTATE_BYTES of
        # weight copies (more than the last-level cache holds).
        n0 = len(c.packed)
        c.packed += [c.packed[0].clone() for _ in range(max(0, copies_for(c.weight_bytes) - n0))]
        us = per_case_rate(c, reps=5)
        breakdown.append({"M": c.M, "N": c.N, "K": c.K, "us": round(us, 2),
                          "weight_GBps": round(c.weight_bytes / us / 1e3, 1),
                          "frac_of_hbm_peak": round(c.weight_bytes / us / 1e3 / HBM_PEAK_GBS, 4),
                          "copies": len(c.packed), **per_case_spread(c)})
        del c.packed[n0:]
        torch.cuda.empty_cache()

    traffic = measured_traffic()
    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": "decode-shape symmetric W4A16 GEMM: M in {1,4,8,16} x (N,K) in "
                        "{(4096,4096),(14336,4096),(4096,14336)}, G=128, uint4b8, fp16 (12 GEMMs per step)",
            "weight_bytes_per_step": step_weight_bytes,
            "weight_copies": copies,
            "rotation_bytes": step_weight_bytes * copies,
            "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        },
        "roofline": {
            "kernel": "skinny decode GEMM (wide-weight register, LDS and split-K variants)",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "avg_launch_us": round(avg_launch_us, 3),
            "algorithmic_bytes_per_launch": step_algo_bytes / launches,
        },
        "decode_breakdown": breakdown,
    }
    del graphs
    if not args.no_extras:
        result["extras"] = extras(args.warmup)
        pre = result["extras"]["prefill"]
        # The other half of the metric: the tiled MFMA kernel on the prefill
        # workload, 2*M*N*K per GEMM over its measured duration, summed over
        # the 16 prefill GEMMs, against the dense fp16/bf16 MFMA peak.
        result["roofline_prefill"] = {
            "kernel": "tiled MFMA GEMM (128 x 512 and 128 x 256 tiles), prefill workload",
            "bound": "mfma",
            "achieved": pre["tflops"],
            "peak": MFMA_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": pre["frac_of_peak"],
            "traffic": None,
            "algorithmic_flops": sum(2.0 * r["M"] * r["N"] * r["K"] for r in pre["rows"]),
        }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
