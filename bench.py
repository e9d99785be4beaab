#!/usr/bin/env python3
"""Benchmark: exact attention forward + backward on one MI355X.

One step = one forward (fa_forward) and one backward (fa_backward: the dQ
kernel, which also forms D and LSE*log2e, then the dK/dV kernel) over one batch
of the N=4096, d=128, causal bf16 workload (B=2, H=16, K with 5% outlier rows
x8), inputs resident in device memory.  Prints one JSON line: whole-step TFLOPS
(algorithmic FLOPs: forward 4*N^2*d, backward 10*N^2*d per head, halved for
causal), its fraction of the dense bf16 MFMA peak, per-kernel times measured
with HIP events on the launch stream, the roofline of the dominant kernel, and
the float64 CPU oracle timed on a bounded sample.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 4] [--prewarm S]
                  [--no-cpu-baseline] [--copy-calibration] [--sweep] [--decode]
                  [--fp8-quant] [--fp8]

--decode times the split-K decode workload (32 heads, one query, a 128K-token
cache) instead, against the HBM roofline.  --fp8-quant times the FP8 input
stage (Hadamard rotation and per-row E4M3 codes) on the N=4096 workload's Q
and K, also against the HBM roofline.  --fp8 times the FP8 forward path (that
stage on Q and K, then the attention kernel with Q K^T on E4M3) on the same
workload, against the mixed E4M3/bf16 MFMA peak.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2500.0, "fp16": 2500.0, "fp32": 157.3}  # MI355X dense MFMA
PEAK_HBM_GBPS = 8000.0
METRIC = "attention fwd+bwd TFLOPS at N=4K d=128 bf16, 1 GPU; % of MFMA peak"
# One training step's kernels in launch order: the dQ kernel also forms D and
# LSE*log2(e) (the backward preprocess) for the dK/dV kernel that follows it.
KERNELS = ("fwd", "bwd_dq", "bwd_dkdv")
BWD_ORDER = ("bwd_dq", "bwd_dkdv")
# Untimed steps before the warm-up steps, in seconds of wall time (see main()).
PREWARM_S = 0.3
CSRC = os.path.join(ROOT, "exact_io_aware_forward_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


# The FLOP and byte arithmetic of the measurement, written once.  Per head of a
# sequence of S tokens with head dimension d and b-byte elements (Lecture 9
# notes, cs2680.com, sections 9.2 and 9.6):
def matmul_flop(m: int, n: int, k: int) -> int:
    """A dense (m x k) @ (k x n) product: 2 m n k FLOPs."""
    return 2 * m * n * k


def score_matrix_bytes(s: int, b: int) -> int:
    """One S x S score (or probability) matrix in b-byte elements."""
    return s * s * b


def attention_flop(s: int, d: int) -> int:
    """The forward's irreducible work: Q K^T and A V, 4 S^2 d."""
    return matmul_flop(s, s, d) + matmul_flop(s, d, s)


def unfused_intensity(s: int, d: int, b: int) -> float:
    """FLOP per byte of attention run as separate kernels: S and A are each
    written once and read once (4 S^2 b bytes), so 4 S^2 d / 4 S^2 b = d / b."""
    return attention_flop(s, d) / (4 * score_matrix_bytes(s, b))


def fused_intensity(s: int, d: int, b: int) -> float:
    """FLOP per byte of the fused kernel: Q, K, V read and O written once
    (4 S d b bytes), so S / b."""
    return attention_flop(s, d) / (4 * s * d * b)


def crossover_seq_len(ridge_flop_per_byte: float, b: int) -> float:
    """Sequence length at which the fused kernel reaches a device's ridge point
    (S / b = ridge)."""
    return ridge_flop_per_byte * b


def lecture9_arithmetic() -> dict:
    """The values the Lecture 9 notes print (section 9.2, section 9.6, exercise 1
    and the key-takeaways table), recomputed with the functions above; keys as in
    tests/golden/lecture9_arithmetic.json."""
    s4k, s32k, d, b = 4096, 32768, 128, 2
    recompute = matmul_flop(s4k, s4k, d)                   # one extra Q K^T
    store = 2 * score_matrix_bytes(s4k, b)                 # written once, read once
    return {
        "recompute_flops_S4096_d128_gflop": recompute / 1e9,
        "score_matrix_bytes_S4096_bf16_mb": score_matrix_bytes(s4k, b) / 1e6,
        "store_traffic_S4096_mb": store / 1e6,
        "store_time_us_at_3350GBps": store / 3350e9 * 1e6,
        "recompute_time_us_at_494p5TFs": recompute / 494.5e12 * 1e6,
        "unfused_intensity_flop_per_byte": unfused_intensity(s4k, d, b),
        "fused_intensity_S4096": fused_intensity(s4k, d, b),
        "fused_intensity_S32768": fused_intensity(s32k, d, b),
        "crossover_h100_bf16": crossover_seq_len(295, 2),
        "crossover_a100_bf16": crossover_seq_len(153, 2),
        "crossover_h100_fp32": crossover_seq_len(295, 4),
        "score_matrix_S32768_gb": score_matrix_bytes(s32k, b) / 1e9,
        "one_layer_32_heads_S32768_gb": 32 * score_matrix_bytes(s32k, b) / 1e9,
        "flash_footprint_S32768_mb": 4 * s32k * d * b / 1e6,
    }


def work_model(w) -> dict:
    """Algorithmic work per launch of each kernel (per-head figure x B*H heads)."""
    bh, n, d = w.B * w.H, w.N, w.d
    b = 2 if w.dtype in ("bf16", "fp16") else 4
    cf = 0.5 if w.causal else 1.0
    nn = n * n * d * bh * cf
    assert attention_flop(n, d) == 4 * n * n * d
    return {
        "fwd": {"flop": 4 * nn, "bytes": bh * (4 * n * d * b + 4 * n)},
        # the standalone preprocess (backward stage 0): reads O, dO and LSE;
        # writes D and LSE*log2(e)
        "bwd_pre": {"flop": 2 * n * d * bh, "bytes": bh * (2 * n * d * b + 12 * n)},
        "bwd_dkdv": {"flop": 8 * nn, "bytes": bh * (6 * n * d * b + 8 * n)},
        # dQ recomputes S and dP (4*N^2*d) on top of its own 2*N^2*d product; it
        # also reads O and LSE and writes D and LSE*log2(e) (the preprocess).
        "bwd_dq": {"flop": 2 * nn, "flop_executed": 6 * nn, "bytes": bh * (6 * n * d * b + 12 * n)},
        "step_flop": 14 * nn,
        "fwd_flop": 4 * nn,
        "bwd_flop": 10 * nn,
    }


def cpu_baseline(w, x, budget_s: float = 12.0) -> dict:
    """Float64 oracle (as it stands) on whole heads of the same workload, until the
    time budget is spent; reported in the same unit as the GPU value."""
    import numpy as np
    import oracle
    blas = blas_info()
    threads = blas.get("threads") or os.cpu_count()
    t0 = time.perf_counter()
    heads = 0
    for bh in range(w.B * w.H):
        b, h = divmod(bh, w.H)
        q, k, v, do = (x[n][b, h].double().numpy() for n in ("q", "k", "v", "do"))
        oracle.forward_head(q, k, v, w.causal, w.scale)
        oracle.backward_head(q, k, v, do, w.causal, w.scale)
        heads += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    cf = 0.5 if w.causal else 1.0
    flop = 14 * w.N * w.N * w.d * cf * heads
    return {"value": round(flop / dt / 1e12, 6), "unit": "TFLOPS", "cores": threads,
            "kind": "oracle",
            "sample": f"{heads} of {w.B * w.H} heads (b,h in row-major order), forward + "
                      f"backward in float64 numpy, {dt:.2f} s wall; same algorithmic FLOP "
                      f"convention as the GPU value",
            "cpu": cpu_model(), "blas": blas}


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), else the machine type."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def blas_info() -> dict:
    """The BLAS numpy runs on and the thread count it uses, as threadpoolctl
    reports them once numpy is loaded ({} if it cannot tell)."""
    import numpy  # noqa: F401  (threadpoolctl only sees loaded libraries)
    try:
        from threadpoolctl import threadpool_info
        pools = [p for p in threadpool_info() if p.get("user_api") == "blas"]
    except Exception:  # threadpoolctl is optional
        return {}
    if not pools:
        return {}
    p = pools[0]
    return {"library": f"{p.get('internal_api')} {p.get('version')}",
            "threads": int(p.get("num_threads", 0)),
            "threads_from": "threadpoolctl (the BLAS pool numpy uses; OMP_NUM_THREADS / "
                            "OPENBLAS_NUM_THREADS set it when present)"}


def load_traffic(dominant: str) -> float | None:
    """HBM bytes per launch from the recorded FETCH_SIZE/WRITE_SIZE counter runs,
    only if they were taken on the current kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha") != kernel_source_sha():
        return None
    k = rec.get("kernels", {}).get(dominant)
    if not k:
        return None
    return float(k["hbm_bytes_per_launch"])


def settle_clock(step, seconds: float) -> int:
    """Untimed calls of step() for `seconds` of wall time, synchronising every
    10: after idle the GPU's clock settles only after ~40 ms of sustained work,
    so timed regions that follow see the settled clock.  Returns the calls made."""
    import torch
    n, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(10):
            step()
        torch.cuda.synchronize()
        n += 10
    return n


def visited_tiles(n: int, br: int, bc: int, causal: bool) -> int:
    """Tiles (br query rows x bc keys) a kernel runs: all of them, or under the
    causal mask those with at least one key at or before their last row."""
    nq, nk = -(-n // br), -(-n // bc)
    if not causal:
        return nq * nk
    return sum(min(nk, (min((i + 1) * br, n) - 1) // bc + 1) for i in range(nq))


def device_peak_tflops(dtype: str) -> dict:
    """Peak recomputed from the device's CU count and its reported maximum shader
    clock: CUs x clock x MFMA FLOP per CU per cycle (4 SIMDs; 1024 dense
    16-bit FLOP per SIMD per cycle, 64 for fp32)."""
    import ctypes
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    khz = ctypes.c_int(0)
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        hip.hipDeviceGetAttribute(ctypes.byref(khz), 5, 0)   # hipDeviceAttributeClockRate, kHz
    except OSError:
        pass
    per_cu = 4 * (64 if dtype == "fp32" else 1024)
    ghz = khz.value / 1e6
    return {"cus": cus, "max_clock_ghz": round(ghz, 3),
            "peak_tflops": round(cus * ghz * 1e9 * per_cu / 1e12, 1) if ghz else None}


def sweep(reps: int, warmup: int, prewarm: float = PREWARM_S) -> int:
    """Every workload: forward and backward stage times (HIP events, median and
    min over `reps`), algorithmic and executed TFLOPS, and for
    the smallest workload a launch floor.  One JSON line per workload."""
    import statistics
    import torch
    import exact_io_aware_forward_amd as fa
    import workloads

    dev = torch.device("cuda", 0)
    for cid, w in sorted(workloads.WORKLOADS.items()):
        print(f"sweep: workload {w.name}", file=sys.stderr, flush=True)
        x = workloads.workload_inputs(cid)
        q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
        do = x["do"].to(dev) if w.backward else None
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
        if w.backward:
            dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
            ws = fa.new_workspace(q)
        names = ["fwd"] + (list(BWD_ORDER) if w.backward else [])
        times = {n: [] for n in names}

        def plain():
            fa.forward(q, k, v, w.causal, w.scale, out=o, lse=lse)
            if w.backward:
                fa.backward(q, k, v, o, do, lse, w.causal, w.scale, workspace=ws, out=(dq, dk, dv))

        settle_clock(plain, prewarm)
        for r in range(warmup + reps):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
            ev[0].record()
            fa.forward(q, k, v, w.causal, w.scale, out=o, lse=lse)
            ev[1].record()
            if w.backward:
                for j, s in enumerate((fa.BWD_DQ, fa.BWD_DKDV)):
                    fa.backward_stage(s, q, k, v, o, do, lse, dq, dk, dv, ws, w.causal, w.scale)
                    ev[2 + j].record()
            torch.cuda.synchronize()
            if r >= warmup:
                for j, n in enumerate(names):
                    times[n].append(ev[j].elapsed_time(ev[j + 1]))
        wm = work_model(w)
        peak = PEAK_TFLOPS[w.dtype]
        bh = w.B * w.H
        br, bc = fa.tile_config(0 if w.causal else 3, w.d, w.torch_dtype)
        fwd_exec = visited_tiles(w.N, br, bc, w.causal) * 4 * br * bc * w.d * bh
        med = {n: statistics.median(t) for n, t in times.items()}
        res = {"workload": w.name, "dtype": w.dtype, "reps": reps,
               "fwd_ms_median": round(med["fwd"], 5), "fwd_ms_min": round(min(times["fwd"]), 5),
               "fwd_tflops": round(wm["fwd_flop"] / med["fwd"] / 1e9, 2),
               "fwd_pct_peak": round(100 * wm["fwd_flop"] / med["fwd"] / 1e9 / peak, 2),
               "fwd_executed_tflops": round(fwd_exec / med["fwd"] / 1e9, 2),
               "fwd_gbps_algorithmic": round(wm["fwd"]["bytes"] / med["fwd"] / 1e6, 1)}
        if w.backward:
            b1r, b1c = fa.tile_config(1, w.d, w.torch_dtype)
            b2r, b2c = fa.tile_config(2, w.d, w.torch_dtype)
            bwd_exec = (visited_tiles(w.N, b1r, b1c, w.causal) * 8 * b1r * b1c
                        + visited_tiles(w.N, b2r, b2c, w.causal) * 6 * b2r * b2c) * w.d * bh
            bwd = [sum(t[i] for n, t in times.items() if n != "fwd") for i in range(reps)]
            tot = [times["fwd"][i] + bwd[i] for i in range(reps)]
            mb, mt = statistics.median(bwd), statistics.median(tot)
            res.update({
                "bwd_ms_median": round(mb, 5), "bwd_ms_min": round(min(bwd), 5),
                "bwd_tflops": round(wm["bwd_flop"] / mb / 1e9, 2),
                "bwd_executed_tflops": round(bwd_exec / mb / 1e9, 2),
                "bwd_stage_ms_median": {n: round(med[n], 5) for n in names[1:]},
                "fwdbwd_ms_median": round(mt, 5), "fwdbwd_ms_min": round(min(tot), 5),
                "fwdbwd_tflops": round(wm["step_flop"] / mt / 1e9, 2),
                "fwdbwd_pct_peak": round(100 * wm["step_flop"] / mt / 1e9 / peak, 2)})
        if not w.backward:
            # Cold runs: a 1 GiB write between repetitions evicts the inputs from
            # the last-level (MALL) cache, so the forward reads them from HBM.
            flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
            cold = []
            for r in range(reps):
                flush.fill_(float(r))
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                fa.forward(q, k, v, w.causal, w.scale, out=o, lse=lse)
                e1.record()
                torch.cuda.synchronize()
                cold.append(e0.elapsed_time(e1))
            del flush
            res["fwd_ms_cold_median"] = round(statistics.median(cold), 5)
            res["fwd_gbps_algorithmic_cold"] = round(
                wm["fwd"]["bytes"] / statistics.median(cold) / 1e6, 1)
        if cid == min(workloads.WORKLOADS):
            # Launch floor: a one-element fill kernel timed the same way.
            t1 = torch.zeros(1, device=dev)
            fl = []
            for r in range(warmup + reps):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                t1.fill_(1.0)
                e1.record()
                torch.cuda.synchronize()
                if r >= warmup:
                    fl.append(e0.elapsed_time(e1))
            res["launch_floor_ms_median"] = round(statistics.median(fl), 5)
        res["peak_tflops_nominal"] = peak
        res["device_peak"] = device_peak_tflops(w.dtype)
        print(json.dumps(res), flush=True)
        del x, q, k, v, do, o, lse
        if w.backward:
            del dq, dk, dv, ws
        torch.cuda.empty_cache()
    return 0


DECODE_METRIC = ("split-K decode: KV-cache GB/s at B=1 H=32 Nq=1 Nk=128K d=128 bf16, 1 GPU; "
                 "% of HBM peak")


def decode_work_model(w) -> dict:
    """Algorithmic work of one decode call (Lecture 9 notes §9.8): FLOPs 4*d per
    visible (query, key) pair, bytes = the cache (K and V, 2*Nk*d*b per key/value
    head) plus Q read and O, LSE written.  At Nq = 1 in 16-bit types this is 1 FLOP
    per byte of cache, the page's figure; g query heads sharing a key/value head
    raise it to g."""
    bh, b = w.B * w.H, 2
    if w.causal:
        pairs = sum(w.Nk - w.Nq + i + 1 for i in range(w.Nq))
    else:
        pairs = w.Nq * w.Nk
    cache = w.B * w.kv_heads * 2 * w.Nk * w.d * b   # grouped heads share one cache
    return {"flop": 4 * w.d * pairs * bh, "cache_bytes": cache,
            "split_bytes": cache + bh * w.Nq * w.d * b,
            "bytes": cache + bh * w.Nq * (2 * w.d * b + 4)}


def decode_cpu_baseline(w, x, budget_s: float) -> dict:
    """Float64 oracle decode (as it stands) on whole heads until the budget is spent,
    in the GPU line's unit (cache bytes per second)."""
    import oracle
    t0 = time.perf_counter()
    heads = 0
    for bh in range(w.B * w.H):
        b, h = divmod(bh, w.H)
        q, k, v = (x[n][b, h].double().numpy() for n in ("q", "k", "v"))
        oracle.decode_head(q, k, v, w.causal, w.scale)
        heads += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    cache = heads * 2 * w.Nk * w.d * 2
    blas = blas_info()
    return {"value": round(cache / dt / 1e9, 3), "unit": "GB/s",
            "cores": blas.get("threads") or os.cpu_count(), "kind": "oracle",
            "cpu": cpu_model(), "blas": blas,
            "sample": f"{heads} of {w.B * w.H} heads, float64 numpy decode, {dt:.2f} s wall; "
                      f"bytes counted as the 16-bit cache the GPU reads"}


def decode_dispatch(calls: int) -> list:
    """decode_dispatch_one at a 256-token and a 4096-token cache."""
    return [decode_dispatch_one(calls, nk) for nk in (256, 4096)]


def decode_dispatch_one(calls: int, nk: int) -> dict:
    """Dispatch cost of a short-context decode step (Lecture 9 notes §9.8: decode is
    launch-bound as well as bandwidth-bound, and graph capture is the remedy): the
    wall time per call of `calls` back-to-back eager calls (binding + two kernel
    launches each) against the same calls replayed from one captured HIP graph,
    and the GPU time per call from HIP events."""
    import torch
    import exact_io_aware_forward_amd as fa
    import workloads

    B, H, hkv, d = 1, 32, 32, 128
    x = workloads.draw_decode(B, H, 1, nk, d, "bf16", seed=108, hkv=hkv)
    q, k, v = (x[n].to("cuda") for n in ("q", "k", "v"))
    ws = fa.new_decode_workspace(q, k)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")

    def call():
        fa.decode(q, k, v, True, workspace=ws, out=o, lse=lse)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(3):
            call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(calls):
            call()
    for _ in range(3):
        call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(calls):
        call()
    torch.cuda.synchronize()
    eager = (time.perf_counter() - t0) / calls
    graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    graph.replay()
    torch.cuda.synchronize()
    replay = (time.perf_counter() - t0) / calls
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(calls):
        call()
    e1.record()
    torch.cuda.synchronize()
    return {"workload": f"decode_bf16_B{B}_H{H}_Nq1_Nk{nk}_d{d}", "calls": calls,
            "eager_wall_us_per_call": round(eager * 1e6, 2),
            "graph_wall_us_per_call": round(replay * 1e6, 2),
            "gpu_event_us_per_call": round(e0.elapsed_time(e1) * 1e3 / calls, 2),
            "cache_bytes_per_call": 2 * B * hkv * nk * d * 2}


def decode_bench(steps: int, warmup: int, cpu: bool, cpu_budget: float) -> int:
    """The split-K decode workload: split and combine kernels timed separately with
    HIP events on the launch stream, at the default slice count and at one slice
    per head (the occupancy contrast of Lecture 9 §9.8), plus the same shape with
    32 query heads on 4 key/value heads (packed groups of 8).  One JSON line; its
    value is the multi-head case at the default slice count."""
    import torch
    import exact_io_aware_forward_amd as fa
    import workloads

    dev = torch.device("cuda", 0)
    runs = {}
    for label, w, splits in (("default", workloads.DECODE_WORKLOAD, 0),
                             ("one_slice", workloads.DECODE_WORKLOAD, 1),
                             ("gqa8", workloads.DECODE_WORKLOAD_GQA, 0)):
        if label != "one_slice":
            x = workloads.draw_decode(w.B, w.H, w.Nq, w.Nk, w.d, w.dtype, w.seed, hkv=w.kv_heads)
            q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
            o = torch.empty_like(q)
            lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
            if label == "default":
                x_mha = x
        wm = decode_work_model(w)
        ws = fa.new_decode_workspace(q, k, splits)
        eff = splits or fa.decode_num_splits(w.B, w.H, w.kv_heads, w.Nq, w.Nk, w.d)

        def call(ev=None):
            if ev is not None:
                ev[0].record()
            fa.decode_stage(fa.DEC_SPLIT, q, k, v, None, None, w.causal, w.scale, splits, ws)
            if ev is not None:
                ev[1].record()
            fa.decode_stage(fa.DEC_COMBINE, q, k, v, o, lse, w.causal, w.scale, splits, ws)
            if ev is not None:
                ev[2].record()

        for _ in range(warmup):
            call()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        torch.cuda.synchronize()
        for i in range(steps):
            call(evs[i])
        torch.cuda.synchronize()
        t_split = sum(e[0].elapsed_time(e[1]) for e in evs) / steps
        t_comb = sum(e[1].elapsed_time(e[2]) for e in evs) / steps
        t_all = sum(e[0].elapsed_time(e[2]) for e in evs) / steps
        runs[label] = {"workload": w.name, "splits": eff, "workgroups": w.B * w.kv_heads * eff,
                       "split_ms": round(t_split, 5), "combine_ms": round(t_comb, 5),
                       "decode_ms": round(t_all, 5),
                       "split_gbps": round(wm["split_bytes"] / t_split / 1e6, 1),
                       "decode_gbps": round(wm["cache_bytes"] / t_all / 1e6, 1),
                       "tflops_algorithmic": round(wm["flop"] / t_all / 1e9, 3)}
        del ws
    dispatch = decode_dispatch(steps)
    w = workloads.DECODE_WORKLOAD
    wm = decode_work_model(w)
    d = runs["default"]
    achieved = wm["split_bytes"] / d["split_ms"] / 1e6
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS,
            "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4), "kernel": "dec_split",
            "traffic": load_traffic("dec_split")}
    value = wm["cache_bytes"] / d["decode_ms"] / 1e6
    result = {
        "metric": DECODE_METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": steps, "warmup": warmup, "ms_per_step": d["decode_ms"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "Nq": w.Nq, "Nk": w.Nk, "d": w.d,
                   "causal": w.causal, "scale": w.scale, "seed": w.seed,
                   "parallelism": "none (1 GPU)"},
        "pct_hbm_peak": round(100 * value / PEAK_HBM_GBPS, 2),
        "tflops_algorithmic": round(wm["flop"] / d["decode_ms"] / 1e9, 3),
        "runs": runs, "dispatch": dispatch, "roofline": roof,
        "kernel_source_sha": kernel_source_sha(),
        "device": torch.cuda.get_device_name(0)}
    if cpu:
        result["cpu_baseline"] = decode_cpu_baseline(w, x_mha, cpu_budget)
    print(json.dumps(result))
    return 0


FP8_METRIC = ("FP8 input stage (Hadamard rotation + per-row E4M3): GB/s over Q and K at "
              "B=2 H=16 N=4096 d=128 bf16, 1 GPU; % of HBM peak")


def fp8_quant_bytes(rows: int, d: int) -> int:
    """Algorithmic bytes of one fa_fp8_quantize_rows launch: the 16-bit rows read,
    one code byte per value and one fp32 scale per row written."""
    return rows * d * 2 + rows * d + rows * 4


def fp8_quant_bench(steps: int, warmup: int, cpu: bool, cpu_budget: float) -> int:
    """The FP8 input stage on the causal N=4096 d=128 bf16 workload's Q and K
    (CMU 11-868 FlashAttention notes, slide page 24): one launch per tensor,
    timed with HIP events on the launch stream."""
    import torch
    import exact_io_aware_forward_amd as fa
    import workloads

    w = workloads.WORKLOADS[4]
    x = workloads.workload_inputs(4)
    dev = torch.device("cuda", 0)
    q, k = x["q"].to(dev), x["k"].to(dev)
    signs = workloads.draw_signs(w.d, 4).to(dev)
    outs = [(torch.empty(t.shape, dtype=torch.uint8, device=dev),
             torch.empty(t.shape[:-1], dtype=torch.float32, device=dev)) for t in (q, k)]

    def call(ev=None):
        for j, t in enumerate((q, k)):
            if ev is not None:
                ev[j].record()
            fa.fp8_quantize_rows(t, signs, *outs[j])
        if ev is not None:
            ev[2].record()

    for _ in range(warmup):
        call()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        call(evs[i])
    torch.cuda.synchronize()
    t_launch = sum(e[0].elapsed_time(e[1]) + e[1].elapsed_time(e[2]) for e in evs) / (2 * steps)
    t_step = sum(e[0].elapsed_time(e[2]) for e in evs) / steps
    rows = w.B * w.H * w.N
    per_launch = fp8_quant_bytes(rows, w.d)
    achieved = per_launch / t_launch / 1e6
    value = 2 * per_launch / t_step / 1e6
    result = {
        "metric": FP8_METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": steps, "warmup": warmup, "ms_per_step": round(t_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": "fp8_quant_" + w.name, "rows_per_launch": rows, "d": w.d,
                   "launches_per_step": 2, "parallelism": "none (1 GPU)"},
        "pct_hbm_peak": round(100 * value / PEAK_HBM_GBPS, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4),
                     "kernel": "fp8_quant", "traffic": load_traffic("fp8_quant")},
        "kernel_source_sha": kernel_source_sha(),
        "device": torch.cuda.get_device_name(0)}
    if cpu:
        result["cpu_baseline"] = fp8_quant_cpu_baseline(x["q"], signs.cpu().double().numpy(),
                                                        cpu_budget)
    print(json.dumps(result))
    return 0


def fp8_quant_cpu_baseline(q, signs, budget_s: float) -> dict:
    """The float64 oracle's rotation and per-row E4M3 quantisation (as it stands) on
    blocks of 4096 rows until the budget is spent, in the GPU line's byte count."""
    from oracle import fp8
    rows2d = q.reshape(-1, q.shape[-1])
    d = rows2d.shape[1]
    t0 = time.perf_counter()
    done = 0
    while done < rows2d.shape[0]:
        blk = rows2d[done:done + 4096].double().numpy()
        fp8.quantize_rows(blk @ fp8.rotation(signs))
        done += blk.shape[0]
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    blas = blas_info()
    return {"value": round(fp8_quant_bytes(done, d) / dt / 1e9, 3), "unit": "GB/s",
            "cores": blas.get("threads") or os.cpu_count(), "kind": "oracle",
            "cpu": cpu_model(), "blas": blas,
            "sample": f"{done} of {rows2d.shape[0]} Q rows, float64 numpy, {dt:.2f} s wall; "
                      f"bytes counted as the GPU launch's (16-bit in, codes and scales out)"}


FP8_FWD_METRIC = ("FP8 attention forward TFLOPS (Q K^T on E4M3 after the Hadamard rotation, "
                  "P V on bf16) at N=4K d=128 causal, 1 GPU; % of the mixed FP8/bf16 MFMA peak")
PEAK_FP8_TFLOPS = 5000.0   # MI355X dense E4M3 MFMA


def fp8_mixed_peak(flop_qk: float, flop_pv: float) -> float:
    """Peak TFLOP/s of a kernel doing flop_qk on the E4M3 matrix pipe and flop_pv
    on the bf16 one, each at its own published dense peak."""
    return (flop_qk + flop_pv) / (flop_qk / PEAK_FP8_TFLOPS + flop_pv / PEAK_TFLOPS["bf16"])


def fp8_fwd_bench(steps: int, warmup: int, cpu: bool, cpu_budget: float,
                  prewarm: float = PREWARM_S) -> int:
    """The FP8 forward path on the causal N=4096 d=128 bf16 workload (K with 5 %
    outlier rows x8): one step = the rotation and E4M3 quantisation of Q and of K
    (fa_fp8_quantize_rows) and the FP8 attention kernel (fa_forward_fp8), each
    timed with HIP events on the launch stream.  value = the forward's
    algorithmic FLOPs (4 N^2 d per head, half under the causal mask) over the
    step time."""
    import torch
    import exact_io_aware_forward_amd as fa
    import workloads

    w = workloads.WORKLOADS[4]
    x = workloads.workload_inputs(4)
    dev = torch.device("cuda", 0)
    q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
    signs = workloads.draw_signs(w.d, 4).to(dev)
    qc, qs = fa.fp8_quantize_rows(q, signs)
    kc, ks = fa.fp8_quantize_rows(k, signs)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        fa.fp8_quantize_rows(q, signs, qc, qs)
        fa.fp8_quantize_rows(k, signs, kc, ks)
        if ev is not None:
            ev[1].record()
        fa.forward_fp8(qc, qs, kc, ks, v, w.causal, w.scale, out=o, lse=lse)
        if ev is not None:
            ev[2].record()
        fa.forward(q, k, v, w.causal, w.scale, out=o, lse=lse)   # the bf16 forward, for context
        if ev is not None:
            ev[3].record()

    settle_clock(step, prewarm)
    for _ in range(warmup):
        step()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    t_quant = sum(e[0].elapsed_time(e[1]) for e in evs) / steps
    t_attn = sum(e[1].elapsed_time(e[2]) for e in evs) / steps
    t_bf16 = sum(e[2].elapsed_time(e[3]) for e in evs) / steps
    wm = work_model(w)
    flop = wm["fwd_flop"]
    t_step = t_quant + t_attn
    peak = fp8_mixed_peak(flop / 2, flop / 2)
    achieved = flop / (t_attn * 1e-3) / 1e12
    result = {
        "metric": FP8_FWD_METRIC, "value": round(flop / (t_step * 1e-3) / 1e12, 2),
        "unit": "TFLOPS", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": round(t_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8_e4m3+bf16", "data": "synthetic",
        "config": {"workload": "fp8_fwd_" + w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                   "causal": w.causal, "scale": w.scale, "k_outlier_frac": w.outlier_frac,
                   "seed": w.cid, "signs_seed": 4, "parallelism": "none (1 GPU)"},
        "kernels": {"fp8_quantize_q_and_k": {"avg_ms": round(t_quant, 5)},
                    "fwd_fp8": {"avg_ms": round(t_attn, 5),
                                "tflops_algorithmic": round(achieved, 2)},
                    "fwd_bf16_same_inputs": {"avg_ms": round(t_bf16, 5),
                                             "tflops_algorithmic": round(
                                                 flop / (t_bf16 * 1e-3) / 1e12, 2)}},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": round(peak, 1),
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "kernel": "fwd_fp8",
                     "peak_basis": "half the FLOPs (Q K^T) at the 5.0 PFLOP/s E4M3 peak, half "
                                   "(P V) at the 2.5 PFLOP/s bf16 peak",
                     "traffic": load_traffic("fwd_fp8")},
        "kernel_source_sha": kernel_source_sha(),
        "device": torch.cuda.get_device_name(0)}
    if cpu:
        result["cpu_baseline"] = fp8_fwd_cpu_baseline(w, x, signs.cpu().double().numpy(),
                                                      cpu_budget)
    print(json.dumps(result))
    return 0


def fp8_fwd_cpu_baseline(w, x, signs, budget_s: float) -> dict:
    """The float64 FP8 oracle (rotation, E4M3 quantisation, plain forward; as it
    stands) on whole heads of the same workload until the budget is spent, in the
    GPU line's FLOP convention."""
    from oracle import fp8
    blas = blas_info()
    t0 = time.perf_counter()
    heads = 0
    for bh in range(w.B * w.H):
        b, h = divmod(bh, w.H)
        q, k, v = (x[n][b, h].double().numpy() for n in ("q", "k", "v"))
        fp8.fp8_forward_head(q, k, v, w.causal, w.scale, signs)
        heads += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    flop = 4 * w.N * w.N * w.d * (0.5 if w.causal else 1.0) * heads
    return {"value": round(flop / dt / 1e12, 6), "unit": "TFLOPS",
            "cores": blas.get("threads") or os.cpu_count(), "kind": "oracle",
            "sample": f"{heads} of {w.B * w.H} heads, float64 numpy FP8 forward (rotation, "
                      f"E4M3 codes, plain forward), {dt:.2f} s wall",
            "cpu": cpu_model(), "blas": blas}


def copy_calibration(steps: int) -> None:
    """A plain 1 GiB device-to-device copy, for scaling FETCH_SIZE / WRITE_SIZE."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").random_(0, 255)
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": steps}))


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--prewarm", type=float, default=PREWARM_S,
                    help="seconds of untimed steps before the warm-up steps (counter runs use 0)")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--sweep", action="store_true",
                    help="time every workload (median/min over --steps reps) instead of the "
                         "benchmark step; one JSON line per workload")
    ap.add_argument("--fp8-quant", action="store_true",
                    help="time the FP8 input stage on Q and K of the N=4096 workload")
    ap.add_argument("--decode", action="store_true",
                    help="time the split-K decode workload instead of the benchmark step")
    ap.add_argument("--fp8", action="store_true",
                    help="time the FP8 forward path (rotation, E4M3 codes, attention) on the "
                         "N=4096 workload")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this path has no multi-GPU mode "
              "(no collectives); run with --gpus 1", file=sys.stderr)
        return 2

    import torch
    if args.copy_calibration:
        copy_calibration(args.steps)
        return 0
    if args.sweep:
        return sweep(args.steps, args.warmup, args.prewarm)
    if args.decode:
        return decode_bench(args.steps, args.warmup, not args.no_cpu_baseline, args.cpu_budget)
    if args.fp8_quant:
        return fp8_quant_bench(args.steps, args.warmup, not args.no_cpu_baseline, args.cpu_budget)
    if args.fp8:
        return fp8_fwd_bench(args.steps, args.warmup, not args.no_cpu_baseline, args.cpu_budget,
                             args.prewarm)

    import exact_io_aware_forward_amd as fa
    import workloads

    w = workloads.WORKLOADS[args.workload]
    if not w.backward:
        print("the benchmark step is forward + backward; pick a workload with a backward pass",
              file=sys.stderr)
        return 2
    x = workloads.workload_inputs(args.workload)
    dev = torch.device("cuda", 0)
    q, k, v, do = (x[n].to(dev) for n in ("q", "k", "v", "do"))
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = fa.new_workspace(q)
    causal, scale = w.causal, w.scale

    def step():
        fa.forward(q, k, v, causal, scale, out=o, lse=lse)
        fa.backward(q, k, v, o, do, lse, causal, scale, workspace=ws, out=(dq, dk, dv))

    def step_by_kernel(ev):
        # The same kernels, launched stage by stage with a HIP event between
        # kernels (fa_backward is exactly these two stages in this order).
        ev[0].record()
        fa.forward(q, k, v, causal, scale, out=o, lse=lse)
        ev[1].record()
        for j, s in enumerate((fa.BWD_DQ, fa.BWD_DKDV)):
            fa.backward_stage(s, q, k, v, o, do, lse, dq, dk, dv, ws, causal, scale)
            ev[2 + j].record()

    # The GPU's clock settles only after ~50 steps (~40 ms) of this work
    # following idle (a step takes ~850 us in the first 20, ~635 us from the
    # 60th on), so untimed steps run for --prewarm seconds first; then the
    # W warm-up steps and the K timed ones all see the settled clock.
    prewarm_steps = settle_clock(step, args.prewarm)
    for _ in range(args.warmup):
        step()
    # Timed region 1 (the reported value): K plain steps between two events.
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for _ in range(args.steps):
        step()
    t_end.record()
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / args.steps
    # Timed region 2 (per-kernel times and the roofline): K more steps with an
    # event between kernels; kept out of region 1, whose step it would lengthen.
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(KERNELS) + 1)]
              for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step_by_kernel(events[i])
    torch.cuda.synchronize()
    per_kernel_ms = {name: sum(ev[j].elapsed_time(ev[j + 1]) for ev in events) / args.steps
                     for j, name in enumerate(KERNELS)}
    ms_step_by_kernel = sum(per_kernel_ms.values())

    wm = work_model(w)
    peak = PEAK_TFLOPS[w.dtype]
    tflops = wm["step_flop"] / (ms_step * 1e-3) / 1e12
    kernels = {}
    for name in KERNELS:
        t = per_kernel_ms[name] * 1e-3
        kernels[name] = {"avg_ms": round(per_kernel_ms[name], 5),
                         "tflops_algorithmic": round(wm[name]["flop"] / t / 1e12, 2),
                         "gbps_algorithmic": round(wm[name]["bytes"] / t / 1e9, 1)}
        if name in ("fwd", "bwd_dkdv", "bwd_dq"):
            kernels[name]["frac_mfma_peak"] = round(wm[name]["flop"] / t / 1e12 / peak, 4)
    dominant = max(KERNELS, key=lambda n: per_kernel_ms[n])
    t_dom = per_kernel_ms[dominant] * 1e-3
    achieved = wm[dominant]["flop"] / t_dom / 1e12
    roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
            "unit": "TFLOP/s", "frac": round(achieved / peak, 4)}
    roof["kernel"] = dominant
    roof["traffic"] = load_traffic(dominant)

    fwd_t = per_kernel_ms["fwd"] * 1e-3
    result = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                   "causal": w.causal, "scale": scale, "k_outlier_frac": w.outlier_frac,
                   "seed": w.cid, "parallelism": "none (1 GPU)"},
        "pct_mfma_peak": round(100 * tflops / peak, 2),
        "fwd_tflops": round(wm["fwd_flop"] / fwd_t / 1e12, 2),
        "fwd_pct_mfma_peak": round(100 * wm["fwd_flop"] / fwd_t / 1e12 / peak, 2),
        "kernels": kernels,
        "prewarm": {"seconds": args.prewarm, "steps": prewarm_steps},
        "kernel_times_from": ("a second run of the same number of steps with a HIP event between "
                              f"kernels ({ms_step_by_kernel:.5f} ms per step there); "
                              "ms_per_step and value come from plain steps"),
        "roofline": roof,
        "kernel_source_sha": kernel_source_sha(),
        "device": torch.cuda.get_device_name(0),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, x, args.cpu_budget)
    print(json.dumps(result))
    return 0


if __name__ == "__main__":
    sys.exit(main())
