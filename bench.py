#!/usr/bin/env python3
"""Attention forward benchmark on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload long] [--no-cpu-baseline]
                    [--op forward|backward] [--seq-len N] [--kv-heads G]

One step = one fa_forward launch over the whole workload (every query row of
every head) with Q, K, V, O and LSE already resident in HBM.  Prints one JSON
line: TFLOP/s counted as 4*B*H*N^2*d (non-causal), the kernel's roofline
against the MFMA peak, and the CPU oracle timed on a bounded sample of the
same workload on this host's cores.  The oracle's results are compared with
the GPU's on every row it computed (the long workload: every row of every
head); "parity" in the JSON line gives the max-abs errors against the bar
(O 1e-4 fp32 / 2e-2 fp16, bf16; LSE 1e-3), and the process exits with status
1 after printing the line when they exceed it.

--op backward times one fa_backward call instead (its three kernels, with
O and LSE from one forward launch made before timing) and counts
10*B*H*N^2*d: the five N x N x d products of the gradient (S, dP, dV, dQ,
dK), recomputation of S included, as is usual for attention backward.
--op split times one fa_forward_split call (forward kernel over key ranges
plus the merge kernel; workspace allocated before timing) with --splits
ranges (0: the library's suggestion), counts 4*B*H*N^2*d like the forward,
and also reports the unsplit forward on the same inputs.
--op fp8 times one fa_forward_fp8 launch on the workload's draws quantised
per tensor to OCP e4m3 (bf16 output), counts 4*B*H*N^2*d and takes the
5000 TFLOP/s dense fp8 MFMA peak.
--seq-len replaces the workload's N (same seeds and other sizes).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

METRIC = "attention fwd TFLOP/s (4·B·H·N²·d) bf16 at 1 GPU + % of MFMA peak"
METRIC_BWD = "attention bwd TFLOP/s (10·B·H·N²·d) at 1 GPU + % of MFMA peak"
METRIC_FP8 = "attention fwd TFLOP/s (4·B·H·N²·d) fp8 e4m3 inputs at 1 GPU + % of fp8 MFMA peak"
# MI355X published dense matrix peaks (TFLOP/s) and HBM bandwidth (GB/s).
PEAK_TFLOPS = {"bf16": 2500.0, "fp16": 2500.0, "fp32": 157.3, "fp8_e4m3": 5000.0}
PEAK_HBM_GBS = 8000.0
# Parity bar of the forward (max-abs error over every checked element).
O_TOL = {"fp32": 1e-4, "fp16": 2e-2, "bf16": 2e-2}
LSE_TOL = 1e-3
# Oracle worker threads: at most the CPU share that one GPU of the host is
# given (16 threads), and no more than this process may run on.
CPU_SHARE = 16
KERNEL_SOURCE = os.path.join(HERE, "tiled_online_softmax_06_amd", "csrc", "flash_fwd.hip")
FP8_SOURCE = os.path.join(HERE, "tiled_online_softmax_06_amd", "csrc", "flash_fwd_fp8.hip")
BWD_SOURCE = os.path.join(HERE, "tiled_online_softmax_06_amd", "csrc", "flash_bwd.hip")


def kernel_hash(path: str = KERNEL_SOURCE) -> str:
    """First 16 hex digits of sha256 over a kernel source and the compiler
    flags it is built with (paths left out), so a record taken on another
    build of the kernel is not used."""
    from tiled_online_softmax_06_amd import build_lib
    flags = " ".join(f for f in build_lib.FLAGS if "/" not in f and f != "-I")
    with open(path, "rb") as f:
        return hashlib.sha256(f.read() + flags.encode()).hexdigest()[:16]


def kernel_name(w) -> str:
    """The kernel fa_forward dispatches for a workload's dtype and head size."""
    if w.dtype == "fp32":
        return f"flash_fwd_32<d={w.d}>"
    return f"flash_fwd_pp<{w.dtype}, d=128>" if w.d == 128 else f"flash_fwd_16<{w.dtype}, d={w.d}>"


def traffic_record(workload: str):
    """HBM bytes per launch from committed PMC counter runs, if they were taken
    on the current kernel source; else None."""
    path = os.path.join(HERE, "profiles", f"flash_fwd_{workload}_hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_sha256_16") != kernel_hash():
        return None
    return rec


def device_info(props, peak_spec, fp8):
    """Name, CU count and peak engine clock (hipDeviceGetAttribute), with the
    dense MFMA peak derived from them (bf16/fp16: 4096 flop per clock per CU,
    fp8 twice that) beside the published figure."""
    import ctypes

    info = {"name": props.name, "cu": props.multi_processor_count, "gcn_arch": getattr(props, "gcnArchName", "")}
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        val = ctypes.c_int(0)
        dev = ctypes.c_int(0)
        hip.hipGetDevice(ctypes.byref(dev))
        # hipDeviceAttributeClockRate (kHz): the sixth entry of hipDeviceAttribute_t
        if hip.hipDeviceGetAttribute(ctypes.byref(val), 5, dev.value) == 0 and 1e5 < val.value < 1e7:
            ghz = val.value / 1e6
            per_clk = 4096 * (2 if fp8 else 1)
            info["peak_clock_ghz"] = round(ghz, 3)
            info["derived_peak_tflops"] = round(props.multi_processor_count * ghz * 1e9 * per_clk / 1e12, 1)
            info["published_peak_tflops"] = peak_spec
    except OSError:
        pass
    return info


def oracle_pool():
    """(workers, cpus available to this process) for the oracle's thread pool."""
    avail = len(os.sched_getaffinity(0))
    return max(1, min(CPU_SHARE, avail)), avail


def pool_fields(workers: int, avail: int) -> dict:
    return {"cores": workers, "host_cpus_available": avail, "os_cpu_count": os.cpu_count(),
            "pool": f"thread pool of {workers} workers (numpy releases the GIL), one BLAS thread each; "
                    f"capped at {CPU_SHARE}, the CPU share of one GPU on this host"}


def cpu_baseline_backward(w, q, k, v, do, heads: int, workers: int):
    """The backward oracle, untuned, on a bounded sample: the first `heads`
    (b, h) heads of the workload (whole heads: every query and key), one head
    per worker thread with one BLAS thread each."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    from tiled_online_softmax_06_amd import inputs

    g = w.H // k.shape[1]
    heads = max(1, min(heads, w.B * w.H))
    scale = float(np.float32(w.scale))
    qf, dof = (t.reshape(1, w.B * w.H, w.N, w.d) for t in (q, do))
    kf, vf = (t.reshape(1, -1, w.N, w.d) for t in (k, v))

    def job(h):
        sl = (slice(0, 1), slice(h, h + 1))
        kv = (slice(0, 1), slice(h // g, h // g + 1))
        return oracle.attention_bwd_ref(inputs.to_float64(qf[sl]), inputs.to_float64(kf[kv]),
                                        inputs.to_float64(vf[kv]), inputs.to_float64(dof[sl]), scale)

    with threadpool_limits(1):
        t0 = time.perf_counter()
        with ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(job, range(heads)))
        dt = time.perf_counter() - t0
    flops = 10 * heads * w.N * w.N * w.d
    out = {"value": flops / dt / 1e12, "unit": "TFLOP/s", "kind": "oracle",
           "sample": f"first {heads} of {w.B * w.H} heads, every query and key "
                     f"({flops / 1e9:.1f} GFLOP counted as 10*N^2*d per head, float64)",
           "seconds": round(dt, 3)}
    out.update(pool_fields(min(workers, heads), len(os.sched_getaffinity(0))))
    return out


def cpu_baseline_rows(w, q, k, v, workers: int, gpu_out=None):
    """The oracle on the workload's seeded sample of query rows (workloads
    whose parity is checked on sampled rows), one row chunk per worker, with
    the full-workload time extrapolated from it and labelled as such."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    from tiled_online_softmax_06_amd import inputs

    rows = inputs.sample_rows(w)
    q64, k64, v64 = (inputs.to_float64(t) for t in (q, k, v))
    scale = float(np.float32(w.scale))
    parts = np.array_split(rows, workers)
    with threadpool_limits(1):
        t0 = time.perf_counter()
        with ThreadPoolExecutor(max_workers=workers) as ex:
            results = list(ex.map(lambda r: (r, oracle.attention_ref(q64, k64, v64, scale, rows=r)), parts))
        dt = time.perf_counter() - t0
    flops = 4 * rows.size * w.N * w.d
    out = {"value": flops / dt / 1e12, "unit": "TFLOP/s", **pool_fields(workers, len(os.sched_getaffinity(0))),
           "kind": "oracle",
           "sample": f"{rows.size} seeded query rows of {w.B * w.H * w.N} (default_rng(2005)), each against "
                     f"its head's {w.N} keys ({flops / 1e9:.2f} GFLOP in float64)",
           "seconds": round(dt, 3),
           "extrapolated_full_workload_seconds": round(dt * w.flops / flops, 1)}
    if gpu_out is not None:
        o_gpu = gpu_out[0].reshape(-1, w.d)
        lse_gpu = gpu_out[1].reshape(-1)
        eo = el = 0.0
        for r, (o_ref, lse_ref) in results:
            eo = max(eo, float(np.abs(o_gpu[r].double().numpy() - o_ref).max()))
            el = max(el, float(np.abs(lse_gpu[r].double().numpy() - lse_ref).max()))
        out["sample_max_abs_err"] = {"O": eo, "LSE": el}
        out["rows_compared"] = int(rows.size)
    return out


def cpu_baseline(w, q, k, v, heads: int, chunk: int, workers: int, gpu_out=None):
    """The oracle, untuned, on a bounded sample: the first `heads` heads of the
    workload, every query row, split into row chunks over a thread pool with
    one BLAS thread per worker."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    from tiled_online_softmax_06_amd import inputs

    g = w.H // k.shape[1]                     # query heads per K/V head
    heads = w.B * w.H if heads <= 0 else max(g, min(heads, w.B * w.H) // g * g)
    # flattened (1, B*H) query heads use flattened K/V head f // g
    q64 = inputs.to_float64(q.reshape(1, w.B * w.H, w.N, w.d)[:, :heads])
    k64, v64 = (inputs.to_float64(t.reshape(1, -1, w.N, w.d)[:, :heads // g]) for t in (k, v))
    scale = float(np.float32(w.scale))
    tasks = [(h, i0) for h in range(heads) for i0 in range(0, w.N, chunk)]

    def job(t):
        h, i0 = t
        rows = np.arange(h * w.N + i0, h * w.N + min(i0 + chunk, w.N))
        return rows, oracle.attention_ref(q64, k64, v64, scale, rows=rows)

    with threadpool_limits(1):
        t0 = time.perf_counter()
        with ThreadPoolExecutor(max_workers=workers) as ex:
            results = list(ex.map(job, tasks))
        dt = time.perf_counter() - t0
    flops = 4 * heads * w.N * w.N * w.d
    out = {"value": flops / dt / 1e12, "unit": "TFLOP/s", **pool_fields(workers, len(os.sched_getaffinity(0))),
           "kind": "oracle",
           "sample": f"first {heads} of {w.B * w.H} heads, all {w.N} query rows each "
                     f"({flops / 1e9:.1f} GFLOP in float64; {len(tasks)} row chunks of {chunk})",
           "seconds": round(dt, 3)}
    if gpu_out is not None:
        o_gpu, lse_gpu = gpu_out
        o_gpu = o_gpu.reshape(-1, w.d)
        lse_gpu = lse_gpu.reshape(-1)
        eo = el = 0.0
        for rows, (o_ref, lse_ref) in results:
            eo = max(eo, float(np.abs(o_gpu[rows].double().numpy() - o_ref).max()))
            el = max(el, float(np.abs(lse_gpu[rows].double().numpy() - lse_ref).max()))
        out["sample_max_abs_err"] = {"O": eo, "LSE": el}
        out["rows_compared"] = heads * w.N
    return out


def parity_verdict(w, base, fixed_bar: bool):
    """The oracle comparison the CPU-baseline leg made, against the parity
    bar (max-abs error on O and LSE over every compared element)."""
    if base is None or "sample_max_abs_err" not in base:
        return {"checked": False, "note": "no oracle comparison in this run"}
    err = base["sample_max_abs_err"]
    out = {"checked": True, "O_max_abs_err": err["O"], "LSE_max_abs_err": err["LSE"],
           "rows_compared": base.get("rows_compared"), "rows_total": w.B * w.H * w.N}
    if not fixed_bar:
        out["note"] = ("FP8 inputs: no fixed bar; tests/test_gpu_fp8.py asserts the derived per-element bar")
        return out
    out["O_tol"] = O_TOL[w.dtype]
    out["LSE_tol"] = LSE_TOL
    out["pass"] = bool(err["O"] <= O_TOL[w.dtype] and err["LSE"] <= LSE_TOL)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="long")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kv-heads", type=int, default=0,
                    help="K/V heads for a grouped-query run (0: one per query head)")
    ap.add_argument("--cpu-heads", type=int, default=0,
                    help="heads the CPU oracle computes in full (0: every head of the workload)")
    ap.add_argument("--op", choices=("forward", "backward", "split", "fp8"), default="forward")
    ap.add_argument("--splits", type=int, default=0, help="key ranges for --op split (0: suggested)")
    ap.add_argument("--seq-len", type=int, default=0, help="override the workload's N (0: keep it)")
    ap.add_argument("--graph", action="store_true",
                    help="time the K steps as one replay of a HIP graph holding them instead of "
                         "back-to-back launches (both figures are then reported)")
    ap.add_argument("--min-warmup-ms", type=float, default=200.0,
                    help="after the W warm-up steps, keep warming up until this much time has "
                         "passed: the chip's power controller takes about 10-15 ms of sustained "
                         "load to settle its clock")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 512 MiB device copy (for HBM counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on exactly one GPU (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "this attention forward is a single-GPU kernel and no multi-GPU path is built.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from tiled_online_softmax_06_amd import fa, inputs

    import dataclasses

    w = inputs.WORKLOADS[args.workload]
    if args.seq_len > 0:
        w = dataclasses.replace(w, N=args.seq_len)
    backward = args.op == "backward"
    if backward and w.dtype == "fp32":
        print("the backward kernels take fp16 / bf16 inputs", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    kv_heads = args.kv_heads or w.H
    if w.H % kv_heads:
        print(f"--kv-heads {kv_heads} must divide H={w.H}", file=sys.stderr)
        sys.exit(2)
    q, k, v = inputs.make_inputs(w, kv_heads=kv_heads)
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    o = torch.empty_like(qd)
    lse = torch.empty(qd.shape[:3], dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        fa.forward_into(qd, kd, vd, o, lse, w.scale, stream=None)

    fp8 = args.op == "fp8"
    if fp8:
        q8, k8, v8, descale = inputs.make_fp8_inputs(w, kv_heads=kv_heads)
        q8d, k8d, v8d = (t.to(dev) for t in (q8, k8, v8))
        o = torch.empty(q8.shape, dtype=torch.bfloat16, device=dev)
        # the oracle (cpu_baseline) sees the dequantised values
        q, k, v = (torch.from_numpy(inputs.dequantize(c, s_)) for c, s_ in zip((q8, k8, v8), descale))

        def step():  # noqa: F811
            fa.forward_fp8_into(q8d, k8d, v8d, descale, o, lse, w.scale, stream=None)

    if backward:
        do = inputs.make_grad(w)
        dod = do.to(dev)
        step()
        dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
        dws = torch.empty(qd.shape[:3], dtype=torch.float32, device=dev)

        def step():  # noqa: F811
            fa.backward_into(qd, kd, vd, o, dod, lse, dq, dk, dv, dws, w.scale, stream=None)

    split = args.op == "split"
    unsplit_ms = None
    if split:
        splits = args.splits or fa.split_suggest(w.B, w.H, w.N, w.d, qd.dtype)
        ws = torch.empty(max(fa.split_workspace_bytes(w.B, w.H, w.N, w.d, splits), 16), dtype=torch.uint8,
                         device=dev)

        def time_it(fn, steps):
            for _ in range(args.warmup):
                fn()
            torch.cuda.synchronize()
            t0 = torch.cuda.Event(enable_timing=True)
            t1 = torch.cuda.Event(enable_timing=True)
            t0.record(stream)
            for _ in range(steps):
                fn()
            t1.record(stream)
            torch.cuda.synchronize()
            return t0.elapsed_time(t1) / max(steps, 1)

        unsplit_ms = time_it(step, args.steps)

        def step():  # noqa: F811
            fa.forward_split_into(qd, kd, vd, o, lse, ws, splits, w.scale, stream=None)

    if args.calibrate_copy:
        src = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    # Warm-up: W steps, then more until min-warmup-ms have passed, so that
    # the timed steps run at the clock the power limit settles at (the first
    # ~10 ms of sustained load run at a transient clock, up to 15 % slower).
    warm_start = time.perf_counter()
    warm_steps = 0
    for _ in range(args.warmup):
        step()
        warm_steps += 1
    torch.cuda.synchronize()
    while (time.perf_counter() - warm_start) * 1e3 < args.min_warmup_ms:
        for _ in range(max(args.steps, 1)):
            step()
            warm_steps += 1
        torch.cuda.synchronize()
    warm_ms = (time.perf_counter() - warm_start) * 1e3

    def timed(run):
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        run()
        end.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(end) / max(args.steps, 1)

    def eager():
        for _ in range(args.steps):
            step()

    # With --graph the K steps are captured once into a HIP graph (the
    # library allocates nothing and records no memset), replayed once
    # untimed, then timed as one replay, with no host work between the
    # launches; the same K steps launched back to back are timed right after.
    graph = None
    if args.graph:
        try:
            graph = torch.cuda.CUDAGraph()
            cap = torch.cuda.Stream(dev)
            cap.wait_stream(stream)
            with torch.cuda.graph(graph, stream=cap):
                eager()
            stream.wait_stream(cap)
            graph.replay()
            torch.cuda.synchronize()
        except RuntimeError as exc:   # capture unavailable: time the launches themselves
            print(f"graph capture failed ({exc}); timing back-to-back launches", file=sys.stderr)
            graph = None
            torch.cuda.synchronize()
    if graph is not None:
        ms = timed(graph.replay)
        eager_ms = timed(eager)
    else:
        ms = timed(eager)
        eager_ms = ms

    # Per-launch spread, after and outside the timed region: each launch
    # bracketed by its own pair of events on the launch stream.
    per = []
    for _ in range(min(args.steps, 50)):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        step()
        b.record(stream)
        per.append((a, b))
    torch.cuda.synchronize()
    per_ms = sorted(a.elapsed_time(b) for a, b in per)

    flops = w.flops
    if backward:
        flops = 10 * w.B * w.H * w.N * w.N * w.d
    tflops = flops / (ms * 1e-3) / 1e12
    props = torch.cuda.get_device_properties(dev)
    peak = PEAK_TFLOPS["fp8_e4m3" if fp8 else w.dtype]
    roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak, "unit": "TFLOP/s",
            "frac": round(tflops / peak, 4), "traffic": None,
            "kernel": kernel_name(w),
            "avg_launch_ms": round(ms, 5)}
    if fp8:
        roof["kernel"] = f"flash_fwd_fp8<d={w.d}, bf16 out>"
    if split:
        roof["kernel"] = f"{kernel_name(w)} over {splits} key ranges + fa_merge_rows (one fa_forward_split call)"
        roof["avg_launch_ms_note"] = "the two kernels of one call, stream order"
    if backward:
        roof["kernel"] = (f"flash_bwd_dot + flash_bwd_dq + flash_bwd_dkdv <{w.dtype}, d={w.d}> "
                          "(one fa_backward call)")
        roof["avg_launch_ms_note"] = "the three kernels of one call, stream order"
    rec = None if backward or split or fp8 or args.seq_len else traffic_record(w.name)
    if rec is not None:
        roof["traffic"] = rec["hbm_bytes_per_launch"]
        roof["traffic_note"] = rec.get("note", "")

    result = {
        "metric": METRIC_BWD if backward else (METRIC_FP8 if fp8 else METRIC),
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3" if fp8 else w.dtype,
        "data": "synthetic (seeded iid normal inputs, see tiled_online_softmax_06_amd/inputs.py)",
        "config": {"workload": f"{w.name}: B={w.B} H={w.H} N={w.N} d={w.d} {w.dtype}, non-causal, "
                               f"scale=1/sqrt({w.d})" + (f", {kv_heads} K/V heads" if kv_heads != w.H else ""),
                   "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": False, "kv_heads": kv_heads},
        "timing": ("one replay of a HIP graph holding the K steps" if graph is not None
                   else "K steps launched back to back"),
        "eager_ms_per_step": round(eager_ms, 5),
        "warmup_run": {"steps": warm_steps, "ms": round(warm_ms, 1),
                       "note": "W steps, then more until --min-warmup-ms had passed"},
        "pct_of_mfma_peak": round(100 * tflops / peak, 2),
        "roofline": roof,
        "launch_ms": ({"median": round(per_ms[len(per_ms) // 2], 5), "min": round(per_ms[0], 5),
                       "max": round(per_ms[-1], 5), "n": len(per_ms),
                       "note": "separately evented launches after the timed region"} if per_ms else None),
        "device": device_info(props, peak, fp8),
        "kernel_sha256_16": kernel_hash(BWD_SOURCE if backward else (FP8_SOURCE if fp8 else KERNEL_SOURCE)),
    }
    if backward:
        result["op"] = "backward"
        result["config"]["op"] = "backward"
    if fp8:
        result["op"] = "fp8"
        result["config"]["op"] = "fp8"
        result["config"]["descale"] = [round(x, 8) for x in descale]
    if split:
        result["op"] = "split"
        result["config"]["op"] = "split"
        result["config"]["splits"] = splits
        result["unsplit"] = {"ms_per_step": round(unsplit_ms, 5),
                             "value": round(flops / (unsplit_ms * 1e-3) / 1e12, 2)}
    workers, _ = oracle_pool()
    if not args.no_cpu_baseline and (split or fp8):
        result["cpu_baseline"] = cpu_baseline(w, q, k, v, args.cpu_heads, 512, workers,
                                              gpu_out=(o.cpu(), lse.cpu()))
    elif not args.no_cpu_baseline and backward:
        result["cpu_baseline"] = cpu_baseline_backward(w, q, k, v, do, args.cpu_heads or min(8, workers), workers)
    elif not args.no_cpu_baseline and w.sample_rows and not args.seq_len:
        result["cpu_baseline"] = cpu_baseline_rows(w, q, k, v, workers, gpu_out=(o.cpu(), lse.cpu()))
    elif not args.no_cpu_baseline:
        chunk = 512 if w.N >= 4096 else max(64, w.N // 4)
        result["cpu_baseline"] = cpu_baseline(w, q, k, v, args.cpu_heads, chunk, workers,
                                              gpu_out=(o.cpu(), lse.cpu()))
    if not backward:
        result["parity"] = parity_verdict(w, result.get("cpu_baseline"), fixed_bar=not fp8)
    print(json.dumps(result), flush=True)
    if result.get("parity", {}).get("pass") is False:
        print(f"parity FAILED: {result['parity']}", file=sys.stderr, flush=True)
        sys.exit(1)


if __name__ == "__main__":
    main()
