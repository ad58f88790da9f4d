#!/usr/bin/env python3
"""Benchmark of the FlashAttention-2 forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--splits S] [--backward]

A step is one fa2_fwd call over the whole batch of the workload (inputs already
resident in device memory); with --splits, one fa2_fwd_splitkv call (partial
kernel + merge kernel, workspace allocated before the timed region); with
--backward, one fa2_bwd call (prep, dK/dV and dQ kernels) on o and lse from a
forward call made before the timed region, counted as 2.5x the forward's work
(10*B*H*Lq*Lk*d, halved for causal: the five products S, dP, dV, dK, dQ).  Prints ONE JSON line with the throughput in
attention-forward TFLOP/s (4*B*H*Lq*Lk*d, halved for causal), the roofline
position of the kernel (HIP events on the launch stream), the HBM traffic taken
from rocprofv3 counters (profiles/), and the CPU oracle timed on a bounded
sample of the same workload.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOPS (4·B·H·Lq·Lk·d) bf16 at N=2K–16K; % of MFMA peak"
METRIC_BWD = "attention bwd TFLOPS (10·B·H·Lq·Lk·d, halved for causal) bf16; % of MFMA peak"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
PEAK_FP32_MFMA_TFLOPS = 157.3  # MI355X fp32, published
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fa2_fwd_bf16_B2_H32_L4096_d128_causal_traffic.md")
COUNTERS_FILE = os.path.join(ROOT, "profiles", "fa2_fwd_bf16_B2_H32_L4096_d128_causal_counters.md")
CONTEXT = {
    "a100_fp16_tensor_tflops": 312, "a100_hbm_gbs": 1555, "a100_sram_tbs": 19,
    "claimed_matmul_utilisation_fa1_to_fa2": "30-50% -> >70%",
    "note": "figures quoted by the pages for NVIDIA A100; context only, not a target",
}


def kernel_source_digest():
    """sha256 over the code of the one-pass forward kernel and its launch (the
    kernel file, the shared headers and the entry points; comments and blank
    space removed), to tell whether stored counters are stale.  The backward,
    merge and fp32 sources do not enter it."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "flashattention_forward_fwd_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith(".h") or name in ("fa2_fwd_bf16.hip", "fa2_api.hip"):
            with open(os.path.join(csrc, name)) as f:
                text = f.read()
            text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)      # block comments
            text = re.sub(r"//[^\n]*", " ", text)                    # line comments
            text = " ".join(text.split())
            h.update(name.encode() + b"\0" + text.encode())
    return h.hexdigest()[:16]


def stored_fields(path, workload_name):
    """The machine-readable fields of a committed rocprofv3 summary, or None when
    the summary is missing, covers another workload, or predates the kernel."""
    try:
        text = open(path).read()
    except OSError:
        return None
    fields = dict(re.findall(r"^- (\w+): `([^`]*)`", text, flags=re.M))
    if fields.get("workload") != workload_name:
        return None
    if fields.get("kernel_source_sha256") != kernel_source_digest():
        return None
    return fields


def stored_traffic(workload_name):
    """HBM bytes per launch from the committed counter summary (or None)."""
    fields = stored_fields(TRAFFIC_FILE, workload_name)
    try:
        return float(fields["hbm_bytes_per_launch"]) if fields else None
    except (KeyError, ValueError):
        return None


def stored_counters(workload_name):
    """MFMA-busy fraction, VALU and LDS instruction mix and LDS bank conflicts of
    the forward kernel, from the committed counter summary (or None)."""
    fields = stored_fields(COUNTERS_FILE, workload_name)
    if not fields:
        return None
    keys = ("mfma_busy_frac", "clock_ghz", "valu_coexec_frac", "valu_insts_per_score_element",
            "trans_insts_per_score_element", "lds_insts_per_wave_tile", "lds_bank_conflict_cycles")
    optional = ("lds_busy_frac", "wave_wait_any_frac", "wave_wait_issue_frac", "wave_issue_frac",
                "lds_latency_cycles", "vmem_latency_cycles")
    try:
        out = {k: float(fields[k]) for k in keys}
        out.update({k: float(fields[k]) for k in optional if k in fields})
    except (KeyError, ValueError):
        return None
    out["source"] = os.path.join("profiles", os.path.basename(COUNTERS_FILE))
    return out


def device_peak():
    """Compute units and peak shader clock of device 0, read through the HIP
    runtime this process already uses, and the dense bf16 MFMA peak they imply
    (gfx950: 4096 FLOP per clock per CU).  The roofline's peak stays MI355X's
    published 2.5 PFLOP/s; this is the cross-check."""
    import ctypes
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    clock_khz = None
    try:
        with open("/proc/self/maps") as f:
            path = next((ln.split()[-1] for ln in f if "libamdhip64.so" in ln), None)
        if path:
            hip = ctypes.CDLL(path)
            val = ctypes.c_int(0)
            # hipDeviceGetAttribute(&val, hipDeviceAttributeClockRate (5), device 0): kHz
            if hip.hipDeviceGetAttribute(ctypes.byref(val), 5, 0) == 0 and 100000 < val.value < 10000000:
                clock_khz = val.value
    except (OSError, AttributeError):
        clock_khz = None
    out = {"cus": cus, "max_sclk_mhz": clock_khz / 1000.0 if clock_khz else None,
           "bf16_flop_per_clk_per_cu": 4096}
    out["bf16_peak_tflops"] = round(cus * clock_khz * 1e3 * 4096 / 1e12, 1) if clock_khz else None
    return out


def warm_up(fn, call, stream, min_launches, min_seconds=1.0, max_seconds=10.0, window_ms=20.0):
    """Untimed launches until at least min_launches have run, at least min_seconds
    have passed, and the last three windows of about window_ms of GPU work each
    agree within 0.5 % (max over min): the shader clock of MI355X settles only
    after about a hundred milliseconds of load (the first launches of a run take
    ~12 % longer).  Returns (launches, seconds, settled)."""
    import torch
    n, per_window, recent = 0, 5, []
    t0 = time.perf_counter()
    while True:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(per_window):
            fn(*call)
        b.record(stream)
        torch.cuda.synchronize()
        n += per_window
        per_launch = a.elapsed_time(b) / per_window
        recent = (recent + [per_launch])[-3:]
        per_window = max(5, int(window_ms / max(per_launch, 1e-3)))
        dt = time.perf_counter() - t0
        settled = len(recent) == 3 and max(recent) <= 1.005 * min(recent)
        if (n >= min_launches and dt >= min_seconds and settled) or dt >= max_seconds:
            return n, dt, settled


def cpu_baseline(w, q, k, v, rows_per_head):
    """The oracle, as it stands, on a seeded sample of query rows of every head."""
    import numpy as np
    import torch
    from flashattention_forward_fwd_amd.inputs import head_row_samples
    from oracle import ref

    rows = head_row_samples(w, rows_per_head)
    qd, kd, vd = (t.to(torch.float64).numpy() for t in (q, k, v))
    threads = ref.default_threads()
    ref.attention_f64(qd[:, :1], kd[:, :1], vd[:, :1], w.scale, w.causal, rows=rows[:1, :8], nthreads=threads)
    t0 = time.perf_counter()
    ref.attention_f64(qd, kd, vd, w.scale, w.causal, rows=rows, nthreads=threads)
    dt = time.perf_counter() - t0
    vis = np.minimum(rows + 1, w.Lk) if w.causal else np.full(rows.shape, w.Lk)
    flops = float(4.0 * w.d * vis.sum())
    return {
        "value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
        "sample": "%d seeded query rows of each of the %d (batch, head) pairs (%.1f%% of rows), "
                  "each against all its visible keys; %.3g FLOP in %.2f s, fp64"
                  % (rows.shape[1], w.B * w.H, 100.0 * rows.shape[1] / w.Lq, flops, dt),
    }


def cpu_baseline_bwd(w, q, k, v, do):
    """The backward oracle, as it stands, on every row and key of the first (batch, head)."""
    import torch
    from oracle import ref

    sl = (slice(0, 1), slice(0, 1))
    qd, kd, vd, dod = (t[sl].to(torch.float64).numpy() for t in (q, k, v, do))
    threads = ref.default_threads()
    t0 = time.perf_counter()
    ref.attention_bwd_f64(qd, kd, vd, dod, w.scale, w.causal, nthreads=threads)
    dt = time.perf_counter() - t0
    flops = 2.5 * w.flops / (w.B * w.H)
    return {
        "value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
        "sample": "full gradients (dq, dk, dv) of 1 of the %d (batch, head) pairs; %.3g FLOP "
                  "(2.5x the forward count) in %.2f s, fp64" % (w.B * w.H, flops, dt),
    }


def calibrate_copy(nbytes):
    """A plain device copy of known size, for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "launches": 3}))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    # Warm-up: at least --warmup launches, and more until the per-launch time has
    # settled (see warm_up); the JSON line reports how many ran.
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default=None, help="workload name (default: the headline causal N=4096, d=128)")
    ap.add_argument("--shape", default=None, metavar="B,H,Lq,Lk,d,causal",
                    help="time another shape instead of a named workload: inputs drawn by the same recipe "
                         "(bf16, seed 7)")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="omit the oracle timing (profiling runs)")
    ap.add_argument("--cpu-rows-per-head", type=int, default=0,
                    help="query rows per (batch, head) for the oracle timing (0: every row)")
    ap.add_argument("--splits", type=int, default=None, metavar="S",
                    help="time the split-KV path with S K/V ranges (0: the library's choice)")
    ap.add_argument("--window", default=None, metavar="WL,WR",
                    help="time the sliding-window forward fa2_fwd_window (key j visible to query i iff "
                         "i-WL <= j <= i+WR; negative: unbounded) on a bf16 workload; the window "
                         "replaces the workload's causal flag")
    ap.add_argument("--fp16", action="store_true",
                    help="run a bf16 workload's shapes in fp16 (fa2_fwd_f16 / fa2_bwd_f16): inputs drawn the same "
                         "way, rounded to IEEE half")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward pass fa2_bwd (bf16 workloads) instead of the forward")
    ap.add_argument("--dropout", type=float, default=None, metavar="P",
                    help="time the dropout entry point (fa2_fwd_dropout, or fa2_bwd_dropout with --backward) "
                         "with drop probability P on a bf16 workload; seed and offset fixed")
    ap.add_argument("--flush-l2", action="store_true",
                    help="after the timed steps, time K more calls, each after a read of 512 MiB on the "
                         "launch stream (evicts the L2s and the 256 MiB Infinity Cache); reported as "
                         "roofline.l2_flushed_*")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run a plain copy of BYTES bytes (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py: the library and this bench run on one GPU; --gpus %d is not supported "
              "(the forward pass would shard by (batch, head) and query tile with no exchange; "
              "there is no multi-GPU path)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return

    import torch
    import flashattention_forward_fwd_amd as fa
    from flashattention_forward_fwd_amd.inputs import DECODE_WORKLOADS, HEADLINE, WORKLOADS, workload_inputs

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    fa.lib()   # fail loudly if the HIP library is missing
    if args.shape is not None:
        if args.workload is not None:
            print("bench.py: --shape replaces --workload", file=sys.stderr)
            sys.exit(2)
        from flashattention_forward_fwd_amd.inputs import Workload
        B, H, Lq, Lk, d, causal = (int(x) for x in args.shape.split(","))
        name = "B%d_H%d_Lq%d_Lk%d_d%d_bf16%s" % (B, H, Lq, Lk, d, "_causal" if causal else "")
        w = Workload(name, B, H, Lq, Lk, d, "bf16", bool(causal), 7)
    else:
        w = dict(WORKLOADS, **DECODE_WORKLOADS)[args.workload or HEADLINE]
    if args.fp16:
        import dataclasses
        if w.dtype != "bf16":
            print("bench.py: --fp16 takes a bf16 workload", file=sys.stderr)
            sys.exit(2)
        w = dataclasses.replace(w, dtype="fp16")
    q, k, v = workload_inputs(w)
    dq, dk, dv = q.cuda(), k.cuda(), v.cuda()
    o = torch.empty_like(dq)
    lse = torch.empty((w.B, w.H, w.Lq), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    args_common = (dq, dk, dv, o, lse, w.B, w.H, w.Lq, w.Lk, w.d, w.scale, int(w.causal))
    # the fp16 twin of a 16-bit entry point
    f16 = (lambda name: getattr(fa, name + "_f16")) if w.dtype == "fp16" else (lambda name: getattr(fa, name))
    split_info = None
    bwd_info = None
    win_info = None
    flops_override = None
    drop_info = None
    if args.dropout is not None:
        if w.dtype not in ("bf16", "fp16") or args.splits is not None or args.window is not None:
            print("bench.py: --dropout takes a bf16 (or --fp16) workload, without --splits or --window",
                  file=sys.stderr)
            sys.exit(2)
        drop_args = (float(args.dropout), 0x5EED, 0)
        drop_info = {"p": float(args.dropout), "seed": 0x5EED, "offset": 0,
                     "flops_count": "as without dropout (the mask adds no matrix work)"}
    if args.window is not None:
        if w.dtype not in ("bf16", "fp16") or args.splits is not None or args.backward:
            print("bench.py: --window takes a bf16 (or --fp16) workload, without --splits or --backward",
                  file=sys.stderr)
            sys.exit(2)
        import numpy as np
        wl, wr = (int(x) for x in args.window.split(","))
        i = np.arange(w.Lq, dtype=np.int64)
        lo = np.maximum(0, i - wl) if wl >= 0 else np.zeros_like(i)
        hi = np.minimum(w.Lk, i + wr + 1) if wr >= 0 else np.full_like(i, w.Lk)
        pairs = int(np.maximum(hi - lo, 0).sum())
        flops_override = 4.0 * w.B * w.H * w.d * pairs
        fn = f16("fa2_fwd_window")
        call = (dq, dk, dv, o, lse, w.B, w.H, w.Lq, w.Lk, w.d, w.scale, wl, wr, stream.cuda_stream)
        win_info = {"window_left": wl, "window_right": wr, "visible_pairs_per_head": pairs,
                    "flops_count": "4*d per visible (query, key) pair"}
    elif args.backward:
        if w.dtype not in ("bf16", "fp16") or args.splits is not None:
            print("bench.py: --backward takes a bf16 (or --fp16) workload and no --splits", file=sys.stderr)
            sys.exit(2)
        from flashattention_forward_fwd_amd.inputs import random_dout
        do = random_dout(w.B, w.H, w.Lq, w.d, w.dtype, seed=w.seed)
        ddo = do.cuda()
        if drop_info is not None:
            f16("fa2_fwd_dropout")(*(args_common + drop_args + (stream.cuda_stream,)))
        else:
            (fa.fa2_fwd_f16 if w.dtype == "fp16" else fa.fa2_fwd)(*(args_common + (stream.cuda_stream,)))
        gq, gk, gv = torch.empty_like(dq), torch.empty_like(dk), torch.empty_like(dv)
        ws_bytes = fa.fa2_bwd_workspace_bytes(w.B, w.H, w.Lq)
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
        fn = fa.fa2_bwd_f16 if w.dtype == "fp16" else fa.fa2_bwd
        call = (dq, dk, dv, o, lse, ddo, gq, gk, gv, w.B, w.H, w.Lq, w.Lk, w.d, w.scale, int(w.causal),
                workspace, ws_bytes, stream.cuda_stream)
        if drop_info is not None:
            fn = f16("fa2_bwd_dropout")
            call = call[:16] + drop_args + call[16:]
        bwd_info = {"timed_call": "fa2_bwd = prep + dK/dV + dQ kernels", "workspace_bytes": ws_bytes,
                    "flops_count": "2.5x forward (S, dP, dV, dK, dQ); the dQ pass recomputes S and dP, "
                                   "so the device executes 3.5x"}
    elif drop_info is not None:
        fn = f16("fa2_fwd_dropout")
        call = args_common + drop_args + (stream.cuda_stream,)
    elif args.splits is None:
        fn = {"bf16": fa.fa2_fwd, "fp16": fa.fa2_fwd_f16, "fp32": fa.fa2_fwd_f32}[w.dtype]
        call = args_common + (stream.cuda_stream,)
    else:
        if w.dtype not in ("bf16", "fp16"):
            print("bench.py: the split-KV path takes bf16 (or --fp16) workloads", file=sys.stderr)
            sys.exit(2)
        S = args.splits or fa.fa2_splitkv_num_splits(w.B, w.H, w.Lq, w.Lk, w.d, int(w.causal))
        ws_bytes = fa.fa2_splitkv_workspace_bytes(w.B, w.H, w.Lq, w.Lk, w.d, int(w.causal), S)
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
        fn = f16("fa2_fwd_splitkv")
        call = args_common + (S, workspace, ws_bytes, stream.cuda_stream)
        split_info = {"num_splits": S, "requested": args.splits, "workspace_bytes": ws_bytes,
                      "timed_call": "fa2_fwd_splitkv = partial kernel + merge kernel"}

    K = args.steps
    # events made before the warm-up, so nothing but a synchronisation separates it
    # from the timed launches (an idle GPU lowers its clock within milliseconds)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    warm_launches, warm_s, warm_settled = warm_up(fn, call, stream, args.warmup)

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(K):
        ev[i][0].record(stream)
        fn(*call)
        ev[i][1].record(stream)
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = start.elapsed_time(stop) / K
    launch_ms = [a.elapsed_time(b) for a, b in ev]
    avg_launch_ms = sum(launch_ms) / K
    med_launch_ms = sorted(launch_ms)[K // 2] if K % 2 else 0.5 * sum(sorted(launch_ms)[K // 2 - 1:K // 2 + 1])

    flops = flops_override if flops_override is not None else w.flops * (2.5 if bwd_info else 1.0)
    value = flops / (ms_step * 1e-3) / 1e12
    # dense fp16 MFMA has the same published peak as bf16 on MI355X
    peak = PEAK_FP32_MFMA_TFLOPS if w.dtype == "fp32" else PEAK_BF16_TFLOPS
    traffic = (stored_traffic(w.name) if split_info is None and bwd_info is None and win_info is None
               and drop_info is None and not args.fp16 else None)
    algo_bytes = (4 if w.dtype == "fp32" else 2) * w.B * w.H * (2 * w.Lq + 2 * w.Lk) * w.d + 4 * w.B * w.H * w.Lq
    if bwd_info:
        # reads q, k, v, o, dout, lse; writes dq, dk, dv
        algo_bytes = 2 * w.B * w.H * (3 * w.Lq + 2 * w.Lk) * w.d + 4 * w.B * w.H * w.Lq \
            + 2 * w.B * w.H * (w.Lq + 2 * w.Lk) * w.d
    # Bound by whichever roof is lower at this arithmetic intensity.
    if flops / algo_bytes >= (peak * 1e12) / (PEAK_HBM_GBS * 1e9):
        roof = {"bound": "mfma", "achieved": round(flops / (avg_launch_ms * 1e-3) / 1e12, 2), "peak": peak,
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": round(algo_bytes / (avg_launch_ms * 1e-3) / 1e9, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof.update({"traffic": traffic, "avg_launch_ms": round(avg_launch_ms, 5),
                 "median_launch_ms": round(med_launch_ms, 5), "min_launch_ms": round(min(launch_ms), 5),
                 "launch_timing": "HIP events on the launch stream around each of the K timed calls",
                 "l2_flushed": False,
                 "l2_note": "no cache flush between calls: consecutive calls find part of Q, K, V in the "
                            "256 MiB Infinity Cache, as a model running attention back to back would"})
    # HBM bytes moved per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, committed summary)
    # over the kernel's average launch time, against the 8 TB/s HBM3E peak.
    if traffic is not None:
        roof["hbm_achieved_gbs"] = round(traffic / (avg_launch_ms * 1e-3) / 1e9, 1)
        roof["hbm_peak_gbs"] = PEAK_HBM_GBS
        roof["hbm_frac"] = round(roof["hbm_achieved_gbs"] / PEAK_HBM_GBS, 4)
        roof["traffic_over_algorithmic"] = round(traffic / algo_bytes, 3)
    if roof["bound"] == "mfma" and w.dtype != "fp32":
        roof["peak_derivation"] = device_peak()
    if args.flush_l2:
        # Cold-cache calls: Q, K and V come from HBM, not from the Infinity Cache.  The
        # flush reads (a sum over a 512 MiB buffer): it leaves clean lines, whose
        # eviction costs nothing, where a fill would leave dirty ones to write back
        # during the timed call.
        flush = torch.zeros(128 << 20, dtype=torch.float32, device="cuda")
        fev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
        for _ in range(3):      # the zero fill's dirty lines are written back here, untimed
            flush.sum()
            fn(*call)
        torch.cuda.synchronize()
        for i in range(K):
            flush.sum()
            fev[i][0].record(stream)
            fn(*call)
            fev[i][1].record(stream)
        torch.cuda.synchronize()
        fms = sorted(a.elapsed_time(b) for a, b in fev)
        favg = sum(fms) / K
        roof["l2_flushed_avg_launch_ms"] = round(favg, 5)
        roof["l2_flushed_median_launch_ms"] = round(fms[K // 2] if K % 2 else 0.5 * (fms[K // 2 - 1] + fms[K // 2]), 5)
        if roof["bound"] == "mfma":
            roof["l2_flushed_frac"] = round(flops / (favg * 1e-3) / 1e12 / peak, 4)
        else:
            roof["l2_flushed_frac"] = round(algo_bytes / (favg * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
        roof["l2_flush"] = ("K further calls, each after a read of 512 MiB on the launch stream (more than "
                            "the 256 MiB Infinity Cache and the eight 4 MiB L2s); value and frac above "
                            "are the calls without it")
        del flush

    out = {
        "metric": METRIC_BWD if bwd_info else METRIC, "value": round(value, 2), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup, "warmup_launches_run": warm_launches,
        "warmup_s": round(warm_s, 3), "warmup_settled": warm_settled, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "Lq": w.Lq, "Lk": w.Lk, "d": w.d,
                   "causal": w.causal, "flops_per_step": flops, "algorithmic_bytes_per_step": algo_bytes,
                   "wall_s_timed_region": round(wall, 4), "parallelism": "single GPU"},
        "roofline": roof,
        "context_pages": CONTEXT,
    }
    plain = split_info is None and bwd_info is None and win_info is None and drop_info is None and not args.fp16
    counters = stored_counters(w.name) if plain else None
    if counters is not None:
        counters["measured_in_this_run"] = False
        counters["note"] = ("stored: rocprofv3 counters of the same kernel source on this workload, "
                            "from the committed summary; counter collection serialises dispatches, "
                            "so they are taken in a run of their own")
        out["counters_stored"] = counters
    if split_info is not None:
        out["config"]["split_kv"] = split_info
    if args.fp16:
        out["metric"] = out["metric"].replace("bf16", "fp16")
    if win_info is not None:
        out["config"]["window"] = win_info
        out["metric"] = "attention fwd TFLOPS (4·d per visible query-key pair) bf16, sliding window"
    if drop_info is not None:
        out["config"]["dropout"] = drop_info
        out["metric"] = out["metric"] + ", dropout"
    if bwd_info is not None:
        out["config"]["backward"] = bwd_info
        if not args.no_cpu_baseline and drop_info is None:
            out["cpu_baseline"] = cpu_baseline_bwd(w, q, k, v, do)
    elif not args.no_cpu_baseline and win_info is None and drop_info is None:
        n = args.cpu_rows_per_head if args.cpu_rows_per_head > 0 else w.Lq
        out["cpu_baseline"] = cpu_baseline(w, q, k, v, min(n, w.Lq))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
