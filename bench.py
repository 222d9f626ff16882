#!/usr/bin/env python3
"""Benchmark of the Q8_0 block contraction on one MI355X.

One step = one ``q8_qdot`` call (the whole path: Q8_0 operands -> int32 block
sums -> f32 block-scale epilogue -> C) on the decode workload M=1, N=14336,
K=4096 (FFN up-projection shape).  Inputs are seeded synthetic f32 drawn by
``synth`` and quantized on the GPU by the library's own ``q8_quantize``; R
distinct device copies of every operand are rotated so that no launch finds
its operands in the 256 MB last-level cache or the L2s: each step reads its
weights from HBM, as a decode step would.

Printed: one JSON line with the headline metric (weight GB/s of the M=1
matvec), the roofline of the dominant kernel (HBM), the batched M=512 qGEMM
as a second measured workload (int8 TOPS, MFMA and VALU rooflines), the
other workloads, entry points and the GPU quantizer timed briefly, and the
CPU oracle timed on this host on a bounded sample of the headline workload.
The GEMMs are timed last.
"""
from __future__ import annotations

import argparse
import gc
import json
import os
import platform
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, published
INT8_PEAK_TOPS = 5000.0          # MI355X dense int8 MFMA, published (5.0 POP/s)
# VALU f32 FMA lane-op rate: 256 CU x 4 SIMD x 32 lanes x 2.4 GHz, the published
# 157.3 TFLOP/s FP32 vector figure.  Plain v_fma_f32 (packed forms are not used)
# reaches it on this part: measured, a SIMD with two or more waves issuing
# independent wave64 FMAs completes one every 2.0-2.4 clocks.
VALU_LANE_OPS_PER_S = 256 * 4 * 32 * 2.4e9
EPILOGUE_VALU_OPS = 2            # f32 VALU ops per (i, j, block) in the MFMA epilogue
CACHE_DEFEAT_BYTES = 1 << 30     # rotate >= 1 GiB of distinct operand copies
KERNEL_NAMES = ("matvec", "qgemm_ksplit", "qgemm_staged", "qgemm_splitk")              # by q8_qdot_path
# Launches per timing window of the secondary figures (the other workloads,
# the variants, the shard shares, the quantizer): at least 50, so that the
# window's fixed cost (~1.5 us for the events and the first dispatch) stays
# near 1 % of the small kernels' figures; the headline takes --steps.
MIN_WINDOW = 50
KERNEL_SOURCES = ("matvec.hip", "qgemm_ksplit.hip", "qgemm.hip", "qgemm_splitk.hip")   # their csrc files


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=1, help="index into synth.WORKLOADS for the headline")
    ap.add_argument("--second", type=int, default=4, help="second measured workload (-1: none)")
    ap.add_argument("--others", default="0,2,3", help="other workloads timed briefly ('' for none)")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the qmma_t / Q5_0 / small-batch timings")
    ap.add_argument("--cpu-seconds", type=float, default=16.0, help="CPU oracle sample budget (0: skip)")
    ap.add_argument("--no-rotate", action="store_true", help="reuse one copy (cache-warm number)")
    ap.add_argument("--profile", action="store_true",
                    help="only launch the headline kernel (for rocprofv3 counter passes)")
    ap.add_argument("--shape", default="", metavar="M,N,K",
                    help="with --profile: launch this shape instead (generators and seeds of --workload)")
    ap.add_argument("--entry", default="qdot", choices=("qdot", "qmma", "q50"),
                    help="with --profile: the entry to launch (q50: Q5_0 weights)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="run a plain device copy of MIB MiB 10 times and exit (counter calibration)")
    return ap.parse_args()


class Operands:
    """R device copies of (A, AS, W, WS, C) for one workload, quantized on the GPU.

    ``kind``: "qdot" (W int8, WS [N, K/32]), "qdotws" (the same through the
    workspace entry), "qmma" (the same weights, scales stored [K/32, N]) or
    "q50" (W as Q5_0 blocks, 20 bytes per 32 values, seeded uniform codes;
    scales from the Q8_0 quantization of the weights).
    """

    def __init__(self, torch, q8, w: synth.Workload, rotate: bool, kind: str = "qdot"):
        self.w = w
        self.kind = kind
        dev = torch.device("cuda:0")
        a32, w32 = synth.workload_f32(w)
        Xa = torch.from_numpy(a32).to(dev)
        Xw = torch.from_numpy(w32).to(dev)
        A, AS = q8.q8_quantize(Xa)
        W, WS = q8.q8_quantize(Xw)
        del Xa, Xw
        if kind == "qmma":
            WS = WS.t().contiguous()
        elif kind == "q50":
            W = torch.from_numpy(synth.random_q50(w.N, w.K, 4000 + w.index)).to(dev)
        per_copy = A.numel() + AS.numel() * 4 + W.numel() + WS.numel() * 4 + w.M * w.N * 4
        self.R = max(1, -(-CACHE_DEFEAT_BYTES // per_copy)) if rotate else 1
        self.copies = []
        for r in range(self.R):
            if r == 0:
                cA, cAS, cW, cWS = A, AS, W, WS
            else:
                cA, cAS, cW, cWS = A.clone(), AS.clone(), W.clone(), WS.clone()
            C = torch.empty((w.M, w.N), dtype=torch.float32, device=dev)
            self.copies.append((cA, cAS, cW, cWS, C))
        torch.cuda.synchronize()
        self.weight_bytes = W.numel() + WS.numel() * 4
        self.act_bytes = A.numel() + AS.numel() * 4
        self.out_bytes = w.M * w.N * 4
        self.algo_bytes = self.weight_bytes + self.act_bytes + self.out_bytes
        self.int8_ops = 2 * w.M * w.N * w.K
        self.element_blocks = w.M * w.N * w.KB


def settle_copies(torch, ops: Operands, first: int):
    """Read every byte of every rotated copy once, with a plain torch reduction (max).

    Creating the copies leaves up to the last-level cache's size of them
    dirty in that cache; without this pass, the first timed launches would
    also pay for writing those lines back to HBM.  The copies are read in
    the order first, first + 1, ..., wrapping round, so the ones read last
    are those the warmup launches use (copies 0 .. first - 1): the timed
    launches, which start at copy `first`, find nothing of theirs cached.
    Not a step of the path: no library call is made.
    """
    R = len(ops.copies)
    acc = []
    for r in range(R):
        for t in ops.copies[(first + r) % R][:4]:
            acc.append(t.view(torch.uint8).max())
    torch.cuda.synchronize()
    del acc


_SPIN_CYCLES_PER_US = None


def hold_stream(torch, us: float):
    """Occupy the current stream with a spin kernel of about `us` microseconds.

    Enqueued right before the start event, it keeps the GPU busy while the
    host enqueues the timed launches, so the start event fires with the
    launches already queued: the events then bracket back-to-back kernels,
    not the host's latency to its first launch (several microseconds per
    ctypes call), which would otherwise be spread over the steps.  The spin
    rate (clock cycles per microsecond) is measured once with HIP events.
    """
    global _SPIN_CYCLES_PER_US
    if not hasattr(torch.cuda, "_sleep"):
        log("[bench] torch.cuda._sleep is missing: timed windows start without a held stream")
        return
    stream = torch.cuda.current_stream()
    if _SPIN_CYCLES_PER_US is None:
        cyc = 2_000_000
        torch.cuda._sleep(cyc // 10)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        torch.cuda._sleep(cyc)
        e1.record(stream)
        torch.cuda.synchronize()
        _SPIN_CYCLES_PER_US = cyc / max(e0.elapsed_time(e1) * 1e3, 1.0)
    torch.cuda._sleep(int(us * _SPIN_CYCLES_PER_US))


def time_launches(torch, q8, ops: Operands, steps: int, warmup: int):
    """Warm up, then time exactly `steps` launches between two HIP events.

    Launch k (warmup and timed alike, k = 0, 1, ...) reads rotated copy
    k mod R, so a timed launch never re-reads a copy a warmup launch just
    read unless there are fewer copies than launches.  The host's garbage
    collector is held off while launches are issued.  After the warmup the
    stream is drained (synchronize), then held by a spin kernel long enough
    for the host to enqueue every timed launch (1.5x the per-launch enqueue
    time the warmup showed, plus 100 us), so that the two events bracket K
    back-to-back kernels.
    """
    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream
    cps = ops.copies
    w = ops.w
    if ops.kind == "qdotws":
        wsb = q8.workspace(w.M, w.N, w.K, torch.device("cuda:0"))
        wsp, wsn = wsb.data_ptr(), wsb.numel()

        def raw(A, AS, W, WS, C, M, N, K, s):
            return q8.q8_qdot_ws_raw(A, AS, W, WS, C, M, N, K, wsp, wsn, s)
    else:
        raw = {"qdot": q8.q8_qdot_raw, "qmma": q8.q8_qmma_raw, "q50": q8.q8_q50_qdot_raw}[ops.kind]
    ptrs = [(a.data_ptr(), s.data_ptr(), b.data_ptr(), t.data_ptr(), c.data_ptr()) for a, s, b, t, c in cps]
    R = len(ptrs)
    settle_copies(torch, ops, warmup % R)
    gc.collect()
    gc.disable()
    try:
        tw = time.perf_counter()
        for k in range(warmup):
            st = raw(*ptrs[k % R], w.M, w.N, w.K, sptr)
            if st:
                raise RuntimeError("%s failed: %s" % (ops.kind, q8.q8_strerror(st)))
        enqueue_us = (time.perf_counter() - tw) * 1e6 / max(warmup, 1) if warmup else 50.0
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        hold_stream(torch, min(1.5 * enqueue_us * steps + 100.0, 50_000.0))
        t0 = time.perf_counter()
        start.record(stream)
        for k in range(warmup, warmup + steps):
            raw(*ptrs[k % R], w.M, w.N, w.K, sptr)
        end.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    finally:
        gc.enable()
    ms = start.elapsed_time(end)
    return ms / steps, wall


def time_quantize(torch, q8, rows: int, K: int, steps: int, warmup: int, rotate: bool):
    """q8_quantize of seeded N(0, 1) f32 rows: X f32 [rows, K] -> Q int8, D f32.

    Algorithmic bytes per launch: 4 per value read, 1 per value + 4 per 32
    values written.  R distinct copies of X (and outputs) rotate so that X
    comes from HBM.
    """
    dev = torch.device("cuda:0")
    X = torch.from_numpy(synth.random_f32((rows, K), 6000 + rows)).to(dev)
    per = rows * K * 4 + rows * K + rows * (K // 32) * 4
    R = max(1, -(-CACHE_DEFEAT_BYTES // per)) if rotate else 1
    bufs = []
    for r in range(R):
        x = X if r == 0 else X.clone()
        bufs.append((x, torch.empty((rows, K), dtype=torch.int8, device=dev),
                     torch.empty((rows, K // 32), dtype=torch.float32, device=dev)))
    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream
    ptrs = [(x.data_ptr(), q.data_ptr(), d.data_ptr()) for x, q, d in bufs]
    tw = time.perf_counter()
    for k in range(warmup):
        st = q8.q8_quantize_raw(*ptrs[k % R], rows, K, sptr)
        if st:
            raise RuntimeError("q8_quantize failed: %s" % q8.q8_strerror(st))
    enqueue_us = (time.perf_counter() - tw) * 1e6 / max(warmup, 1) if warmup else 50.0
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    hold_stream(torch, min(1.5 * enqueue_us * steps + 100.0, 50_000.0))
    start.record(stream)
    for k in range(steps):
        q8.q8_quantize_raw(*ptrs[k % R], rows, K, sptr)
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    gbs = per / (ms * 1e-3) / 1e9
    del bufs
    return {"entry": "q8_quantize", "rows": rows, "K": K, "us_per_launch": round(ms * 1e3, 3),
            "bytes": per, "hbm_gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
            "rotated_copies": R}


def kernel_source_sha(path: str) -> str:
    """SHA-256 of the sources a kernel is built from (ties counters to code)."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gemm_q8_qdot_amd", "csrc")
    for name in (path, "q8_device.h"):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, source: str):
    """HBM bytes per launch from the committed counter record, or None.

    profiles/traffic.json holds FETCH_SIZE and WRITE_SIZE per dispatch for a
    workload, each scaled by the factor the same counter gives on a plain
    copy of known size, with the hash of the kernel source they were taken
    on; a changed kernel makes the record stale (None).
    """
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("kernel_source_sha") != kernel_source_sha(source):
        return None
    return int(rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"])


def copy_calibration(torch, mib: int):
    """A plain device copy of known size, for scaling FETCH_SIZE/WRITE_SIZE."""
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(10):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_each_way": n * 4, "launches": 10}), flush=True)


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor()


def _time_oracle(fn, budget_s: float, min_runs: int = 3):
    """Median seconds of repeated calls of fn, for about budget_s (at least min_runs)."""
    times = []
    t_all = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        fn()
        times.append(time.perf_counter() - t0)
        if len(times) >= min_runs and time.perf_counter() - t_all >= budget_s:
            break
    return statistics.median(times), len(times), sum(times)


def cpu_baseline(ops_w: synth.Workload, gemm_w, budget_s: float):
    """The oracle as it stands, on this host, on bounded samples of the workloads.

    Headline: full passes of the decode workload on all the oracle's threads
    (the reported value) and on one thread.  GEMM: the first rows of the
    prompt-size workload against the whole weight, on all threads, in int8
    TOPS.  Quantization is outside every timed call.
    """
    import oracle
    a32, w32 = synth.workload_f32(ops_w)
    A, AS = oracle.quantize_rows(a32)
    W, WS = oracle.quantize_rows(w32)
    del a32, w32
    threads = oracle.num_threads()
    wbytes = W.nbytes + WS.nbytes
    per, n, tot = _time_oracle(lambda: oracle.qdot_f64(A, AS, W, WS), 0.45 * budget_s)
    rec = {
        "value": round(wbytes / per / 1e9, 3),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": "%d full passes of %s (M=%d N=%d K=%d), median %.2f ms each, %.1f s total; "
                  "host %s, %d CPUs in affinity; oracle built with '%s'"
                  % (n, ops_w.name, ops_w.M, ops_w.N, ops_w.K, per * 1e3, tot, _cpu_model(),
                     len(os.sched_getaffinity(0)), oracle.BUILD_FLAGS),
    }
    oracle.set_num_threads(1)
    try:
        per1, n1, tot1 = _time_oracle(lambda: oracle.qdot_f64(A, AS, W, WS), 0.2 * budget_s)
    finally:
        oracle.set_num_threads(threads)
    rec["one_thread"] = {"value": round(wbytes / per1 / 1e9, 3), "unit": "GB/s", "cores": 1,
                         "sample": "%d full passes of %s, median %.1f ms each, %.1f s total"
                                   % (n1, ops_w.name, per1 * 1e3, tot1)}
    del A, AS, W, WS
    if gemm_w is not None:
        a32, w32 = synth.workload_f32(gemm_w)
        rows = min(gemm_w.M, 32)
        A, AS = oracle.quantize_rows(a32[:rows])
        W, WS = oracle.quantize_rows(w32)
        del a32, w32
        perg, ng, totg = _time_oracle(lambda: oracle.qdot_f64(A, AS, W, WS), 0.35 * budget_s)
        ops = 2.0 * rows * gemm_w.N * gemm_w.K
        rec["gemm"] = {"value": round(ops / perg / 1e12, 4), "unit": "int8 TOPS", "cores": threads,
                       "sample": "%d passes over the first %d of %d activation rows of %s "
                                 "(N=%d K=%d), median %.1f ms each, %.1f s total"
                                 % (ng, rows, gemm_w.M, gemm_w.name, gemm_w.N, gemm_w.K,
                                    perg * 1e3, totg)}
    return rec


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(--gpus %d requested)." % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import gemm_q8_qdot_amd as q8

    if not torch.cuda.is_available():
        print("bench.py needs a visible gfx950 GPU", file=sys.stderr)
        sys.exit(1)
    q8.ensure_built()
    q8.load()
    if args.copy_calibration:
        copy_calibration(torch, args.copy_calibration)
        return
    if args.profile:
        args.second = -1
        args.others = ""
        args.cpu_seconds = 0
        args.steps = min(args.steps, 50)
        args.warmup = min(args.warmup, 5)

    head_w = synth.WORKLOADS[args.workload]
    if args.shape:
        if not args.profile:
            sys.exit("bench.py: --shape is for --profile runs only (the headline is a listed workload)")
        M, N, K = (int(x) for x in args.shape.split(","))
        head_w = synth.Workload(head_w.index, "q8_shape_m%d_n%d_k%d" % (M, N, K), M, N, K, head_w.outliers)
    if args.entry != "qdot" and not args.profile:
        sys.exit("bench.py: --entry is for --profile runs only (the headline is q8_qdot)")
    log("[bench] preparing %s" % head_w.name)
    head = Operands(torch, q8, head_w, rotate=not args.no_rotate, kind=args.entry)
    log("[bench] %s: %d rotated copies; timing %d steps after %d warmup"
        % (head_w.name, head.R, args.steps, args.warmup))
    ms, wall = time_launches(torch, q8, head, args.steps, args.warmup)
    achieved = head.algo_bytes / (ms * 1e-3) / 1e9
    weight_gbs = head.weight_bytes / (ms * 1e-3) / 1e9
    path = q8.q8_qdot_path(head_w.M, head_w.N, head_w.K)
    source = KERNEL_SOURCES[path]
    traffic = measured_traffic(head_w.name, source)
    dtype = "i8xi8->i32, f32 scales"
    result = {
        "metric": "Q8_0 matvec weight GB/s (M=1)",
        "value": round(weight_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) activations, Q8_0-quantized on GPU)",
        "config": {"workload": head_w.name, "M": head_w.M, "N": head_w.N, "K": head_w.K,
                   "kernel": KERNEL_NAMES[path],
                   "rotated_copies": head.R, "arith": dtype},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "algorithmic_bytes_per_launch": head.algo_bytes,
                     "kernel_us": round(ms * 1e3, 3)},
    }
    log("[bench] headline %.3f us/launch, %.1f GB/s weights, %.1f GB/s total (%.1f%% of HBM)"
        % (ms * 1e3, weight_gbs, achieved, 100 * achieved / HBM_PEAK_GBS))
    del head
    torch.cuda.empty_cache()
    if not args.profile and not args.no_rotate:
        # The same launches on one copy read over and over: after the first
        # launch the operands come from the 256 MB last-level cache.  A
        # cache-warm figure, for context only (never the headline).
        warm = Operands(torch, q8, head_w, rotate=False)
        msw, _ = time_launches(torch, q8, warm, args.steps, args.warmup)
        result["cache_warm"] = {"us_per_launch": round(msw * 1e3, 3),
                                "gbs": round(warm.algo_bytes / (msw * 1e-3) / 1e9, 1),
                                "note": "one operand copy re-read by every launch (served from the "
                                        "last-level cache); context only"}
        log("[bench] headline cache-warm: %.3f us/launch" % (msw * 1e3))
        del warm
        torch.cuda.empty_cache()

    # The small workloads, before the GEMMs.
    others = [int(x) for x in args.others.split(",") if x.strip() != ""]
    if others:
        result["others"] = []
    for idx in others:
        ow = synth.WORKLOADS[idx]
        ops = Operands(torch, q8, ow, rotate=not args.no_rotate)
        ms3, _ = time_launches(torch, q8, ops, max(MIN_WINDOW, args.steps // 4), max(3, args.warmup // 4))
        rec = {"workload": ow.name, "M": ow.M, "N": ow.N, "K": ow.K,
               "kernel": KERNEL_NAMES[q8.q8_qdot_path(ow.M, ow.N, ow.K)],
               "us_per_launch": round(ms3 * 1e3, 3),
               "hbm_gbs": round(ops.algo_bytes / (ms3 * 1e-3) / 1e9, 1),
               "hbm_frac": round(ops.algo_bytes / (ms3 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
               "int8_tops": round(ops.int8_ops / (ms3 * 1e-3) / 1e12, 2)}
        result["others"].append(rec)
        log("[bench] %s: %.3f us/launch, %.1f GB/s (%.1f%% HBM), %.1f int8 TOPS"
            % (ow.name, rec["us_per_launch"], rec["hbm_gbs"], 100 * rec["hbm_frac"], rec["int8_tops"]))
        del ops
        torch.cuda.empty_cache()

    # One GPU's share of an 8-way split: the kernel at the shape each GPU
    # would run (N split: a slab of weight rows; K split: 1/8 of the blocks,
    # whose f32 partial outputs an all-reduce would sum).  No collective is
    # timed; same generators, seeds of the full workload, fewer rows or k.
    shares = [] if (args.no_variants or args.profile) else [
        ("N/8", synth.WORKLOADS[1], synth.Workload(1, "q8_matvec_m1_n1792_k4096", 1, 1792, 4096, False)),
        ("K/8", synth.WORKLOADS[2], synth.Workload(2, "q8_matvec_m1_n4096_k1792_outliers", 1, 4096, 1792, True)),
        ("N/8", synth.WORKLOADS[3], synth.Workload(3, "q8_qgemm_m64_n512_k4096", 64, 512, 4096, False)),
        ("N/8", synth.WORKLOADS[4], synth.Workload(4, "q8_qgemm_m512_n1792_k4096", 512, 1792, 4096, False)),
    ]
    if shares:
        result["shard_share"] = []
    for split, full, sw_ in shares:
        ops = Operands(torch, q8, sw_, rotate=not args.no_rotate)
        ms3, _ = time_launches(torch, q8, ops, max(MIN_WINDOW, args.steps // 4), max(3, args.warmup // 4))
        rec = {"split": split, "of": full.name, "workload": sw_.name, "M": sw_.M, "N": sw_.N, "K": sw_.K,
               "kernel": KERNEL_NAMES[q8.q8_qdot_path(sw_.M, sw_.N, sw_.K)],
               "us_per_launch": round(ms3 * 1e3, 3),
               "hbm_gbs": round(ops.algo_bytes / (ms3 * 1e-3) / 1e9, 1),
               "hbm_frac": round(ops.algo_bytes / (ms3 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
               "int8_tops": round(ops.int8_ops / (ms3 * 1e-3) / 1e12, 2)}
        result["shard_share"].append(rec)
        log("[bench] %s share of %s (%s): %.3f us/launch, %.1f GB/s (%.1f%% HBM), %.1f int8 TOPS"
            % (split, full.name, sw_.name, rec["us_per_launch"], rec["hbm_gbs"], 100 * rec["hbm_frac"],
               rec["int8_tops"]))
        del ops
        torch.cuda.empty_cache()

    # The other entry points and dispatch paths, on the same workload shapes:
    # qmma_t (transposed scales), Q5_0 weights, and a small decode batch.
    # The qmma_t GEMM is timed with the other GEMM, last.
    variants = [] if (args.no_variants or args.profile) else [
        ("qmma", synth.WORKLOADS[1]),
        ("q50", synth.WORKLOADS[1]), ("q50", synth.WORKLOADS[2]), ("q50", synth.WORKLOADS[3]),
        ("qdot", synth.Workload(1, "q8_batch_m4_n14336_k4096", 4, 14336, 4096, False)),
        ("q50", synth.Workload(1, "q8_batch_m4_n14336_k4096", 4, 14336, 4096, False)),
        # the long-contraction weights against a 32-row batch: the one-tile
        # GEMM, then the split form of the workspace entry
        ("qdot", synth.Workload(2, "q8_qgemm_m32_n4096_k14336_outliers", 32, 4096, 14336, True)),
        ("qdotws", synth.Workload(2, "q8_qgemm_m32_n4096_k14336_outliers", 32, 4096, 14336, True)),
    ]
    # Last, the GEMMs: qmma_t on the prompt workload, Q5_0 weights on it (the
    # 64 x 64-tile ring GEMM, decoding in LDS), and a medium prompt
    # projection on that kernel's two-workgroups-per-unit form.
    late_variants = [] if (args.no_variants or args.profile) else [
        ("qmma", synth.WORKLOADS[4]),
        ("q50", synth.WORKLOADS[4]),
        ("qdot", synth.Workload(4, "q8_qgemm_m512_n4096_k4096", 512, 4096, 4096, False)),
    ]
    if variants or late_variants:
        result["variants"] = []

    def time_variants(todo):
        for kind, vw in todo:
            ops = Operands(torch, q8, vw, rotate=not args.no_rotate, kind=kind)
            ms3, _ = time_launches(torch, q8, ops, max(MIN_WINDOW, args.steps // 4), max(3, args.warmup // 4))
            rec = {"entry": {"qdot": "q8_qdot", "qmma": "q8_qmma", "q50": "q8_q50_qdot",
                             "qdotws": "q8_qdot_ws"}[kind],
                   "workload": vw.name, "M": vw.M, "N": vw.N, "K": vw.K,
                   "us_per_launch": round(ms3 * 1e3, 3),
                   "weight_bytes": ops.weight_bytes,
                   "hbm_gbs": round(ops.algo_bytes / (ms3 * 1e-3) / 1e9, 1),
                   "hbm_frac": round(ops.algo_bytes / (ms3 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                   "int8_tops": round(ops.int8_ops / (ms3 * 1e-3) / 1e12, 2)}
            result["variants"].append(rec)
            log("[bench] %s %s: %.3f us/launch, %.1f GB/s (%.1f%% HBM), %.1f int8 TOPS"
                % (rec["entry"], vw.name, rec["us_per_launch"], rec["hbm_gbs"], 100 * rec["hbm_frac"],
                   rec["int8_tops"]))
            del ops
            torch.cuda.empty_cache()

    time_variants(variants)

    # The GPU Q8_0 quantizer (the step that makes A and AS): the prompt's
    # activation rows and a whole weight, f32 in, int8 + f32 scales out.
    quant = [] if (args.no_variants or args.profile) else [(512, 4096), (14336, 4096)]
    if quant:
        result["quantize"] = []
    for rows, K in quant:
        rec = time_quantize(torch, q8, rows, K, max(MIN_WINDOW, args.steps // 4), max(3, args.warmup // 4),
                            rotate=not args.no_rotate)
        result["quantize"].append(rec)
        log("[bench] q8_quantize %dx%d: %.3f us/launch, %.1f GB/s (%.1f%% HBM)"
            % (rows, K, rec["us_per_launch"], rec["hbm_gbs"], 100 * rec["hbm_frac"]))
        torch.cuda.empty_cache()

    # The GEMMs last.
    if args.second >= 0:
        sw = synth.WORKLOADS[args.second]
        log("[bench] preparing %s" % sw.name)
        sec = Operands(torch, q8, sw, rotate=not args.no_rotate)
        steps2 = max(10, args.steps // 4)
        ms2, _ = time_launches(torch, q8, sec, steps2, max(3, args.warmup // 4))
        # and sustained: a long run of back-to-back launches (the clock
        # settles lower under the epilogue's load)
        steps_sus = max(60, args.steps // 2)
        ms_sus, _ = time_launches(torch, q8, sec, steps_sus, 0)
        tops = sec.int8_ops / (ms2 * 1e-3) / 1e12
        valu_floor_us = sec.element_blocks * EPILOGUE_VALU_OPS / VALU_LANE_OPS_PER_S * 1e6
        hbm_gbs = sec.algo_bytes / (ms2 * 1e-3) / 1e9
        result["second"] = {
            "workload": sw.name, "M": sw.M, "N": sw.N, "K": sw.K, "steps": steps2,
            "us_per_launch": round(ms2 * 1e3, 3),
            "int8_tops": round(tops, 2),
            "roofline_mfma": {"bound": "mfma", "achieved": round(tops, 2), "peak": INT8_PEAK_TOPS,
                              "unit": "TOPS", "frac": round(tops / INT8_PEAK_TOPS, 4)},
            "valu_epilogue_floor_us": round(valu_floor_us, 2),
            "valu_floor_frac": round(valu_floor_us / (ms2 * 1e3), 4),
            "hbm_gbs": round(hbm_gbs, 1), "hbm_frac": round(hbm_gbs / HBM_PEAK_GBS, 4),
            "rotated_copies": sec.R,
            "traffic": measured_traffic(sw.name, KERNEL_SOURCES[q8.q8_qdot_path(sw.M, sw.N, sw.K)]),
            "sustained": {"steps": steps_sus, "us_per_launch": round(ms_sus * 1e3, 3),
                          "int8_tops": round(sec.int8_ops / (ms_sus * 1e-3) / 1e12, 2),
                          "frac_int8_peak": round(sec.int8_ops / (ms_sus * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4),
                          "valu_floor_frac": round(valu_floor_us / (ms_sus * 1e3), 4)},
        }
        log("[bench] second %s: %.3f us/launch, %.1f int8 TOPS (%.1f%% of peak), VALU floor %.1f us; "
            "sustained over %d launches %.3f us"
            % (sw.name, ms2 * 1e3, tops, 100 * tops / INT8_PEAK_TOPS, valu_floor_us, steps_sus, ms_sus * 1e3))
        del sec
        torch.cuda.empty_cache()

    time_variants(late_variants)

    if args.cpu_seconds > 0:
        log("[bench] CPU oracle baseline (~%.0f s)" % args.cpu_seconds)
        gemm_w = synth.WORKLOADS[args.second] if args.second >= 0 else None
        result["cpu_baseline"] = cpu_baseline(head_w, gemm_w, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
