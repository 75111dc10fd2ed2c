#!/usr/bin/env python3
"""Decode-step benchmark on one MI355X.

A step is the whole hot path for one batch: the per-step schedule (64-token
tiles spread evenly over the persistent grid), the decode kernel, and the
log-sum-exp merge of split sequences.  With --schedule device (default) the
decode kernel derives the schedule from the lengths on the GPU and writes one
merge record per (sequence, KV head) for the merge kernel that follows; with
--schedule host one native call per step runs the C++ planner on the host,
queues the plan's upload and launches the decode and merge kernels, which
read it.  Default workload: the skewed batch of one
131072-token sequence and 31 sequences of 4096 tokens, 8 query heads over one
KV head, head dim 128, bf16 KV in 64-token pages, shuffled block table
("vLLM x HPC-Ops ...", §Attention Decode under Mixed-Length Batches).

Inputs are resident in HBM before timing starts.  The KV cache is replicated
into several copies that successive steps rotate through, so that no step
finds its KV in the 256 MB Infinity Cache left behind by the previous one.

Prints one JSON line on stdout; progress goes to stderr.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

METRIC = "decode-attn µs/step & achieved HBM TB/s on 1×128K+31×4K mixed batch"
HBM_PEAK_GBPS = 8000.0
ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_kernel_traffic_skewed-1x128k+31x4k.json")
KERNEL_SOURCES = ("load_balanced_paged_step_amd/csrc/decode_kernels.hip",
                  "load_balanced_paged_step_amd/csrc/device_schedule.h")


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload_name: str, schedule: str, n_workers: int, entry_price: int = 0):
    """HBM bytes per decode launch from the committed counter summary, or None
    when it was taken for another configuration or an older kernel."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if (t.get("kernel_source_sha256") != kernel_source_hash() or t.get("workload") != workload_name
            or t.get("schedule") != schedule or t.get("n_workers") != n_workers
            or t.get("entry_price", 0) != entry_price):
        return None
    return t.get("hbm_bytes_per_launch")


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=4, help="workload number (1-5); 4 = 1x128K+31x4K")
    ap.add_argument("--n-workers", type=int, default=0,
                    help="persistent workgroups (0: the library's worker-count rule, hpc_decode_pick_workers, for "
                         "the step; one per CU for the sweeps)")
    ap.add_argument("--entry-price", type=int, default=-1,
                    help="the partition's price of a unit start in quarter tiles (-1: the library's rule, "
                         "hpc_decode_pick_entry_price, for the step's worker count)")
    ap.add_argument("--plan-in-place", action="store_true",
                    help="--schedule host: the kernels read the plan from the pinned host buffer (no upload)")
    ap.add_argument("--copies", type=int, default=0, help="rotating KV copies (0: enough for >= 1 GiB)")
    ap.add_argument("--cpu-baseline", choices=["on", "off"], default="on")
    ap.add_argument("--probe", choices=["on", "off"], nargs="?", const="on", default="on",
                    help="also measure the HBM streaming-read ceiling and a plain read of the step's bytes")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run the plain copy kernel over MIB MiB (hardware-counter calibration) and exit")
    ap.add_argument("--skew-sweep", action="store_true",
                    help="instead of the bench line: time the balanced schedule against static split-KV "
                         "schedules on batches from uniform 64x512 to 1x128K+31x4K, print one JSON line")
    ap.add_argument("--tile-math", choices=["mfma", "valu"], default="mfma",
                    help="tile arithmetic: matrix cores (default) or vector ALU dot2 products")
    ap.add_argument("--merge", choices=["rule", "kernel", "in-kernel"], default="rule",
                    help="device schedule: how split sequences are merged -- the library's rule "
                         "(hpc_decode_pick_merge), a separate merge kernel, or in the decode kernel by the worker "
                         "that finishes a split sequence last; the host schedule always uses the merge kernel")
    ap.add_argument("--fused-merge", action="store_true", help="the same as --merge in-kernel")
    ap.add_argument("--merge-sweep", action="store_true",
                    help="instead of the bench line: time the device-scheduled step with the merge kernel and "
                         "with the in-kernel merge on batches of 2 to 128 workers per unit, print one JSON line")
    ap.add_argument("--tile-math-sweep", action="store_true",
                    help="time the decode kernel with MFMA and with VALU tile math on workloads 2-5 "
                         "(device schedule) and print one JSON line")
    ap.add_argument("--prefill", nargs="?", const="all", default=None, metavar="WORKLOAD",
                    help="instead of the bench line: time causal prefill/extend attention on the prefill "
                         "workloads (all, or one by name) and print one JSON line")
    ap.add_argument("--prefill-group-sweep", action="store_true",
                    help="instead of the bench line: time causal extend attention at 1-16 query heads per KV head "
                         "on extend-8x512's contexts, print one JSON line")
    ap.add_argument("--prefill-workers", type=int, default=None, metavar="W",
                    help="with --prefill: time only the plan balanced over W workers (0: whole units)")
    ap.add_argument("--phase-trace", action="store_true",
                    help="instead of the bench line: per-worker phase durations of the decode kernel on --workload "
                         "from the tracing window's stamps, print one JSON line")
    ap.add_argument("--workers-sweep", action="store_true",
                    help="instead of the bench line: time the device-scheduled step at one and two workers per CU "
                         "and at hpc_decode_pick_workers' choice on batches of both KV dtypes, print one JSON line")
    ap.add_argument("--price-sweep", action="store_true",
                    help="instead of the bench line: time the device-scheduled step at entry prices 0, 2, 4, 8, 16 "
                         "at hpc_decode_pick_workers' count on the sweep batches, print one JSON line")
    ap.add_argument("--prologue", action="store_true",
                    help="instead of the bench line: time the fused prologue (QK-norm, RoPE, paged append) "
                         "alone and before the decode step on workloads 4 and 5, print one JSON line")
    ap.add_argument("--schedule", choices=["device", "host"], default="device",
                    help="device: kernels derive the per-step schedule from the lengths on the GPU; "
                         "host: C++ planner on the host + plan upload every step")
    return ap.parse_args()


def native_planner_us(seq_lens, num_kv_heads: int, n_workers: int, calls: int = 200, entry_price: int = 0) -> float:
    """Mean time of one hpc_decode_plan_priced call into a preallocated
    buffer, as hpc_decode_plan_attn makes it (no Python-side argument
    conversion)."""
    import ctypes
    import numpy as np
    import load_balanced_paged_step_amd as hd
    from load_balanced_paged_step_amd import _lib
    i32p = ctypes.POINTER(ctypes.c_int32)
    lens = np.ascontiguousarray(seq_lens, dtype=np.int32).reshape(-1)
    cap = hd.hpc_decode_plan_size(lens.shape[0], num_kv_heads, n_workers)
    buf = np.empty(cap, dtype=np.int32)
    fn = _lib.lib().hpc_decode_plan_priced
    lp, bp, B = lens.ctypes.data_as(i32p), buf.ctypes.data_as(i32p), lens.shape[0]
    _lib.check(fn(lp, B, num_kv_heads, n_workers, entry_price, bp, cap), "hpc_decode_plan_priced")
    t0 = time.perf_counter()
    for _ in range(calls):
        fn(lp, B, num_kv_heads, n_workers, entry_price, bp, cap)
    return (time.perf_counter() - t0) / calls * 1e6


def plan_upload_us(seq_lens, num_kv_heads: int, n_workers: int, dev, copies: int = 200) -> float:
    """Mean time, on the stream, of one upload of this step's plan words from
    pinned host memory to the device: the copy the host-planned step queues
    before its kernels (hpc_decode_plan_attn without an in-place plan)."""
    import torch
    import load_balanced_paged_step_amd as hd
    words = hd.hpc_decode_plan(seq_lens, num_kv_heads, n_workers)
    host = torch.from_numpy(words.copy()).pin_memory()
    dst = torch.empty_like(host, device=dev)
    for _ in range(10):
        dst.copy_(host, non_blocking=True)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(copies):
        dst.copy_(host, non_blocking=True)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / copies * 1e3


def cpu_baseline(inp, alg_bytes: int):
    """The float64 oracle on the host cores, over the same workload (median of repeated runs)."""
    from oracle import decode_attention
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:   # threadpoolctl missing: report the affinity size
        threads = len(os.sched_getaffinity(0))
    args = (inp.q_bits(), inp.k_bits(), inp.v_bits(), inp.block_table.numpy(), inp.seq_lens.numpy())
    kw = dict(num_q_heads=inp.num_q_heads, num_kv_heads=inp.num_kv_heads, kv_format=inp.kv_dtype,
              sm_scale=inp.sm_scale, k_scale=inp.k_scale, v_scale=inp.v_scale)
    times = []
    t_start = time.perf_counter()
    while len(times) < 3 or (time.perf_counter() - t_start < 10.0 and len(times) < 30):
        t0 = time.perf_counter()
        decode_attention(*args, **kw)
        times.append(time.perf_counter() - t0)
    med = statistics.median(times)
    result = {"value": alg_bytes / med / 1e12, "unit": "TB/s", "cores": int(threads), "kind": "oracle",
              "sample": f"whole workload, {len(times)} runs of the float64 oracle, median {med:.3f} s/step",
              "s_per_step": med}
    try:   # the same oracle held to one BLAS thread
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            one = []
            t_start = time.perf_counter()
            while len(one) < 3 and (time.perf_counter() - t_start < 20.0 or not one):
                t0 = time.perf_counter()
                decode_attention(*args, **kw)
                one.append(time.perf_counter() - t0)
        m1 = statistics.median(one)
        result["single_thread"] = {"value": alg_bytes / m1 / 1e12, "s_per_step": m1, "runs": len(one)}
    except ImportError:
        pass
    return result


def main() -> int:
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): the decode path runs on a "
              "single GPU and has no multi-GPU mode", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import load_balanced_paged_step_amd as hd
    from workloads import WORKLOADS, workload_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    if args.calibrate_copy:
        nbytes = args.calibrate_copy << 20
        src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            hd.hpc_probe_copy(src, dst)
        torch.cuda.synchronize()
        log(f"copied {nbytes} bytes x 3 with the probe copy kernel")
        return 0
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(dev)
    cus = props.multi_processor_count
    W = args.n_workers or cus
    if args.skew_sweep:
        print(json.dumps(skew_sweep(dev, W, cus, args.steps, args.warmup)), flush=True)
        return 0
    if args.fused_merge:
        args.merge = "in-kernel"
    if args.merge == "in-kernel" and args.schedule != "device":
        print("--merge in-kernel needs the device schedule", file=sys.stderr)
        return 2
    if args.phase_trace:
        print(json.dumps(phase_trace(dev, cus, args.workload, args.n_workers, min(args.steps, 200), args.warmup,
                                     args.entry_price)), flush=True)
        return 0
    if args.price_sweep:
        print(json.dumps(price_sweep(dev, cus, args.steps, args.warmup)), flush=True)
        return 0
    if args.prefill_group_sweep:
        print(json.dumps(prefill_group_sweep(dev, cus, args.steps, args.warmup)), flush=True)
        return 0
    if args.merge_sweep:
        print(json.dumps(merge_sweep(dev, cus, args.steps, args.warmup)), flush=True)
        return 0
    if args.workers_sweep:
        print(json.dumps(workers_sweep(dev, cus, args.steps, args.warmup)), flush=True)
        return 0
    if args.tile_math_sweep:
        print(json.dumps(tile_math_sweep(dev, W, args.steps, args.warmup)), flush=True)
        return 0
    if args.prefill:
        print(json.dumps(prefill_bench(dev, cus, args.prefill, args.steps, args.warmup, args.prefill_workers)),
              flush=True)
        return 0
    if args.prologue:
        print(json.dumps(prologue_bench(dev, cus, W, args.steps, args.warmup)), flush=True)
        return 0
    wl = WORKLOADS[args.workload]

    log(f"building inputs for workload {args.workload} ({wl.name})")
    inp = workload_inputs(args.workload)
    kv_bytes_total = inp.k_cache.numel() * inp.k_cache.element_size() * 2
    copies = args.copies or max(1, min(16, math.ceil((1 << 30) / kv_bytes_total)))
    alg_bytes = inp.algorithmic_bytes()
    if args.n_workers:
        w_rule = "given (--n-workers)"
    else:
        # the library's worker-count rule: the count over [CUs / 2, CUs] whose
        # costliest worker (tiles plus an entry price) is cheapest, or two per
        # CU for an fp8 cache with dense entries
        W = hd.hpc_decode_pick_workers(inp.seq_lens, inp.num_kv_heads, inp.kv_dtype, cus)
        w_rule = (f"hpc_decode_pick_workers ({cus} CUs; hpc_decode_choose_workers over [{cus // 2}, {cus}], "
                  f"entry cost {hd.ENTRY_COST_TILES} tile, or {2 * cus} for fp8 with >= 1.5 entries per worker)")
    if args.entry_price >= 0:
        price, price_rule = args.entry_price, "given (--entry-price)"
    else:
        # the library's price rule for this W: the partition price (quarter
        # tiles per unit start) whose costliest worker prices lowest
        price = hd.hpc_decode_pick_entry_price(inp.seq_lens, inp.num_kv_heads, inp.kv_dtype, W)
        price_rule = (f"hpc_decode_pick_entry_price (prices 0, 2, 4, 8, 16; entry cost "
                      f"{0.5 if inp.kv_dtype == 'bf16' else 2.0} tiles on {inp.kv_dtype})")
    if args.schedule != "device":
        fused, merge_rule = False, "the host schedule merges in the merge kernel"
    elif args.merge == "rule":
        # the library's merge rule: in the decode kernel when no sequence-head
        # unit of this partition is shared by more than FUSED_MAX_SHARES workers
        fused = hd.hpc_decode_pick_merge(inp.seq_lens, inp.num_kv_heads, W, price)
        merge_rule = (f"hpc_decode_pick_merge (in the decode kernel when no unit is shared by more than "
                      f"{hd.FUSED_MAX_SHARES} workers)")
    else:
        fused, merge_rule = args.merge == "in-kernel", "given (--merge)"
    log(f"device {props.name}, {cus} CUs; W={W} ({w_rule}); entry price {price} ({price_rule}); "
        f"merge {'in the decode kernel' if fused else 'kernel'} ({merge_rule}); "
        f"KV {kv_bytes_total / 1e6:.1f} MB x {copies} copies; algorithmic bytes/step {alg_bytes}")

    q = inp.q.to(dev)
    bt = inp.block_table.to(dev)
    sl = inp.seq_lens.to(dev)
    k0 = inp.k_cache.to(dev)
    v0 = inp.v_cache.to(dev)
    ks = [k0] + [k0.clone() for _ in range(copies - 1)]
    vs = [v0] + [v0.clone() for _ in range(copies - 1)]
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=dev)
    lens_host = inp.seq_lens.numpy()
    scales = dict(sm_scale=inp.sm_scale, k_scale=inp.k_scale, v_scale=inp.v_scale)
    if args.schedule == "device":
        ws = torch.zeros(hd.hpc_decode_step_workspace_size(inp.batch, inp.num_q_heads, inp.num_kv_heads, W),
                         dtype=torch.uint8, device=dev)
        launchers = [hd.StepLauncher(q, ks[c], vs[c], bt, sl, out, lse, num_kv_heads=inp.num_kv_heads,
                                     n_workers=W, workspace=ws, tile_math=args.tile_math,
                                     fused_merge=fused, entry_price=price, **scales)
                     for c in range(copies)]

        def one_step(i: int) -> None:
            launchers[i % copies]()
    else:
        ws = torch.empty(hd.hpc_decode_plan_workspace_bound(inp.batch, inp.num_q_heads, inp.num_kv_heads, W),
                         dtype=torch.uint8, device=dev)
        planned = [hd.PlannedStepLauncher(q, ks[c], vs[c], bt, sl, out, lse, num_kv_heads=inp.num_kv_heads,
                                          n_workers=W, workspace=ws, in_place=args.plan_in_place,
                                          tile_math=args.tile_math, entry_price=price, **scales)
                   for c in range(copies)]
        lens_np = np.ascontiguousarray(lens_host, dtype=np.int32)

        def one_step(i: int) -> None:
            planned[i % copies](lens_np)

    clock_warmup(dev, cus, inputs=ks + vs)
    log(f"warmup {args.warmup} steps")
    for i in range(args.warmup):
        one_step(i)
    torch.cuda.synchronize()

    # timed region: K whole steps, bracketed by device synchronisation
    log(f"timed region: {args.steps} steps")
    s = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(s)
    t0 = time.perf_counter()
    for i in range(args.steps):
        one_step(i)
    ev1.record(s)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev_ms = ev0.elapsed_time(ev1)
    ms_per_step = max(wall * 1e3, ev_ms) / args.steps
    log(f"{ms_per_step * 1e3:.2f} us/step (host clock {wall / args.steps * 1e6:.2f}, stream events "
        f"{ev_ms / args.steps * 1e3:.2f})")

    # kernel durations: the same steps again with the library bracketing every
    # decode and merge launch by HIP events on the launch stream
    hd.hpc_decode_profile_start(args.steps)
    for i in range(args.steps):
        one_step(i)
    torch.cuda.synchronize()
    decode_ms, combine_ms, n_calls = hd.hpc_decode_profile_stop()
    decode_us = decode_ms / max(n_calls, 1) * 1e3
    combine_us = combine_ms / max(n_calls, 1) * 1e3

    # the native host planner alone, called as the one-call host step calls it
    # (preallocated buffers; part of every --schedule host step, overlapping
    # the previous step's kernels), and one upload of its plan; taken after the
    # timed steps, so the GPU does not idle between the warm-up and the timing
    plan_us = native_planner_us(lens_host, inp.num_kv_heads, W, calls=200, entry_price=price)
    upload_us = plan_upload_us(lens_host, inp.num_kv_heads, W, dev)
    log(f"decode kernel {decode_us:.2f} us, merge kernel {combine_us:.2f} us (HIP events, {n_calls} calls)")

    step_tbps = alg_bytes / (ms_per_step * 1e-3) / 1e12
    achieved_gbps = alg_bytes / (decode_us * 1e-6) / 1e9
    result = {
        "metric": METRIC,
        "value": round(step_tbps, 4),
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "us_per_step": round(ms_per_step * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": inp.kv_dtype if inp.kv_dtype == "bf16" else f"fp8-e4m3 KV, bf16 {args.tile_math.upper()}",
        "data": "synthetic (seeded N(0,1) Q/K/V, shuffled block table)",
        "config": {
            "workload": wl.name, "batch": inp.batch, "kv_lens": _lens_summary(lens_host),
            "num_q_heads": inp.num_q_heads, "num_kv_heads": inp.num_kv_heads, "head_dim": 128,
            "page_size": 64, "kv_dtype": inp.kv_dtype, "n_workers": W, "n_workers_from": w_rule,
            "entry_price": price, "entry_price_from": price_rule,
            "kv_copies": copies,
            "algorithmic_bytes": alg_bytes,
            "schedule": args.schedule + (", plan in place" if args.schedule == "host" and args.plan_in_place else ""),
            "parallelism": "single GPU", "tile_math": args.tile_math,
            "merge": "in the decode kernel" if fused else "separate kernel", "merge_from": merge_rule,
        },
        "step_clocks_us": {"host_clock": round(wall / args.steps * 1e6, 3),
                           "stream_events": round(ev_ms / args.steps * 1e3, 3)},
        "kernels": {"decode_us": round(decode_us, 3), "merge_us": round(combine_us, 3),
                    "plan_host_us": round(plan_us, 2), "plan_upload_us": round(upload_us, 2),
                    "timed_calls": n_calls},
        "roofline": {"bound": "hbm", "achieved": round(achieved_gbps, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": (measured_traffic(wl.name, args.schedule, W, price)
                                 if args.tile_math == "mfma" and not fused else None),
                     "kernel": "decode_kernel", "bytes_per_launch": alg_bytes,
                     "kernel_us_hip_events": round(decode_us, 3),
                     "duration_source": ("decode kernel alone: mean of HIP events stamped by each launch's "
                                         "dispatch (kernel start to end), on the launch stream, in a pass of "
                                         "the same steps right after the timed region"),
                     "step_frac": round(step_tbps * 1e3 / HBM_PEAK_GBPS, 4),
                     "step_frac_source": "whole step (decode + merge + gaps): algorithmic bytes / us_per_step"},
    }

    if args.probe == "on":
        nbytes = 1 << 30
        buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        buf.fill_(1)
        sink = torch.empty(4096, dtype=torch.float32, device=dev)
        best = 0.0
        for nwg in (cus * 2, cus * 4, cus * 16):
            for _ in range(3):
                hd.hpc_probe_read(buf, sink, nwg)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(10):
                hd.hpc_probe_read(buf, sink, nwg)
            e1.record()
            torch.cuda.synchronize()
            gbps = nbytes * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9
            best = max(best, gbps)
            log(f"read probe, {nwg} workgroups: {gbps:.0f} GB/s")
        # the same bytes as one decode step: a plain streaming read of exactly
        # the algorithmic bytes, rotating over disjoint chunks of the buffer
        # as the steps rotate over KV copies; each launch timed from its
        # dispatch to its end, like the decode kernel above
        n_same = min(alg_bytes, nbytes) // 16 * 16
        chunks = max(1, nbytes // n_same)
        same = {}
        for nwg in (cus, cus * 2, cus * 4):
            ts = []
            for i in range(40):
                c = i % chunks
                t = hd.hpc_probe_read_timed(buf[c * n_same:(c + 1) * n_same], sink, nwg)
                if i >= 10:
                    ts.append(t * 1e3)
            same[str(nwg)] = round(float(np.median(ts)), 3)
            log(f"read probe over {n_same} bytes, {nwg} workgroups: {same[str(nwg)]:.2f} us")
        result["probe"] = {"read_GBps": round(best, 1), "bytes": nbytes,
                           "same_bytes_us": same, "same_bytes": n_same,
                           "same_bytes_GBps": round(n_same / (min(same.values()) * 1e-6) / 1e9, 1)}

    if args.cpu_baseline == "on":
        log("timing the float64 oracle on the host (cpu_baseline)")
        result["cpu_baseline"] = cpu_baseline(inp, alg_bytes)
    print(json.dumps(result), flush=True)
    return 0


def clock_warmup(dev, cus: int, seconds: float = 0.2, inputs=()) -> None:
    """About `seconds` of streaming reads, so that nothing is timed while the
    GPU's clocks are still ramping up (set-up, outside every timed region).
    The reads go over `inputs` (device tensors, e.g. every rotating KV copy)
    when given, so that each is touched once before timing: the first decode
    step on a copy never read before ran 5-6 us slower than later ones."""
    import torch

    import load_balanced_paged_step_amd as hd
    bufs = [t for t in inputs if (t.numel() * t.element_size()) % 16 == 0 and t.numel() > 0]
    if not bufs:
        bufs = [torch.empty(256 << 20, dtype=torch.uint8, device=dev)]
    sink = torch.empty(cus * 4, dtype=torch.float32, device=dev)
    t_end = time.perf_counter() + seconds
    i = 0
    while time.perf_counter() < t_end or i < len(bufs):
        hd.hpc_probe_read(bufs[i % len(bufs)], sink, cus * 4)
        torch.cuda.synchronize()
        i += 1
    del bufs, sink


def tile_math_sweep(dev, W: int, steps: int, warmup: int) -> dict:
    """Decode-kernel time with the MFMA and with the VALU tile math, same
    inputs, same device-scheduled step, alternating rounds of the two so
    that clock or thermal drift hits both alike."""
    import numpy as np
    import torch

    import load_balanced_paged_step_amd as hd
    from workloads import WORKLOADS, workload_inputs

    clock_warmup(dev, torch.cuda.get_device_properties(dev).multi_processor_count)
    rows = []
    for cfg in (2, 3, 4, 5):
        inp = workload_inputs(cfg)
        kv_bytes = inp.k_cache.numel() * inp.k_cache.element_size() * 2
        copies = max(1, min(16, math.ceil((1 << 30) / kv_bytes)))
        q, bt, sl = inp.q.to(dev), inp.block_table.to(dev), inp.seq_lens.to(dev)
        k0, v0 = inp.k_cache.to(dev), inp.v_cache.to(dev)
        ks = [k0] + [k0.clone() for _ in range(copies - 1)]
        vs = [v0] + [v0.clone() for _ in range(copies - 1)]
        # every copy read once before timing (a copy's first step runs slower)
        clock_warmup(dev, torch.cuda.get_device_properties(dev).multi_processor_count, inputs=ks + vs)
        out = torch.empty_like(q)
        lse = torch.empty(q.shape[:2], dtype=torch.float32, device=dev)
        ws = torch.zeros(hd.hpc_decode_step_workspace_size(inp.batch, inp.num_q_heads, inp.num_kv_heads, W),
                         dtype=torch.uint8, device=dev)
        scales = dict(sm_scale=inp.sm_scale, k_scale=inp.k_scale, v_scale=inp.v_scale)
        launch = {m: [hd.StepLauncher(q, ks[c], vs[c], bt, sl, out, lse, num_kv_heads=inp.num_kv_heads,
                                      n_workers=W, workspace=ws, tile_math=m, **scales) for c in range(copies)]
                  for m in ("mfma", "valu")}
        alg = inp.algorithmic_bytes()
        times = {"mfma": [], "valu": []}
        for rnd in range(3):
            for m in ("mfma", "valu"):
                for i in range(warmup):
                    launch[m][i % copies]()
                torch.cuda.synchronize()
                hd.hpc_decode_profile_start(steps)
                for i in range(steps):
                    launch[m][i % copies]()
                torch.cuda.synchronize()
                d_ms, c_ms, n = hd.hpc_decode_profile_stop()
                times[m].append((d_ms / max(n, 1) * 1e3, c_ms / max(n, 1) * 1e3))
        row = {"workload": WORKLOADS[cfg].name, "kv_dtype": inp.kv_dtype,
               "heads": f"{inp.num_q_heads}q/{inp.num_kv_heads}kv", "algorithmic_bytes": alg}
        for m in ("mfma", "valu"):
            d = float(np.median([t[0] for t in times[m]]))
            c = float(np.median([t[1] for t in times[m]]))
            row[m] = {"decode_us": round(d, 3), "merge_us": round(c, 3),
                      "decode_GBps": round(alg / (d * 1e-6) / 1e9, 1),
                      "rounds_decode_us": [round(t[0], 3) for t in times[m]]}
        row["valu_over_mfma"] = round(row["valu"]["decode_us"] / row["mfma"]["decode_us"], 3)
        log(f"{row['workload']}: decode MFMA {row['mfma']['decode_us']:.2f} us, "
            f"VALU {row['valu']['decode_us']:.2f} us ({row['valu_over_mfma']:.3f}x)")
        rows.append(row)
        del launch, ks, vs
        torch.cuda.empty_cache()
    return {"mode": "tile-math-sweep", "n_workers": W, "steps": steps, "warmup": warmup,
            "schedule": "device", "timing": "decode kernel, dispatch-stamped HIP events, median of 3 rounds",
            "rows": rows}


MFMA_BF16_PEAK_TFLOPS = 2500.0


def _events_us(fn, steps: int, warmup: int, reps: int = 3) -> float:
    """Time per call of `fn`: the mean over `steps` back-to-back calls on the
    current stream, bracketed by events (after `warmup` calls), taken `reps`
    times; the median of those means (a single pass of a launch this short
    was seen to double now and then)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    means = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        means.append(e0.elapsed_time(e1) / steps * 1e3)
    return sorted(means)[len(means) // 2]


def _step_us(one_step, steps: int, warmup: int, reps: int = 3) -> float:
    """Time per step of `one_step(i)` (all of a step's launches): the mean
    over `steps` back-to-back steps between two events on the current stream,
    after `warmup` steps, taken `reps` times; the median.  No per-kernel
    events: bracketing every launch with events lengthens each kernel, so a
    step of two kernels would pay that twice and a step of one kernel once."""
    import torch
    for i in range(warmup):
        one_step(i)
    torch.cuda.synchronize()
    means = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(steps):
            one_step(i)
        e1.record()
        torch.cuda.synchronize()
        means.append(e0.elapsed_time(e1) / steps * 1e3)
    return sorted(means)[len(means) // 2]


def _blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:
        return len(os.sched_getaffinity(0))


def prefill_oracle_baseline(pi) -> dict:
    """The float64 prefill oracle on the host, on a bounded sample: the whole
    step when it holds one sequence, else its first sequence alone (queries
    and cache as they are); the rate is that sample's FLOPs / time."""
    import numpy as np
    from oracle import prefill_attention
    from workloads import PrefillInputs
    c = pi.cache
    qs = pi.q_start.numpy()
    if c.batch == 1:
        sample, desc = pi, "the whole step"
    else:
        sub = make_sub_prefill(pi, 0)
        sample, desc = sub, f"sequence 0 alone ({int(qs[1] - qs[0])} queries over {int(c.seq_lens[0])} tokens)"
    sc = sample.cache
    t0 = time.perf_counter()
    prefill_attention(sample.q_bits(), sc.k_bits(), sc.v_bits(), sc.block_table.numpy(), sc.seq_lens.numpy(),
                      sample.q_start.numpy(), num_q_heads=sc.num_q_heads, num_kv_heads=sc.num_kv_heads,
                      kv_format=sc.kv_dtype, sm_scale=sc.sm_scale, k_scale=sc.k_scale, v_scale=sc.v_scale)
    dt = time.perf_counter() - t0
    return {"value": sample.flops() / dt / 1e12, "unit": "TFLOP/s", "cores": _blas_threads(), "kind": "oracle",
            "sample": f"{desc}, one run of the float64 oracle, {dt:.2f} s"}


def make_sub_prefill(pi, b: int):
    """Sequence b of a prefill step as a one-sequence step (same cache tensors)."""
    import numpy as np
    import torch
    from dataclasses import replace
    from workloads import PrefillInputs
    c = pi.cache
    qs = pi.q_start.numpy()
    r0, r1 = int(qs[b]), int(qs[b + 1])
    sub_cache = replace(c, q=c.q[b:b + 1], block_table=c.block_table[b:b + 1], seq_lens=c.seq_lens[b:b + 1])
    return PrefillInputs(cache=sub_cache, q=pi.q[r0:r1], q_start=torch.tensor([0, r1 - r0], dtype=torch.int32))


def prefill_bench(dev, cus: int, which: str, steps: int, warmup: int, only_workers: int | None = None) -> dict:
    """Causal prefill / extend attention: mean kernel time over back-to-back
    launches (events on the launch stream; the work list is planned and
    uploaded once, outside the timing), algorithmic FLOPs (4 * 128 per query
    head and visible token) against the bf16 MFMA peak.  Each workload runs
    with whole units (n_workers = 0) and with balanced plans over 1, 2 and 4
    workers per CU; the roofline object is that of the balanced plan at 2
    workers per CU (two workgroups of one group fit a CU).  only_workers
    times that one plan alone (for profiler runs)."""
    import torch

    from load_balanced_paged_step_amd.prefill import PrefillStep, hpc_prefill_units
    from workloads import PREFILL_WORKLOADS, prefill_workload_inputs

    clock_warmup(dev, cus)
    names = list(PREFILL_WORKLOADS) if which == "all" else [which]
    rows = []
    W_default = 2 * cus if only_workers is None else only_workers
    sweep = (0, cus, 2 * cus, 4 * cus) if only_workers is None else (only_workers,)
    for name in names:
        pi = prefill_workload_inputs(name)
        c = pi.cache
        q, qs = pi.q.to(dev), pi.q_start.to(dev)
        k, v = c.k_cache.to(dev), c.v_cache.to(dev)
        bt, sl = c.block_table.to(dev), c.seq_lens.to(dev)
        out = torch.empty_like(q)
        lse = torch.empty(q.shape[:2], dtype=torch.float32, device=dev)
        flops = pi.flops()
        plans = {}
        for W in sweep:
            t0 = time.perf_counter()
            step = PrefillStep(pi.q_start, c.seq_lens, c.num_q_heads, c.num_kv_heads, c.max_pages_per_seq,
                               n_workers=W, device=dev)
            plan_us = (time.perf_counter() - t0) * 1e6
            one = step.bind(q, qs, k, v, bt, sl, out, lse, sm_scale=c.sm_scale, k_scale=c.k_scale,
                            v_scale=c.v_scale)
            us = _events_us(one, max(steps, 20), max(warmup, 5))
            plans[W] = {"n_workers": W, "entries": step.n_entries, "cut_units": step.n_merge,
                        "longest_entry_tiles": int(step.entries[:, 3].max()) if step.n_entries else 0,
                        "us": round(us, 3), "TFLOPs": round(flops / (us * 1e-6) / 1e12, 1),
                        "plan_and_upload_us": round(plan_us, 1)}
            del one, step
        main = plans[W_default]
        tflops = main["TFLOPs"]
        row = {"workload": name, "heads": f"{c.num_q_heads}q/{c.num_kv_heads}kv", "kv_dtype": c.kv_dtype,
               "queries": pi.total, "kv_lens": _lens_summary(c.seq_lens.numpy()),
               "units": hpc_prefill_units(pi.q_start, c.num_kv_heads), "flops": flops, "n_workers": W_default,
               "us": main["us"], "TFLOPs": tflops,
               "whole_units_us": plans[0]["us"] if 0 in plans else None,
               "balanced_speedup": round(plans[0]["us"] / main["us"], 3) if 0 in plans else None,
               "roofline": {"bound": "mfma", "achieved": tflops, "peak": MFMA_BF16_PEAK_TFLOPS,
                            "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4)},
               "plans": list(plans.values())}
        row["cpu_baseline"] = prefill_oracle_baseline(pi)
        log(f"prefill {name}: " + ", ".join(f"W={p['n_workers']} {p['us']:.2f} us ({p['entries']} entries)"
                                            for p in plans.values())
            + f"; {tflops:.1f} TFLOP/s at W={W_default} ({row['roofline']['frac']:.3f} of bf16 MFMA peak); "
            f"oracle {row['cpu_baseline']['value']:.4f} TFLOP/s")
        rows.append(row)
        del q, k, v, out, lse
        torch.cuda.empty_cache()
    return {"mode": "prefill", "timing": "mean of back-to-back launches, HIP events on the launch stream; median of three passes",
            "peak_note": "fp8 KV widens to bf16 in LDS; all products run on bf16 MFMA", "rows": rows}


def prologue_bench(dev, cus: int, W: int, steps: int, warmup: int) -> dict:
    """The fused prologue (QK-norm, RoPE, paged append of the new token) on
    the decode workloads' shapes: its mean time over back-to-back launches,
    its algorithmic bytes (new q/k/v read, q written, the new K/V rows
    written, norm weights), and the whole decode step with it in front
    (prologue + decode + merge, device schedule) against the step without."""
    import numpy as np
    import torch

    import load_balanced_paged_step_amd as hd
    from load_balanced_paged_step_amd.prologue import PrologueLauncher
    from workloads import WORKLOADS, make_prologue_inputs, workload_inputs

    clock_warmup(dev, cus)
    rows = []
    for cfg in (4, 5):
        base = workload_inputs(cfg)
        lens = base.seq_lens.numpy().astype(np.int64)
        pi = make_prologue_inputs(lens - 1, base.num_q_heads, base.num_kv_heads, base.kv_dtype, seed=cfg)
        c = pi.cache
        q_in, k_in, v_in = pi.q_in.to(dev), pi.k_in.to(dev), pi.v_in.to(dev)
        wq, wk = pi.q_norm_w.to(dev), pi.k_norm_w.to(dev)
        pos, bt, sl = pi.positions.to(dev), c.block_table.to(dev), c.seq_lens.to(dev)
        k, v = c.k_cache.to(dev), c.v_cache.to(dev)
        q_out = torch.empty_like(q_in)
        q_fp8 = torch.empty(q_in.shape, dtype=torch.float8_e4m3fn, device=dev) if c.kv_dtype != "bf16" else None

        pro = PrologueLauncher(q_in, k_in, v_in, wq, wk, pos, bt, k, v, q_out, q_fp8, eps=pi.eps, theta=pi.theta,
                               k_scale=c.k_scale, v_scale=c.v_scale, q_scale=pi.q_scale)
        ws = torch.zeros(hd.hpc_decode_step_workspace_size(c.batch, c.num_q_heads, c.num_kv_heads, W),
                         dtype=torch.uint8, device=dev)
        out = torch.empty_like(q_out)
        lse = torch.empty(q_out.shape[:2], dtype=torch.float32, device=dev)
        decode = hd.StepLauncher(q_out, k, v, bt, sl, out, lse, num_kv_heads=c.num_kv_heads, n_workers=W,
                                 workspace=ws, sm_scale=c.sm_scale, k_scale=c.k_scale, v_scale=c.v_scale)

        def both():
            pro()
            decode()
        B, Hq, Hkv = c.batch, c.num_q_heads, c.num_kv_heads
        kv_elem = 1 if c.kv_dtype != "bf16" else 2
        nbytes = (B * (Hq + 2 * Hkv) * 128 * 2 + 2 * 128 * 2 + B * 4 * 2 + B * Hq * 128 * 2
                  + (B * Hq * 128 if q_fp8 is not None else 0) + 2 * B * Hkv * 128 * kv_elem)
        n = max(steps, 50)
        pro_us = _events_us(pro, n, max(warmup, 10))
        dec_us = _events_us(decode, n, max(warmup, 10))
        both_us = _events_us(both, n, max(warmup, 10))
        row = {"workload": WORKLOADS[cfg].name, "heads": f"{Hq}q/{Hkv}kv", "kv_dtype": c.kv_dtype,
               "fp8_query": q_fp8 is not None, "prologue_us": round(pro_us, 3), "prologue_bytes": nbytes,
               "prologue_GBps": round(nbytes / (pro_us * 1e-6) / 1e9, 1),
               "roofline": {"bound": "latency", "achieved": round(nbytes / (pro_us * 1e-6) / 1e9, 1),
                            "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                            "frac": round(nbytes / (pro_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 5)},
               "decode_step_us": round(dec_us, 3), "prologue_plus_decode_step_us": round(both_us, 3)}
        from oracle import decode_prologue
        t0 = time.perf_counter()
        decode_prologue(pi.bits(pi.q_in), pi.bits(pi.k_in), pi.bits(pi.v_in), pi.bits(pi.q_norm_w),
                        pi.bits(pi.k_norm_w), pi.positions.numpy(), c.block_table.numpy(), c.k_bits(), c.v_bits(),
                        kv_format=c.kv_dtype, eps=pi.eps, theta=pi.theta, k_scale=c.k_scale, v_scale=c.v_scale,
                        q_scale=pi.q_scale if q_fp8 is not None else None)
        dt = time.perf_counter() - t0
        row["cpu_baseline"] = {"value": round(dt * 1e6, 1), "unit": "us per step", "cores": _blas_threads(),
                               "kind": "oracle", "sample": "the whole batch, one run of the float64 oracle (it "
                               "copies both caches, which dominates its time)"}
        log(f"prologue {row['workload']}: {pro_us:.2f} us ({nbytes} B); decode step {dec_us:.2f} us, "
            f"with prologue {both_us:.2f} us; oracle {dt * 1e3:.1f} ms")
        rows.append(row)
    return {"mode": "prologue", "n_workers": W,
            "timing": "mean of back-to-back launches, HIP events on the launch stream (KV resident, one copy); median of three passes",
            "rows": rows}


SKEW_BATCHES = (
    ("64x512", [512] * 64),
    ("32x4K", [4096] * 32),
    ("1x8K+31x4K", [8192] + [4096] * 31),
    ("1x16K+31x4K", [16384] + [4096] * 31),
    ("1x32K+31x4K", [32768] + [4096] * 31),
    ("1x64K+31x4K", [65536] + [4096] * 31),
    ("1x128K+31x4K", [131072] + [4096] * 31),
)
STATIC_SPLITS = (1, 2, 4, 8, 16, 32, 64, 128)


def skew_sweep(dev, W: int, cus: int, steps: int, warmup: int) -> dict:
    """Balanced step (device-scheduled, and from a prebuilt host plan) against
    static split-KV plans with S splits per sequence, on batches from uniform
    to one long sequence among short ones (8 query heads over one KV head,
    bf16).  Times are whole steps (all of a step's launches, gaps between
    kernels included), the mean over back-to-back steps between two events,
    median of three passes, KV rotated over >= 1 GiB of copies; host plans
    are built and uploaded once, outside the timing; ratio = static /
    balanced (device-scheduled), and static / balanced host plan (the same
    host-planned kernel as the static plans).  The device-scheduled step is
    also timed as the library's rules set it up (hpc_decode_pick_workers,
    hpc_decode_pick_entry_price, hpc_decode_pick_merge) where that differs.
    Every KV copy of a batch is read once before its first timing."""
    import torch

    import load_balanced_paged_step_amd as hd
    from workloads import make_inputs

    steps = min(steps, 50)
    clock_warmup(dev, cus)   # the first batch is not timed while clocks ramp up
    rows = []
    for name, lens in SKEW_BATCHES:
        inp = make_inputs(lens, 8, 1, "bf16", seed=4)
        kv_bytes = inp.k_cache.numel() * inp.k_cache.element_size() * 2
        copies = max(1, min(64, math.ceil((1 << 30) / kv_bytes)))
        q, bt, sl = inp.q.to(dev), inp.block_table.to(dev), inp.seq_lens.to(dev)
        ks = [inp.k_cache.to(dev) for _ in range(copies)]
        vs = [inp.v_cache.to(dev) for _ in range(copies)]
        clock_warmup(dev, cus, inputs=ks + vs)   # every copy read once before timing
        out = torch.empty_like(q)
        lse = torch.empty(q.shape[:2], dtype=torch.float32, device=dev)
        scales = dict(sm_scale=inp.sm_scale, k_scale=inp.k_scale, v_scale=inp.v_scale)

        def kernel_us(one_step) -> float:
            # small batches: let clocks and caches settle first
            return _step_us(one_step, steps, max(warmup, 20))

        ws = torch.zeros(hd.hpc_decode_step_workspace_size(inp.batch, 8, 1, W), dtype=torch.uint8, device=dev)
        launchers = [hd.StepLauncher(q, ks[c], vs[c], bt, sl, out, lse, num_kv_heads=1, n_workers=W,
                                     workspace=ws, **scales) for c in range(copies)]
        balanced = kernel_us(lambda i: launchers[i % copies]())
        lens_np = inp.seq_lens.numpy()
        # the device-scheduled step as the library's rules set it up: worker
        # count, entry price and merge mode (when that differs from the above)
        w_rule = hd.hpc_decode_pick_workers(lens_np, 1, "bf16", cus)
        price_rule = hd.hpc_decode_pick_entry_price(lens_np, 1, "bf16", w_rule)
        fused_rule = hd.hpc_decode_pick_merge(lens_np, 1, w_rule, price_rule)
        if w_rule == W and price_rule == 0 and not fused_rule:
            balanced_rule = balanced
        else:
            ws_r = torch.zeros(hd.hpc_decode_step_workspace_size(inp.batch, 8, 1, w_rule), dtype=torch.uint8,
                               device=dev)
            launchers_r = [hd.StepLauncher(q, ks[c], vs[c], bt, sl, out, lse, num_kv_heads=1, n_workers=w_rule,
                                           workspace=ws_r, entry_price=price_rule, fused_merge=fused_rule,
                                           **scales) for c in range(copies)]
            balanced_rule = kernel_us(lambda i: launchers_r[i % copies]())
            del launchers_r

        def planned_us(plan) -> float:
            """step time of a prebuilt host plan (uploaded once) through hpc_decode_attn, its arguments
            marshalled once per KV copy (AttnLauncher), as the device step's are (StepLauncher)"""
            plan_dev = torch.from_numpy(plan.copy()).to(dev)
            nb = hd.hpc_decode_workspace_size(plan, 8, 1)
            sws = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev) if nb > 0 else None
            ls = [hd.AttnLauncher(q, ks[c], vs[c], bt, sl, plan, plan_dev, sws, out, lse, num_kv_heads=1, **scales)
                  for c in range(copies)]
            return kernel_us(lambda i: ls[i % copies]())

        balanced_host = planned_us(hd.hpc_decode_plan(lens_np, 1, W))
        rule_S = hd.hpc_decode_static_splits(lens_np, 1, cus)
        static = {S: planned_us(hd.hpc_decode_plan_static(lens_np, 1, S))
                  for S in sorted(set(STATIC_SPLITS) | {rule_S})}
        best_S = min(static, key=static.get)
        row = {"batch": name, "balanced_us": round(balanced, 2), "balanced_host_plan_us": round(balanced_host, 2),
               "static_us": {str(S): round(t, 2) for S, t in static.items()},
               "rule_splits": rule_S, "ratio_rule": round(static[rule_S] / balanced, 3),
               "best_splits": best_S, "ratio_best": round(static[best_S] / balanced, 3),
               # the balanced plan through the same host-planned kernel the static plans run through
               "ratio_rule_host_plan": round(static[rule_S] / balanced_host, 3),
               "ratio_best_host_plan": round(static[best_S] / balanced_host, 3),
               "rules": {"n_workers": w_rule, "entry_price": price_rule,
                         "merge": "in the decode kernel" if fused_rule else "merge kernel"},
               "balanced_rules_us": round(balanced_rule, 2),
               "ratio_best_rules": round(static[best_S] / balanced_rule, 3)}
        log(f"skew sweep {name}: balanced {balanced:.1f} us (host-planned {balanced_host:.1f}); "
            f"static S={rule_S} (rule) "
            f"{static[rule_S]:.1f} us = {row['ratio_rule']}x; best static S={best_S} {static[best_S]:.1f} us "
            f"= {row['ratio_best']}x; host-planned balanced vs best static {row['ratio_best_host_plan']}x; "
            f"device-scheduled by the rules (W={w_rule}, price {price_rule}, "
            f"{'in-kernel merge' if fused_rule else 'merge kernel'}) {balanced_rule:.1f} us = "
            f"{row['ratio_best_rules']}x")
        rows.append(row)
        del ks, vs, launchers
        torch.cuda.empty_cache()
    return {"metric": "static split-KV / balanced schedule step time, uniform -> skewed batches",
            "unit": "ratio", "higher_is_better": True, "n_workers": W, "steps": steps, "warmup": warmup,
            "heads": "8 q / 1 kv, head dim 128, bf16 KV, page 64",
            "static_rule": "smallest power of two S with units x S >= CUs, S <= 128 and <= the longest unit's tiles",
            "rows": rows}


def phase_trace(dev, cus: int, cfg: int, n_workers: int, steps: int, warmup: int, entry_price: int = -1) -> dict:
    """Per-worker phases of the device-scheduled decode kernel from the
    tracing window's wall-clock stamps (100 MHz), over `steps` traced steps
    (KV rotated over >= 1 GiB of copies): entry -> first loads issued
    (schedule), entry -> first tile consumed (first data), first -> last tile
    consumed (steady state, per tile), last tile -> end (entry merges), entry
    -> end.  Medians and maxima over the workers of each step, then the
    median over steps; the traced launches' kernel time by events beside."""
    import numpy as np
    import torch

    import load_balanced_paged_step_amd as hd
    from workloads import WORKLOADS, workload_inputs

    inp = workload_inputs(cfg)
    W = n_workers or hd.hpc_decode_pick_workers(inp.seq_lens, inp.num_kv_heads, inp.kv_dtype, cus)
    price = (entry_price if entry_price >= 0
             else hd.hpc_decode_pick_entry_price(inp.seq_lens, inp.num_kv_heads, inp.kv_dtype, W))
    kv_bytes = inp.k_cache.numel() * inp.k_cache.element_size() * 2
    copies = max(1, min(16, math.ceil((1 << 30) / kv_bytes)))
    q, bt, sl = inp.q.to(dev), inp.block_table.to(dev), inp.seq_lens.to(dev)
    ks = [inp.k_cache.to(dev) for _ in range(copies)]
    vs = [inp.v_cache.to(dev) for _ in range(copies)]
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=dev)
    ws = torch.zeros(hd.hpc_decode_step_workspace_size(inp.batch, inp.num_q_heads, inp.num_kv_heads, W),
                     dtype=torch.uint8, device=dev)
    launchers = [hd.StepLauncher(q, ks[c], vs[c], bt, sl, out, lse, num_kv_heads=inp.num_kv_heads, n_workers=W,
                                 workspace=ws, sm_scale=inp.sm_scale, k_scale=inp.k_scale, v_scale=inp.v_scale,
                                 entry_price=price)
                 for c in range(copies)]
    clock_warmup(dev, cus, inputs=ks + vs)
    for i in range(max(warmup, 20)):
        launchers[i % copies]()
    torch.cuda.synchronize()
    rate_hz = hd.hpc_decode_wall_clock_hz()
    buf = torch.zeros(8 * W, dtype=torch.int64, device=dev)
    names = ("schedule_us", "first_tile_us", "steady_us_per_tile", "entry_merges_us", "worker_us")
    per_step = {n: {"median": [], "max": []} for n in names}
    hd.hpc_decode_profile_start(steps)
    hd.hpc_decode_trace_start(buf)
    try:
        for i in range(steps):
            buf.zero_()
            launchers[i % copies]()
            st = buf.cpu().numpy().view(np.uint64).reshape(W, 8).astype(np.int64)
            busy = st[:, 5] > 0
            t = st[busy, :5] * (1e6 / rate_hz)
            tiles = st[busy, 5]
            vals = {"schedule_us": t[:, 1] - t[:, 0], "first_tile_us": t[:, 2] - t[:, 0],
                    "steady_us_per_tile": (t[:, 3] - t[:, 2]) / np.maximum(tiles - 1, 1),
                    "entry_merges_us": t[:, 4] - t[:, 3], "worker_us": t[:, 4] - t[:, 0]}
            for n in names:
                per_step[n]["median"].append(float(np.median(vals[n])))
                per_step[n]["max"].append(float(np.max(vals[n])))
    finally:
        hd.hpc_decode_trace_stop()
    d_ms, c_ms, n = hd.hpc_decode_profile_stop()
    summary = {n: {"median_over_workers": round(float(np.median(per_step[n]["median"])), 3),
                   "max_over_workers": round(float(np.median(per_step[n]["max"])), 3)} for n in names}
    log(f"phase trace {WORKLOADS[cfg].name}, W={W}, entry price {price}: " + "; ".join(
        f"{n} {v['median_over_workers']} (max {v['max_over_workers']})" for n, v in summary.items())
        + f"; traced decode kernel {d_ms / max(n, 1) * 1e3:.2f} us by events")
    return {"mode": "phase-trace", "workload": WORKLOADS[cfg].name, "n_workers": W, "entry_price": price,
            "steps": steps,
            "clock_hz": rate_hz, "phases": summary,
            "traced_decode_kernel_us": round(d_ms / max(n, 1) * 1e3, 3),
            "traced_merge_kernel_us": round(c_ms / max(n, 1) * 1e3, 3),
            "note": "stamps are taken by wave 0 of each worker; workers on different XCDs have offset clocks, so "
                    "only durations within a worker are used"}


WORKER_SWEEP_BATCHES = (
    # (name, lengths or ("loguniform", seed, batch), Hq, Hkv, kv dtype)
    ("fp8 64q/8kv 32 x log-uniform [128, 65536] (seed 5)", ("loguniform", 5, 32), 64, 8, "fp8_e4m3"),
    ("bf16 64q/8kv 32 x log-uniform [128, 65536] (seed 5)", ("loguniform", 5, 32), 64, 8, "bf16"),
    ("fp8 64q/8kv 16 x 32K", [32768] * 16, 64, 8, "fp8_e4m3"),
    ("bf16 64q/8kv 16 x 32K", [32768] * 16, 64, 8, "bf16"),
    ("fp8 64q/8kv 64 x 4K", [4096] * 64, 64, 8, "fp8_e4m3"),
    ("bf16 8q/1kv 64 x log-uniform [128, 65536] (seed 1)", ("loguniform", 1, 64), 8, 1, "bf16"),
    ("fp8 8q/1kv 1 x 128K + 31 x 4K", [131072] + [4096] * 31, 8, 1, "fp8_e4m3"),
    ("bf16 8q/1kv 1 x 128K + 31 x 4K", [131072] + [4096] * 31, 8, 1, "bf16"),
)


def workers_sweep(dev, cus: int, steps: int, warmup: int) -> dict:
    """The device-scheduled step at one and at two workers per CU and at
    hpc_decode_pick_workers' choice, on batches that differ in KV dtype and
    in entries per worker: decode + merge kernel time per step
    (dispatch-stamped events), KV rotated over >= 1 GiB of copies, two
    rounds per count."""
    import numpy as np
    import torch

    import load_balanced_paged_step_amd as hd
    from workloads import draw_loguniform_lengths, make_inputs

    clock_warmup(dev, cus)
    steps = max(steps, 50)
    rows = []
    for name, lens, hq, hkv, kv in WORKER_SWEEP_BATCHES:
        if isinstance(lens, tuple):
            lens = list(draw_loguniform_lengths(np.random.default_rng(lens[1]), lens[2], 128, 65536))
        inp = make_inputs(lens, hq, hkv, kv, seed=4)
        kv_bytes = inp.k_cache.numel() * inp.k_cache.element_size() * 2
        copies = max(1, min(16, math.ceil((1 << 30) / kv_bytes)))
        q, bt, sl = inp.q.to(dev), inp.block_table.to(dev), inp.seq_lens.to(dev)
        ks = [inp.k_cache.to(dev) for _ in range(copies)]
        vs = [inp.v_cache.to(dev) for _ in range(copies)]
        clock_warmup(dev, cus, inputs=ks + vs)   # every copy read once before timing
        out = torch.empty_like(q)
        lse = torch.empty(q.shape[:2], dtype=torch.float32, device=dev)
        scales = dict(sm_scale=inp.sm_scale, k_scale=inp.k_scale, v_scale=inp.v_scale)
        picked = hd.hpc_decode_pick_workers(inp.seq_lens, hkv, kv, cus)
        words = hd.hpc_decode_plan(inp.seq_lens.numpy(), hkv, cus)
        times = {}
        for W in sorted({cus, 2 * cus, picked}):
            ws = torch.zeros(hd.hpc_decode_step_workspace_size(inp.batch, hq, hkv, W), dtype=torch.uint8, device=dev)
            launchers = [hd.StepLauncher(q, ks[c], vs[c], bt, sl, out, lse, num_kv_heads=hkv, n_workers=W,
                                         workspace=ws, **scales) for c in range(copies)]
            rounds = []
            for _ in range(2):
                for i in range(max(warmup, 20)):
                    launchers[i % copies]()
                torch.cuda.synchronize()
                hd.hpc_decode_profile_start(steps)
                for i in range(steps):
                    launchers[i % copies]()
                torch.cuda.synchronize()
                d_ms, c_ms, n = hd.hpc_decode_profile_stop()
                rounds.append(round((d_ms + c_ms) / max(n, 1) * 1e3, 2))
            times[W] = rounds
            del launchers, ws
        row = {"batch": name, "entries_per_worker_at_cus": round(int(words[5]) / cus, 3), "picked_workers": picked,
               "kernel_us": {str(W): t for W, t in times.items()}}
        log(f"workers sweep {name}: " + ", ".join(f"W={W} {t} us" for W, t in times.items()) + f"; picked W={picked}")
        rows.append(row)
        del ks, vs
        torch.cuda.empty_cache()
    return {"mode": "workers-sweep", "cus": cus, "steps": steps,
            "timing": "decode + merge kernel time per step, dispatch-stamped HIP events, two rounds per count",
            "rows": rows}


PRICE_SWEEP_PRICES = (0, 2, 4, 8, 16)


def price_sweep(dev, cus: int, steps: int, warmup: int) -> dict:
    """The device-scheduled step at entry prices 0, 2, 4, 8 and 16 quarter
    tiles, at hpc_decode_pick_workers' count, on the worker-sweep batches:
    decode + merge kernel time per step (dispatch-stamped events), KV
    rotated over >= 1 GiB of copies, prices taken in turn for three rounds
    so that drift hits all alike."""
    import numpy as np
    import torch

    import load_balanced_paged_step_amd as hd
    from workloads import draw_loguniform_lengths, make_inputs

    clock_warmup(dev, cus)
    steps = max(steps, 50)
    rows = []
    for name, lens, hq, hkv, kv in WORKER_SWEEP_BATCHES:
        if isinstance(lens, tuple):
            lens = list(draw_loguniform_lengths(np.random.default_rng(lens[1]), lens[2], 128, 65536))
        inp = make_inputs(lens, hq, hkv, kv, seed=4)
        kv_bytes = inp.k_cache.numel() * inp.k_cache.element_size() * 2
        copies = max(1, min(16, math.ceil((1 << 30) / kv_bytes)))
        q, bt, sl = inp.q.to(dev), inp.block_table.to(dev), inp.seq_lens.to(dev)
        ks = [inp.k_cache.to(dev) for _ in range(copies)]
        vs = [inp.v_cache.to(dev) for _ in range(copies)]
        clock_warmup(dev, cus, inputs=ks + vs)   # every copy read once before timing
        out = torch.empty_like(q)
        lse = torch.empty(q.shape[:2], dtype=torch.float32, device=dev)
        scales = dict(sm_scale=inp.sm_scale, k_scale=inp.k_scale, v_scale=inp.v_scale)
        W = hd.hpc_decode_pick_workers(inp.seq_lens, hkv, kv, cus)
        picked = hd.hpc_decode_pick_entry_price(inp.seq_lens, hkv, kv, W)
        lens_np = inp.seq_lens.numpy()
        ws = torch.zeros(hd.hpc_decode_step_workspace_size(inp.batch, hq, hkv, W), dtype=torch.uint8, device=dev)
        launchers = {c: [hd.StepLauncher(q, ks[i], vs[i], bt, sl, out, lse, num_kv_heads=hkv, n_workers=W,
                                         workspace=ws, entry_price=c, **scales) for i in range(copies)]
                     for c in PRICE_SWEEP_PRICES}
        applied = {c: int(hd.hpc_decode_plan(lens_np, hkv, W, entry_price=c)[9]) for c in PRICE_SWEEP_PRICES}
        entries = {c: int(hd.hpc_decode_plan(lens_np, hkv, W, entry_price=c)[5]) for c in PRICE_SWEEP_PRICES}
        times = {c: [] for c in PRICE_SWEEP_PRICES}
        for _ in range(3):
            for c in PRICE_SWEEP_PRICES:
                for i in range(max(warmup, 20)):
                    launchers[c][i % copies]()
                torch.cuda.synchronize()
                hd.hpc_decode_profile_start(steps)
                for i in range(steps):
                    launchers[c][i % copies]()
                torch.cuda.synchronize()
                d_ms, c_ms, n = hd.hpc_decode_profile_stop()
                times[c].append(round((d_ms + c_ms) / max(n, 1) * 1e3, 2))
        med = {c: float(np.median(t)) for c, t in times.items()}
        best = min(med, key=med.get)
        row = {"batch": name, "kv_dtype": kv, "n_workers": W, "picked_price": picked,
               "applied": {str(c): applied[c] for c in PRICE_SWEEP_PRICES},
               "entries": {str(c): entries[c] for c in PRICE_SWEEP_PRICES},
               "kernel_us": {str(c): t for c, t in times.items()},
               "picked_over_best": round(med[picked] / med[best], 4)}
        log(f"price sweep {name} (W={W}): " + ", ".join(f"c={c} {med[c]:.2f} us" for c in PRICE_SWEEP_PRICES)
            + f"; picked {picked} ({row['picked_over_best']}x the best)")
        rows.append(row)
        del launchers, ks, vs, ws
        torch.cuda.empty_cache()
    return {"mode": "price-sweep", "cus": cus, "steps": steps,
            "timing": "decode + merge kernel time per step, dispatch-stamped HIP events, median of three rounds",
            "rows": rows}


def _lens_summary(lens) -> str:
    from collections import Counter
    c = Counter(int(x) for x in lens)
    if len(c) > 6:
        return f"{len(lens)} seqs, {int(min(lens))}..{int(max(lens))} (sum {int(sum(lens))})"
    return " + ".join(f"{n}x{L}" for L, n in sorted(c.items(), key=lambda kv: -kv[0]))


def prefill_group_sweep(dev, cus: int, steps: int, warmup: int) -> dict:
    """Causal extend attention at 1, 2, 4, 8 and 16 query heads per KV head
    (8 KV heads, bf16): the contexts and chunks of extend-8x512 (8 chunks of
    512 new tokens after log-uniform [64, 16384] cached, seed 7), whole units
    (W = 0) and the balanced plan at 2 workers per CU; launch time by events,
    median of three passes."""
    import numpy as np
    import torch

    from load_balanced_paged_step_amd.prefill import PrefillStep
    from workloads import PREFILL_WORKLOADS, draw_loguniform_lengths, make_prefill_inputs

    w = PREFILL_WORKLOADS["extend-8x512"]
    clock_warmup(dev, cus)
    rng = np.random.default_rng(7)
    ctx = draw_loguniform_lengths(rng, len(w.q_lens), *w.ctx_loguniform)
    qn = np.asarray(w.q_lens, dtype=np.int64)
    rows = []
    for hq in (8, 16, 32, 64, 128):
        pi = make_prefill_inputs(ctx, qn, hq, 8, "bf16", seed=7)
        c = pi.cache
        q, qs = pi.q.to(dev), pi.q_start.to(dev)
        k, v = c.k_cache.to(dev), c.v_cache.to(dev)
        bt, sl = c.block_table.to(dev), c.seq_lens.to(dev)
        out = torch.empty_like(q)
        lse = torch.empty(q.shape[:2], dtype=torch.float32, device=dev)
        flops = pi.flops()
        row = {"heads": f"{hq}q/8kv", "group": hq // 8, "flops": flops}
        for W in (0, 2 * cus):
            step = PrefillStep(pi.q_start, c.seq_lens, c.num_q_heads, c.num_kv_heads, c.max_pages_per_seq,
                               n_workers=W, device=dev)
            one = step.bind(q, qs, k, v, bt, sl, out, lse, sm_scale=c.sm_scale, k_scale=c.k_scale,
                            v_scale=c.v_scale)
            us = _events_us(one, max(steps, 20), max(warmup, 5))
            row[f"W={W}"] = {"us": round(us, 2), "TFLOPs": round(flops / (us * 1e-6) / 1e12, 1)}
            del one, step
        log(f"prefill group sweep {hq}q/8kv (G={hq // 8}): " + ", ".join(
            f"{k} {v['us']:.1f} us ({v['TFLOPs']:.0f} TFLOP/s)" for k, v in row.items() if k.startswith("W=")))
        rows.append(row)
        del q, k, v, out, lse
        torch.cuda.empty_cache()
    return {"mode": "prefill-group-sweep", "contexts": "extend-8x512's (seed 7)",
            "timing": "mean of back-to-back launches, HIP events on the launch stream; median of three passes",
            "rows": rows}


MERGE_SWEEP_BATCHES = (
    # (name, lengths, q heads, kv heads, kv dtype): 2 to 32 workers per unit at one worker per CU
    ("bf16 8q/1kv 128x256", [256] * 128, 8, 1, "bf16"),
    ("bf16 8q/1kv 64x512", [512] * 64, 8, 1, "bf16"),
    ("bf16 8q/1kv 32x1K", [1024] * 32, 8, 1, "bf16"),
    ("bf16 8q/1kv 16x2K", [2048] * 16, 8, 1, "bf16"),
    ("bf16 8q/1kv 8x4K", [4096] * 8, 8, 1, "bf16"),
    ("bf16 8q/1kv 64x1K", [1024] * 64, 8, 1, "bf16"),
    ("bf16 8q/1kv 32x2K", [2048] * 32, 8, 1, "bf16"),
    ("bf16 64q/8kv 8x1K", [1024] * 8, 64, 8, "bf16"),
    ("bf16 64q/8kv 4x2K", [2048] * 4, 64, 8, "bf16"),
    ("fp8 64q/8kv 16x512", [512] * 16, 64, 8, "fp8_e4m3"),
    ("fp8 64q/8kv 8x1K", [1024] * 8, 64, 8, "fp8_e4m3"),
    ("fp8 64q/8kv 4x2K", [2048] * 4, 64, 8, "fp8_e4m3"),
    ("fp8 64q/8kv 2x4K", [4096] * 2, 64, 8, "fp8_e4m3"),
    ("bf16 8q/1kv 4 short (37-200)", [37, 80, 150, 200], 8, 1, "bf16"),
    # fewer tiles than workers: every worker holds at most one tile
    ("bf16 8q/1kv 8x128", [128] * 8, 8, 1, "bf16"),
    ("bf16 8q/1kv 16x256", [256] * 16, 8, 1, "bf16"),
    ("bf16 8q/1kv 8x512", [512] * 8, 8, 1, "bf16"),
    ("bf16 8q/1kv 32x256", [256] * 32, 8, 1, "bf16"),
    ("bf16 8q/1kv 8x1K", [1024] * 8, 8, 1, "bf16"),
    ("fp8 64q/8kv 2x512", [512] * 2, 64, 8, "fp8_e4m3"),
    ("bf16 8q/1kv 1x8K+31x4K", [8192] + [4096] * 31, 8, 1, "bf16"),
    ("bf16 8q/1kv 1x16K+31x4K", [16384] + [4096] * 31, 8, 1, "bf16"),
    ("bf16 8q/1kv 1x128K+31x4K", [131072] + [4096] * 31, 8, 1, "bf16"),
)


def plan_max_shares(words) -> int:
    """Most workers sharing one unit in a host plan (its merge records hold
    each split unit's worker count; header of 16 words, then W + 1 worker
    pointers, 4 words per entry, 3 per merge record)."""
    W, E, C = int(words[3]), int(words[5]), int(words[7])
    o = 16 + W + 1 + 4 * E
    return max([1] + [int(words[o + 3 * i + 1]) for i in range(C)])


def merge_sweep(dev, cus: int, steps: int, warmup: int) -> dict:
    """The device-scheduled step with the merge kernel and with the in-kernel
    merge, at the rules' worker count and entry price, on batches whose
    units are shared by 2 to 128 workers: whole-step time (the mean over
    back-to-back steps between two events, gaps between kernels included),
    KV rotated over >= 1 GiB of copies, the two modes taken in turn for three
    rounds, medians."""
    import numpy as np
    import torch

    import load_balanced_paged_step_amd as hd
    from workloads import make_inputs

    clock_warmup(dev, cus)
    steps = max(steps, 50)
    rows = []
    for name, lens, hq, hkv, kv in MERGE_SWEEP_BATCHES:
        inp = make_inputs(lens, hq, hkv, kv, seed=4)
        kv_bytes = inp.k_cache.numel() * inp.k_cache.element_size() * 2
        copies = max(1, min(16, math.ceil((1 << 30) / kv_bytes)))
        q, bt, sl = inp.q.to(dev), inp.block_table.to(dev), inp.seq_lens.to(dev)
        ks = [inp.k_cache.to(dev) for _ in range(copies)]
        vs = [inp.v_cache.to(dev) for _ in range(copies)]
        clock_warmup(dev, cus, inputs=ks + vs)   # every copy read once before timing
        out = torch.empty_like(q)
        lse = torch.empty(q.shape[:2], dtype=torch.float32, device=dev)
        scales = dict(sm_scale=inp.sm_scale, k_scale=inp.k_scale, v_scale=inp.v_scale)
        lens_np = inp.seq_lens.numpy()
        W = hd.hpc_decode_pick_workers(lens_np, hkv, kv, cus)
        price = hd.hpc_decode_pick_entry_price(lens_np, hkv, kv, W)
        picked = hd.hpc_decode_pick_merge(lens_np, hkv, W, price)
        shares = plan_max_shares(hd.hpc_decode_plan(lens_np, hkv, W, entry_price=price))
        ws = torch.zeros(hd.hpc_decode_step_workspace_size(inp.batch, hq, hkv, W), dtype=torch.uint8, device=dev)
        launchers = {f: [hd.StepLauncher(q, ks[i], vs[i], bt, sl, out, lse, num_kv_heads=hkv, n_workers=W,
                                         workspace=ws, entry_price=price, fused_merge=f, **scales)
                         for i in range(copies)] for f in (False, True)}
        times = {f: [] for f in (False, True)}
        for _ in range(3):
            for f in (False, True):
                times[f].append(round(_step_us(lambda i: launchers[f][i % copies](), steps, max(warmup, 20),
                                               reps=1), 2))
        med = {f: float(np.median(t)) for f, t in times.items()}
        row = {"batch": name, "n_workers": W, "entry_price": price, "max_shares": shares,
               "merge_kernel_us": times[False], "in_kernel_us": times[True],
               "picked": "in the decode kernel" if picked else "merge kernel",
               "picked_over_best": round(med[picked] / min(med.values()), 4)}
        log(f"merge sweep {name} (W={W}, price {price}, up to {shares} workers per unit): merge kernel "
            f"{med[False]:.2f} us, in-kernel {med[True]:.2f} us; picked {row['picked']}")
        rows.append(row)
        del launchers, ks, vs, ws
        torch.cuda.empty_cache()
    return {"mode": "merge-sweep", "cus": cus, "steps": steps,
            "timing": "whole step, the mean over back-to-back steps between two events, three rounds",
            "rows": rows}


if __name__ == "__main__":
    sys.exit(main())
