#!/usr/bin/env python3
"""Benchmark of the varlen attention backward on one MI355X.

One step = one fa_varlen_bwd call over the whole workload (for 16-bit inputs the dQ kernel,
which also computes the row statistics, then the dK/dV kernel) with every input already
resident in HBM.
Default workload: bf16, 4 sequences x 16384 tokens, 16 heads, D = 128,
bottom-right causal mask, keep_prob 1.

Metric: useful TFLOP/s = 10 * N * D * (admitted query/key pairs) / step time
(five contractions of 2*D flops per admitted pair and head).

Also reported:
  roofline      the dominant kernel's algorithmic flops per launch over its
                average duration (HIP events on the launch stream, recorded by
                the library during the timed steps) against the bf16 MFMA peak;
  kernels       the same figure for every kernel (GB/s for the HBM-bound ones);
  cold_layout   calls whose sequence layout is new to the library (work lists
                built and uploaded in the call), device and host time per call;
  workloads     (default run) ms per call and useful TFLOP/s of the other 16-bit
                workloads: 2 (bf16 causal, 16 sequences), 4 (bf16 band 2048/0,
                8 x 8192), 5 (fp16 causal with dropout, 32 sequences);
  cpu_baseline  the fp64 oracle timed on this host on a bounded sample of the
                same workload (a few (sequence, head) units), as a baseline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
# input preparation shared with the tests (torch fp32 forward for Y and the statistics, pair counts)
TESTS = os.path.join(ROOT, "tests")
if TESTS not in sys.path:
    sys.path.append(TESTS)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 / fp16 MFMA, published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
KERNEL_SOURCES = [os.path.join(ROOT, "variable_length_flashattention_fa_amd", "csrc", f)
                  for f in ("fa_kernels.hip", "fa_bwd16.hip", "fa_fwd.hip", "fa_device.h", "fa_kernels.h", "build.py",
                            "fa_worklist.cpp")]  # the work-list order decides which tiles share an L2
# kernel name fragment in a counter trace -> the name bench reports it under
PMC_KERNELS = {"bwd_dkdv16_kernel": "bwd_dkdv16_kernel", "bwd_dq16_kernel": "bwd_dq16_kernel",
               "preprocess_kernel": "preprocess", "bwd_main_kernel": "bwd_main_kernel", "fwd16_kernel": "fwd16_kernel"}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` from committed counter runs, if taken on this kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    entry = rec.get(workload, {}).get(kernel)
    if not entry or entry.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return entry.get("hbm_bytes_per_launch")


def ingest_pmc(fetch_dir: str, write_dir: str, workload: str, copy_mib: int) -> dict:
    """Turn two rocprofv3 --pmc CSV runs (FETCH_SIZE, then WRITE_SIZE) of this script into HBM bytes per launch.

    Both runs must have been made with --calibration-copy-mib `copy_mib`: the copy through torch's elementwise
    kernel (``neg``) of known size gives the factor from counter KiB to bytes moved.
    """
    import collections
    import csv

    def load(d, counter):
        per = collections.OrderedDict()
        for r in csv.DictReader(open(os.path.join(d, "run_counter_collection.csv"))):
            if r["Counter_Name"] != counter:
                continue
            k = int(r["Dispatch_Id"])
            per.setdefault(k, [r["Kernel_Name"], 0.0])[1] += float(r["Counter_Value"])
        return [per[k] for k in sorted(per)]

    def calib(rows):
        for i, (n, v) in enumerate(rows):
            if "neg_kernel" in n:
                return rows[i - 1][1], v  # the blit copy right before, and the elementwise copy
        raise SystemExit("no calibration copy in the counter trace")

    f, w = load(fetch_dir, "FETCH_SIZE"), load(write_dir, "WRITE_SIZE")
    cf_blit, cf_elem = calib(f)
    cw_blit, cw_elem = calib(w)
    kib = copy_mib * 1024.0
    ff, wf = kib / cf_elem, kib / cw_elem
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        rec = {}
    rec["_calibration"] = {
        "copy_mib": copy_mib,
        "fetch_size_kib": {"runtime_blit_copy": cf_blit, "elementwise_copy": cf_elem},
        "write_size_kib": {"runtime_blit_copy": cw_blit, "elementwise_copy": cw_elem},
        "fetch_factor": ff, "write_factor": wf,
        "note": "a plain copy of copy_mib MiB reads and writes copy_mib MiB; factor = true KiB / counter KiB"}
    ent = rec.setdefault(workload, {})
    for frag, label in PMC_KERNELS.items():
        fv = [v for n, v in f if frag in n]
        wv = [v for n, v in w if frag in n]
        if not fv or not wv:
            continue
        fa, wa = sum(fv) / len(fv), sum(wv) / len(wv)
        ent[label] = {"fetch_size_kib_per_dispatch": fv, "write_size_kib_per_dispatch": wv,
                      "hbm_read_bytes_per_launch": fa * 1024 * ff, "hbm_write_bytes_per_launch": wa * 1024 * wf,
                      "hbm_bytes_per_launch": (fa * ff + wa * wf) * 1024,
                      "kernel_source_sha256_16": kernel_source_hash()}
        log(f"{label}: read {fa * 1024 * ff / 1e9:.3f} GB, write {wa * 1024 * wf / 1e9:.3f} GB per launch")
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(rec, fh, indent=1)
    return rec


def cpu_baseline(inp, y_host, smax_h, ssum_h, wl, units_wanted: int):
    """Time the oracle backward on the first `units` (sequence, head) units of the workload."""
    import numpy as np

    from oracle import fa_oracle as O
    from variable_length_flashattention_fa_amd import synth
    from inputs_forward import pair_count

    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    workers = max(1, min(16, cores, units_wanted))
    nb = len(inp.cu_q) - 1
    units = [(b, n) for n in range(wl.heads) for b in range(nb)][:workers]
    q, k, v, dy = (synth.as_float_array(x) for x in (inp.q, inp.k, inp.v, inp.dy))
    flops = 0
    for b, _ in units:
        cq = inp.cu_q[b:b + 2] - inp.cu_q[b]
        ck = inp.cu_kv[b:b + 2] - inp.cu_kv[b]
        flops += 10 * wl.head_dim * pair_count(cq, ck, wl.mode, wl.pre, wl.nxt)
    log(f"cpu baseline: oracle on {len(units)} (sequence, head) units with {workers} worker processes")
    t0 = time.perf_counter()
    O.backward(q, k, v, dy, y_host, smax_h, ssum_h, inp.cu_q, inp.cu_kv, mode=wl.mode, pre=wl.pre, nxt=wl.nxt,
               keep_prob=wl.keep_prob, drop_mask=inp.drop_mask, scale=wl.scale, head_num=wl.heads,
               workers=workers, units=units)
    dt = time.perf_counter() - t0
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": workers,
        "kind": "oracle",
        "sample": (f"{len(units)} of {nb * wl.heads} (sequence, head) units of the same workload "
                   f"(each one sequence x one head, fp64 numpy, one BLAS thread per worker process); "
                   f"{dt:.1f} s wall"),
        "seconds": dt,
        "useful_tflop": flops / 1e12,
    }


def cold_layout_calls(B, q, k, v, dy, y, smax, ssum, inp, wl, drop, dq, dk, dv, stream, count: int = 8) -> dict:
    """Calls whose sequence layout the library has not seen: the first two sequences' boundary
    moves by 1..count tokens (same tensors, same total), so each call builds its work lists and
    uploads them.  Reports device time per call (HIP events), host time per call, and the host
    time of the same number of calls with a cached layout."""
    import numpy as np
    import torch

    lens = np.diff(inp.cu_q)
    if len(lens) < 2 or wl.keep_prob < 1.0:
        return None
    layouts = []
    for i in range(1, count + 1):
        l2 = lens.copy()
        l2[0] += i
        l2[1] -= i
        layouts.append(np.concatenate([[0], np.cumsum(l2)]).astype(np.int64))

    def call(cu):
        B.fa_varlen_bwd(q, k, v, dy, y, smax, ssum, cu, cu, wl.mode, wl.pre, wl.nxt, wl.keep_prob, drop, wl.scale,
                        wl.heads, dq, dk, dv, stream=stream)

    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    host = 0.0
    ev[0].record(stream)
    for cu in layouts:
        t0 = time.perf_counter()
        call(cu)
        host += time.perf_counter() - t0
    ev[1].record(stream)
    torch.cuda.synchronize()
    cold_ms = ev[0].elapsed_time(ev[1]) / count
    host_cached = 0.0
    for _ in range(count):
        t0 = time.perf_counter()
        call(inp.cu_q)
        host_cached += time.perf_counter() - t0
    torch.cuda.synchronize()
    return {"ms_per_call": cold_ms, "host_us_per_call": host / count * 1e6,
            "cached_host_us_per_call": host_cached / count * 1e6, "calls": count,
            "note": "each call has a sequence layout not seen before (the boundary of the first two sequences "
                    "moves by 1..calls tokens): its work lists are built and uploaded asynchronously"}


def other_workload(number: int, steps: int, warmup: int) -> dict:
    """ms per call and useful TFLOP/s of another workload, timed like the headline one."""
    import torch

    from variable_length_flashattention_fa_amd import binding as B
    from variable_length_flashattention_fa_amd import synth
    from inputs_forward import forward_stats, pair_count

    wl = synth.workload(number)
    t0 = time.time()
    log(f"workload {number}: {wl.name}; drawing inputs")
    inp = synth.make(wl)
    dev = torch.device("cuda:0")
    q, k, v, dy = (x.to(dev) for x in (inp.q, inp.k, inp.v, inp.dy))
    drop = torch.from_numpy(inp.drop_mask).to(dev) if inp.drop_mask is not None else None
    y, smax, ssum = forward_stats(q, k, v, inp.cu_q, inp.cu_kv, mode=wl.mode, pre=wl.pre, nxt=wl.nxt,
                                  keep_prob=wl.keep_prob, drop_mask=drop, scale=wl.scale)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    stream = torch.cuda.current_stream(dev)

    def step():
        B.fa_varlen_bwd(q, k, v, dy, y, smax, ssum, inp.cu_q, inp.cu_kv, wl.mode, wl.pre, wl.nxt, wl.keep_prob,
                        drop, wl.scale, wl.heads, dq, dk, dv, stream=stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    B.profile_read()
    B.profile_enable(True)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for _ in range(steps):
        step()
    ev[1].record(stream)
    torch.cuda.synchronize()
    B.profile_enable(False)
    prof = B.profile_read()
    ms = ev[0].elapsed_time(ev[1]) / steps
    pairs = pair_count(inp.cu_q, inp.cu_kv, wl.mode, wl.pre, wl.nxt)
    tflops = 10.0 * wl.heads * wl.head_dim * pairs / (ms * 1e-3) / 1e12
    kernels = {name: ms_ / max(n, 1) for name, (ms_, n) in prof.items() if n}
    log(f"workload {number}: {ms:.3f} ms/call, {tflops:.0f} useful TFLOP/s ({time.time() - t0:.1f}s)")
    del q, k, v, dy, y, smax, ssum, dq, dk, dv, drop
    torch.cuda.empty_cache()
    return {"workload": wl.name, "ms_per_call": ms, "useful_TFLOP/s": tflops,
            "pct_of_bf16_peak": 100.0 * tflops / PEAK_BF16_TFLOPS, "dtype": wl.dtype, "steps": steps,
            "kernel_avg_ms": {("bwd_dkdv16_kernel" if k_ == "bwd_main" else "bwd_dq16_kernel" if k_ == "bwd_dq"
                               else k_): v_ for k_, v_ in kernels.items()},
            "config": {"sequences": len(wl.lengths), "tokens": wl.tokens, "heads": wl.heads,
                       "head_dim": wl.head_dim, "mask": ["none", "causal", "band"][wl.mode],
                       "pre_tokens": wl.pre, "next_tokens": wl.nxt, "keep_prob": wl.keep_prob,
                       "admitted_pairs_per_head": pairs}}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=3, help="workload number 1..5 (default 3)")
    ap.add_argument("--cpu-units", type=int, default=16, help="(sequence, head) units for the CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra-workloads", action="store_true",
                    help="skip the other 16-bit workloads (2, 4, 5) reported under 'workloads'")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="copy this many MiB device-to-device once before the timed steps, with the runtime's "
                         "blit kernel and with an elementwise kernel (plain copies of known size, for "
                         "scaling HBM byte counters)")
    ap.add_argument("--ingest-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU run: turn two rocprofv3 --pmc output folders (FETCH_SIZE, WRITE_SIZE) of this "
                         "script, run with --calibration-copy-mib, into per-launch HBM bytes in profiles/")
    args = ap.parse_args(argv)
    if args.ingest_pmc:
        from variable_length_flashattention_fa_amd import synth
        if args.calibration_copy_mib <= 0:
            ap.error("--ingest-pmc needs the --calibration-copy-mib the counter runs used")
        ingest_pmc(*args.ingest_pmc, synth.workload(args.workload).name, args.calibration_copy_mib)
        return 0

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (each (sequence, head) unit is "
              "independent, so heads or sequences would shard across GPUs with no communication). Run with --gpus 1.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from variable_length_flashattention_fa_amd import binding as B
    from variable_length_flashattention_fa_amd import synth
    from inputs_forward import forward_stats, pair_count

    B.load()  # fail loudly before any work if the library is missing
    wl = synth.workload(args.workload)
    t0 = time.time()
    log(f"workload {args.workload}: {wl.name}; drawing inputs")
    inp = synth.make(wl)
    dev = torch.device("cuda:0")
    q, k, v, dy = (x.to(dev) for x in (inp.q, inp.k, inp.v, inp.dy))
    drop = torch.from_numpy(inp.drop_mask).to(dev) if inp.drop_mask is not None else None
    log(f"inputs on device ({time.time() - t0:.1f}s); forward for Y and statistics")
    y, smax, ssum = forward_stats(q, k, v, inp.cu_q, inp.cu_kv, mode=wl.mode, pre=wl.pre, nxt=wl.nxt,
                                  keep_prob=wl.keep_prob, drop_mask=drop, scale=wl.scale)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)

    def step():
        B.fa_varlen_bwd(q, k, v, dy, y, smax, ssum, inp.cu_q, inp.cu_kv, wl.mode, wl.pre, wl.nxt, wl.keep_prob,
                        drop, wl.scale, wl.heads, dq, dk, dv, stream=stream)

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.calibration_copy_mib > 0:
        nel = args.calibration_copy_mib * (1 << 20) // 4
        src = torch.ones(nel, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)          # runtime blit kernel: reads and writes nel*4 bytes
        torch.cuda.synchronize()
        torch.neg(src, out=dst)  # elementwise kernel: the same bytes through an ordinary kernel
        torch.cuda.synchronize()
        del src, dst
        log(f"calibration copy of {args.calibration_copy_mib} MiB done")
    B.profile_read()  # drop anything recorded before the timed region
    B.profile_enable(True)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    marks[0].record(stream)
    for i in range(args.steps):
        step()
        marks[i + 1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    B.profile_enable(False)
    prof = B.profile_read()
    ms_per_step = elapsed * 1e3 / args.steps
    call_ms = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps))
    log(f"timed {args.steps} steps: {ms_per_step:.3f} ms/step")
    # the varlen forward on the same inputs (Y and statistics into scratch tensors)
    y_f = torch.empty_like(y)
    smax_f, ssum_f = torch.empty_like(smax), torch.empty_like(ssum)

    def fwd_step():
        B.fa_varlen_fwd(q, k, v, inp.cu_q, inp.cu_kv, wl.mode, wl.pre, wl.nxt, wl.keep_prob, drop, wl.scale,
                        wl.heads, y_f, smax_f, ssum_f, stream=stream)

    for _ in range(args.warmup):
        fwd_step()
    torch.cuda.synchronize()
    B.profile_read()
    B.profile_enable(True)
    t_f = time.perf_counter()
    for _ in range(args.steps):
        fwd_step()
    torch.cuda.synchronize()
    fwd_ms = (time.perf_counter() - t_f) * 1e3 / args.steps
    B.profile_enable(False)
    fwd_prof = B.profile_read()
    log(f"forward: {fwd_ms:.3f} ms/call")

    pairs = pair_count(inp.cu_q, inp.cu_kv, wl.mode, wl.pre, wl.nxt)
    useful = 10.0 * wl.heads * wl.head_dim * pairs
    value = useful / (ms_per_step * 1e-3) / 1e12
    tq, heads, d = q.shape
    esz = q.element_size()
    pair_flops = 2.0 * wl.heads * wl.head_dim * pairs  # one contraction over all admitted pairs
    if q.dtype == torch.float32:
        # dK/dV kernel: S, dP, dV, dK on fp32 MFMA; dQ kernel: S, dP (recomputed) and dQ on the VALU
        mfma = {"bwd_main": ("bwd_main_kernel", 4 * pair_flops), "bwd_dq": ("bwd_dq32_kernel", 3 * pair_flops)}
        hbm = {"preprocess": tq * heads * (2 * d * esz + 2 * 4 + 8)}
    else:
        # dK/dV kernel: S, dP, dV, dK; dQ kernel: S, dP (recomputed) and dQ
        mfma = {"bwd_main": ("bwd_dkdv16_kernel", 4 * pair_flops), "bwd_dq": ("bwd_dq16_kernel", 3 * pair_flops)}
        hbm = {}  # the row pass (D and beta) runs inside the dQ kernel on this path
    kernels = {}
    for name, (kname, flops) in mfma.items():
        ms, n = prof[name]
        avg = ms / max(n, 1)
        kernels[kname] = {"avg_ms": avg, "launches": n, "algorithmic_tflop": flops / 1e12,
                          "TFLOP/s": flops / (avg * 1e-3) / 1e12 if avg > 0 else None}
    for name, nbytes in hbm.items():
        ms, n = prof[name]
        avg = ms / max(n, 1)
        gbs = nbytes / (avg * 1e-3) / 1e9 if avg > 0 else None
        kernels[name] = {"avg_ms": avg, "launches": n, "algorithmic_bytes": nbytes, "GB/s": gbs,
                         "hbm_frac": gbs / PEAK_HBM_GBS if gbs else None}
    dominant = max((k for k in kernels if "TFLOP/s" in kernels[k]), key=lambda k: kernels[k]["avg_ms"])
    achieved = kernels[dominant]["TFLOP/s"]
    main_avg = kernels[dominant]["avg_ms"]

    dtype_name = {torch.bfloat16: "bf16", torch.float16: "fp16", torch.float32: "fp32"}[q.dtype]
    out = {
        "metric": "attn-bwd useful TFLOP/s (varlen TND, causal) and % of bf16 MFMA peak, 1 GPU",
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype_name,
        "data": "synthetic (seeded normal Q/K/V/dY; Y and softmax stats from a device forward)",
        "config": {"workload": wl.name, "sequences": len(wl.lengths), "tokens": wl.tokens, "heads": wl.heads,
                   "head_dim": wl.head_dim, "mask": ["none", "causal", "band"][wl.mode], "pre_tokens": wl.pre,
                   "next_tokens": wl.nxt, "keep_prob": wl.keep_prob, "admitted_pairs_per_head": pairs},
        "pct_of_bf16_peak": 100.0 * value / PEAK_BF16_TFLOPS,
        "call_ms": {"median": call_ms[len(call_ms) // 2], "min": call_ms[0], "max": call_ms[-1]},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": traffic_for(wl.name, dominant),
                     "kernel": dominant, "avg_ms": main_avg},
        "kernels": kernels,
        "forward": {
            "ms_per_call": fwd_ms,
            "kernel_avg_ms": fwd_prof["fwd"][0] / max(fwd_prof["fwd"][1], 1),
            "traffic": traffic_for(wl.name, "fwd16_kernel"),
            "useful_TFLOP/s": 4.0 * wl.heads * wl.head_dim * pairs / (fwd_ms * 1e-3) / 1e12,
            "pct_of_bf16_peak": 100.0 * 4.0 * wl.heads * wl.head_dim * pairs / (fwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "note": "Y and statistics for the same inputs; useful work 4*N*D per admitted pair (two contractions)",
        },
    }

    out["cold_layout"] = cold_layout_calls(B, q, k, v, dy, y, smax, ssum, inp, wl, drop, dq, dk, dv, stream)
    log(f"cold layout: {out['cold_layout']['ms_per_call']:.3f} ms/call, host "
        f"{out['cold_layout']['host_us_per_call']:.0f} us vs {out['cold_layout']['cached_host_us_per_call']:.0f} us cached")
    if args.workload == 3 and not args.no_extra_workloads:
        out["workloads"] = {}
        for number in (2, 4, 5):
            r = other_workload(number, steps=min(args.steps, 10), warmup=args.warmup)
            out["workloads"][r.pop("workload")] = r

    if not args.no_cpu_baseline:
        y_host = synth.as_float_array(y.cpu())
        smax_h, ssum_h = smax.cpu().numpy(), ssum.cpu().numpy()
        del q, k, v, dy, y, dq, dk, dv
        out["cpu_baseline"] = cpu_baseline(inp, y_host, smax_h, ssum_h, wl, args.cpu_units)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
