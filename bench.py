#!/usr/bin/env python3
"""Throughput of LRKV compressed-cache decode (and prefill) on one MI355X.

A step is one lrkv_decode call over the whole batch (the split-K scan, then
the merge and B^V epilogue, enqueued together), on seeded synthetic inputs
already resident in HBM.  Before the warmup steps the step is repeated,
untimed, for --settle-s seconds so that the timed steps run at the GPU's
steady clock.  Every time reported is the median of --trials trials, each
the average over --steps back-to-back launches between two HIP events on
the launch stream; each kernel's own duration is timed the same way over
launches of lrkv_decode_partial and lrkv_decode_combine alone.

`value` is the 8K-context bf16 decode: 32 sequences x 8192 cached tokens,
H=32 heads, d_h=128, r=16 (cache 671 MB, larger than the 256 MB Infinity
Cache, so every step streams it from HBM).  The default run also measures,
under `configs`, the other synthetic workloads: the tiny fp32 decode (a
latency), the small bf16 decode (L2-resident latency, and throughput over
rotated copies whose working set exceeds twice L2 plus the Infinity
Cache), the ragged 1K-64K-token decode (checked in full against the
oracle), decode at rank 54 (a rank the pages train, on the any-rank scan),
the causal prefill (TFLOP/s against the bf16 MFMA peak, sampled rows
checked against the oracle) and a training step (forward and backward),
each with the oracle timed beside it.

Prints one JSON line.  `roofline` prices the dominant kernel (the scan)
against the HBM peak using the algorithmic bytes of one launch and its
duration; `cpu_baseline` times the float64 oracle on the host cores (all of
them, and one thread for the small configs) as a reported baseline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBPS = 8000.0
ROOT = os.path.dirname(os.path.abspath(__file__))
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "rank_compressed_kv_lrkv_amd", "csrc")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--settle-s", type=float, default=0.5,
                    help="before the warmup steps, repeat the step (untimed) for this many seconds: "
                         "the GPU takes tens of ms of sustained work to reach its steady clock")
    ap.add_argument("--mode", choices=("decode", "prefill", "chunk", "rank-sweep", "project", "vendor", "train"),
                    default="decode",
                    help="decode (the headline line); the causal-prefill MFMA path; a prefill chunk over a "
                         "4096-token history; decode at ranks 0/8/16/32 and plain MHA on the headline shape; "
                         "the fused projection + append of 4 x 4096 tokens from d = 4096; the vendor "
                         "libraries (hipBLASLt GEMM, PyTorch flash attention) timed beside the two MFMA kernels; or "
                         "one training step (forward with log-sum-exp, backward) of the prefill workload")
    ap.add_argument("--workload", default=None, help="default: mid_bf16_T8k (decode), prefill_bf16_L4k (prefill)")
    ap.add_argument("--split-tokens", type=int, default=0, help="0 = library default")
    ap.add_argument("--engine", type=int, default=0, choices=(0, 1, 2, 3, 4),
                    help="decode scan: 0 the default for the shape, 1 the vector-ALU scan, 2 the MFMA scan, "
                         "3 the any-rank scan, 4 the any-rank MFMA scan")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="wall-clock budget of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--trials", type=int, default=5, help="timed trials per figure (the median is reported)")
    ap.add_argument("--headline-only", action="store_true",
                    help="decode mode: measure the selected workload only (no `configs` section)")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="after timing, run `steps` plain device copies of this many MB (untimed), "
                         "a known-size reference for the HBM byte counters")
    return ap.parse_args()


# kernel -> the sources its code comes from (the counter summaries record their digest)
KERNEL_SOURCES = {
    "decode_mfma_kernel": ("decode_mfma.hip", "decode_balance.h", "lrkv_device.h"),
    "decode_split_kernel": ("decode.hip", "lrkv_device.h"),
    "prefill_kernel": ("prefill.hip", "lrkv_device.h"),
    "project_gemm_kernel": ("project.hip", "lrkv_device.h"),
    "decode_generic_kernel": ("decode_generic.hip", "lrkv_device.h"),
    "decode_mfma_any_kernel": ("decode_mfma_any.hip", "lrkv_device.h"),
    "train_dkv_kernel": ("train.hip", "lrkv_device.h"),
    "train_dq_kernel": ("train.hip", "lrkv_device.h"),
}


def source_digest(names):
    """sha256 (first 16 hex digits) of the named kernel sources, concatenated in order."""
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(counters, kernel, workload, split=None):
    """HBM bytes per launch of a kernel from a committed rocprofv3 counter
    summary (profiles/<counters>.json: FETCH_SIZE + WRITE_SIZE per dispatch,
    each divided by the same counter's reading for a copy of known size), if
    it was taken on the current sources of that kernel for this workload;
    else None."""
    path = os.path.join(PROFILES, counters + ".json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel", "").split("<")[0] != kernel or rec.get("workload") != workload:
        return None
    if rec.get("source_sha256_16") != source_digest(KERNEL_SOURCES[kernel]):
        return None
    if split is not None and rec.get("split_tokens") != split:
        return None
    return rec.get("hbm_bytes_per_launch")


def timed(stream, n, fn):
    """Average milliseconds of `fn` (which enqueues GPU work on `stream`) over
    n back-to-back calls, from HIP events on that stream."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(n):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def timed_median(stream, n, fn, trials):
    """Median (and spread) of `trials` runs of timed(stream, n, fn)."""
    runs = sorted(timed(stream, n, fn) for _ in range(max(1, trials)))
    return float(np.median(runs)), runs


def settle(fn, seconds):
    """Repeat `fn` (untimed) until `seconds` of wall clock have passed; returns
    the number of calls.  Steps timed straight after an idle period run up to
    ~20% slower until the GPU's clock has ramped, which takes some tens of ms
    of sustained work."""
    import torch
    n, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            fn()
        n += 8
        torch.cuda.synchronize()
    return n


def copy_reference(args, rec):
    """Untimed plain device copies of a known size after the measurement: the
    calibration reference for the FETCH_SIZE/WRITE_SIZE counters."""
    if args.copy_mb <= 0:
        return
    import torch
    src = torch.empty(args.copy_mb << 20, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(args.steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    rec["copy_reference_bytes"] = args.copy_mb << 20


def thread_count():
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 1) for i in threadpool_info()]
        return max(n) if n else 1
    except Exception:
        return 1


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}); "
              "the LRKV decode path here is single-GPU.", file=sys.stderr)
        sys.exit(2)

    import torch
    import rank_compressed_kv_lrkv_amd as L
    from rank_compressed_kv_lrkv_amd.workloads import DECODE_WORKLOADS, as_f64, decode_inputs

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    L.library()     # fails loudly if the HIP library is missing
    if args.mode == "prefill":
        return bench_prefill(args)
    if args.mode == "chunk":
        return bench_chunk(args)
    if args.mode == "rank-sweep":
        return bench_rank_sweep(args)
    if args.mode == "project":
        return bench_project(args)
    if args.mode == "vendor":
        return bench_vendor(args)
    if args.mode == "train":
        return bench_train(args)
    wl = DECODE_WORKLOADS[args.workload or "mid_bf16_T8k"]
    d = decode_inputs(wl)
    m = measure_decode(args, wl, d, engine=args.engine)
    rec = {
        "metric": "compressed-cache decode: cache tokens/s and achieved HBM GB/s (% of peak)",
        "value": m["tokens_per_s"],
        "unit": "cache tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "trials": args.trials,
        "settle": {"seconds": args.settle_s, "steps": m["settled"]},
        "ms_per_step": m["step_ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": m["dtype"],
        "data": "synthetic (seeded N(0,1) queries, bases and latents; B ~ N(0, 1/r))",
        "config": m["config"],
        "hbm_GBps_step": m["hbm_GBps_step"],
        "hbm_frac_step": m["hbm_frac_step"],
        "kernels_ms": m["kernels_ms"],
        "step_ms_trials": m["step_ms_trials"],
        "wall_s_timed": m["wall_s_timed"],
        "roofline": m["roofline"],
    }
    copy_reference(args, rec)
    progress(f"{wl.name} measured")
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(d, m["out"], args.cpu_seconds, as_f64)
        rec["cpu_baseline"].update(cpu_identity())
        progress("cpu baseline done")
    del m
    if not args.headline_only and args.workload is None and args.engine == 0:
        rec["configs"] = other_configs(args)
    print(json.dumps(rec), flush=True)


def _dev(a, dtype):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def measure_decode(args, wl, d, rotate_mb: float = 0.0, engine: int = 0):
    """Decode steps of one workload: step, scan and merge times (medians of
    the trials), bytes and the roofline of the scan.  With rotate_mb > 0 the
    steps cycle over enough copies of the cache (and queries) that their
    working set exceeds rotate_mb, so no step finds its cache in L2 or the
    Infinity Cache."""
    import torch
    import rank_compressed_kv_lrkv_amd as L

    dt = torch.bfloat16 if d["dtype"] == "bf16" else torch.float32
    B, H, d_h, r = wl.batch, wl.heads, wl.head_dim, wl.rank
    es = 2 if d["dtype"] == "bf16" else 4
    lens_np = np.asarray(d["seq_lens"], np.int32)
    max_len = int(d["capacity"])
    tokens = int(np.minimum(lens_np, max_len).sum())
    cache_bytes = tokens * 2 * (d_h + H * r) * es
    copies = 1
    if rotate_mb > 0:
        per_copy = (d["k_s"].nbytes + d["v_s"].nbytes + d["z_k"].nbytes + d["z_v"].nbytes) / 1e6
        copies = int(np.ceil(rotate_mb / per_copy)) + 1
    lens = torch.from_numpy(lens_np).cuda()
    out = torch.empty((B, H, d_h), dtype=dt, device="cuda")
    calls = []
    keep = []
    for c in range(copies):
        cache = L.LrkvCache(_dev(d["k_s"], d["dtype"]), _dev(d["v_s"], d["dtype"]), _dev(d["z_k"], d["dtype"]),
                            _dev(d["z_v"], d["dtype"]))
        q, b_k, b_v = _dev(d["q"], d["dtype"]), _dev(d["b_k"], d["dtype"]), _dev(d["b_v"], d["dtype"])
        ws = L.decode_workspace(cache, max_len, args.split_tokens, engine)
        calls.append(L.DecodeCall(cache, lens, max_len, q, b_k, b_v, split_tokens=args.split_tokens, out=out,
                                  workspace=ws, engine=engine))
        keep.append((cache, q, b_k, b_v, ws))
    state = {"i": 0}

    def rotating(kind):
        def fn():
            call = calls[state["i"]]
            state["i"] = (state["i"] + 1) % copies
            getattr(call, kind)()
        return fn

    both, scan, combine = rotating("both"), rotating("partial"), rotating("combine")
    settled = settle(both, args.settle_s)
    for _ in range(args.warmup):
        both()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()       # the library launches on torch's current stream
    t0 = time.perf_counter()
    # a step is one lrkv_decode call (scan + merge enqueued together)
    step_ms, step_runs = timed_median(stream, args.steps, both, args.trials)
    wall = time.perf_counter() - t0
    # each kernel's duration: back-to-back launches between one event pair
    scan_ms, _ = timed_median(stream, args.steps, scan, args.trials)
    comb_ms, _ = timed_median(stream, args.steps, combine, args.trials)
    calls[0].both()
    torch.cuda.synchronize()

    scan_bytes = cache_bytes + B * H * d_h * es + H * d_h * r * es          # cache + q + B^K
    step_bytes = cache_bytes + 2 * B * H * d_h * es + 2 * H * d_h * r * es  # + out + B^V
    achieved = scan_bytes / (scan_ms * 1e-3) / 1e9
    scan_kernel = {1: "decode_split_kernel", 2: "decode_mfma_kernel", 3: "decode_generic_kernel",
                   4: "decode_mfma_any_kernel"}.get(engine) or \
        L.lrkv_decode_scan_kernel(dt, H, d_h, r)
    # the any-rank scans merge with decode_merge_generic_kernel; the MFMA one's
    # scan phase also runs decode_absorb_kernel (the absorbed queries) first
    merge_kernel = ("decode_merge_generic_kernel" if scan_kernel in ("decode_generic_kernel", "decode_mfma_any_kernel")
                    else "decode_merge_kernel")
    traffic = None
    for rec_name in ("decode_scan_counters", "decode_valu_scan_counters", "decode_ragged_counters",
                     "decode_any_rank_counters"):
        traffic = traffic or traffic_from_profiles(rec_name, scan_kernel, wl.name, args.split_tokens)
    return {
        "tokens": tokens, "tokens_per_s": tokens / (step_ms * 1e-3), "step_ms": step_ms,
        "step_ms_trials": step_runs, "wall_s_timed": wall, "settled": settled,
        "dtype": "bf16" if d["dtype"] == "bf16" else "f32",
        "config": {"workload": wl.name, "batch": B, "heads": H, "head_dim": d_h, "rank": r,
                   "context": max_len, "cache_tokens": tokens, "split_tokens": args.split_tokens or "default",
                   "cache_MB": cache_bytes / 1e6},
        "hbm_GBps_step": step_bytes / (step_ms * 1e-3) / 1e9,
        "hbm_frac_step": step_bytes / (step_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "kernels_ms": {scan_kernel: scan_ms, merge_kernel: comb_ms},
        "scan_phase_kernels": (["decode_absorb_kernel", scan_kernel] if scan_kernel == "decode_mfma_any_kernel"
                               else [scan_kernel]),
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic,
                     "kernel": scan_kernel, "algorithmic_bytes_per_launch": scan_bytes},
        "copies": copies, "out": out,
    }


def progress(msg):
    print(f"bench: {msg}", file=sys.stderr, flush=True)


def other_configs(args):
    """The synthetic configurations besides the headline: each measured on
    the GPU and checked against the oracle, with the oracle's own rate on
    this host beside it."""
    import torch
    from rank_compressed_kv_lrkv_amd.workloads import DECODE_WORKLOADS, as_f64, decode_inputs

    res = {}
    # Causal prefill (MFMA) first: it runs at the part's power limit, and is
    # measured before the long host-side oracle checks and HBM-bound decodes.
    res["prefill_bf16_L4k"] = prefill_record(args)
    torch.cuda.empty_cache()
    progress("prefill_bf16_L4k done")
    res["train_bf16_L4k"] = train_record(args)
    torch.cuda.empty_cache()
    progress("train_bf16_L4k done")
    # Tiny fp32 decode: latency-bound (19 KB of cache).
    wl = DECODE_WORKLOADS["tiny_f32_T64"]
    d = decode_inputs(wl)
    m = measure_decode(args, wl, d)
    o = oracle_decode_check(d, m["out"], as_f64, budget_s=5.0)
    res[wl.name] = {"kind": "latency", "step_us": m["step_ms"] * 1e3, "kernels_us":
                    {k: v * 1e3 for k, v in m["kernels_ms"].items()}, "cache_tokens": m["tokens"],
                    "gpu_vs_oracle_max_err_over_inf_norm": o["err"], "oracle": o["rate"]}
    progress("tiny_f32_T64 done")
    # Small bf16 decode: the 8.4 MB cache stays in L2 when one copy is reused
    # (a latency); over rotated copies (working set above 2 x (L2 + MALL))
    # each step reads its cache from HBM.
    wl = DECODE_WORKLOADS["small_bf16_T2k"]
    d = decode_inputs(wl)
    m = measure_decode(args, wl, d)
    o = oracle_decode_check(d, m["out"], as_f64, budget_s=5.0)
    mr = measure_decode(args, wl, d, rotate_mb=2 * (32 + 256))
    res[wl.name] = {
        "kind": "latency (L2-resident) and rotated-buffer throughput",
        "l2_resident": {"step_us": m["step_ms"] * 1e3,
                        "kernels_us": {k: v * 1e3 for k, v in m["kernels_ms"].items()}},
        "rotated": {"copies": mr["copies"], "step_us": mr["step_ms"] * 1e3, "cache_tokens_per_s": mr["tokens_per_s"],
                    "hbm_GBps_step": mr["hbm_GBps_step"], "hbm_frac_step": mr["hbm_frac_step"],
                    "kernels_us": {k: v * 1e3 for k, v in mr["kernels_ms"].items()},
                    "scan_frac": mr["roofline"]["frac"]},
        "gpu_vs_oracle_max_err_over_inf_norm": o["err"], "oracle": o["rate"]}
    del m, mr
    torch.cuda.empty_cache()
    progress("small_bf16_T2k done")
    # The headline decode on the vector-ALU scan (no MFMA in decode), for
    # comparison with the default MFMA scan.
    wl = DECODE_WORKLOADS["mid_bf16_T8k"]
    d = decode_inputs(wl)
    m = measure_decode(args, wl, d, engine=1)
    o = oracle_decode_check(d, m["out"], as_f64, budget_s=3.0)
    progress("mid_bf16_T8k on the vector-ALU scan measured")
    res["mid_bf16_T8k_vector_alu_scan"] = {
        "kind": "throughput (the headline shape on decode_split_kernel)", "cache_tokens_per_s": m["tokens_per_s"],
        "step_ms": m["step_ms"], "kernels_ms": m["kernels_ms"], "hbm_GBps_step": m["hbm_GBps_step"],
        "hbm_frac_step": m["hbm_frac_step"], "roofline": m["roofline"],
        "gpu_vs_oracle_max_err_over_inf_norm": o["err"], "checked": o["checked"]}
    del m, d
    torch.cuda.empty_cache()
    # Ragged long-context decode: 16 sequences of 1K-64K tokens, r = 32.
    wl = DECODE_WORKLOADS["ragged_bf16_T1k_64k"]
    d = decode_inputs(wl)
    m = measure_decode(args, wl, d)
    o = oracle_decode_check(d, m["out"], as_f64, budget_s=1e9)    # every (sequence, head) pair
    res[wl.name] = {"kind": "throughput", "cache_tokens": m["tokens"], "cache_tokens_per_s": m["tokens_per_s"],
                    "step_ms": m["step_ms"], "kernels_ms": m["kernels_ms"], "hbm_GBps_step": m["hbm_GBps_step"],
                    "hbm_frac_step": m["hbm_frac_step"], "roofline": m["roofline"],
                    "gpu_vs_oracle_max_err_over_inf_norm": o["err"], "checked": o["checked"], "oracle": o["rate"]}
    del m, d
    torch.cuda.empty_cache()
    progress("ragged_bf16_T1k_64k done")
    # Decode at a rank the pages train (Table 7's largest model: 32 heads,
    # rank 54), on the any-rank MFMA scan.
    wl = DECODE_WORKLOADS["rank54_bf16_T8k"]
    d = decode_inputs(wl)
    m = measure_decode(args, wl, d)
    o = oracle_decode_check(d, m["out"], as_f64, budget_s=5.0)
    res[wl.name] = {"kind": "throughput (any-rank MFMA scan)", "cache_tokens": m["tokens"],
                    "cache_tokens_per_s": m["tokens_per_s"], "step_ms": m["step_ms"], "kernels_ms": m["kernels_ms"],
                    "hbm_GBps_step": m["hbm_GBps_step"], "hbm_frac_step": m["hbm_frac_step"],
                    "roofline": m["roofline"], "config": m["config"],
                    "gpu_vs_oracle_max_err_over_inf_norm": o["err"], "checked": o["checked"], "oracle": o["rate"]}
    del m, d
    torch.cuda.empty_cache()
    progress("rank54_bf16_T8k done")
    return res


def oracle_decode_check(d, out_dev, as_f64, budget_s):
    """The oracle, one whole sequence (all heads) at a time until budget_s of
    wall clock is spent, against the GPU output; its rate on this host."""
    sys.path.insert(0, ROOT)
    import oracle as O
    got = out_dev.float().cpu().numpy().astype(np.float64)
    dt = d["dtype"]
    f = lambda k: as_f64(d[k], dt)
    bk, bv, q = f("b_k"), f("b_v"), f("q")
    lens = np.asarray(d["seq_lens"])
    toks, secs, err, done = 0, 0.0, 0.0, 0
    for b in range(len(lens)):
        L_ = int(lens[b])
        args = (q[b:b + 1], as_f64(d["k_s"][b:b + 1, :L_], dt), as_f64(d["v_s"][b:b + 1, :L_], dt),
                as_f64(d["z_k"][b:b + 1, :L_], dt), as_f64(d["z_v"][b:b + 1, :L_], dt), bk, bv, lens[b:b + 1])
        t = time.perf_counter()
        want = O.decode(*args)
        secs += time.perf_counter() - t
        toks += L_
        done += 1
        err = max(err, float(np.max(np.abs(got[b] - want[0])) / max(np.max(np.abs(want[0])), 1e-30)))
        if secs >= budget_s:
            break
    return {"err": err, "checked": f"{done} of {len(lens)} sequences, all heads",
            "rate": {"value": toks / secs, "unit": "cache tokens/s", "cores": thread_count(), "kind": "oracle",
                     "sample": f"{done} of {len(lens)} sequences, all heads ({toks} cache tokens), float64 numpy, "
                               f"{secs:.2f} s"}}


def cpu_identity():
    """The host CPU model and the single-thread oracle rate on the small decode configs."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    single = {}
    try:
        from threadpoolctl import threadpool_limits
        from rank_compressed_kv_lrkv_amd.workloads import DECODE_WORKLOADS, as_f64, decode_inputs
        sys.path.insert(0, ROOT)
        import oracle as O
        with threadpool_limits(limits=1):
            for name, budget in (("tiny_f32_T64", 1.0), ("small_bf16_T2k", 3.0), ("mid_bf16_T8k", 5.0)):
                d = decode_inputs(DECODE_WORKLOADS[name])
                dt = d["dtype"]
                f = lambda k: as_f64(d[k], dt)
                lens = np.asarray(d["seq_lens"])
                toks, secs, done = 0, 0.0, 0
                for b in range(len(lens)):
                    L_ = int(lens[b])
                    a = (f("q")[b:b + 1], as_f64(d["k_s"][b:b + 1, :L_], dt), as_f64(d["v_s"][b:b + 1, :L_], dt),
                         as_f64(d["z_k"][b:b + 1, :L_], dt), as_f64(d["z_v"][b:b + 1, :L_], dt), f("b_k"),
                         f("b_v"), lens[b:b + 1])
                    t = time.perf_counter()
                    O.decode(*a)
                    secs += time.perf_counter() - t
                    toks += L_
                    done += 1
                    if secs >= budget:
                        break
                single[name] = {"cache_tokens_per_s": toks / secs, "sample": f"{done} of {len(lens)} sequences",
                                "seconds": secs}
    except Exception as e:      # the baseline is a report; never fail the bench for it
        single["error"] = str(e)[:200]
    return {"cpu_model": model, "logical_cpus_visible": len(os.sched_getaffinity(0)),
            "single_thread": single}


MFMA_BF16_PEAK_TFLOPS = 2500.0
FP32_VECTOR_PEAK_TFLOPS = 157.3   # published fp32 vector peak (packed fp32 FMAs)


def prefill_record(args):
    """Causal prefill of the 4 x 4096-token workload (H=32, d_h=128, r=16):
    the attention kernel alone (its TFLOP/s priced against the bf16 MFMA
    peak) and lrkv_prefill with the cache written (the step); sampled query
    rows checked against the oracle, and the oracle's rate on this host."""
    import torch
    import rank_compressed_kv_lrkv_amd as L
    from rank_compressed_kv_lrkv_amd.workloads import PREFILL_WORKLOADS, as_f64, prefill_inputs

    wl = PREFILL_WORKLOADS[args.workload if args.mode == "prefill" and args.workload else "prefill_bf16_L4k"]
    d = prefill_inputs(wl)
    t = {k: _dev(d[k], "bf16") for k in ("q", "k_s", "v_s", "z_k", "z_v", "b_k", "b_v")}
    B, Lq, H, d_h, r = wl.batch, wl.seq_len, wl.heads, wl.head_dim, wl.rank
    cache = L.LrkvCache.empty(B, H, d_h, r, Lq, dtype=torch.bfloat16)
    out = torch.empty_like(t["q"])

    def step(with_cache=True):
        L.lrkv_prefill(t["q"], t["k_s"], t["v_s"], t["z_k"], t["z_v"], t["b_k"], t["b_v"],
                       cache=cache if with_cache else None, out=out)

    settled = settle(step, args.settle_s)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    steps = max(1, min(args.steps, 20))
    step_ms, _ = timed_median(stream, steps, step, args.trials)
    kern_ms, kern_runs = timed_median(stream, steps, lambda: step(with_cache=False), args.trials)
    torch.cuda.synchronize()

    pairs = B * H * Lq * (Lq + 1) // 2                       # causal (query, key) pairs
    flops = pairs * 4 * (d_h + r) + B * H * Lq * 4 * d_h * r  # Eq. (6)-(7) contractions + absorption
    tflops = flops / (kern_ms * 1e-3) / 1e12
    kernel = L.lrkv_prefill_kernel(torch.bfloat16, H, d_h, r)
    # the MFMA kernels are priced against the bf16 MFMA peak, the vector-ALU
    # kernel (fp32 FMAs) against the fp32 vector peak
    mfma = kernel in ("prefill_kernel", "prefill_wide_kernel")
    bound, peak = ("mfma", MFMA_BF16_PEAK_TFLOPS) if mfma else ("alu", FP32_VECTOR_PEAK_TFLOPS)
    rec = {
        "value": B * Lq / (step_ms * 1e-3), "unit": "prefill tokens/s (cache written)",
        "settle": {"seconds": args.settle_s, "steps": settled}, "ms_per_step": step_ms, "steps": steps,
        "config": {"workload": wl.name, "batch": B, "seq_len": Lq, "heads": H, "head_dim": d_h, "rank": r},
        "kernels_ms": {kernel: kern_ms}, "prefill_kernel_ms_trials": kern_runs,
        "causal_pairs_per_s": pairs / (kern_ms * 1e-3),
        "roofline": {"bound": bound, "achieved": tflops, "peak": peak, "unit": "TFLOP/s",
                     "frac": tflops / peak,
                     "traffic": traffic_from_profiles("prefill_counters", kernel, wl.name),
                     "kernel": kernel, "algorithmic_flops_per_launch": flops},
    }
    if not args.no_cpu_baseline:
        rec.update(oracle_prefill_check(d, out, as_f64))
    return rec


def train_record(args):
    """One training step of LRKV attention on the 4 x 4096-token prefill
    workload (H=32, d_h=128, r=16): lrkv_train_forward (the causal prefill
    kernel, also writing each row's log-sum-exp) and lrkv_train_backward
    (fp32 gradients of q, K_s, V_s, Z^K, Z^V, B^K, B^V), timed apart.  Their
    TFLOP/s are priced against the bf16 MFMA peak with the algorithmic flops
    of the absorbed products: 2 per causal pair and inner dimension (d_h + r)
    for each of S and P.V in the forward, and of S, dP, dV, dK, dQ in the
    backward.  Sampled (sequence, head) pairs of dq, dz_k, dz_v are checked
    against the float64 gradient oracle, whose rate is reported beside."""
    import torch
    import rank_compressed_kv_lrkv_amd as L
    from rank_compressed_kv_lrkv_amd.workloads import PREFILL_WORKLOADS, as_f64, train_inputs

    wl = PREFILL_WORKLOADS["prefill_bf16_L4k"]
    d = train_inputs(wl)
    names = ("q", "k_s", "v_s", "z_k", "z_v", "b_k", "b_v")
    t = {k: _dev(d[k], "bf16") for k in names + ("d_out",)}
    B, Lq, H, d_h, r = wl.batch, wl.seq_len, wl.heads, wl.head_dim, wl.rank
    ins = [t[k] for k in names]
    out, lse = L.lrkv_train_forward(*ins)
    ws = torch.empty(L.lrkv_train_backward_workspace_size(torch.bfloat16, B, H, d_h, r, Lq), dtype=torch.uint8,
                     device="cuda")
    grads = L.lrkv_train_backward(*ins, out, lse, t["d_out"], workspace=ws)

    def fwd():
        L.lrkv_train_forward(*ins, out=out, lse=lse)

    def bwd():
        L.lrkv_train_backward(*ins, out, lse, t["d_out"], workspace=ws, grads=grads)

    def step():
        fwd()
        bwd()

    settled = settle(step, args.settle_s)
    for _ in range(max(1, args.warmup // 4)):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    steps = max(1, min(args.steps, 5))
    step_ms, step_runs = timed_median(stream, steps, step, args.trials)
    fwd_ms, _ = timed_median(stream, steps, fwd, args.trials)
    bwd_ms, _ = timed_median(stream, steps, bwd, args.trials)
    fwd(); bwd()
    torch.cuda.synchronize()
    pairs = B * H * Lq * (Lq + 1) // 2
    fwd_flops = pairs * 4 * (d_h + r)
    bwd_flops = pairs * 10 * (d_h + r)
    tf = lambda fl, ms: fl / (ms * 1e-3) / 1e12
    rec = {
        "kind": "training step (forward + backward), throughput",
        "value": B * Lq / (step_ms * 1e-3), "unit": "training tokens/s (forward + backward)",
        "step_ms": step_ms, "step_ms_trials": step_runs, "settle": {"seconds": args.settle_s, "steps": settled},
        "config": {"workload": wl.name, "batch": B, "seq_len": Lq, "heads": H, "head_dim": d_h, "rank": r},
        "forward_ms": fwd_ms, "backward_ms": bwd_ms,
        "forward_tflops": tf(fwd_flops, fwd_ms), "backward_tflops": tf(bwd_flops, bwd_ms),
        "roofline": {"bound": "mfma", "achieved": tf(bwd_flops, bwd_ms), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": tf(bwd_flops, bwd_ms) / MFMA_BF16_PEAK_TFLOPS, "traffic": None,
                     "kernel": "lrkv_train_backward (all its kernels)", "algorithmic_flops_per_launch": bwd_flops},
    }
    if not args.no_cpu_baseline:
        sys.path.insert(0, ROOT)
        import oracle as O
        f = lambda k: as_f64(d[k], "bf16")
        got = {k: v.cpu().numpy().astype(np.float64) for k, v in grads.items()}
        err, secs, npairs = 0.0, 0.0, 0
        for b, h in ((0, 0), (B - 1, H - 1)):
            sl = lambda k: f(k)[b:b + 1][:, :, [h]]
            t0 = time.perf_counter()
            want = O.prefill_backward(sl("q"), f("k_s")[b:b + 1], f("v_s")[b:b + 1], sl("z_k"), sl("z_v"),
                                      f("b_k")[[h]], f("b_v")[[h]], sl("d_out"))
            secs += time.perf_counter() - t0
            npairs += Lq * (Lq + 1) // 2
            for k in ("dq", "dz_k", "dz_v"):
                g = got[k][b:b + 1][:, :, [h]]
                err = max(err, float(np.max(np.abs(g - want[k])) / np.max(np.abs(want[k]))))
        rec["gpu_vs_oracle_max_err_over_inf_norm"] = err
        rec["checked"] = "dq, dz_k, dz_v of (sequence, head) = (0, 0) and (3, 31), every query and key"
        rec["oracle"] = {"value": npairs / secs, "unit": "causal pairs/s (forward recompute + backward)",
                         "cores": thread_count(), "kind": "oracle",
                         "sample": f"float64 numpy backward of 2 (sequence, head) pairs at 4096 tokens, {secs:.1f} s"}
    return rec


def bench_train(args):
    """--mode train: the training step as the headline line."""
    r = train_record(args)
    rec = {
        "metric": "LRKV attention training step: tokens/s, forward and backward TFLOP/s",
        "value": r.pop("value"), "unit": r.pop("unit"), "n_gpus": 1, "steps": max(1, min(args.steps, 5)),
        "warmup": args.warmup, "trials": args.trials, "ms_per_step": r.pop("step_ms"),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) queries, bases, latents and upstream gradient; B ~ N(0, 1/r))",
        **r,
    }
    copy_reference(args, rec)
    print(json.dumps(rec), flush=True)


def oracle_prefill_check(d, out_dev, as_f64, budget_s=8.0):
    """Sampled rows of the prefill output against the oracle (query row i of
    head h over keys 0..i, one by one), and the oracle's rate in causal
    (query, key) pairs per second on this host (whole rows, all heads, until
    budget_s is spent)."""
    sys.path.insert(0, ROOT)
    import oracle as O
    got = out_dev.float().cpu().numpy().astype(np.float64)
    f = lambda k: as_f64(d[k], "bf16")
    q, b_k, b_v = f("q"), f("b_k"), f("b_v")
    B, Lq, H, _ = q.shape
    err, checked = 0.0, 0
    for b, h in ((0, 0), (B - 1, H - 1), (B // 2, H // 2 + 1)):
        for i in (0, 1, 31, 32, 33, Lq // 4, Lq // 2 - 1, Lq - 1):
            n = i + 1
            want = O.decode(q[b:b + 1, i][:, [h]], as_f64(d["k_s"][b:b + 1, :n], "bf16"),
                            as_f64(d["v_s"][b:b + 1, :n], "bf16"), as_f64(d["z_k"][b:b + 1, :n][:, :, [h]], "bf16"),
                            as_f64(d["z_v"][b:b + 1, :n][:, :, [h]], "bf16"), b_k[[h]], b_v[[h]], [n])[0, 0]
            err = max(err, float(np.max(np.abs(got[b, i, h] - want)) / np.max(np.abs(want))))
            checked += 1
    # oracle rate: the plain prefill of the first n rows of sequence 0, all
    # heads, for n = 256, 512, ... while the next size (about 4x the cost of
    # the last) still fits the budget
    t0 = time.perf_counter()
    secs, rows, pairs, last, n = 0.0, 0, 0, 0.0, 256
    while n <= Lq and secs + 4.5 * last < budget_s:
        t = time.perf_counter()
        O.prefill(q[:1, :n], f("k_s")[:1, :n], f("v_s")[:1, :n], f("z_k")[:1, :n], f("z_v")[:1, :n], b_k, b_v)
        last = time.perf_counter() - t
        secs += last
        pairs += H * n * (n + 1) // 2
        rows = n
        n *= 2
    return {"gpu_vs_oracle_max_err_over_inf_norm": err, "checked": f"{checked} (sequence, head, query row) samples",
            "oracle": {"value": pairs / secs, "unit": "causal pairs/s", "cores": thread_count(), "kind": "oracle",
                       "sample": f"plain causal prefill of the first 256..{rows} tokens of sequence 0, all {H} heads, "
                                 f"float64 numpy, {secs:.1f} s"},
            "oracle_wall_s": time.perf_counter() - t0}


def bench_prefill(args):
    """--mode prefill: the prefill workload as the headline line."""
    r = prefill_record(args)
    rec = {
        "metric": "causal prefill over the LRKV cache: TFLOP/s and MFMA utilisation",
        "value": r.pop("value"), "unit": r.pop("unit"),
        "n_gpus": 1, "steps": r.pop("steps"), "warmup": args.warmup, "trials": args.trials,
        "settle": r.pop("settle"), "ms_per_step": r.pop("ms_per_step"),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) queries, bases and latents; B ~ N(0, 1/r))",
        **r,
    }
    copy_reference(args, rec)
    print(json.dumps(rec), flush=True)


def bench_chunk(args):
    """A prefill chunk over cached history: 4 sequences with 4096 cached
    tokens each take 512 new tokens (H=32, d_h=128, r=16); a step is one
    lrkv_prefill_chunk call (cache write + attention over 4096 + i + 1 keys)."""
    import torch
    import rank_compressed_kv_lrkv_amd as L
    from rank_compressed_kv_lrkv_amd.workloads import chunk_inputs

    B, H, d_h, r, hist, n = 4, 32, 128, 16, 4096, 512
    d = chunk_inputs(batch=B, heads=H, head_dim=d_h, rank=r, capacity=hist + n, starts=[hist] * B, n_new=n,
                     seed=20261207)

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

    cache = L.LrkvCache(*(dev(d["cache_" + k]) for k in ("k_s", "v_s", "z_k", "z_v")))
    t = {k: dev(d[k]) for k in ("q", "k_s", "v_s", "z_k", "z_v", "b_k", "b_v")}
    start = torch.full((B,), hist, dtype=torch.int32, device="cuda")
    out = torch.empty_like(t["q"])

    def step():
        L.lrkv_prefill_chunk(cache, start, hist, t["q"], t["k_s"], t["v_s"], t["z_k"], t["z_v"], t["b_k"], t["b_v"],
                             out=out)

    settled = settle(step, args.settle_s)
    for _ in range(args.warmup):
        step()
    stream = torch.cuda.current_stream()
    step_ms = timed(stream, args.steps, step)
    pairs = B * H * (n * hist + n * (n + 1) // 2)             # (query, key) pairs under the shifted causal mask
    flops = pairs * 4 * (d_h + r) + B * H * n * 4 * d_h * r
    tflops = flops / (step_ms * 1e-3) / 1e12
    rec = {
        "metric": "prefill chunk over a cached history: new tokens/s and TFLOP/s",
        "value": B * n / (step_ms * 1e-3), "unit": "new tokens/s (cache written)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "settle": {"seconds": args.settle_s, "steps": settled}, "ms_per_step": step_ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) history, queries, rows and latents; B ~ N(0, 1/r))",
        "config": {"workload": "chunk_bf16_hist4k_new512", "batch": B, "history": hist, "new_tokens": n,
                   "heads": H, "head_dim": d_h, "rank": r},
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": tflops / MFMA_BF16_PEAK_TFLOPS, "traffic": None,
                     "kernel": "append_kernel + prefill_kernel", "algorithmic_flops_per_launch": flops},
    }
    print(json.dumps(rec), flush=True)


def bench_project(args):
    """Fused projection + append: the cache rows of 4 sequences x 4096 new
    tokens computed from hidden states of width d = H d_h = 4096 (H=32,
    d_h=128, r=16: 1280 outputs per token) and written into the cache; a step
    is one lrkv_project_append call (one bf16 MFMA GEMM with the cache
    scatter in its epilogue).  The same call for one token per sequence over
    32 sequences (a decode step's projection) is timed beside it."""
    import torch
    import rank_compressed_kv_lrkv_amd as L
    from rank_compressed_kv_lrkv_amd.workloads import projection_inputs

    B, n, d, H, d_h, r = 4, 4096, 4096, 32, 128, 16
    inp = projection_inputs(batch=B, n_new=n, d_model=d, heads=H, head_dim=d_h, rank=r, dtype="bf16",
                            seed=20261208)

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

    w = L.lrkv_pack_projection(dev(inp["wk"]), dev(inp["wv"]), dev(inp["uk"]), dev(inp["uv"]))
    x = dev(inp["x"])
    cache = L.LrkvCache.empty(B, H, d_h, r, n, dtype=torch.bfloat16, zero=False)
    pos = torch.zeros(B, dtype=torch.int32, device="cuda")

    def step():
        L.lrkv_project_append(cache, pos, x, w, workspace=None)

    settled = settle(step, args.settle_s)
    for _ in range(args.warmup):
        step()
    stream = torch.cuda.current_stream()
    step_ms = timed(stream, args.steps, step)
    N = 2 * (d_h + H * r)
    flops = 2 * B * n * N * d
    kernel = L.lrkv_project_kernel(torch.bfloat16, B, n, H, d_h, r, d)
    tflops = flops / (step_ms * 1e-3) / 1e12
    # decode-step shape: 32 sequences, one token each, same weights
    Bd = 32
    xd = torch.randn(Bd, 1, d, device="cuda").to(torch.bfloat16)
    cache_d = L.LrkvCache.empty(Bd, H, d_h, r, 64, dtype=torch.bfloat16, zero=False)
    pos_d = torch.full((Bd,), 5, dtype=torch.int32, device="cuda")
    ws_d = torch.empty(max(L.lrkv_project_workspace_size(torch.bfloat16, Bd, 1, H, d_h, r, d), 16),
                       dtype=torch.uint8, device="cuda")
    dec = lambda: L.lrkv_project_append(cache_d, pos_d, xd, w, workspace=ws_d)
    for _ in range(args.warmup):
        dec()
    dec_ms = timed(stream, args.steps, dec)
    dec_bytes = N * d * 2 + Bd * d * 2 + Bd * N * 2
    rec = {
        "metric": "fused projection + append: new tokens/s and TFLOP/s",
        "value": B * n / (step_ms * 1e-3), "unit": "new tokens/s (cache written)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "settle": {"seconds": args.settle_s, "steps": settled}, "ms_per_step": step_ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded hidden states N(0,1), projection weights N(0, 1/d))",
        "config": {"workload": "project_bf16_B4_L4096_d4096", "batch": B, "new_tokens": n, "d_model": d,
                   "heads": H, "head_dim": d_h, "rank": r, "outputs_per_token": N},
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": tflops / MFMA_BF16_PEAK_TFLOPS,
                     "traffic": traffic_from_profiles("project_counters", kernel, "project_bf16_B4_L4096_d4096"),
                     "kernel": kernel, "algorithmic_flops_per_launch": flops},
        "decode_shape": {"batch": Bd, "new_tokens": 1, "ms": dec_ms, "algorithmic_bytes": dec_bytes,
                         "kernel": L.lrkv_project_kernel(torch.bfloat16, Bd, 1, H, d_h, r, d, True),
                         "GB_per_s": dec_bytes / (dec_ms * 1e-3) / 1e9},
    }
    copy_reference(args, rec)
    print(json.dumps(rec), flush=True)


def bench_vendor(args):
    """Vendor libraries at the shapes of the two MFMA kernels, timed beside
    them in one process (context, not the LRKV computation):
    - hipBLASLt (torch.matmul, bf16) on the projection GEMM, 16384 x 4096 x
      1280, against lrkv_project_append of the same size (random packed W);
    - PyTorch's flash-attention backend (forced: no fallback to the math
      path) on dense causal MHA of the prefill workload's shape (B=4, H=32,
      L=4096, d=128), against lrkv_prefill's attention kernel (no cache
      write) on LRKV inputs of that shape with r = 16.
    Inputs are torch.randn on the device; each call is settled, warmed up
    and timed like the other modes."""
    import torch
    import torch.nn.functional as F
    import rank_compressed_kv_lrkv_amd as L
    from torch.nn.attention import SDPBackend, sdpa_kernel

    stream = torch.cuda.current_stream()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(20261209)

    def randn(*shape, scale=1.0):
        return (torch.randn(*shape, device="cuda", generator=gen) * scale).to(torch.bfloat16)

    def run(fn):
        settle(fn, args.settle_s)
        for _ in range(args.warmup):
            fn()
        return timed(stream, args.steps, fn)

    B, n, d, H, d_h, r = 4, 4096, 4096, 32, 128, 16
    N, M = 2 * (d_h + H * r), B * n
    gemm_flops = 2 * M * N * d
    x = randn(B, n, d)
    w = randn(N, d, scale=d ** -0.5)                          # the packed layout [N][d]
    wt = w.t().contiguous()
    out = torch.empty(M, N, device="cuda", dtype=torch.bfloat16)
    x2 = x.view(M, d)
    blas_ms = run(lambda: torch.matmul(x2, wt, out=out))
    cache = L.LrkvCache.empty(B, H, d_h, r, n, dtype=torch.bfloat16, zero=False)
    pos = torch.zeros(B, dtype=torch.int32, device="cuda")
    proj_ms = run(lambda: L.lrkv_project_append(cache, pos, x, w, workspace=None))
    del x, x2, w, wt, out, cache

    Lq = n
    pairs = B * H * Lq * (Lq + 1) // 2
    mha_flops = pairs * 4 * d_h
    lrkv_flops = pairs * 4 * (d_h + r) + B * H * Lq * 4 * d_h * r
    q_l = randn(B, Lq, H, d_h)
    t = {"k_s": randn(B, Lq, d_h), "v_s": randn(B, Lq, d_h), "z_k": randn(B, Lq, H, r), "z_v": randn(B, Lq, H, r),
         "b_k": randn(H, d_h, r, scale=r ** -0.5), "b_v": randn(H, d_h, r, scale=r ** -0.5)}
    o_l = torch.empty_like(q_l)
    lrkv_ms = run(lambda: L.lrkv_prefill(q_l, t["k_s"], t["v_s"], t["z_k"], t["z_v"], t["b_k"], t["b_v"], out=o_l))
    del q_l, t, o_l
    q, k, v = randn(B, H, Lq, d_h), randn(B, H, Lq, d_h), randn(B, H, Lq, d_h)
    flash = {"backend": "torch SDPA, FLASH_ATTENTION only", "shape": [B, H, Lq, d_h], "causal": True}
    try:
        with sdpa_kernel([SDPBackend.FLASH_ATTENTION]):
            fa_ms = run(lambda: F.scaled_dot_product_attention(q, k, v, is_causal=True))
        fa_tf = mha_flops / (fa_ms * 1e-3) / 1e12
        flash.update({"ms": fa_ms, "TFLOP/s": fa_tf, "frac": fa_tf / MFMA_BF16_PEAK_TFLOPS})
    except RuntimeError as e:
        flash["unavailable"] = str(e)[:200]

    def entry(ms, flops, **kw):
        tf = flops / (ms * 1e-3) / 1e12
        return {"ms": ms, "TFLOP/s": tf, "frac": tf / MFMA_BF16_PEAK_TFLOPS, **kw}

    rec = {
        "metric": "vendor libraries beside the LRKV MFMA kernels (context)",
        "peak_TFLOPs": MFMA_BF16_PEAK_TFLOPS, "dtype": "bf16", "steps": args.steps, "warmup": args.warmup,
        "projection_gemm": {
            "shape_MxKxN": [M, d, N],
            "hipblaslt_torch_matmul": entry(blas_ms, gemm_flops),
            "lrkv_project_append": entry(proj_ms, gemm_flops,
                                         kernel=L.lrkv_project_kernel(torch.bfloat16, B, n, H, d_h, r, d)),
        },
        "causal_prefill": {
            "mha_flash_attention": flash,
            "lrkv_prefill_kernel": entry(lrkv_ms, lrkv_flops, rank=r),
        },
    }
    print(json.dumps(rec), flush=True)


def bench_rank_sweep(args):
    """Decode on the headline shape (32 sequences x 8192 tokens, H=32, d_h=128)
    at ranks 0 (the MQA cache), 8, 16 and 32: cache elements per token
    2(d_h + H r) and the measured step, to show how the cache ratio turns
    into time; then the plain MHA decode (2 H d_h elements per token) at the
    same shape.  One JSON line per point."""
    import torch
    import rank_compressed_kv_lrkv_amd as L
    from rank_compressed_kv_lrkv_amd.workloads import DecodeWorkload, decode_inputs

    for r in (0, 8, 16, 32):
        wl = DecodeWorkload(f"mid_bf16_T8k_r{r}", 32, 32, 128, r, 8192, "bf16", 20261204)
        d = decode_inputs(wl)

        def dev(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

        cache = L.LrkvCache(dev(d["k_s"]), dev(d["v_s"]), dev(d["z_k"]), dev(d["z_v"]))
        q, b_k, b_v = dev(d["q"]), dev(d["b_k"]), dev(d["b_v"])
        lens = torch.from_numpy(np.asarray(d["seq_lens"], np.int32)).cuda()
        call = L.DecodeCall(cache, lens, 8192, q, b_k, b_v)
        settle(call.both, args.settle_s)
        for _ in range(args.warmup):
            call.both()
        stream = torch.cuda.current_stream()
        step_ms = timed(stream, args.steps, call.both)
        scan_ms = timed(stream, args.steps, call.partial)
        elems = L.lrkv_cache_elems_per_token(32, 128, r)
        cache_bytes = 32 * 8192 * elems * 2
        print(json.dumps({
            "metric": "decode step vs rank", "workload": wl.name, "rank": r, "cache_elems_per_token": elems,
            "cache_ratio_vs_mha": elems / (2 * 32 * 128), "cache_MB": cache_bytes / 1e6,
            "scan_kernel": L.lrkv_decode_scan_kernel(torch.bfloat16, 32, 128, r),
            "ms_per_step": step_ms, "scan_ms": scan_ms,
            "cache_tokens_per_s": 32 * 8192 / (step_ms * 1e-3),
            "scan_hbm_frac": cache_bytes / (scan_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        }), flush=True)
        del cache, q, b_k, b_v, call
        torch.cuda.empty_cache()

    # the plain MHA cache at the same shape: every head's own K and V rows
    B, T, H, d_h = 32, 8192, 32, 128
    gen = torch.Generator(device="cuda").manual_seed(20261209)
    k = torch.randn(B, T, H, d_h, device="cuda", generator=gen).to(torch.bfloat16)
    v = torch.randn(B, T, H, d_h, device="cuda", generator=gen).to(torch.bfloat16)
    q = torch.randn(B, H, d_h, device="cuda", generator=gen).to(torch.bfloat16)
    lens = torch.full((B,), T, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    ws = torch.empty(max(L.lrkv_mha_decode_workspace_size(torch.bfloat16, B, H, d_h, T, T), 16), dtype=torch.uint8,
                     device="cuda")
    step = lambda: L.lrkv_mha_decode(k, v, lens, T, q, out=out, workspace=ws)
    settle(step, args.settle_s)
    for _ in range(args.warmup):
        step()
    step_ms = timed(torch.cuda.current_stream(), args.steps, step)
    elems = 2 * H * d_h
    cache_bytes = B * T * elems * 2
    print(json.dumps({
        "metric": "decode step vs rank", "workload": "mha_bf16_T8k", "rank": None, "mechanism": "mha",
        "cache_elems_per_token": elems, "cache_ratio_vs_mha": 1.0, "cache_MB": cache_bytes / 1e6,
        "scan_kernel": "mha_split_kernel", "ms_per_step": step_ms,
        "cache_tokens_per_s": B * T / (step_ms * 1e-3),
        "step_hbm_frac": cache_bytes / (step_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
    }), flush=True)


def cpu_baseline(d, out_dev, budget_s, as_f64):
    """Time the float64 oracle, one whole sequence (all heads) at a time, on
    the host cores until the budget is spent; compare with the GPU output."""
    sys.path.insert(0, ROOT)
    import oracle as O
    got = out_dev.float().cpu().numpy().astype(np.float64)
    dt = d["dtype"]
    f = lambda k: as_f64(d[k], dt)
    bk, bv = f("b_k"), f("b_v")
    q = f("q")
    lens = np.asarray(d["seq_lens"])
    toks, secs, errs, done = 0, 0.0, [], 0
    for b in range(len(lens)):
        L_ = int(lens[b])
        args = (q[b:b + 1], as_f64(d["k_s"][b:b + 1, :L_], dt), as_f64(d["v_s"][b:b + 1, :L_], dt),
                as_f64(d["z_k"][b:b + 1, :L_], dt), as_f64(d["z_v"][b:b + 1, :L_], dt), bk, bv, lens[b:b + 1])
        t = time.perf_counter()
        want = O.decode(*args)
        secs += time.perf_counter() - t
        toks += L_
        done += 1
        errs.append(float(np.max(np.abs(got[b] - want[0])) / max(np.max(np.abs(want[0])), 1e-30)))
        if secs >= budget_s:
            break
    return {"value": toks / secs, "unit": "cache tokens/s", "cores": thread_count(), "kind": "oracle",
            "sample": f"{done} of {len(lens)} sequences, all heads ({toks} cache tokens), float64 numpy, "
                      f"{secs:.1f} s",
            "gpu_vs_oracle_max_err_over_inf_norm": max(errs)}


if __name__ == "__main__":
    main()
