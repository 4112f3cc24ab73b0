"""Benchmark of the FlashMask forward path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--warmup-seconds S] [--config C2]
                    [--no-per-config] [--no-cpu-baseline] [--no-backward] [--no-fp8]

A step is one fm_attn_fwd call (interval preprocessor + scheduler + attention
kernel) over one batch of the workload, inputs resident in HBM.  Untimed
warm-up: W steps, then more until S seconds (default 1) have run, so that the
GPU's clocks have reached their sustained level (S / 4 for the other legs).
Prints ONE
JSON line: effective TFLOP/s counting 4*d FLOPs per attended (query, key)
pair, the attention kernel's roofline figures (its own duration measured with
HIP events the library records on its stream), the other workloads' figures
under "per_config", the backward pass (fm_attn_bwd, 10*d FLOPs per attended
pair) under "backward", the FP8-input forward (fm_attn_fwd_fp8) under
"fp8_forward" (bf16 weights) and "fp8_all_forward" (e4m3 weights), and the CPU
oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

METRIC = "effective masked-attn fwd TFLOP/s (unmasked FLOPs) + % of bf16 MFMA peak"
DEFAULT_CONFIG = "C2"
HERE = os.path.dirname(os.path.abspath(__file__))


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--warmup-seconds", type=float, default=1.0,
                    help="after the W warm-up steps, keep warming up (untimed) until this many seconds of "
                         "GPU work have run (the main workload; other legs use a quarter of it): the "
                         "GPU's clocks take a while to reach their sustained level")
    ap.add_argument("--config", default=DEFAULT_CONFIG)
    ap.add_argument("--no-per-config", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward-pass figures")
    ap.add_argument("--no-fp8", action="store_true", help="skip the FP8-input forward figures")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="after timing, run a plain device copy of this many MiB three times "
                         "(a known-size reference for hardware byte counters)")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def tile_stats(fm, spec, cfg, dev):
    """Skip / partial ratios at the kernel's tile shape, from the GPU class table."""
    import torch
    Br, Bc = fm.fm_attn_tile_shape(cfg.d)
    skip = part = total = 0
    nonskip = 0
    multi = spec.col_start.ndim == 3
    for b in range(cfg.B):
        s = torch.from_numpy(spec.col_start[b]).to(dev)
        e = torch.from_numpy(spec.col_end[b]).to(dev)
        classify = fm.fm_classify_tiles_multi if multi else fm.fm_classify_tiles
        tab = classify(s, e, Br, Bc).cpu().numpy()
        skip += int((tab == fm.FM_TILE_SKIP).sum())
        part += int((tab == fm.FM_TILE_PARTIAL).sum())
        total += tab.size
        nonskip += int((tab != fm.FM_TILE_SKIP).sum())
    executed = 4 * cfg.d * Br * Bc * nonskip * cfg.H
    return {"Br": Br, "Bc": Bc, "skip_ratio": skip / total, "partial_ratio": part / total,
            "tile_executed_flops": executed}


def warm_up(step, count, seconds):
    """count untimed calls of step(), then more until `seconds` of wall time have passed."""
    import torch
    for _ in range(count):
        step()
    torch.cuda.synchronize()
    t0 = time.time()
    while time.time() - t0 < seconds:
        for _ in range(8):
            step()
        torch.cuda.synchronize()


def time_config(cfg, steps, warmup, with_kernel_timer=True, warm_s=0.0):
    import torch
    from masked_attention_fm_amd import flashmask as fm
    from masked_attention_fm_amd import inputs, metrics

    dev = torch.device("cuda:0")
    spec = inputs.config_intervals(cfg)
    t0 = time.time()
    q, k, v = inputs.make_qkv(cfg.B, cfg.H, cfg.N, cfg.d, cfg.seed)
    q, k, v = (x.to(dev) for x in (q, k, v))
    cs = torch.from_numpy(spec.col_start).to(dev)
    ce = torch.from_numpy(spec.col_end).to(dev)
    out = torch.empty_like(q)
    lse = torch.empty(cfg.B, cfg.H, cfg.N, dtype=torch.float32, device=dev)
    scale = inputs.default_scale(cfg.d)
    log(f"{cfg.key}: inputs ready in {time.time() - t0:.1f}s ({cfg.describe()})")

    U = metrics.spec_attended_pairs(spec.col_start, spec.col_end, cfg.N) * cfg.H
    flops = 4 * cfg.d * U
    stream = torch.cuda.current_stream()
    # rows with several ranges ([B, K, N] intervals) take the multi-range entry point
    attn = fm.fm_attn_fwd_multi if spec.col_start.ndim == 3 else fm.fm_attn_fwd

    warm_up(lambda: attn(q, k, v, cs, ce, scale, out=out, lse=lse, stream=stream), warmup, warm_s)
    fm.fm_profile_read()                       # drop anything recorded before

    # Pass 1: the timed steps, uninstrumented.
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(steps):
        attn(q, k, v, cs, ce, scale, out=out, lse=lse, stream=stream)
    stop.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)

    # Pass 2: the same steps with the library's per-launch event pair, for the
    # attention kernel's own duration (the event pair adds a few microseconds
    # per call, so this pass is not the step time).
    kern_ms, launches = 0.0, 0
    if with_kernel_timer:
        fm.fm_profile_enable(True)
        for _ in range(steps):
            attn(q, k, v, cs, ce, scale, out=out, lse=lse, stream=stream)
        torch.cuda.synchronize()
        fm.fm_profile_enable(False)
        kern_ms, launches = fm.fm_profile_read()
    ms_step = total_ms / steps
    res = {
        "key": cfg.key,
        "workload": cfg.name,
        "B": cfg.B, "H": cfg.H, "N": cfg.N, "d": cfg.d, "mask": cfg.mask, "seed": cfg.seed,
        "ranges_per_row": spec.col_start.shape[1] if spec.col_start.ndim == 3 else 1,
        "attended_pairs": U,
        "effective_flops": flops,
        "ms_per_step": ms_step,
        "effective_tflops": flops / (ms_step * 1e-3) / 1e12,
    }
    if launches:
        kms = kern_ms / launches
        res["attn_kernel_ms"] = kms
        res["attn_kernel_tflops"] = flops / (kms * 1e-3) / 1e12
    res["pct_of_bf16_peak"] = 100.0 * res["effective_tflops"] / metrics.MI355X_BF16_DENSE_TFLOPS
    res.update(tile_stats(fm, spec, cfg, dev))
    res["tile_executed_tflops"] = res["tile_executed_flops"] / (ms_step * 1e-3) / 1e12
    if cfg.mask.startswith("doc"):
        res["documents"] = [len(L) for L in spec.doc_lengths]
    if cfg.mask == "prefix_lm":
        res["prefix"] = spec.prefix
    del q, k, v, out, lse
    torch.cuda.empty_cache()
    return res


def time_backward(cfg, steps, warmup, warm_s=0.0):
    """fm_attn_bwd steps on the workload (inputs resident: q, k, v, the forward's out and
    lse, and a bf16 N(0,1) upstream gradient).  Algorithmic work: 10 d FLOPs per attended
    pair (five products of 2 d: the recomputed scores, dV, dP, dK, dQ)."""
    import torch
    from masked_attention_fm_amd import flashmask as fm
    from masked_attention_fm_amd import inputs, metrics

    dev = torch.device("cuda:0")
    spec = inputs.config_intervals(cfg)
    q, k, v = (x.to(dev) for x in inputs.make_qkv(cfg.B, cfg.H, cfg.N, cfg.d, cfg.seed))
    cs = torch.from_numpy(spec.col_start).to(dev)
    ce = torch.from_numpy(spec.col_end).to(dev)
    scale = inputs.default_scale(cfg.d)
    multi = spec.col_start.ndim == 3
    fwd = fm.fm_attn_fwd_multi if multi else fm.fm_attn_fwd
    bwd = fm.fm_attn_bwd_multi if multi else fm.fm_attn_bwd
    out, lse = fwd(q, k, v, cs, ce, scale)
    g = torch.Generator(device=dev).manual_seed(cfg.seed)
    dout = torch.randn(q.shape, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    dq, dk, dv = (torch.empty(q.shape, dtype=torch.float32, device=dev) for _ in range(3))
    stream = torch.cuda.current_stream()
    warm_up(lambda: bwd(q, k, v, out, dout, lse, cs, ce, scale, dq=dq, dk=dk, dv=dv, stream=stream), warmup,
            warm_s)
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(steps):
        bwd(q, k, v, out, dout, lse, cs, ce, scale, dq=dq, dk=dk, dv=dv, stream=stream)
    stop.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    U = metrics.spec_attended_pairs(spec.col_start, spec.col_end, cfg.N) * cfg.H
    flops = 10 * cfg.d * U
    del q, k, v, out, lse, dout, dq, dk, dv
    torch.cuda.empty_cache()
    return {"ms_per_step": ms, "effective_flops": flops, "effective_tflops": flops / (ms * 1e-3) / 1e12}


def time_fp8(cfg, steps, warmup, mode, warm_s=0.0):
    """fm_attn_fwd_fp8 steps in the given mode on the workload's draws quantized per tensor
    to e4m3 (inputs resident); same 4 d FLOPs per attended pair as the bf16 forward."""
    import torch
    from masked_attention_fm_amd import flashmask as fm
    from masked_attention_fm_amd import inputs, metrics

    dev = torch.device("cuda:0")
    spec = inputs.config_intervals(cfg)
    (q8, qs), (k8, ks), (v8, vs) = inputs.make_qkv_fp8(cfg.B, cfg.H, cfg.N, cfg.d, cfg.seed)
    q8, k8, v8 = (x.to(dev) for x in (q8, k8, v8))
    cs = torch.from_numpy(spec.col_start).to(dev)
    ce = torch.from_numpy(spec.col_end).to(dev)
    out = torch.empty(q8.shape, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(q8.shape[:3], dtype=torch.float32, device=dev)
    scale = inputs.default_scale(cfg.d)
    stream = torch.cuda.current_stream()
    warm_up(lambda: fm.fm_attn_fwd_fp8(q8, k8, v8, qs, ks, vs, cs, ce, scale, out=out, lse=lse, stream=stream,
                                       mode=mode), warmup, warm_s)
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(steps):
        fm.fm_attn_fwd_fp8(q8, k8, v8, qs, ks, vs, cs, ce, scale, out=out, lse=lse, stream=stream, mode=mode)
    stop.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    flops = 4 * cfg.d * metrics.spec_attended_pairs(spec.col_start, spec.col_end, cfg.N) * cfg.H
    del q8, k8, v8, out, lse
    torch.cuda.empty_cache()
    return {"ms_per_step": ms, "effective_flops": flops, "effective_tflops": flops / (ms * 1e-3) / 1e12}


def load_counters(key):
    """Hardware-counter record of the attention kernel on this workload, if it was taken
    from the current kernel source (profiles/attn_fwd_<key>_counters.json)."""
    from masked_attention_fm_amd import counters
    path = os.path.join(HERE, "profiles", f"attn_fwd_{key}_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("attn_source_sha256_16") != counters.attn_source_hash():
        log(f"{path} was taken from another kernel version: traffic reported as null")
        return None
    rec["file"] = os.path.relpath(path, HERE)
    return rec


def cpu_baseline(cfg, target_s):
    """The float64 oracle on whole heads of the workload, head after head (and pass after
    pass over all heads when one pass is shorter), until about target_s seconds."""
    import oracle
    from masked_attention_fm_amd import inputs, metrics
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = 1
    spec = inputs.config_intervals(cfg)
    scale = inputs.default_scale(cfg.d)
    per_b_pairs = {b: metrics.spec_attended_pairs(spec.col_start[b:b + 1], spec.col_end[b:b + 1], cfg.N)
                   for b in range(cfg.B)}
    heads = [(b, h) for b in range(cfg.B) for h in range(cfg.H)]
    secs = 0.0
    flops = 0
    runs = 0
    while secs < target_s:
        b, h = heads[runs % len(heads)]
        sl = [inputs.qkv_slice(cfg.seed, n, b, h, cfg.N, cfg.d).float().numpy()[None, None] for n in "qkv"]
        t1 = time.time()
        oracle.attention(*sl, spec.col_start[b:b + 1], spec.col_end[b:b + 1], scale)
        secs += time.time() - t1
        flops += 4 * cfg.d * per_b_pairs[b]
        runs += 1
    passes = runs / len(heads)
    what = (f"{runs} of {len(heads)} (b,h) heads" if runs < len(heads) else
            f"{passes:.2f} passes over all {len(heads)} (b,h) heads")
    return {"value": flops / secs / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{what} of {cfg.key}, all rows, {secs:.1f}s float64 numpy (dense mask per 128-row block)",
            "seconds": secs, "host_cpus": len(os.sched_getaffinity(0))}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "this build has no multi-GPU path", file=sys.stderr)
        sys.exit(2)
    sys.path.insert(0, HERE)
    import torch
    from masked_attention_fm_amd import inputs, metrics
    from masked_attention_fm_amd import flashmask as fm

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if not os.path.exists(fm.LIB_PATH):
        from masked_attention_fm_amd import build as _build
        _build.build()
    fm.lib()

    cfg = inputs.CONFIGS[args.config]
    leg_s = args.warmup_seconds / 4
    main_res = time_config(cfg, args.steps, args.warmup, warm_s=args.warmup_seconds)
    log(f"{cfg.key}: {main_res['effective_tflops']:.1f} TFLOP/s effective, {main_res['ms_per_step']:.4f} ms/step")

    per_config = {}
    if not args.no_per_config:
        for key, c in inputs.CONFIGS.items():
            if key == cfg.key:
                continue
            steps = 200 if c.N <= 1024 else max(5, min(args.steps, 20))
            r = time_config(c, steps, min(args.warmup, 5), warm_s=leg_s)
            log(f"{key}: {r['effective_tflops']:.1f} TFLOP/s effective, {r['ms_per_step']:.4f} ms/step")
            per_config[key] = {k: r[k] for k in ("workload", "ranges_per_row", "ms_per_step", "effective_tflops",
                                                 "pct_of_bf16_peak", "attn_kernel_ms", "attn_kernel_tflops",
                                                 "skip_ratio", "partial_ratio", "tile_executed_tflops")
                               if k in r}

    backward = {}
    if not args.no_backward:
        for key, c in inputs.CONFIGS.items():
            if key != cfg.key and args.no_per_config:
                continue
            steps = 100 if c.N <= 1024 else max(5, min(args.steps, 20))
            r = time_backward(c, steps, min(args.warmup, 3), warm_s=leg_s)
            log(f"{key} backward: {r['effective_tflops']:.1f} TFLOP/s effective, {r['ms_per_step']:.4f} ms/step")
            backward[key] = r

    fp8, fp8_all = {}, {}
    if not args.no_fp8:
        for key, c in inputs.CONFIGS.items():
            if key != cfg.key and args.no_per_config:
                continue
            steps = 200 if c.N <= 1024 else max(5, min(args.steps, 20))
            r = time_fp8(c, steps, min(args.warmup, 5), fm.FM_FP8_SCORES, warm_s=leg_s)
            log(f"{key} fp8: {r['effective_tflops']:.1f} TFLOP/s effective, {r['ms_per_step']:.4f} ms/step")
            fp8[key] = r
            r = time_fp8(c, steps, min(args.warmup, 5), fm.FM_FP8_ALL, warm_s=leg_s)
            log(f"{key} fp8 weights: {r['effective_tflops']:.1f} TFLOP/s effective, {r['ms_per_step']:.4f} ms/step")
            fp8_all[key] = r

    if args.copy_mib:
        n = args.copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"reference copy: 3 x {args.copy_mib} MiB")
        del src, dst

    kms = main_res.get("attn_kernel_ms")
    counters = load_counters(cfg.key)
    roofline = {
        "bound": "mfma",
        "achieved": main_res.get("attn_kernel_tflops"),
        "peak": metrics.MI355X_BF16_DENSE_TFLOPS,
        "unit": "TFLOP/s",
        "frac": (main_res["attn_kernel_tflops"] / metrics.MI355X_BF16_DENSE_TFLOPS) if kms else None,
        "traffic": counters.get("hbm_bytes_per_launch") if counters else None,
        "traffic_source": counters.get("file") if counters else None,
        "mfma_busy": counters.get("mfma_busy_per_cu_busy") if counters else None,
        "lds_bank_conflict_cycles": counters.get("lds_bank_conflict_cycles") if counters else None,
        "kernel": f"attn_fwd_kernel<{cfg.d}, {main_res['ranges_per_row']}, 0>",   # <d, ranges per row, bf16>
        "kernel_ms": kms,
        "algorithmic_flops_per_launch": main_res["effective_flops"],
    }
    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        cpu = cpu_baseline(cfg, args.cpu_seconds)

    line = {
        "metric": METRIC,
        "value": main_res["effective_tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_seconds": args.warmup_seconds,
        "ms_per_step": main_res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{cfg.key} {cfg.name}", "B": cfg.B, "H": cfg.H, "N": cfg.N, "d": cfg.d,
                   "mask": cfg.mask, "seed": cfg.seed, "global_batch": cfg.B, "seq_len": cfg.N,
                   "parallelism": "single-gpu"},
        "pct_of_bf16_peak": main_res["pct_of_bf16_peak"],
        "skip_ratio": main_res["skip_ratio"],
        "partial_ratio": main_res["partial_ratio"],
        "tile_shape": [main_res["Br"], main_res["Bc"]],
        "tile_executed_tflops": main_res["tile_executed_tflops"],
        "roofline": roofline,
        "cpu_baseline": cpu,
        "per_config": per_config,
        "backward": backward,
        "fp8_forward": fp8,
        "fp8_all_forward": fp8_all,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
