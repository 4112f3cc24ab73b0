"""Benchmark of the FlashMask forward path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--warmup-seconds S] [--config C4]
                    [--no-per-config] [--no-cpu-baseline] [--no-backward] [--no-fp8]

A step is one fm_attn_fwd call (interval preprocessor + scheduler + attention
kernel) over one batch of the workload, inputs resident in HBM.  The headline
workload is the prefix-LM one (B=2, H=32, N=16384, d=128), the largest of the
five by attended work.  Untimed warm-up: W steps, then more until S seconds
(default 1) have run, so that the GPU's clocks have reached their sustained
level (S / 4 for the other legs).  Prints ONE JSON line: effective TFLOP/s
counting 4*d FLOPs per attended (query, key) pair over exactly K steps, the
median step, the attention kernel's roofline figures (its own duration measured
with HIP events the library records on its stream; HBM traffic and matrix-unit
figures from the committed rocprofv3 counter records when those were taken
from the current kernel source), the same for every other workload under
"per_config", the backward pass (fm_attn_bwd, 10*d FLOPs per attended pair)
under "backward", the FP8-input forward (fm_attn_fwd_fp8) under "fp8_forward"
(bf16 weights) and "fp8_all_forward" (e4m3 weights), and the float64 CPU oracle
timed on a bounded sample of every workload on the host's cores.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import threading
import time

import numpy as np

METRIC = "effective masked-attn fwd TFLOP/s (unmasked FLOPs) + % of bf16 MFMA peak"
DEFAULT_CONFIG = "C4"
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
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target wall time of the oracle sample of the main workload")
    ap.add_argument("--cpu-seconds-other", type=float, default=4.0,
                    help="target wall time of the oracle sample of each other workload")
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


def timed_steps(step, stream, steps):
    """Exactly `steps` calls of step() between two events on `stream`, with the device
    synchronized on both sides (the timed region: the mean step), then the same number
    of calls with an event after each one (the per-step times, for the median; these
    events are not in the timed region)."""
    import torch
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(steps):
        step()
    stop.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    evs[0].record(stream)
    for i in range(steps):
        step()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    per = [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]
    return total_ms / steps, float(np.median(per))


def time_config(cfg, steps, warmup, warm_s=0.0):
    """bf16 forward: step time (mean over exactly `steps`, and the median), then the
    attention kernel's own duration from the library's event pair in a third pass."""
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
    step = lambda: attn(q, k, v, cs, ce, scale, out=out, lse=lse, stream=stream)

    warm_up(step, warmup, warm_s)
    fm.fm_profile_read()                       # drop anything recorded before
    ms_step, ms_median = timed_steps(step, stream, steps)

    # The attention kernel's own duration: the library's per-launch event pair (it adds
    # a few microseconds per call, so this pass is not the step time).
    fm.fm_profile_enable(True)
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    fm.fm_profile_enable(False)
    kern_ms, launches = fm.fm_profile_read()
    n_ranges = spec.col_start.shape[1] if spec.col_start.ndim == 3 else 1
    res = {
        "key": cfg.key,
        "workload": cfg.name,
        "B": cfg.B, "H": cfg.H, "N": cfg.N, "d": cfg.d, "mask": cfg.mask, "seed": cfg.seed,
        "ranges_per_row": n_ranges,
        "attended_pairs": U,
        "effective_flops": flops,
        "algorithmic_bytes": metrics.algorithmic_bytes(cfg.B, cfg.H, cfg.N, cfg.d, n_ranges),
        # matrix instructions the kernel issues (every wavefront's computed key blocks)
        "mfma_instructions": metrics.wave_mfma_instructions(spec.col_start, spec.col_end, cfg.N, cfg.H, cfg.d),
        "ms_per_step": ms_step,
        "ms_median": ms_median,
        "effective_tflops": flops / (ms_step * 1e-3) / 1e12,
        "effective_tflops_median": flops / (ms_median * 1e-3) / 1e12,
        "steps": steps,
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
    step = lambda: bwd(q, k, v, out, dout, lse, cs, ce, scale, dq=dq, dk=dk, dv=dv, stream=stream)
    warm_up(step, warmup, warm_s)
    ms, ms_median = timed_steps(step, stream, steps)
    U = metrics.spec_attended_pairs(spec.col_start, spec.col_end, cfg.N) * cfg.H
    flops = 10 * cfg.d * U
    del q, k, v, out, lse, dout, dq, dk, dv
    torch.cuda.empty_cache()
    return {"ms_per_step": ms, "ms_median": ms_median, "effective_flops": flops,
            "effective_tflops": flops / (ms * 1e-3) / 1e12,
            "pct_of_bf16_peak": 100.0 * flops / (ms * 1e-3) / 1e12 / metrics.MI355X_BF16_DENSE_TFLOPS}


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
    step = lambda: fm.fm_attn_fwd_fp8(q8, k8, v8, qs, ks, vs, cs, ce, scale, out=out, lse=lse, stream=stream,
                                      mode=mode)
    warm_up(step, warmup, warm_s)
    ms, ms_median = timed_steps(step, stream, steps)
    flops = 4 * cfg.d * metrics.spec_attended_pairs(spec.col_start, spec.col_end, cfg.N) * cfg.H
    del q8, k8, v8, out, lse
    torch.cuda.empty_cache()
    return {"ms_per_step": ms, "ms_median": ms_median, "effective_flops": flops,
            "effective_tflops": flops / (ms * 1e-3) / 1e12}


def load_counters(key):
    """Hardware-counter record of the bf16 attention kernel on this workload, if it was
    taken from the current kernel and launch code (profiles/attn_fwd_<key>_counters.json)."""
    from masked_attention_fm_amd import counters
    path = os.path.join(HERE, "profiles", f"attn_fwd_{key}_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("attn_source_sha256_16") != counters.attn_source_hash():
        log(f"{os.path.relpath(path, HERE)} was taken from another kernel version: traffic reported as null")
        return None
    rec["file"] = os.path.relpath(path, HERE)
    return rec


def attn_kernel_name(res):
    """The bf16 attention kernel instance the default options launch: <d, ranges per row, 0>
    after the preprocessor; a problem of at most 256 query-block workgroups runs alone, as
    the 32-row slice kernel when it has at most 512 slices, else as <.., 3>, or <.., 4>
    (two wavefront groups) at d = 128 with at least 32 key blocks."""
    items = res["B"] * res["H"] * -(-res["N"] // 128)
    slices = res["B"] * res["H"] * -(-res["N"] // 32)
    if items <= 256 and slices <= 512:
        return f"attn_fwd_rows_kernel<{res['d']}, {res['ranges_per_row']}>"
    prec = 0
    if items <= 256:
        prec = 4 if res["d"] == 128 and -(-res["N"] // 64) >= 32 else 3
    return f"attn_fwd_kernel<{res['d']}, {res['ranges_per_row']}, {prec}>"


def roofline_of(res):
    """The attention kernel's roofline figures on one workload.  achieved = algorithmic
    FLOPs (4 d per attended pair) over the kernel's own average duration; traffic = the
    bytes beyond L2 per launch from the counter record (FETCH_SIZE + WRITE_SIZE, each
    scaled by what the counter reads for a device copy of known size), an upper bound on
    the HBM bytes since the MALL serves part of those misses."""
    from masked_attention_fm_amd import metrics
    kms = res.get("attn_kernel_ms")
    rec = load_counters(res["key"])
    achieved = res["effective_flops"] / (kms * 1e-3) / 1e12 if kms else None
    traffic = rec.get("l2_miss_bytes_per_launch") if rec else None
    alg = res["algorithmic_bytes"]
    out = {
        "bound": "mfma",
        "achieved": achieved,
        "peak": metrics.MI355X_BF16_DENSE_TFLOPS,
        "unit": "TFLOP/s",
        "frac": achieved / metrics.MI355X_BF16_DENSE_TFLOPS if achieved else None,
        "traffic": traffic,
        "kernel": attn_kernel_name(res),
        "kernel_ms": kms,
        "algorithmic_flops_per_launch": res["effective_flops"],
        "algorithmic_bytes_per_launch": alg,
        "algorithmic_GBps": alg / (kms * 1e-3) / 1e9 if kms else None,
        "traffic_GBps": traffic / (kms * 1e-3) / 1e9 if (kms and traffic) else None,
        "traffic_over_algorithmic": traffic / alg if traffic else None,
        "hbm_peak_GBps": metrics.MI355X_HBM_TBPS * 1e3,
        "mfma_busy": rec.get("mfma_busy_per_cu_busy") if rec else None,
        "executed_flops_per_launch": res["mfma_instructions"] * 32768,
        "executed_TFLOPs": res["mfma_instructions"] * 32768 / (kms * 1e-3) / 1e12 if kms else None,
        "mfma_instructions_per_launch": res["mfma_instructions"],
        "mfma_instructions_counted_per_launch": rec["attention"].get("SQ_INSTS_MFMA") if rec else None,
        "mfma_valu_coexec_per_mfma_busy": rec.get("mfma_valu_coexec_per_mfma_busy") if rec else None,
        "lds_bank_conflict_cycles": rec.get("lds_bank_conflict_cycles") if rec else None,
        "lds_bank_conflict_per_lds_active": rec.get("lds_bank_conflict_per_lds_active") if rec else None,
        "counter_record": rec.get("file") if rec else None,
    }
    return out


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or None


def cpu_baseline(cfg, target_s):
    """The float64 oracle as it stands, timed on a bounded sample of the workload.

    Jobs are chunks of up to 1024 consecutive query rows of one (b, h) head, taken from
    a seeded choice of heads in a seeded order (cycling when the sample is shorter than
    the target), run by a pool of threads, one per host core up to 16 (numpy's BLAS held
    to one thread per call), until about target_s seconds of wall time have passed.  The
    throughput counts 4 d FLOPs per attended pair of the rows computed; the inputs of the
    chosen heads are drawn before the clock starts."""
    import oracle
    from concurrent.futures import FIRST_COMPLETED, ThreadPoolExecutor, wait
    from threadpoolctl import threadpool_limits
    from masked_attention_fm_amd import inputs, metrics

    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    spec = inputs.config_intervals(cfg)
    scale = inputs.default_scale(cfg.d)
    rng = np.random.default_rng(cfg.seed)
    all_heads = [(b, h) for b in range(cfg.B) for h in range(cfg.H)]
    heads = [all_heads[i] for i in rng.permutation(len(all_heads))[:min(len(all_heads), 2 * threads)]]
    with ThreadPoolExecutor(threads) as ex:
        slices = dict(zip(heads, ex.map(
            lambda bh: [inputs.qkv_slice(cfg.seed, n, bh[0], bh[1], cfg.N, cfg.d).float().numpy()[None, None]
                        for n in "qkv"], heads)))
    rows = min(1024, cfg.N)
    jobs = [(b, h, r0, min(r0 + rows, cfg.N)) for (b, h) in heads for r0 in range(0, cfg.N, rows)]
    jobs = [jobs[i] for i in rng.permutation(len(jobs))]
    pairs = {}
    for b, h, r0, r1 in jobs:
        if (b, r0) not in pairs:
            pairs[(b, r0)] = metrics.spec_attended_pairs(spec.col_start[b:b + 1, ..., r0:r1],
                                                         spec.col_end[b:b + 1, ..., r0:r1], cfg.N)

    def run(job):
        b, h, r0, r1 = job
        q, k, v = slices[(b, h)]
        oracle.attention(q, k, v, spec.col_start[b:b + 1], spec.col_end[b:b + 1], scale,
                         rows=np.arange(r0, r1))
        return job

    done, flops, rows_done = 0, 0, 0
    lock = threading.Lock()
    with threadpool_limits(1), ThreadPoolExecutor(threads) as ex:
        t0 = time.time()
        pending = set()
        nxt = 0
        while True:
            while len(pending) < threads and time.time() - t0 < target_s:
                pending.add(ex.submit(run, jobs[nxt % len(jobs)]))
                nxt += 1
            if not pending:
                break
            finished, pending = wait(pending, return_when=FIRST_COMPLETED)
            for f in finished:
                b, h, r0, r1 = f.result()
                with lock:
                    done += 1
                    flops += 4 * cfg.d * pairs[(b, r0)]
                    rows_done += r1 - r0
        secs = time.time() - t0
    total_flops = 4 * cfg.d * metrics.spec_attended_pairs(spec.col_start, spec.col_end, cfg.N) * cfg.H
    value = flops / secs / 1e12
    return {"value": value, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": (f"{done} jobs of up to {rows} query rows from {len(heads)} of {len(all_heads)} (b,h) heads "
                       f"of {cfg.key} ({rows_done} rows; their attended pairs are {flops / total_flops:.3f} x the "
                       f"workload's, jobs repeat once all have run), float64 numpy oracle, {secs:.1f} s wall on "
                       f"{threads} threads"),
            "seconds": secs, "cpu_model": cpu_model(), "host_cpus": len(os.sched_getaffinity(0)),
            "full_step_seconds_at_this_rate": total_flops / (value * 1e12) if value > 0 else None}


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

    keep = ("workload", "ranges_per_row", "ms_per_step", "ms_median", "steps", "effective_tflops",
            "effective_tflops_median", "pct_of_bf16_peak", "attn_kernel_ms", "attn_kernel_tflops", "skip_ratio",
            "partial_ratio", "tile_executed_tflops", "attended_pairs")
    per_config = {}
    if not args.no_per_config:
        for key, c in inputs.CONFIGS.items():
            if key == cfg.key:
                continue
            steps = 200 if c.N <= 1024 else max(5, min(args.steps, 20))
            r = time_config(c, steps, min(args.warmup, 5), warm_s=leg_s)
            log(f"{key}: {r['effective_tflops']:.1f} TFLOP/s effective, {r['ms_per_step']:.4f} ms/step")
            per_config[key] = {k: r[k] for k in keep if k in r}
            per_config[key]["roofline"] = roofline_of(r)

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

    cpu = None
    if not args.no_cpu_baseline:
        log(f"timing the CPU oracle on {cfg.key}")
        cpu = cpu_baseline(cfg, args.cpu_seconds)
        log(f"CPU oracle {cfg.key}: {cpu['value'] * 1e3:.2f} GFLOP/s on {cpu['cores']} threads")
        for key in per_config:
            log(f"timing the CPU oracle on {key}")
            per_config[key]["cpu_baseline"] = cpu_baseline(inputs.CONFIGS[key], args.cpu_seconds_other)

    line = {
        "metric": METRIC,
        "value": main_res["effective_tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_seconds": args.warmup_seconds,
        "ms_per_step": main_res["ms_per_step"],
        "ms_median": main_res["ms_median"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{cfg.key} {cfg.name}", "B": cfg.B, "H": cfg.H, "N": cfg.N, "d": cfg.d,
                   "mask": cfg.mask, "seed": cfg.seed, "global_batch": cfg.B, "seq_len": cfg.N,
                   "parallelism": "single-gpu"},
        "pct_of_bf16_peak": main_res["pct_of_bf16_peak"],
        "effective_tflops_median": main_res["effective_tflops_median"],
        "attended_pairs": main_res["attended_pairs"],
        "skip_ratio": main_res["skip_ratio"],
        "partial_ratio": main_res["partial_ratio"],
        "tile_shape": [main_res["Br"], main_res["Bc"]],
        "tile_executed_tflops": main_res["tile_executed_tflops"],
        "roofline": roofline_of(main_res),
        "cpu_baseline": cpu,
        "per_config": per_config,
        "backward": backward,
        "fp8_forward": fp8,
        "fp8_all_forward": fp8_all,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
