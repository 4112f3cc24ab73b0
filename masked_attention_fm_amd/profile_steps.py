"""Run a few forward or backward steps of one workload, for rocprofv3 to trace or count.

    python -m masked_attention_fm_amd.profile_steps --config C4 --pass bwd --steps 3 [--copy-mib 512]

The inputs are the workload's seeded synthetic draws, resident on cuda:0 before the first
step.  --pass fwd runs fm_attn_fwd (fm_attn_fwd_multi for several ranges per row) `steps`
times after `warmup` untimed calls; --pass bwd runs the forward once for O and LSE, then
fm_attn_bwd with a seeded N(0, 1) upstream gradient.  --copy-mib M ends with three plain
device copies of M MiB: the reference of known size that hardware byte counters are
calibrated against (masked_attention_fm_amd.counters).  Nothing is timed or printed beyond
one line per phase.
"""
from __future__ import annotations

import argparse
import sys


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--config", default="C4")
    ap.add_argument("--pass", dest="which", choices=("fwd", "bwd"), default="fwd")
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--copy-mib", type=int, default=0)
    args = ap.parse_args(argv)

    import torch
    from masked_attention_fm_amd import flashmask as fm
    from masked_attention_fm_amd import inputs

    cfg = inputs.CONFIGS[args.config]
    dev = torch.device("cuda:0")
    spec = inputs.config_intervals(cfg)
    q, k, v = (x.to(dev) for x in inputs.make_qkv(cfg.B, cfg.H, cfg.N, cfg.d, cfg.seed))
    cs = torch.from_numpy(spec.col_start).to(dev)
    ce = torch.from_numpy(spec.col_end).to(dev)
    scale = inputs.default_scale(cfg.d)
    multi = spec.col_start.ndim == 3
    fwd = fm.fm_attn_fwd_multi if multi else fm.fm_attn_fwd
    out, lse = fwd(q, k, v, cs, ce, scale)
    if args.which == "fwd":
        step = lambda: fwd(q, k, v, cs, ce, scale, out=out, lse=lse)
    else:
        bwd = fm.fm_attn_bwd_multi if multi else fm.fm_attn_bwd
        g = torch.Generator(device=dev).manual_seed(cfg.seed)
        dout = torch.randn(q.shape, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
        dq, dk, dv = (torch.empty(q.shape, dtype=torch.float32, device=dev) for _ in range(3))
        step = lambda: bwd(q, k, v, out, dout, lse, cs, ce, scale, dq=dq, dk=dk, dv=dv)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    print(f"[profile_steps] {cfg.key} {args.which}: {args.warmup} + {args.steps} steps", flush=True)
    if args.copy_mib:
        n = args.copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[profile_steps] reference copy: 3 x {args.copy_mib} MiB", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
