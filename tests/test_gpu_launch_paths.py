"""Every forward launch path on the same seeded inputs: a sweep of drawn shapes and masks,
each run through the 32-row slice kernel, the 128-row single launch (with its key-range
pieces and wavefront groups), the same unsplit, the preprocessed launch and the
no-allocation entry point, each against the float64 oracle at the usual bars, and the
paths against one another to one bf16 ulp of O (they differ only by the order of fp32
additions where they split a row's key blocks)."""
import numpy as np
import pytest
import torch

import oracle
from masked_attention_fm_amd import flashmask as fm
from masked_attention_fm_amd import inputs

from test_gpu_parity import compare, log, small_intervals, to_dev

pytestmark = pytest.mark.gpu

KINDS = ("causal", "random", "random_empty", "docs", "sliding", "prefix", "out_of_range", "multi")


def draw_cases(n, seed=2024):
    """n (B, H, N, d, kind, K) cases from a fixed generator: sizes that reach every launch
    path (up to 512 slices, up to 256 query blocks, longer ranges that split) while the
    oracle still finishes in about a second each."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        d = (128, 64)[i % 2]
        N = int(rng.integers(1, 2600)) if i % 3 else int(rng.integers(1, 300))
        B = int(rng.integers(1, 3))
        H = int(rng.integers(1, 4))
        kind = KINDS[i % len(KINDS)]
        K = int(rng.integers(2, 5)) if kind == "multi" else 1
        cases.append((B, H, N, d, kind, K, int(rng.integers(0, 1 << 30))))
    return cases


CASES = draw_cases(18)

PATHS = {
    # name: options set before the call (restored afterwards), entry point
    "slices": ({}, "multi"),
    "blocks": ({fm.FM_OPT_ROW_SLICES: 0}, "multi"),
    "unsplit": ({fm.FM_OPT_SPLIT_KEYS: 0}, "multi"),
    "preprocessed": ({fm.FM_OPT_SINGLE_LAUNCH: 0}, "multi"),
    "noalloc": ({}, "noalloc"),
}
DEFAULTS = {fm.FM_OPT_ROW_SLICES: 512, fm.FM_OPT_SPLIT_KEYS: 1, fm.FM_OPT_SINGLE_LAUNCH: 1}


def intervals(case):
    B, H, N, d, kind, K, seed = case
    rng = np.random.default_rng(seed)
    if kind == "multi":
        s, e = inputs.random_multi_intervals(rng, B, K, N, empty_frac=0.15, max_width=max(1, N // 3))
        return s, e
    s, e = small_intervals(kind, B, N, rng)
    return s[:, None, :], e[:, None, :]


def run_path(name, q, k, v, s, e, scale):
    opts, entry = PATHS[name]
    out = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=q.device)
    try:
        for o, val in opts.items():
            fm.fm_set_option(o, val)
        if entry == "noalloc":
            fm.fm_attn_fwd_noalloc(q, k, v, s, e, scale, out, lse)
        else:
            fm.fm_attn_fwd_multi(q, k, v, s, e, scale, out=out, lse=lse)
        torch.cuda.synchronize()
    finally:
        for o in opts:
            fm.fm_set_option(o, DEFAULTS[o])
    return out, lse


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c[:6])))
def test_every_launch_path(case):
    B, H, N, d, kind, K, seed = case
    s, e = intervals(case)
    q, k, v = inputs.make_qkv(B, H, N, d, seed=seed % 100000)
    scale = inputs.default_scale(d)
    log(f"launch paths {case}: {B * H * -(-N // 32)} slices, {B * H * -(-N // 128)} query blocks")
    qd, kd, vd, sd, ed = to_dev(q, k, v, np.ascontiguousarray(s), np.ascontiguousarray(e))
    qf, kf, vf = (x.float().numpy() for x in (q, k, v))
    O_ref, L_ref = oracle.attention(qf, kf, vf, s, e, scale)
    results = {}
    for name in PATHS:
        out, lse = run_path(name, qd, kd, vd, sd, ed, scale)
        results[name] = (out, lse)
        compare(out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), O_ref, L_ref,
                f"{name} {case[:6]}")
    o0, l0 = results["unsplit"]
    fin = torch.isfinite(l0)
    for name, (o, l) in results.items():
        assert torch.equal(torch.isfinite(l), fin), f"{name}: empty rows differ from the unsplit launch"
        dO = (o.float() - o0.float()).abs().max().item() if o.numel() else 0.0
        dL = (l[fin] - l0[fin]).abs().max().item() if fin.any() else 0.0
        assert dO <= 2 ** -7 * max(1.0, o0.float().abs().max().item()) and dL <= 1e-5, \
            f"{name} vs unsplit: max|dO| {dO}, max|dLSE| {dL}"
    # the preprocessed launch and the unsplit single launch give the same bits
    assert torch.equal(results["preprocessed"][0], o0) and torch.equal(results["preprocessed"][1], l0)
