"""GPU parity of the backward pass (dQ, dK, dV through the C ABI) against the
float64 oracle's gradients, on the forward's own outputs (O, LSE)."""
import numpy as np
import pytest
import torch

import oracle
from masked_attention_fm_amd import flashmask as fm
from masked_attention_fm_amd import inputs

from test_gpu_parity import DEV, log, small_intervals, to_dev
from test_gpu_multi import multi_intervals

pytestmark = pytest.mark.gpu

# max |G - G_ref| <= GRAD_TOL * max(1, max |G_ref|) for each of dQ, dK, dV
GRAD_TOL = 2e-2


def dout_for(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(*shape, generator=g, dtype=torch.float32).to(torch.bfloat16)


def run_bwd(q, k, v, do, s, e, scale, multi):
    qd, kd, vd, dod = to_dev(q, k, v, do)
    sd, ed = to_dev(s, e)
    fwd = fm.fm_attn_fwd_multi if multi else fm.fm_attn_fwd
    out, lse = fwd(qd, kd, vd, sd, ed, scale)
    grads = [torch.full(q.shape, float("nan"), dtype=torch.float32, device=DEV) for _ in range(3)]
    bwd = fm.fm_attn_bwd_multi if multi else fm.fm_attn_bwd
    bwd(qd, kd, vd, out, dod, lse, sd, ed, scale, dq=grads[0], dk=grads[1], dv=grads[2])
    torch.cuda.synchronize()
    return [g.cpu().numpy().astype(np.float64) for g in grads]


def compare_grads(got, ref, what):
    worst = 0.0
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        assert np.isfinite(g).all(), f"{what}: non-finite {name}"
        err = float(np.abs(g - r).max()) if r.size else 0.0
        scale = max(1.0, float(np.abs(r).max()) if r.size else 0.0)
        log(f"{what}: {name} max|err|={err:.3e} max|ref|={scale:.3g} rel={err / scale:.3e}")
        assert err <= GRAD_TOL * scale, f"{what}: {name} error {err} > {GRAD_TOL} * {scale}"
        worst = max(worst, err / scale)
    return worst


def check_bwd(q, k, v, s, e, scale, what, multi=False, seed=0):
    do = dout_for(q.shape, seed)
    got = run_bwd(q, k, v, do, s, e, scale, multi)
    ref = oracle.attention_bwd(*(x.float().numpy() for x in (q, k, v, do)), s, e, scale)
    return compare_grads(got, ref, what)


BWD_CASES = [
    # (B, H, N, d, mask)
    (1, 1, 1, 64, "causal"),
    (1, 2, 64, 64, "causal"),
    (1, 2, 130, 128, "random"),
    (2, 2, 333, 128, "random"),
    (1, 2, 1000, 128, "docs"),
    (2, 1, 777, 64, "sliding"),
    (2, 1, 1500, 128, "prefix"),
    (1, 2, 515, 128, "random_empty"),
    (1, 1, 300, 128, "out_of_range"),
]


@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: "-".join(map(str, c)))
def test_bwd_small(case):
    B, H, N, d, mask = case
    rng = np.random.default_rng(N * 11 + d)
    s, e = small_intervals(mask, B, N, rng)
    q, k, v = inputs.make_qkv(B, H, N, d, seed=N + 2 * d)
    log(f"bwd small {case}")
    check_bwd(q, k, v, s, e, inputs.default_scale(d), f"bwd {case}", seed=N)


@pytest.mark.parametrize("d,fused", [(64, 1), (128, 1), (128, 0)])
def test_bwd_key_blocks_no_query_attends(d, fused):
    """Key blocks that no query attends: every row of batch element 0 attends keys [0, 100]
    only, and every row of batch element 1 attends nothing.  Their key blocks have no live
    query chunk (the kernel's start issues their K and V loads, then skips the steps), so
    dK and dV there are exactly 0 and everything else matches the oracle; on both
    preparation paths."""
    B, H, N = 2, 2, 700
    s = np.zeros((B, N), np.int32)
    e = np.full((B, N), 100, np.int32)
    s[1], e[1] = 5, 4                      # empty ranges
    q, k, v = inputs.make_qkv(B, H, N, d, seed=31 + d)
    do = dout_for(q.shape, 77)
    log(f"bwd unattended key blocks d={d} fused={fused}")
    fm.fm_set_option(fm.FM_OPT_BWD_FUSED_PREP, fused)
    try:
        got = run_bwd(q, k, v, do, s, e, inputs.default_scale(d), False)
    finally:
        fm.fm_set_option(fm.FM_OPT_BWD_FUSED_PREP, 1)
    for g in got[1:]:
        assert np.all(g[0, :, 101:] == 0.0) and np.all(g[1] == 0.0), "unattended keys must get zero gradients"
    assert np.all(got[0][1] == 0.0), "rows that attend nothing must get dQ = 0"
    ref = oracle.attention_bwd(*(x.float().numpy() for x in (q, k, v, do)), s, e, inputs.default_scale(d))
    compare_grads(got, ref, f"bwd unattended key blocks d={d} fused={fused}")


BWD_MULTI_CASES = [
    (1, 2, 1000, 128, 2, "sinks"),
    (2, 1, 700, 64, 3, "random"),
    (1, 2, 900, 128, 4, "random_empty"),
]


@pytest.mark.parametrize("case", BWD_MULTI_CASES, ids=lambda c: "-".join(map(str, c)))
def test_bwd_multi_small(case):
    B, H, N, d, K, kind = case
    rng = np.random.default_rng(N * 5 + K)
    s, e = multi_intervals(kind, B, K, N, rng)
    q, k, v = inputs.make_qkv(B, H, N, d, seed=N + K + 7)
    log(f"bwd multi {case}")
    check_bwd(q, k, v, s, e, inputs.default_scale(d), f"bwd multi {case}", multi=True, seed=N + K)


def test_bwd_q_zero_gives_zero_dk():
    """Q = 0: dK = scale dS^T Q is exactly 0."""
    B, H, N, d = 1, 2, 600, 128
    rng = np.random.default_rng(17)
    s, e = inputs.random_intervals(rng, B, N, empty_frac=0.1, max_width=200)
    _, k, v = inputs.make_qkv(B, H, N, d, seed=17)
    q = torch.zeros_like(k)
    do = dout_for(q.shape, 17)
    dq, dk, dv = run_bwd(q, k, v, do, s, e, inputs.default_scale(d), False)
    assert np.all(dk == 0.0)


def test_bwd_deterministic():
    B, H, N, d = 1, 2, 2000, 128
    spec = inputs.make_intervals("doc_uniform", B, N, 3, lo=100, hi=900)
    q, k, v = inputs.make_qkv(B, H, N, d, seed=3)
    do = dout_for(q.shape, 3)
    a = run_bwd(q, k, v, do, spec.col_start, spec.col_end, inputs.default_scale(d), False)
    b = run_bwd(q, k, v, do, spec.col_start, spec.col_end, inputs.default_scale(d), False)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_bwd_doc_packed_workload_heads():
    """The doc-packed workload (N = 8192, d = 128) at full size, six heads, all rows.  Six heads
    make a dK/dV grid of 576 workgroups, so the dQ part runs on the library's second stream."""
    cfg = inputs.CONFIGS["C2"]
    spec = inputs.config_intervals(cfg)
    H = 6
    q, k, v = (x[:, :H].contiguous() for x in inputs.make_qkv(cfg.B, cfg.H, cfg.N, cfg.d, cfg.seed))
    log("bwd C2 six heads")
    worst = check_bwd(q, k, v, spec.col_start, spec.col_end, inputs.default_scale(cfg.d), "bwd C2", seed=cfg.seed)
    log(f"bwd C2: worst relative error {worst:.3e}")


def test_bwd_prefix_lm_workload_full_size_sampled_heads():
    """The prefix-LM workload at its full size and launch (B = 2, H = 32, N = 16384, d = 128,
    every head in one call, as the benchmark runs it); two heads, one per batch element,
    compared in full with the oracle's gradients."""
    cfg = inputs.CONFIGS["C4"]
    spec = inputs.config_intervals(cfg)
    scale = inputs.default_scale(cfg.d)
    q, k, v = inputs.make_qkv(cfg.B, cfg.H, cfg.N, cfg.d, cfg.seed)
    do = dout_for(q.shape, cfg.seed)
    log("bwd C4 full size")
    qd, kd, vd, dod = to_dev(q, k, v, do)
    sd, ed = to_dev(spec.col_start, spec.col_end)
    out, lse = fm.fm_attn_fwd(qd, kd, vd, sd, ed, scale)
    grads = [torch.full(q.shape, float("nan"), dtype=torch.float32, device=DEV) for _ in range(3)]
    fm.fm_attn_bwd(qd, kd, vd, out, dod, lse, sd, ed, scale, dq=grads[0], dk=grads[1], dv=grads[2])
    torch.cuda.synchronize()
    for g in grads:
        assert bool(torch.isfinite(g).all()), "non-finite gradient"
    for b, h in ((0, 5), (1, 30)):
        got = [g[b:b + 1, h:h + 1].cpu().numpy().astype(np.float64) for g in grads]
        ref = oracle.attention_bwd(*(x[b:b + 1, h:h + 1].float().numpy() for x in (q, k, v, do)),
                                   spec.col_start[b:b + 1], spec.col_end[b:b + 1], scale)
        compare_grads(got, ref, f"bwd C4 head ({b}, {h})")


def test_bwd_dv_within_rounding_bound_of_each_weight():
    """dV = P^T dO with every weight rounded to bfloat16 (relative error <= u = 2^-8)
    and exact bf16 dO: each element obeys |dV - dV_ref| <= 2u sum_i P_ij |dO_ic| (+ fp32
    accumulation), with P from the oracle."""
    B, H, N, d = 1, 2, 300, 128
    rng = np.random.default_rng(23)
    s, e = inputs.random_intervals(rng, B, N, empty_frac=0.1, max_width=120)
    q, k, v = inputs.make_qkv(B, H, N, d, seed=23)
    do = dout_for(q.shape, 23)
    _, _, dv = run_bwd(q, k, v, do, s, e, inputs.default_scale(d), False)
    qf, kf, vf, dof = (x.float().numpy().astype(np.float64) for x in (q, k, v, do))
    P = oracle.attention_weights(qf, kf, s, e, inputs.default_scale(d))        # [B, H, N, N]
    ref = np.einsum("bhij,bhic->bhjc", P, dof)
    bound = 2 * 2.0 ** -8 * np.einsum("bhij,bhic->bhjc", P, np.abs(dof)) + 1e-5
    excess = np.abs(dv - ref) - bound
    log(f"dV elementwise: max (err - bound) = {excess.max():.3e}, max err/bound = {(np.abs(dv - ref) / bound).max():.3f}")
    assert excess.max() <= 0.0


# ---------------------------------------------------------------- split key blocks

@pytest.fixture
def forced_split():
    """Split long key blocks into pieces of at least one query chunk (the default piece
    is 32 chunks, which these sizes never reach); the default is restored afterwards."""
    fm.fm_set_option(fm.FM_OPT_BWD_SPLIT_CHUNKS, 1)
    yield
    fm.fm_set_option(fm.FM_OPT_BWD_SPLIT_CHUNKS, 32)


SPLIT_CASES = [
    # (B, H, N, d, ranges, kind): attention sinks make the first key block far longer than the rest
    (1, 2, 2500, 128, 2, "sinks"),
    (2, 2, 1800, 64, 2, "sinks"),
    (1, 2, 1500, 128, 3, "random"),
]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=lambda c: "-".join(map(str, c)))
def test_bwd_split_key_blocks(forced_split, case):
    """Key blocks split into pieces whose partial dK, dV are summed afterwards: the oracle's
    gradients, to the same bar."""
    B, H, N, d, K, kind = case
    rng = np.random.default_rng(N * 7 + K)
    s, e = multi_intervals(kind, B, K, N, rng)
    q, k, v = inputs.make_qkv(B, H, N, d, seed=N + 3 * K)
    log(f"bwd split {case}")
    check_bwd(q, k, v, s, e, inputs.default_scale(d), f"bwd split {case}", multi=True, seed=N + K)


def _split_runs(q, k, v, do, s, e, scale):
    try:
        fm.fm_set_option(fm.FM_OPT_BWD_SPLIT_CHUNKS, 1)
        a = run_bwd(q, k, v, do, s, e, scale, True)
        b = run_bwd(q, k, v, do, s, e, scale, True)
        fm.fm_set_option(fm.FM_OPT_BWD_SPLIT_CHUNKS, 0)
        c = run_bwd(q, k, v, do, s, e, scale, True)
    finally:
        fm.fm_set_option(fm.FM_OPT_BWD_SPLIT_CHUNKS, 32)
    return a, b, c


def test_bwd_split_deterministic_and_equal_to_unsplit_up_to_summation_order():
    """With splitting: bitwise repeatable; against the unsplit kernel, dQ is identical (its
    kernel is unchanged) and dK, dV differ only by the order of the fp32 chunk sums (and do
    differ somewhere, so the split path ran)."""
    B, H, N, d = 1, 2, 2500, 128
    s, e = multi_intervals("sinks", B, 2, N, None)
    q, k, v = inputs.make_qkv(B, H, N, d, seed=29)
    do = dout_for(q.shape, 29)
    a, b, c = _split_runs(q, k, v, do, s, e, inputs.default_scale(d))
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    assert np.array_equal(a[0], c[0])
    for x, y in zip(a[1:], c[1:]):
        assert np.abs(x - y).max() <= 1e-4 * max(1.0, np.abs(y).max())
    assert not (np.array_equal(a[1], c[1]) and np.array_equal(a[2], c[2]))


def oracle_bwd_by_head(q, k, v, do, s, e, scale):
    """oracle.attention_bwd of every head, one head per thread (BLAS at one thread per
    call; no process is forked from the test process, which holds the GPU)."""
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    B, H = q.shape[:2]
    arrays = [x.float().numpy() for x in (q, k, v, do)]

    def one(bh):
        b, h = bh
        return oracle.attention_bwd(*(x[b:b + 1, h:h + 1] for x in arrays), s[b:b + 1], e[b:b + 1], scale)

    heads = [(b, h) for b in range(B) for h in range(H)]
    with threadpool_limits(1), ThreadPoolExecutor(min(16, len(heads))) as ex:
        res = list(ex.map(one, heads))
    grads = [np.zeros(q.shape, np.float64) for _ in range(3)]
    for (b, h), r in zip(heads, res):
        for g, x in zip(grads, r):
            g[b, h] = x[0, 0]
    return grads


@pytest.mark.timeout(600)
def test_bwd_split_sinks_window_workload_heads():
    """The sinks-plus-window workload (B=1, N=32768, d=128), four whole heads, with the
    default piece size (its sink key block is split): dQ, dK, dV against the float64
    oracle's gradients on every row; dK, dV also equal the unsplit kernel's up to the
    order of the fp32 chunk sums, and dQ exactly."""
    cfg = inputs.CONFIGS["S1"]
    spec = inputs.config_intervals(cfg)
    scale = inputs.default_scale(cfg.d)
    H = 4
    q, k, v = (x[:, :H].contiguous() for x in inputs.make_qkv(cfg.B, cfg.H, cfg.N, cfg.d, cfg.seed))
    do = dout_for(q.shape, cfg.seed)
    log("bwd S1 four heads: split against unsplit and against the oracle")
    try:
        fm.fm_set_option(fm.FM_OPT_BWD_SPLIT_CHUNKS, 32)
        a = run_bwd(q, k, v, do, spec.col_start, spec.col_end, scale, True)
        fm.fm_set_option(fm.FM_OPT_BWD_SPLIT_CHUNKS, 0)
        c = run_bwd(q, k, v, do, spec.col_start, spec.col_end, scale, True)
    finally:
        fm.fm_set_option(fm.FM_OPT_BWD_SPLIT_CHUNKS, 32)
    assert np.array_equal(a[0], c[0])
    for name, x, y in zip(("dK", "dV"), a[1:], c[1:]):
        err = float(np.abs(x - y).max())
        log(f"S1 {name}: max|split - unsplit| = {err:.3e}")
        assert err <= 1e-4 * max(1.0, float(np.abs(y).max()))
    assert not (np.array_equal(a[1], c[1]) and np.array_equal(a[2], c[2]))
    ref = oracle_bwd_by_head(q, k, v, do, spec.col_start, spec.col_end, scale)
    worst = compare_grads(a, ref, "bwd S1 four heads (split) vs oracle")
    log(f"bwd S1: worst relative error {worst:.3e}")


FUSED_PREP_CASES = [
    # (B, H, N, d, kind, ranges): small problems whose key blocks cannot split, prepared by one
    # launch; the same bits as the separate preprocessing launches
    (1, 2, 512, 64, "causal", 1),       # the tiny causal workload's shape
    (2, 3, 333, 128, "random", 1),      # ragged tail
    (1, 2, 515, 128, "random_empty", 1),
    (1, 1, 300, 64, "out_of_range", 1),
    (2, 1, 1500, 128, "prefix", 1),
    (1, 2, 700, 64, "random", 3),       # several ranges per row
    (1, 1, 40, 128, "causal", 1),       # one query chunk, one key block
]


@pytest.mark.parametrize("case", FUSED_PREP_CASES, ids=lambda c: "-".join(map(str, c)))
def test_bwd_fused_preparation_matches_separate_launches(case):
    B, H, N, d, kind, K = case
    rng = np.random.default_rng(N + 17 * K)
    if K == 1:
        s, e = small_intervals(kind, B, N, rng)
    else:
        s, e = inputs.random_multi_intervals(rng, B, K, N, empty_frac=0.1, max_width=N // 3)
    q, k, v = inputs.make_qkv(B, H, N, d, seed=N + 5)
    do = dout_for(q.shape, N)
    scale = inputs.default_scale(d)
    log(f"bwd fused preparation {case}")
    fused = run_bwd(q, k, v, do, s, e, scale, K > 1)
    try:
        fm.fm_set_option(fm.FM_OPT_BWD_FUSED_PREP, 0)
        separate = run_bwd(q, k, v, do, s, e, scale, K > 1)
    finally:
        fm.fm_set_option(fm.FM_OPT_BWD_FUSED_PREP, 1)
    for name, a, b in zip(("dQ", "dK", "dV"), fused, separate):
        assert np.array_equal(a, b), f"{case}: {name} differs between the fused and separate preparation"
    if K == 1:
        ref = oracle.attention_bwd(*(x.float().numpy() for x in (q, k, v, do)), s, e, scale)
        compare_grads(fused, ref, f"bwd fused preparation {case}")


def test_bwd_fused_preparation_per_head_sets():
    """One interval set per head: the fused records are numbered by set like the separate ones."""
    B, H, N, d = 2, 3, 400, 64
    rng = np.random.default_rng(41)
    s, e = inputs.random_multi_intervals(rng, B * H, 2, N, empty_frac=0.1, max_width=150)
    s, e = np.ascontiguousarray(s.reshape(B, H, 2, N)), np.ascontiguousarray(e.reshape(B, H, 2, N))
    q, k, v = inputs.make_qkv(B, H, N, d, seed=43)
    do = dout_for(q.shape, 44)
    scale = inputs.default_scale(d)
    qd, kd, vd, dod, sd, ed = to_dev(q, k, v, do, s, e)
    out, lse = fm.fm_attn_fwd_per_head(qd, kd, vd, sd, ed, scale)

    def grads():
        g = [torch.full(q.shape, float("nan"), dtype=torch.float32, device=DEV) for _ in range(3)]
        fm.fm_attn_bwd_per_head(qd, kd, vd, out, dod, lse, sd, ed, scale, dq=g[0], dk=g[1], dv=g[2])
        torch.cuda.synchronize()
        return g

    fused = grads()
    try:
        fm.fm_set_option(fm.FM_OPT_BWD_FUSED_PREP, 0)
        separate = grads()
    finally:
        fm.fm_set_option(fm.FM_OPT_BWD_FUSED_PREP, 1)
    for a, b in zip(fused, separate):
        assert torch.equal(a, b)
