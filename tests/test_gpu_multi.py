"""GPU parity for rows with several key ranges (the row attends their union):
tile classes, work counts and attention through the C ABI against the float64
oracle, with the same bars as the single-range path."""
import numpy as np
import pytest
import torch

import oracle
from masked_attention_fm_amd import flashmask as fm
from masked_attention_fm_amd import inputs

import full_parity
from test_gpu_parity import DEV, LSE_TOL, O_TOL, compare, log, schedule_key, to_dev

pytestmark = pytest.mark.gpu


def run_multi(q, k, v, cs, ce, scale):
    out = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=q.device)
    fm.fm_attn_fwd_multi(q, k, v, cs, ce, scale, out=out, lse=lse)
    torch.cuda.synchronize()
    return out, lse


def check_multi(q, k, v, s, e, scale, what, rows=None):
    qd, kd, vd = to_dev(q, k, v)
    out, lse = run_multi(qd, kd, vd, *to_dev(s, e), scale)
    qf, kf, vf = (x.float().numpy() for x in (q, k, v))
    O_ref, L_ref = oracle.attention(qf, kf, vf, s, e, scale, rows=rows)
    O_gpu = out.float().cpu().numpy().astype(np.float64)
    L_gpu = lse.cpu().numpy().astype(np.float64)
    if rows is not None:
        O_gpu, L_gpu = O_gpu[:, :, rows], L_gpu[:, :, rows]
    return compare(O_gpu, L_gpu, O_ref, L_ref, what)


def sinks_window(B, N, w, sinks):
    s, e = inputs.sinks_window_intervals(N, w, sinks)
    return np.ascontiguousarray(np.tile(s[None], (B, 1, 1))), np.ascontiguousarray(np.tile(e[None], (B, 1, 1)))


# ---------------------------------------------------------------- tile classes


def classify_multi_gpu(s, e, Br, Bc):
    sd, ed = to_dev(np.ascontiguousarray(s), np.ascontiguousarray(e))
    return fm.fm_classify_tiles_multi(sd, ed, Br, Bc).cpu().numpy()


def test_classes_multi_sinks_window():
    for N, w, sinks in ((8192, 1024, 10), (4096, 300, 1), (1000, 64, 200), (777, 1, 3)):
        s, e = inputs.sinks_window_intervals(N, w, sinks)
        for Br, Bc in ((128, 64), (128, 128), (64, 32), (96, 40)):
            log(f"classes multi sinks+window N={N} w={w} sinks={sinks} Br={Br} Bc={Bc}")
            ref = oracle.classes_minmax_multi(s, e, N, Br, Bc)
            assert np.array_equal(classify_multi_gpu(s, e, Br, Bc), ref)


def test_classes_multi_random_ragged():
    rng = np.random.default_rng(91)
    for K in (1, 2, 3, 4):
        for N, Br, Bc in ((1, 1, 1), (7, 3, 2), (300, 128, 64), (1000, 33, 17), (4097, 128, 64)):
            for width in (None, 5, 200):
                s, e = inputs.random_multi_intervals(rng, 1, K, N, max_width=width)
                log(f"classes multi random K={K} N={N} Br={Br} Bc={Bc} width={width}")
                ref = oracle.classes_minmax_multi(s[0], e[0], N, Br, Bc)
                assert np.array_equal(classify_multi_gpu(s[0], e[0], Br, Bc), ref)


def test_classes_multi_one_range_equals_single():
    rng = np.random.default_rng(5)
    s, e = inputs.random_intervals(rng, 1, 2000, max_width=300)
    single = fm.fm_classify_tiles(*to_dev(s[0], e[0]), 128, 64).cpu().numpy()
    multi = classify_multi_gpu(s, e, 128, 64)
    assert np.array_equal(single, multi)


def test_classes_multi_reject_bad_ranges():
    N = 256
    s, e = inputs.sinks_window_intervals(N, 32, 0)        # no sinks: the first range is empty
    out = torch.empty((2, 4), dtype=torch.uint8, device=DEV)
    with pytest.raises(fm.FlashMaskError) as ei:
        fm.fm_classify_tiles_multi(*to_dev(s, e), 128, 64, out=out)
    assert ei.value.status == fm.FM_ERR_BAD_INTERVAL


# ---------------------------------------------------------------- work counts


@pytest.mark.parametrize("B,N,K", [(1, 8192, 2), (2, 1000, 3), (3, 1 << 15, 2), (1, 5000, 4)])
def test_schedule_multi_counts_union(B, N, K):
    """Work = non-SKIP tiles of the query block's row of the union class table
    (both the one-workgroup path and the preprocessor + rank path)."""
    d = 128
    Br, Bc = fm.fm_attn_tile_shape(d)
    rng = np.random.default_rng(B * 1000 + K)
    if K == 2 and N == 8192:
        s, e = sinks_window(B, N, 1024, 10)
    else:
        s, e = inputs.random_multi_intervals(rng, B, K, N, max_width=N // 8)
    log(f"schedule multi B={B} N={N} K={K} items={B * -(-N // Br)}")
    work, order = fm.fm_tile_schedule_multi(*to_dev(s, e), d)
    work, order = work.cpu().numpy(), order.cpu().numpy()
    ref = np.concatenate([(oracle.classes_minmax_multi(s[b], e[b], N, Br, Bc) != oracle.SKIP).sum(1)
                          for b in range(B)])
    assert np.array_equal(work, ref)
    assert np.array_equal(order, np.argsort(-schedule_key(ref), kind="stable"))


# ---------------------------------------------------------------- attention


def test_multi_one_range_bit_identical_to_single():
    B, H, N, d = 2, 3, 1500, 128
    rng = np.random.default_rng(8)
    s, e = inputs.random_intervals(rng, B, N, empty_frac=0.1, max_width=400)
    q, k, v = to_dev(*inputs.make_qkv(B, H, N, d, seed=8))
    sd, ed = to_dev(s, e)
    scale = inputs.default_scale(d)
    o1 = torch.empty_like(q)
    l1 = torch.empty(q.shape[:3], dtype=torch.float32, device=DEV)
    fm.fm_attn_fwd(q, k, v, sd, ed, scale, out=o1, lse=l1)
    o2, l2 = run_multi(q, k, v, sd[:, None].contiguous(), ed[:, None].contiguous(), scale)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_multi_range_order_and_duplicates_do_not_change_results():
    B, H, N, d = 1, 2, 2000, 64
    rng = np.random.default_rng(9)
    s, e = inputs.random_multi_intervals(rng, B, 3, N, max_width=300)
    q, k, v = to_dev(*inputs.make_qkv(B, H, N, d, seed=9))
    scale = inputs.default_scale(d)
    o1, l1 = run_multi(q, k, v, *to_dev(s, e), scale)
    perm = [2, 0, 1]
    o2, l2 = run_multi(q, k, v, *to_dev(np.ascontiguousarray(s[:, perm]), np.ascontiguousarray(e[:, perm])),
                       scale)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    # a range repeated adds no key
    s4 = np.ascontiguousarray(np.concatenate([s, s[:, :1]], axis=1))
    e4 = np.ascontiguousarray(np.concatenate([e, e[:, :1]], axis=1))
    o3, l3 = run_multi(q, k, v, *to_dev(s4, e4), scale)
    assert torch.equal(o1, o3) and torch.equal(l1, l3)


MULTI_CASES = [
    # (B, H, N, d, K, kind)
    (1, 2, 64, 64, 2, "sinks"),
    (1, 2, 1000, 128, 2, "sinks"),
    (2, 2, 2049, 64, 2, "sinks"),
    (1, 2, 333, 128, 2, "random"),
    (2, 2, 1000, 128, 3, "random"),
    (1, 3, 700, 64, 4, "random"),
    (1, 2, 1500, 128, 4, "random_empty"),
    (1, 1, 600, 128, 3, "out_of_range"),
]


def multi_intervals(kind, B, K, N, rng):
    if kind == "sinks":
        return sinks_window(B, N, max(1, N // 8), 5)
    if kind == "random":
        return inputs.random_multi_intervals(rng, B, K, N, max_width=N // 4)
    if kind == "random_empty":
        return inputs.random_multi_intervals(rng, B, K, N, empty_frac=0.3, max_width=150)
    if kind == "out_of_range":
        s = rng.integers(-60, N, size=(B, K, N))
        e = s + rng.integers(-3, 200, size=(B, K, N))
        return s.astype(np.int32), e.astype(np.int32)
    raise ValueError(kind)


@pytest.mark.parametrize("case", MULTI_CASES, ids=lambda c: "-".join(map(str, c)))
def test_attention_multi_small(case):
    B, H, N, d, K, kind = case
    rng = np.random.default_rng(N * 3 + K)
    s, e = multi_intervals(kind, B, K, N, rng)
    q, k, v = inputs.make_qkv(B, H, N, d, seed=N + K)
    log(f"attention multi {case}")
    check_multi(q, k, v, s, e, inputs.default_scale(d), f"multi {case}")


def test_multi_q_zero_is_union_mean():
    """Q = 0: O_r is the mean of v over the union of the row's ranges and LSE_r = ln of
    its size (keys covered twice count once)."""
    B, H, N, d, K = 1, 2, 900, 128, 3
    rng = np.random.default_rng(12)
    s, e = inputs.random_multi_intervals(rng, B, K, N, empty_frac=0.1, max_width=250)
    _, k, v = inputs.make_qkv(B, H, N, d, seed=12)
    q = torch.zeros_like(k)
    out, lse = run_multi(*to_dev(q, k, v), *to_dev(s, e), inputs.default_scale(d))
    vf = v.double().numpy()
    O = out.double().cpu().numpy()
    L = lse.double().cpu().numpy()
    for i in range(N):
        keys = np.zeros(N, bool)
        for kk in range(K):
            if s[0, kk, i] <= e[0, kk, i]:
                keys[s[0, kk, i]:e[0, kk, i] + 1] = True
        n = int(keys.sum())
        if n == 0:
            assert np.all(O[0, :, i] == 0) and np.all(np.isneginf(L[0, :, i]))
            continue
        mean = vf[0][:, keys].mean(axis=1)
        assert np.abs(O[0, :, i] - mean).max() <= O_TOL
        assert np.abs(L[0, :, i] - np.log(n)).max() <= LSE_TOL


@pytest.mark.timeout(900)
def test_sinks_window_workload_every_row():
    """The sinks-plus-window workload at full size, in the launch configuration the
    benchmark times, every row of every head against the float64 oracle."""
    cfg = inputs.CONFIGS["S1"]
    spec = inputs.config_intervals(cfg)
    scale = inputs.default_scale(cfg.d)
    q, k, v = inputs.make_qkv(cfg.B, cfg.H, cfg.N, cfg.d, cfg.seed)
    log(f"workload {cfg.describe()}")
    out, lse = run_multi(*to_dev(q, k, v, spec.col_start, spec.col_end), scale)
    assert not torch.isnan(out).any() and not torch.isnan(lse).any(), "unwritten output"
    del q, k, v
    full_parity.compare_every_row(cfg, spec, out, lse, scale, O_TOL, LSE_TOL, log)
