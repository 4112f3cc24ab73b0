"""GPU parity of the FP8-input forward pass (fm_attn_fwd_fp8): the oracle on the
dequantized e4m3 inputs.  The score product is exact for FP8 inputs up to the FP8
units' accumulation.  Mode FM_FP8_SCORES widens V exactly to bf16, so the bf16
path's error model applies: small cases are held to its elementwise bound (output
and weight rounding), the full-size doc-packed workload to the 1e-2 / 1e-3 bars.
Mode FM_FP8_ALL rounds the weights to e4m3 (relative 2^-4): every case, the
full-size workload included (on a row sample), is held to that mode's elementwise
bound."""
import numpy as np
import pytest
import torch

import oracle
from masked_attention_fm_amd import flashmask as fm
from masked_attention_fm_amd import inputs

from test_gpu_parity import DEV, compare, log, small_intervals, to_dev
from test_gpu_multi import multi_intervals

pytestmark = pytest.mark.gpu


MODES = [fm.FM_FP8_SCORES, fm.FM_FP8_ALL]
MODE_IDS = ["scores", "all"]


def run_fp8(qkv8, s, e, scale, mode=fm.FM_FP8_SCORES):
    (q8, qs), (k8, ks), (v8, vs) = qkv8
    qd, kd, vd = to_dev(q8, k8, v8)
    out = torch.full(q8.shape, float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full(q8.shape[:3], float("nan"), dtype=torch.float32, device=DEV)
    fm.fm_attn_fwd_fp8(qd, kd, vd, qs, ks, vs, *to_dev(s, e), scale, out=out, lse=lse, mode=mode)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def check_fp8(qkv8, s, e, scale, what, rows=None):
    O, L = run_fp8(qkv8, s, e, scale)
    deq = [inputs.dequantize_e4m3(c, sc) for c, sc in qkv8]
    O_ref, L_ref = oracle.attention(*deq, s, e, scale, rows=rows)
    if rows is not None:
        O, L = O[:, :, rows], L[:, :, rows]
    return compare(O, L, O_ref, L_ref, what)


def bf16_half_ulp(x):
    """Half the bf16 spacing at |x| (bf16 keeps 8 significant bits)."""
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.where(ax > 0, 2.0 ** (e - 8), 0.0)


def row_terms(P, v, O_ref):
    """Per output element: sum_j P_ij |v_j - O_i|, P_max,i sum_j |v_j - O_i| (over the
    row's keys), sum_j P_ij |v_j|; per row: the number of keys n_i."""
    B, H, R, N = P.shape
    spread, tail, mag = (np.zeros(O_ref.shape) for _ in range(3))
    n = np.zeros((B, H, R, 1))
    for b in range(B):
        for h in range(H):
            for i in range(R):
                sup = np.flatnonzero(P[b, h, i] > 0)
                if sup.size == 0:
                    continue
                w = P[b, h, i, sup]
                dev = np.abs(v[b, h, sup] - O_ref[b, h, i])
                spread[b, h, i] = w @ dev
                tail[b, h, i] = w.max() * dev.sum(axis=0)
                mag[b, h, i] = w @ np.abs(v[b, h, sup])
                n[b, h, i] = sup.size
    return spread, tail, mag, n


def fp8_bound(mode, P, v, O_ref):
    """Elementwise error bound of the output against the oracle on the dequantized inputs,
    a function of the oracle's values only.

    With the weights w_j rounded to w'_j before the PV product and the output divided by
    sum_j w'_j, the kernel's fp32 output differs from O_ref by exactly
    sum_j (w'_j - w_j)(v_j - O) / sum_j w'_j, plus 1e-4 for the fp32 arithmetic and the
    FP8 score accumulation (the model term below):
      FM_FP8_SCORES: bf16 weights, |w' - w| <= 2^-8 w.
      FM_FP8_ALL: e4m3 weights of 2^8 w (w <= 1 against the running row maximum):
        |w' - w| <= 2^-4 w, or 2^-18 of the row maximum in the subnormal range, so the
        sum of w' is at least (1 - 2^-4 - n 2^-18) sum_j w_j; plus the FP8 units'
        accumulation, within 4e-5 of sum_j |w'_j v_j|.
    Rounding that fp32 value to bf16 then costs at most half the bf16 spacing at its
    magnitude, which is at most |O_ref| + model."""
    spread, tail, mag, n = row_terms(P, v, O_ref)
    if mode == fm.FM_FP8_SCORES:
        model = 2.0 ** -8 * spread + 1e-4
    else:
        u = 2.0 ** -4
        den = 1.0 - u - n * 2.0 ** -18
        model = (u * spread + 2.0 ** -18 * tail + 4e-5 * (1 + u) * mag) / den + 1e-4
    return bf16_half_ulp(np.abs(O_ref) + model) + model


def check_fp8_model(qkv8, s, e, scale, what, mode=fm.FM_FP8_SCORES, rows=None):
    """The output within fp8_bound elementwise (on the chosen rows); LSE within 1e-3."""
    O, L = run_fp8(qkv8, s, e, scale, mode)
    q, k, v = (inputs.dequantize_e4m3(c, sc) for c, sc in qkv8)
    O_ref, L_ref = oracle.attention(q, k, v, s, e, scale, rows=rows)
    if rows is not None:
        O, L = O[:, :, rows], L[:, :, rows]
    P = oracle.attention_weights(q, k, s, e, scale, rows=rows)       # [B, H, R, N]
    bound = fp8_bound(mode, P, v, O_ref)
    err = np.abs(O - O_ref)
    empty = np.isneginf(L_ref)
    assert np.array_equal(np.isneginf(L), empty), f"{what}: -inf LSE pattern differs"
    dL = float(np.abs(L[~empty] - L_ref[~empty]).max()) if (~empty).any() else 0.0
    log(f"{what}: max|dO|={err.max():.3e} max err/bound={(err / bound).max():.3f} max|dLSE|={dL:.3e}")
    assert np.all(err <= bound), f"{what}: {(err > bound).sum()} elements beyond the rounding bound"
    assert dL <= 1e-3


FP8_CASES = [
    (1, 1, 1, 64, "causal"),
    (1, 2, 64, 64, "causal"),
    (1, 2, 130, 128, "random"),
    (2, 2, 333, 128, "random"),
    (1, 2, 1000, 128, "docs"),
    (2, 2, 777, 64, "sliding"),
    (2, 1, 1500, 128, "prefix"),
    (1, 2, 515, 128, "random_empty"),
    (1, 1, 300, 128, "out_of_range"),
]


@pytest.mark.parametrize("mode", MODES, ids=MODE_IDS)
@pytest.mark.parametrize("case", FP8_CASES, ids=lambda c: "-".join(map(str, c)))
def test_fp8_small(case, mode):
    B, H, N, d, mask = case
    rng = np.random.default_rng(N * 13 + d)
    s, e = small_intervals(mask, B, N, rng)
    qkv8 = inputs.make_qkv_fp8(B, H, N, d, seed=N + 3 * d)
    log(f"fp8 small {case} mode {mode}")
    check_fp8_model(qkv8, s, e, inputs.default_scale(d), f"fp8 {case} mode {mode}", mode)


@pytest.mark.parametrize("mode", MODES, ids=MODE_IDS)
def test_fp8_multi_range(mode):
    B, H, N, d, K = 2, 2, 900, 128, 3
    rng = np.random.default_rng(33)
    s, e = multi_intervals("random_empty", B, K, N, rng)
    qkv8 = inputs.make_qkv_fp8(B, H, N, d, seed=33)
    check_fp8_model(qkv8, s, e, inputs.default_scale(d), f"fp8 multi mode {mode}", mode)


def test_fp8_weights_doc_packed_workload_sampled_rows():
    """FM_FP8_ALL on the doc-packed workload (B=1, H=16, N=8192, d=128), the elementwise
    bound on a sample of rows from every query tile (first, last and a random row)."""
    cfg = inputs.CONFIGS["C2"]
    spec = inputs.config_intervals(cfg)
    qkv8 = inputs.make_qkv_fp8(cfg.B, cfg.H, cfg.N, cfg.d, cfg.seed)
    rng = np.random.default_rng(5)
    tiles = np.arange(0, cfg.N, 128)
    rows = np.unique(np.concatenate([tiles, tiles + 127, tiles + rng.integers(0, 128, tiles.size)]))
    log(f"fp8 all C2, {rows.size} rows")
    check_fp8_model(qkv8, spec.col_start, spec.col_end, inputs.default_scale(cfg.d), "fp8 all C2",
                    fm.FM_FP8_ALL, rows=rows)


@pytest.mark.parametrize("mode", MODES, ids=MODE_IDS)
def test_fp8_prefix_lm_workload_full_size_sampled(mode):
    """The prefix-LM workload at full size (B=2, H=32, N=16384, d=128) from FP8 inputs, all
    heads in one launch as the benchmark runs it; the mode's elementwise bound and the LSE
    bar on sampled rows (tile edges, both prefix boundaries, random rows) of four heads of
    each batch element."""
    cfg = inputs.CONFIGS["C4"]
    spec = inputs.config_intervals(cfg)
    scale = inputs.default_scale(cfg.d)
    qkv8 = inputs.make_qkv_fp8(cfg.B, cfg.H, cfg.N, cfg.d, cfg.seed)
    log(f"fp8 C4 full size, mode {mode}")
    O, L = run_fp8(qkv8, spec.col_start, spec.col_end, scale, mode)
    rng = np.random.default_rng(7)
    prefix_edges = [p + o for p in (spec.col_end[:, 0] + 1).tolist() for o in (-1, 0, 1)]
    rows = np.unique(np.concatenate([[0, 127, 128, cfg.N - 1], prefix_edges, rng.integers(0, cfg.N, 22)]))
    heads = [0, 7, 19, 31]
    q, k, v = (inputs.dequantize_e4m3(c, sc)[:, heads] for c, sc in qkv8)
    O_ref, L_ref = oracle.attention(q, k, v, spec.col_start, spec.col_end, scale, rows=rows)
    P = oracle.attention_weights(q, k, spec.col_start, spec.col_end, scale, rows=rows)
    O, L = O[:, heads][:, :, rows], L[:, heads][:, :, rows]
    bound = fp8_bound(mode, P, v, O_ref)
    err = np.abs(O - O_ref)
    empty = np.isneginf(L_ref)
    assert not empty.any()
    dL = float(np.abs(L - L_ref).max())
    log(f"fp8 C4 mode {mode}: {rows.size} rows x {len(heads)} heads x 2: max|dO|={err.max():.3e} "
        f"max err/bound={(err / bound).max():.3f} max|dLSE|={dL:.3e}")
    assert np.all(err <= bound), f"{(err > bound).sum()} elements beyond the rounding bound"
    assert dL <= 1e-3


def test_fp8_doc_packed_workload():
    """The doc-packed workload (B=1, H=16, N=8192, d=128) from FP8 inputs, all rows."""
    cfg = inputs.CONFIGS["C2"]
    spec = inputs.config_intervals(cfg)
    qkv8 = inputs.make_qkv_fp8(cfg.B, cfg.H, cfg.N, cfg.d, cfg.seed)
    log("fp8 C2")
    dO, dL = check_fp8(qkv8, spec.col_start, spec.col_end, inputs.default_scale(cfg.d), "fp8 C2")
    log(f"fp8 C2: max|dO|={dO:.3e} max|dLSE|={dL:.3e}")


@pytest.mark.parametrize("mode", MODES, ids=MODE_IDS)
def test_fp8_zero_q_is_mean_of_v(mode):
    """Q = 0: O_r is the mean of the dequantized v over the row's keys, LSE_r = ln(#keys)
    (every weight is 1, exact in both weight formats)."""
    B, H, N, d = 1, 2, 500, 128
    rng = np.random.default_rng(41)
    s, e = inputs.random_intervals(rng, B, N, empty_frac=0.05, max_width=250)
    qkv8 = list(inputs.make_qkv_fp8(B, H, N, d, seed=41))
    qkv8[0] = (torch.zeros_like(qkv8[0][0]), qkv8[0][1])
    O, L = run_fp8(qkv8, s, e, inputs.default_scale(d), mode)
    v = inputs.dequantize_e4m3(*qkv8[2])
    for i in range(N):
        if s[0, i] > e[0, i]:
            assert np.all(O[0, :, i] == 0) and np.all(np.isneginf(L[0, :, i]))
            continue
        mean = v[0][:, s[0, i]:e[0, i] + 1].mean(axis=1)
        assert np.abs(O[0, :, i] - mean).max() <= 1e-2
        assert np.abs(L[0, :, i] - np.log(e[0, i] - s[0, i] + 1)).max() <= 1e-3
