"""Pins of the float64 attention oracle against what the pages and mathematics fix (CPU).

Each ``pin_*`` takes the attention function under test so that the planted-
mistake tests (test_oracle_mutants.py) can run the same pins against altered
copies of the oracle and show that every plausible mistake is caught.
"""
import math

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import oracle
from masked_attention_fm_amd import inputs

SCALE = inputs.default_scale


def _qkv(B, H, N, d, seed):
    q, k, v = inputs.make_qkv(B, H, N, d, seed, threads=1)
    return q.float().numpy(), k.float().numpy(), v.float().numpy()


def _sdpa(q, k, v, scale, attn_mask=None, is_causal=False):
    """torch's reference attention in float64 on the CPU (one [N, d] slice)."""
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64))[None, None]
    m = None if attn_mask is None else torch.from_numpy(attn_mask)[None, None]
    out = torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), attn_mask=m, is_causal=is_causal, scale=float(np.float32(scale)))
    return out[0, 0].numpy()


# ---------------------------------------------------------------- pins


def pin_bruteforce(attn):
    """Scalar brute force from a hand-built mask, math.fsum / math.exp (tiny N)."""
    rng = np.random.default_rng(11)
    for N in list(range(1, 18)) + [33]:
        B, H, d = 2, 2, 8
        q, k, v = _qkv(B, H, N, d, seed=N)
        s, e = inputs.random_intervals(rng, B, N, empty_frac=0.15)
        scale = SCALE(d)
        O, L = attn(q, k, v, s, e, scale)
        sc = float(np.float32(scale))
        for b in range(B):
            for h in range(H):
                for i in range(N):
                    keys = [j for j in range(N) if s[b, i] <= j and j <= e[b, i]]
                    if not keys:
                        assert np.all(O[b, h, i] == 0.0) and L[b, h, i] == -math.inf
                        continue
                    sc_ij = [sc * math.fsum(float(q[b, h, i, c]) * float(k[b, h, j, c]) for c in range(d))
                             for j in keys]
                    mx = max(sc_ij)
                    w = [math.exp(x - mx) for x in sc_ij]
                    tot = math.fsum(w)
                    for c in range(d):
                        ref = math.fsum(wj * float(v[b, h, j, c]) for wj, j in zip(w, keys)) / tot
                        assert abs(O[b, h, i, c] - ref) <= 1e-12 * (1 + abs(ref))
                    assert abs(L[b, h, i] - (mx + math.log(tot))) <= 1e-12 * (1 + abs(mx))


def pin_q_zero(attn):
    """Q = 0 makes every attended weight equal: O_r is the mean of v over [s_r, e_r]
    (taken from prefix sums) and LSE_r = ln(e_r - s_r + 1)."""
    rng = np.random.default_rng(5)
    B, H, N, d = 2, 3, 130, 16
    _, k, v = _qkv(B, H, N, d, seed=3)
    q = np.zeros_like(k)
    s, e = inputs.random_intervals(rng, B, N, empty_frac=0.1)
    O, L = attn(q, k, v, s, e, SCALE(d))
    csum = np.concatenate([np.zeros((B, H, 1, d)), np.cumsum(v.astype(np.float64), axis=2)], axis=2)
    for b in range(B):
        for i in range(N):
            if s[b, i] > e[b, i]:
                assert np.all(O[b, :, i] == 0) and np.all(L[b, :, i] == -np.inf)
                continue
            n = e[b, i] - s[b, i] + 1
            mean = (csum[b, :, e[b, i] + 1] - csum[b, :, s[b, i]]) / n
            np.testing.assert_allclose(O[b, :, i], mean, rtol=0, atol=1e-12)
            np.testing.assert_allclose(L[b, :, i], math.log(n), rtol=0, atol=1e-13)


def pin_width_one(attn):
    """A one-key window s_r = e_r = r gives O_r = v_r and LSE_r = scale * q_r . k_r."""
    B, H, N, d = 1, 2, 70, 32
    q, k, v = _qkv(B, H, N, d, seed=9)
    r = np.arange(N, dtype=np.int32)[None]
    O, L = attn(q, k, v, r, r, SCALE(d))
    assert np.array_equal(O, v.astype(np.float64))
    ref = float(np.float32(SCALE(d))) * np.einsum("bhnd,bhnd->bhn", q.astype(np.float64), k.astype(np.float64))
    np.testing.assert_allclose(L, ref, rtol=1e-14, atol=1e-14)


def pin_causal_row0(attn):
    """Causal row 0 attends only key 0: O_0 = v_0 exactly, LSE_0 = scale * q_0 . k_0."""
    B, H, N, d = 1, 2, 40, 64
    q, k, v = _qkv(B, H, N, d, seed=1)
    s, e = inputs.causal_intervals(N)
    O, L = attn(q, k, v, s[None], e[None], SCALE(d))
    assert np.array_equal(O[:, :, 0], v[:, :, 0].astype(np.float64))
    ref = float(np.float32(SCALE(d))) * (q[:, :, 0].astype(np.float64) * k[:, :, 0]).sum(-1)
    np.testing.assert_allclose(L[:, :, 0], ref, rtol=1e-14)


def pin_full_and_causal_vs_sdpa(attn):
    """Full mask and causal mask equal torch's scaled_dot_product_attention (float64)."""
    B, H, N, d = 1, 2, 97, 64
    q, k, v = _qkv(B, H, N, d, seed=2)
    full = (np.zeros((1, N), np.int32), np.full((1, N), N - 1, np.int32))
    cs, ce = inputs.causal_intervals(N)
    for (s, e), causal in ((full, False), ((cs[None], ce[None]), True)):
        O, L = attn(q, k, v, s, e, SCALE(d))
        for h in range(H):
            ref = _sdpa(q[0, h], k[0, h], v[0, h], SCALE(d), is_causal=causal)
            np.testing.assert_allclose(O[0, h], ref, rtol=0, atol=1e-12)


def pin_sliding_vs_sdpa(attn):
    """Sliding window equals torch's attention under a band mask built with tril/triu."""
    B, H, N, d, w = 1, 2, 150, 32, 17
    q, k, v = _qkv(B, H, N, d, seed=4)
    s, e = inputs.sliding_window_intervals(N, w)
    O, L = attn(q, k, v, s[None], e[None], SCALE(d))
    ones = torch.ones(N, N, dtype=torch.bool)
    band = (torch.tril(ones) & torch.triu(ones, diagonal=-(w - 1))).numpy()
    for h in range(H):
        ref = _sdpa(q[0, h], k[0, h], v[0, h], SCALE(d), attn_mask=band)
        np.testing.assert_allclose(O[0, h], ref, rtol=0, atol=1e-12)


def pin_doc_packing_is_per_doc_causal(attn):
    """Packed documents = causal attention run separately on each document's slice."""
    lens = [5, 1, 40, 17, 64, 3]
    N = sum(lens)
    B, H, d = 1, 2, 32
    q, k, v = _qkv(B, H, N, d, seed=6)
    s, e = inputs.doc_causal_intervals(lens)
    O, L = attn(q, k, v, s[None], e[None], SCALE(d))
    off = 0
    for Ln in lens:
        sl = slice(off, off + Ln)
        for h in range(H):
            ref = _sdpa(q[0, h, sl], k[0, h, sl], v[0, h, sl], SCALE(d), is_causal=True)
            np.testing.assert_allclose(O[0, h, sl], ref, rtol=0, atol=1e-12)
        off += Ln


def pin_prefix_lm(attn):
    """Prefix rows attend the whole prefix bidirectionally; later rows are causal."""
    N, p, d = 90, 31, 32
    q, k, v = _qkv(1, 1, N, d, seed=8)
    s, e = inputs.prefix_lm_intervals(N, p)
    O, L = attn(q, k, v, s[None], e[None], SCALE(d))
    ref_pre = _sdpa(q[0, 0, :p], k[0, 0, :p], v[0, 0, :p], SCALE(d))
    np.testing.assert_allclose(O[0, 0, :p], ref_pre, rtol=0, atol=1e-12)
    ref_causal = _sdpa(q[0, 0], k[0, 0], v[0, 0], SCALE(d), is_causal=True)
    np.testing.assert_allclose(O[0, 0, p:], ref_causal[p:], rtol=0, atol=1e-12)


def pin_lse_logsumexp(attn):
    """LSE equals scipy's logsumexp of the scaled scores over each row's interval."""
    rng = np.random.default_rng(12)
    B, H, N, d = 1, 2, 77, 16
    q, k, v = _qkv(B, H, N, d, seed=12)
    s, e = inputs.random_intervals(rng, B, N)
    O, L = attn(q, k, v, s, e, SCALE(d))
    sc = float(np.float32(SCALE(d)))
    for h in range(H):
        S = sc * (q[0, h].astype(np.float64) @ k[0, h].astype(np.float64).T)
        for i in range(N):
            assert abs(L[0, h, i] - logsumexp(S[i, s[0, i]:e[0, i] + 1])) < 1e-12


def pin_linearity(attn):
    """Weights sum to one: O(a*v + c) = a*O(v) + c for scalar a and vector c."""
    rng = np.random.default_rng(13)
    B, H, N, d = 1, 2, 50, 8
    q, k, v = _qkv(B, H, N, d, seed=13)
    s, e = inputs.random_intervals(rng, B, N)
    a, c = -1.75, np.linspace(-3, 3, d)
    O1, _ = attn(q, k, v, s, e, SCALE(d))
    O2, _ = attn(q, k, a * v.astype(np.float64) + c, s, e, SCALE(d))
    np.testing.assert_allclose(O2, a * O1 + c, rtol=0, atol=1e-12)


def pin_multi_overlap_is_single(attn):
    """Two overlapping (or touching) ranges per row equal the single range that covers both."""
    rng = np.random.default_rng(40)
    B, H, N, d = 2, 2, 120, 16
    q, k, v = _qkv(B, H, N, d, seed=40)
    a = rng.integers(0, N, size=(B, N))
    dd = np.minimum(N - 1, a + rng.integers(0, 60, size=(B, N)))
    b_ = a + (rng.random((B, N)) * (dd - a + 1)).astype(np.int64)           # a <= b <= d
    c_ = np.minimum(dd, np.maximum(b_ - 1, a + rng.integers(0, 40, size=(B, N))))   # b-1 <= c <= d
    cs = np.stack([a, b_], axis=1).astype(np.int32)
    ce = np.stack([c_, dd], axis=1).astype(np.int32)
    O2, L2 = attn(q, k, v, cs, ce, SCALE(d))
    O1, L1 = attn(q, k, v, a.astype(np.int32), dd.astype(np.int32), SCALE(d))
    np.testing.assert_allclose(O2, O1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(L2, L1, rtol=0, atol=1e-12)


def pin_sinks_window_vs_sdpa(attn):
    """Attention sinks plus a causal window equal torch's attention under a mask built
    from tril/triu and the first columns."""
    B, H, N, d, w, sinks = 1, 2, 130, 32, 20, 5
    q, k, v = _qkv(B, H, N, d, seed=41)
    cs, ce = inputs.sinks_window_intervals(N, w, sinks)
    O, L = attn(q, k, v, cs[None], ce[None], SCALE(d))
    ones = torch.ones(N, N, dtype=torch.bool)
    causal = torch.tril(ones)
    band = causal & torch.triu(ones, diagonal=-(w - 1))
    sink = causal.clone()
    sink[:, sinks:] = False
    mask = (band | sink).numpy()
    for h in range(H):
        ref = _sdpa(q[0, h], k[0, h], v[0, h], SCALE(d), attn_mask=mask)
        np.testing.assert_allclose(O[0, h], ref, rtol=0, atol=1e-12)


def pin_multi_q_zero(attn):
    """Q = 0 with disjoint ranges: O is the mean of v over the union, LSE = ln(|union|)."""
    rng = np.random.default_rng(42)
    B, H, N, d, K = 1, 2, 90, 8, 3
    _, k, v = _qkv(B, H, N, d, seed=42)
    q = np.zeros_like(k)
    cs, ce = inputs.random_multi_intervals(rng, B, K, N, empty_frac=0.2, max_width=15)
    O, L = attn(q, k, v, cs, ce, SCALE(d))
    for i in range(N):
        keys = sorted({j for kk in range(K) for j in range(max(cs[0, kk, i], 0), min(ce[0, kk, i], N - 1) + 1)})
        if not keys:
            assert np.all(O[0, :, i] == 0) and np.all(np.isneginf(L[0, :, i]))
            continue
        np.testing.assert_allclose(O[0, :, i], v[0][:, keys].astype(np.float64).mean(axis=1), rtol=0, atol=1e-12)
        np.testing.assert_allclose(L[0, :, i], math.log(len(keys)), rtol=0, atol=1e-13)


ALL_PINS = [pin_bruteforce, pin_q_zero, pin_width_one, pin_causal_row0,
            pin_multi_overlap_is_single, pin_sinks_window_vs_sdpa, pin_multi_q_zero,
            pin_full_and_causal_vs_sdpa, pin_sliding_vs_sdpa,
            pin_doc_packing_is_per_doc_causal, pin_prefix_lm, pin_lse_logsumexp,
            pin_linearity]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(oracle.attention)


# ---------------------------------------------------------------- weights


def test_weight_invariants():
    """Each attended row's weights sum to 1; weights outside the interval are exactly 0
    and inside strictly positive; empty rows have no weight."""
    rng = np.random.default_rng(21)
    B, H, N, d = 2, 2, 64, 16
    q, k, v = _qkv(B, H, N, d, seed=21)
    s, e = inputs.random_intervals(rng, B, N, empty_frac=0.1)
    P = oracle.attention_weights(q, k, s, e, SCALE(d))
    for b in range(B):
        for i in range(N):
            inside = np.zeros(N, bool)
            inside[s[b, i]:e[b, i] + 1] = True
            for h in range(H):
                row = P[b, h, i]
                assert np.all(row[~inside] == 0.0)
                if inside.any():
                    assert np.all(row[inside] > 0.0)
                    assert abs(row.sum() - 1.0) < 1e-12
                else:
                    assert row.sum() == 0.0
    # the weights reproduce O
    O, _ = oracle.attention(q, k, v, s, e, SCALE(d))
    np.testing.assert_allclose(np.einsum("bhij,bhjd->bhid", P, v.astype(np.float64)), O, atol=1e-12)


def test_sampled_rows_equal_full_rows():
    """Evaluating a subset of rows gives the same values as the full evaluation
    (up to the summation order of the float64 matrix products)."""
    rng = np.random.default_rng(30)
    B, H, N, d = 2, 2, 300, 16
    q, k, v = _qkv(B, H, N, d, seed=30)
    s, e = inputs.random_intervals(rng, B, N, empty_frac=0.05, max_width=40)
    O, L = oracle.attention(q, k, v, s, e, SCALE(d), row_block=64)
    rows = np.array([0, 1, 63, 64, 65, 150, 299])
    Os, Ls = oracle.attention(q, k, v, s, e, SCALE(d), rows=rows, row_block=3)
    np.testing.assert_allclose(Os, O[:, :, rows], rtol=0, atol=1e-14)
    np.testing.assert_allclose(Ls, L[:, :, rows], rtol=0, atol=1e-14)
    P = oracle.attention_weights(q, k, s, e, SCALE(d))
    Ps = oracle.attention_weights(q, k, s, e, SCALE(d), rows=rows)
    np.testing.assert_allclose(Ps, P[:, :, rows], rtol=0, atol=1e-15)


def test_bf16_round_matches_torch():
    x = np.random.default_rng(0).standard_normal(100000) * 10.0
    x = x.astype(np.float32).astype(np.float64)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(oracle.bf16_round(x), ref)
    assert oracle.bf16_round(np.array([1.0 + 2 ** -8]))[0] == 1.0          # tie -> even
    assert oracle.bf16_round(np.array([1.0 + 3 * 2 ** -8]))[0] == 1.0 + 2 ** -6
