"""Pins of the tile-class oracle and the unmasked-entry count (CPU).

Closed forms: a causal mask with square T x T tiles and n = N/T blocks has
n(n+1)/2 non-skip tiles, so the skipped share (n-1)/(2n) tends to the "about
half" the FlashMask article (§1 item 2 and §2.2) states for causal masks.
"""
import numpy as np
import pytest

import oracle
from oracle import SKIP, FULL, PARTIAL
from masked_attention_fm_amd import inputs


def _counts(tab):
    return {c: int((tab == c).sum()) for c in (SKIP, FULL, PARTIAL)}


def pin_causal_square(classes):
    for N, T in ((512, 128), (512, 64), (1024, 32), (96, 32)):
        n = N // T
        s, e = inputs.causal_intervals(N)
        c = _counts(classes(s, e, N, T, T))
        assert c[SKIP] == n * (n - 1) // 2
        assert c[PARTIAL] == n                   # the diagonal
        assert c[FULL] == n * (n - 1) // 2


def pin_causal_c1_ratio(classes):
    s, e = inputs.causal_intervals(512)
    tab = classes(s, e, 512, 128, 128)
    assert (tab == SKIP).mean() == 0.375


def pin_causal_rect(classes):
    """Br = 2*Bc: query block t keeps key blocks 0..2t+1; 2t full, 2 partial."""
    N, Br, Bc = 1024, 128, 64
    s, e = inputs.causal_intervals(N)
    tab = classes(s, e, N, Br, Bc)
    for t in range(N // Br):
        assert np.all(tab[t, :2 * t] == FULL)
        assert np.all(tab[t, 2 * t:2 * t + 2] == PARTIAL)
        assert np.all(tab[t, 2 * t + 2:] == SKIP)


def pin_sliding_closed_form(classes):
    """w = 1024, T = 128, N = 32768: sum_{t<8}(t+1) + 248*9 = 2268 non-skip tiles, 504 partial."""
    N, w, T = 32768, 1024, 128
    s, e = inputs.sliding_window_intervals(N, w)
    c = _counts(classes(s, e, N, T, T))
    assert c[FULL] + c[PARTIAL] == 2268
    assert c[PARTIAL] == 504
    assert abs(c[SKIP] / (N // T) ** 2 - 0.96539) < 1e-5


def pin_ragged_tail(classes):
    """Ragged last blocks (N = 100, Br = 48, Bc = 40; key blocks [0,39], [40,79], [80,99]).
    A full mask makes every tile FULL; rows attending [80, 99] keep only the short last
    block, as FULL; rows attending only key 99 keep it as PARTIAL."""
    N = 100
    s = np.zeros(N, np.int32)
    e = np.full(N, N - 1, np.int32)
    assert np.all(classes(s, e, N, 48, 40) == FULL)
    tab = classes(np.full(N, 80, np.int32), e, N, 48, 40)
    assert np.all(tab[:, :2] == SKIP) and np.all(tab[:, 2] == FULL)
    tab = classes(np.full(N, 99, np.int32), e, N, 48, 40)
    assert np.all(tab[:, :2] == SKIP) and np.all(tab[:, 2] == PARTIAL)


def pin_against_dense(classes):
    """Full sets equal the dense rule's; min/max skips are a subset of dense-empty tiles."""
    rng = np.random.default_rng(1)
    for N, Br, Bc in ((1, 1, 1), (7, 3, 2), (130, 16, 16), (257, 64, 32), (200, 33, 17), (300, 128, 64)):
        for width in (None, 5, 60):
            s, e = inputs.random_intervals(rng, 1, N, max_width=width)
            a = classes(s[0], e[0], N, Br, Bc)
            b = oracle.classes_dense(s[0], e[0], N, Br, Bc)
            assert np.array_equal(a == FULL, b == FULL)
            assert np.all(b[a == SKIP] == SKIP)


ALL_PINS = [pin_causal_square, pin_causal_c1_ratio, pin_causal_rect, pin_sliding_closed_form,
            pin_ragged_tail, pin_against_dense]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_tile_pin(pin):
    pin(oracle.classes_minmax)


def pin_multi_sinks_window_counts(classes_multi):
    """Sinks (10) + window (1024), N = 32768, 128x128 tiles: the window's 2268 non-skip
    tiles (504 partial) plus key block 0 as a partial tile for the 247 query blocks
    t >= 9 whose window no longer reaches it: 2515 non-skip, 751 partial."""
    N = 32768
    s, e = inputs.sinks_window_intervals(N, 1024, 10)
    c = _counts(classes_multi(s, e, N, 128, 128))
    assert c[FULL] + c[PARTIAL] == 2515
    assert c[PARTIAL] == 751


def pin_multi_against_dense(classes_multi):
    """Union rule vs dense count: FULL implies dense-full, SKIP implies dense-empty; a range
    that covers a tile for every row makes it FULL; one range reproduces the single rule."""
    rng = np.random.default_rng(9)
    for N, Br, Bc in ((130, 16, 16), (257, 64, 32), (200, 33, 17)):
        s, e = inputs.random_multi_intervals(rng, 1, 3, N, max_width=40)
        a = classes_multi(s[0], e[0], N, Br, Bc)
        d = oracle.classes_dense(s[0], e[0], N, Br, Bc)
        assert np.all(d[a == FULL] == FULL)
        assert np.all(d[a == SKIP] == SKIP)
        assert np.array_equal(classes_multi(s[0][:1], e[0][:1], N, Br, Bc),
                              oracle.classes_minmax(s[0][0], e[0][0], N, Br, Bc))
    # a second range covering everything turns every tile FULL
    N = 100
    s0, e0 = inputs.causal_intervals(N)
    s = np.stack([s0, np.zeros(N, np.int32)])
    e = np.stack([e0, np.full(N, N - 1, np.int32)])
    assert np.all(classes_multi(s, e, N, 32, 32) == FULL)


MULTI_PINS = [pin_multi_sinks_window_counts, pin_multi_against_dense]


@pytest.mark.parametrize("pin", MULTI_PINS, ids=lambda f: f.__name__)
def test_multi_tile_pin(pin):
    pin(oracle.classes_minmax_multi)


def test_causal_skip_tends_to_half():
    N, T = 1 << 16, 64
    n = N // T
    s, e = inputs.causal_intervals(N)
    ratio = (oracle.classes_minmax(s, e, N, T, T) == SKIP).mean()
    assert ratio == (n - 1) / (2 * n) and abs(ratio - 0.5) < 1e-3


@pytest.mark.parametrize("key", ["C1", "C2", "C3", "C4"])
@pytest.mark.parametrize("Br,Bc", [(128, 64), (128, 128), (256, 64)])
def test_rules_agree_on_structured_masks(key, Br, Bc):
    """On monotone document-causal, sliding-window and prefix-LM structure the two rules agree."""
    cfg = inputs.CONFIGS[key]
    N = min(cfg.N, 8192)
    params = dict(cfg.params)
    spec = inputs.make_intervals(cfg.mask, cfg.B, N, cfg.seed, **params)
    for b in range(cfg.B):
        a = oracle.classes_minmax(spec.col_start[b], spec.col_end[b], N, Br, Bc)
        d = oracle.classes_dense(spec.col_start[b], spec.col_end[b], N, Br, Bc)
        assert np.array_equal(a, d)


def test_rules_agree_on_lognormal_docs():
    spec = inputs.make_intervals("doc_lognormal", 1, 16384, 1004, median=1024, sigma=1.0, lo=16, hi=8192)
    a = oracle.classes_minmax(spec.col_start[0], spec.col_end[0], 16384, 128, 64)
    d = oracle.classes_dense(spec.col_start[0], spec.col_end[0], 16384, 128, 64)
    assert np.array_equal(a, d)


# ---------------------------------------------------------------- non-skip counts per query block


def pin_nonskip_row_sums(fn):
    """Pinned to the scalar-loop class table (a separate evaluation of the same rule)."""
    for N, Br, Bc in ((1, 1, 1), (7, 3, 2), (300, 128, 64), (1000, 33, 17), (4097, 128, 64)):
        rng = np.random.default_rng(N + Br)
        for width in (None, 3, 200):
            s, e = inputs.random_intervals(rng, 1, N, max_width=width)
            table = oracle.classes_minmax(s[0], e[0], N, Br, Bc)
            for bpp in (1, 5, 64):
                got = fn(s[0], e[0], N, Br, Bc, blocks_per_pass=bpp)
                assert np.array_equal(got, (table != SKIP).sum(axis=1))


def pin_nonskip_causal(fn):
    """Causal, Br = 2 Bc: query block t reaches key block 2t + 1, so 2t + 2 blocks are kept."""
    N, Br, Bc = 1 << 15, 128, 64
    s, e = inputs.causal_intervals(N)
    assert np.array_equal(fn(s, e, N, Br, Bc), 2 * np.arange(N // Br) + 2)


def pin_nonskip_window(fn):
    """Sliding window w = 1024, Br = 128, Bc = 64: from query block 8 on, every block keeps
    its 16 window blocks plus the partly covered block on each side: 18."""
    N, Br, Bc = 1 << 14, 128, 64
    s, e = inputs.sliding_window_intervals(N, 1024)
    got = fn(s, e, N, Br, Bc)
    assert np.all(got[8:] == 18) and np.array_equal(got[:8], 2 * np.arange(8) + 2)


NONSKIP_PINS = [pin_nonskip_row_sums, pin_nonskip_causal, pin_nonskip_window]


@pytest.mark.parametrize("pin", NONSKIP_PINS, ids=lambda f: f.__name__)
def test_nonskip_pin(pin):
    pin(oracle.nonskip_counts)


# ---------------------------------------------------------------- unmasked entries


@pytest.mark.parametrize("N", [1, 2, 17, 512, 3000])
def test_unmasked_causal(N):
    s, e = inputs.causal_intervals(N)
    assert oracle.unmasked_count(s, e, N) == N * (N + 1) // 2


@pytest.mark.parametrize("N,w", [(5000, 1024), (300, 7), (50, 100)])
def test_unmasked_sliding(N, w):
    s, e = inputs.sliding_window_intervals(N, w)
    w_eff = min(w, N)
    assert oracle.unmasked_count(s, e, N) == w_eff * (w_eff + 1) // 2 + (N - w_eff) * w_eff


def test_unmasked_prefix_and_docs():
    N, p = 4096, 1000
    s, e = inputs.prefix_lm_intervals(N, p)
    assert oracle.unmasked_count(s, e, N) == N * (N + 1) // 2 + p * (p - 1) // 2
    lens = [1024, 2048, 512, 7]
    s, e = inputs.doc_causal_intervals(lens)
    assert oracle.unmasked_count(s, e, sum(lens)) == sum(L * (L + 1) // 2 for L in lens)


def test_unmasked_c3_exact():
    """Sliding w = 1024 at N = 32768: w(w+1)/2 + (N-w)w = 33,030,656 per head."""
    s, e = inputs.sliding_window_intervals(32768, 1024)
    assert oracle.unmasked_count(s, e, 32768) == 33030656
