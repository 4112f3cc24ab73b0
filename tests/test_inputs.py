"""Seeded input generators: interval closed forms and random draws (CPU)."""
import json
import os

import numpy as np
import pytest
import torch

from masked_attention_fm_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_causal_matches_page_example():
    with open(os.path.join(GOLDEN, "causal_intervals_example.json")) as f:
        g = json.load(f)
    s, e = inputs.causal_intervals(g["N"])
    assert s.tolist() == g["col_start"]
    assert e.tolist() == g["col_end"]


def test_doc_packing_matches_page_example():
    with open(os.path.join(GOLDEN, "doc_packing_example.json")) as f:
        g = json.load(f)
    s, e = inputs.doc_causal_intervals(g["doc_lengths"])
    assert s.shape == (g["N"],) and e.shape == (g["N"],)
    for blk in g["row_blocks"]:
        rows = np.arange(blk["first_row"], blk["last_row"] + 1)
        assert np.all(s[rows] == blk["col_start"])
        assert np.all(e[rows] == rows)


@pytest.mark.parametrize("N,w", [(1, 1), (10, 1), (10, 3), (64, 64), (100, 1000), (32768, 1024)])
def test_sliding_window_closed_form(N, w):
    s, e = inputs.sliding_window_intervals(N, w)
    for i in [0, 1, w - 2, w - 1, w, N // 2, N - 1]:
        if 0 <= i < N:
            assert s[i] == max(0, i - w + 1) and e[i] == i
    assert np.all(e - s + 1 == np.minimum(np.arange(N) + 1, w))


@pytest.mark.parametrize("N,p", [(16, 0), (16, 1), (16, 5), (16, 16), (16384, 2048)])
def test_prefix_lm_closed_form(N, p):
    s, e = inputs.prefix_lm_intervals(N, p)
    i = np.arange(N)
    assert np.all(s == 0)
    assert np.all(e[i < p] == p - 1)
    assert np.all(e[i >= p] == i[i >= p])


def test_uniform_doc_lengths():
    rng = np.random.default_rng(7)
    for N in (1, 255, 8192, 10000):
        lens = inputs.uniform_doc_lengths(rng, N, 256, 2048)
        assert sum(lens) == N
        assert all(256 <= L <= 2048 for L in lens[:-1])
        assert 1 <= lens[-1] <= 2048


def test_lognormal_doc_lengths():
    rng = np.random.default_rng(3)
    lens = inputs.lognormal_doc_lengths(rng, 1 << 20, 4096, 1.0, 128, 32768)
    assert sum(lens) == 1 << 20
    body = np.array(lens[:-1])
    assert body.min() >= 128 and body.max() <= 32768
    # the median of the clipped draw is the median of the unclipped one
    assert 3000 < np.median(body) < 5500


def test_config_intervals_deterministic_and_valid():
    for key, cfg in inputs.CONFIGS.items():
        a = inputs.config_intervals(cfg)
        b = inputs.config_intervals(cfg)
        assert np.array_equal(a.col_start, b.col_start) and np.array_equal(a.col_end, b.col_end)
        assert a.col_start.dtype == np.int32 and a.col_end.shape == a.col_start.shape
        if cfg.mask == "sinks_window":
            assert a.col_start.shape == (cfg.B, 2, cfg.N)
            s, e = inputs.sinks_window_intervals(cfg.N, cfg.param("window"), cfg.param("sinks"))
            assert all(np.array_equal(a.col_start[b], s) and np.array_equal(a.col_end[b], e)
                       for b in range(cfg.B))
            continue
        assert a.col_start.shape == (cfg.B, cfg.N)
        assert np.all(0 <= a.col_start) and np.all(a.col_start <= a.col_end)
        assert np.all(a.col_end <= cfg.N - 1)
        if cfg.mask == "prefix_lm":
            assert all(cfg.N // 8 <= p <= cfg.N // 2 for p in a.prefix)
        if cfg.mask.startswith("doc"):
            assert all(sum(L) == cfg.N for L in a.doc_lengths)


def test_qkv_deterministic_bf16_normal():
    q, k, v = inputs.make_qkv(1, 2, 256, 64, seed=5, threads=2)
    q2, k2, v2 = inputs.make_qkv(1, 2, 256, 64, seed=5, threads=1)
    for x, y in ((q, q2), (k, k2), (v, v2)):
        assert x.dtype == torch.bfloat16 and x.shape == (1, 2, 256, 64)
        assert torch.equal(x, y)
    assert not torch.equal(q, k)
    allv = torch.cat([q.flatten(), k.flatten(), v.flatten()]).float()
    assert abs(allv.mean().item()) < 0.02 and abs(allv.std().item() - 1) < 0.02
    # a slice regenerated alone equals the slice in the full tensor
    assert torch.equal(inputs.qkv_slice(5, "v", 0, 1, 256, 64), v[0, 1])


def test_sinks_window_closed_form():
    s, e = inputs.sinks_window_intervals(50, 8, 3)
    assert s.shape == (2, 50)
    for i in range(50):
        assert (s[0, i], e[0, i]) == (0, min(2, i))
        assert (s[1, i], e[1, i]) == (max(0, i - 7), i)
    s, e = inputs.sinks_window_intervals(10, 4, 0)      # no sinks: an empty first range
    assert np.all(e[0] < s[0])


def test_random_intervals_valid():
    rng = np.random.default_rng(0)
    s, e = inputs.random_intervals(rng, 2, 333, empty_frac=0.2)
    nonempty = s <= e
    assert np.all(s >= 0) and np.all(e <= 332)
    assert 0.1 < 1 - nonempty.mean() < 0.3


def test_e4m3_decode_known_codes():
    """OCP e4m3fn: bias 7, 3 mantissa bits, largest finite 448, no infinities."""
    codes = torch.tensor([0x00, 0x01, 0x07, 0x08, 0x38, 0x3C, 0x7E, 0x80, 0xB8, 0x7F], dtype=torch.uint8)
    vals = inputs.dequantize_e4m3(codes, 1.0)
    expect = [0.0, 2.0 ** -9, 7 * 2.0 ** -9, 2.0 ** -6, 1.0, 1.5, 448.0, -0.0, -1.0]
    assert vals[:9].tolist() == expect
    assert np.isnan(vals[9])


def test_quantize_e4m3_round_trip():
    x = torch.randn(4096, generator=torch.Generator().manual_seed(1))
    codes, scale = inputs.quantize_e4m3(x)
    assert codes.dtype == torch.uint8 and scale > 0
    back = inputs.dequantize_e4m3(codes, scale)
    assert np.abs(back).max() <= 448.0 * scale * (1 + 1e-7)
    # relative error of a round-to-nearest 4-significant-bit code, away from the subnormals
    big = np.abs(x.numpy()) > 2.0 ** -6 * scale
    rel = np.abs(back[big] - x.numpy()[big]) / np.abs(x.numpy()[big])
    assert rel.max() <= 2.0 ** -4 + 1e-6
