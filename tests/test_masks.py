"""The mask-specification builder (host side): interval arrays against hand-built ones,
their dense masks against hand-written matrices, and agreement with the workload
generators (CPU only)."""
import numpy as np
import pytest

import oracle
from masked_attention_fm_amd import inputs
from masked_attention_fm_amd import masks as mk

N = 8
I = list(range(N))

HAND = {
    # spec: (col_start [K][N], col_end [K][N]) written out by hand for N = 8
    "full": (mk.Full(), [[0] * 8], [[7] * 8]),
    "causal": (mk.Causal(), [[0] * 8], [I]),
    "window3": (mk.SlidingWindow(3), [[0, 0, 0, 1, 2, 3, 4, 5]], [I]),
    "prefix3": (mk.PrefixLM(3), [[0] * 8], [[2, 2, 2, 3, 4, 5, 6, 7]]),
    "docs35": (mk.Documents([3, 5]), [[0, 0, 0, 3, 3, 3, 3, 3]], [I]),
    "sinks2_window3": (mk.SinksWindow(3, 2), [[0] * 8, [0, 0, 0, 1, 2, 3, 4, 5]],
                       [[0, 1, 1, 1, 1, 1, 1, 1], I]),
}

# the same masks as dense N x N matrices, row i listing its attended keys
DENSE = {
    "full": [set(range(8))] * 8,
    "causal": [set(range(i + 1)) for i in range(8)],
    "window3": [set(range(max(0, i - 2), i + 1)) for i in range(8)],
    "prefix3": [set(range(3)) if i < 3 else set(range(i + 1)) for i in range(8)],
    "docs35": [set(range(0, i + 1)) if i < 3 else set(range(3, i + 1)) for i in range(8)],
    "sinks2_window3": [set(range(min(2, i + 1))) | set(range(max(0, i - 2), i + 1)) for i in range(8)],
}


def dense_from_sets(rows):
    M = np.zeros((N, N), bool)
    for i, keys in enumerate(rows):
        M[i, sorted(keys)] = True
    return M


@pytest.mark.parametrize("name", sorted(HAND))
def test_intervals_equal_hand_built_arrays(name):
    spec, s_hand, e_hand = HAND[name]
    s, e = mk.mask_intervals(spec, 2, N)
    assert s.dtype == np.int32 and e.dtype == np.int32 and s.shape == (2, len(s_hand), N)
    for b in range(2):
        assert np.array_equal(s[b], np.array(s_hand)) and np.array_equal(e[b], np.array(e_hand))


@pytest.mark.parametrize("name", sorted(HAND))
def test_dense_meaning_equals_hand_written_matrix(name):
    s, e = mk.mask_intervals(HAND[name][0], 1, N)
    assert np.array_equal(oracle.dense_mask(s[0], e[0], N), dense_from_sets(DENSE[name]))


def test_head_intervals_pad_with_empty_ranges():
    specs = [mk.Causal(), mk.SinksWindow(3, 2), mk.Documents([3, 5]), mk.SlidingWindow(3)]
    s, e = mk.head_intervals(specs, 2, N)
    assert s.shape == (2, 4, 2, N)
    names = ["causal", "sinks2_window3", "docs35", "window3"]
    for h, name in enumerate(names):
        _, s_hand, e_hand = HAND[name]
        k = len(s_hand)
        for b in range(2):
            assert np.array_equal(s[b, h, :k], np.array(s_hand))
            assert np.array_equal(e[b, h, :k], np.array(e_hand))
            assert np.all(s[b, h, k:] == 0) and np.all(e[b, h, k:] == -1)
        # the padded set means the same mask
        assert np.array_equal(oracle.dense_mask(s[0, h], e[0, h], N), dense_from_sets(DENSE[name]))
    s4, _ = mk.head_intervals(specs, 1, N, n_ranges=4)
    assert s4.shape == (1, 4, 4, N)
    with pytest.raises(ValueError):
        mk.head_intervals(specs, 1, N, n_ranges=1)


def test_per_batch_parameters():
    s, e = mk.mask_intervals(mk.PrefixLM([2, 5]), 2, N)
    assert list(e[0, 0]) == [1, 1, 2, 3, 4, 5, 6, 7] and list(e[1, 0]) == [4, 4, 4, 4, 4, 5, 6, 7]
    s, e = mk.mask_intervals(mk.Documents([[8], [1, 7]]), 2, N)
    assert list(s[0, 0]) == [0] * 8 and list(s[1, 0]) == [0, 1, 1, 1, 1, 1, 1, 1]


@pytest.mark.parametrize("key", ["C2", "C4", "C5", "S1"])
def test_agrees_with_the_workload_generators(key):
    cfg = inputs.CONFIGS[key]
    spec = inputs.config_intervals(cfg)
    if cfg.mask.startswith("doc"):
        m = mk.Documents(spec.doc_lengths)
    elif cfg.mask == "prefix_lm":
        m = mk.PrefixLM(spec.prefix)
    else:
        m = mk.SinksWindow(cfg.param("window"), cfg.param("sinks"))
    s, e = mk.mask_intervals(m, cfg.B, cfg.N)
    ref_s = spec.col_start if spec.col_start.ndim == 3 else spec.col_start[:, None]
    ref_e = spec.col_end if spec.col_end.ndim == 3 else spec.col_end[:, None]
    assert np.array_equal(s, ref_s) and np.array_equal(e, ref_e)


def test_layers_mix_shared_and_per_head_masks():
    layers = [mk.SlidingWindow(3), [mk.Causal(), mk.Full()], mk.Ranges(np.array(HAND["docs35"][1]),
                                                                      np.array(HAND["docs35"][2]))]
    out = mk.layer_intervals(layers, 1, N, H=2)
    assert out[0][0].shape == (1, 1, N) and out[1][0].shape == (1, 2, 1, N) and out[2][0].shape == (1, 1, N)
    assert np.array_equal(out[2][0][0], np.array(HAND["docs35"][1]))
    with pytest.raises(ValueError):
        mk.layer_intervals([[mk.Causal()]], 1, N, H=2)


@pytest.mark.parametrize("bad", [mk.SlidingWindow(0), mk.PrefixLM(9), mk.Documents([3, 4]), mk.SinksWindow(2, -1),
                                 mk.PrefixLM([1, 2, 3])])
def test_rejects_bad_specifications(bad):
    with pytest.raises(ValueError):
        mk.mask_intervals(bad, 2, N)
