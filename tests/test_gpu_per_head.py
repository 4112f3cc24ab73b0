"""GPU parity for one interval set per head (fm_attn_fwd_per_head): each head against
the oracle with that head's own intervals; all-equal sets against the shared-set call."""
import numpy as np
import pytest
import torch

import oracle
from masked_attention_fm_amd import flashmask as fm
from masked_attention_fm_amd import inputs

from test_gpu_bwd import GRAD_TOL, compare_grads, dout_for
from test_gpu_parity import DEV, compare, log, to_dev

pytestmark = pytest.mark.gpu


def run_per_head(q, k, v, s, e, scale):
    qd, kd, vd = to_dev(q, k, v)
    out = torch.full_like(qd, float("nan"))
    lse = torch.full(qd.shape[:3], float("nan"), dtype=torch.float32, device=DEV)
    fm.fm_attn_fwd_per_head(qd, kd, vd, *to_dev(s, e), scale, out=out, lse=lse)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def check_per_head(q, k, v, s, e, scale, what, rows=None):
    """s, e: [B, H, K, N]."""
    O, L = run_per_head(q, k, v, s, e, scale)
    qf, kf, vf = (x.float().numpy() for x in (q, k, v))
    worst = (0.0, 0.0)
    for h in range(q.shape[1]):
        O_ref, L_ref = oracle.attention(qf[:, h:h + 1], kf[:, h:h + 1], vf[:, h:h + 1], s[:, h], e[:, h], scale,
                                        rows=rows)
        Oh, Lh = O[:, h:h + 1], L[:, h:h + 1]
        if rows is not None:
            Oh, Lh = Oh[:, :, rows], Lh[:, :, rows]
        dO, dL = compare(Oh, Lh, O_ref, L_ref, f"{what} h={h}")
        worst = (max(worst[0], dO), max(worst[1], dL))
    return worst


def window_per_head(B, H, N, widths):
    s = np.empty((B, H, 1, N), np.int32)
    e = np.empty((B, H, 1, N), np.int32)
    for h in range(H):
        sh, eh = inputs.sliding_window_intervals(N, widths[h % len(widths)])
        s[:, h, 0], e[:, h, 0] = sh, eh
    return s, e


@pytest.mark.parametrize("B,H,N,d", [(1, 4, 700, 128), (2, 3, 333, 64), (1, 8, 8192, 128)])
def test_per_head_windows(B, H, N, d):
    """A different causal window per head; (1, 8, 8192) takes the preprocessor + ranked-segment
    path (512 query blocks) and the XCD-local head order."""
    s, e = window_per_head(B, H, N, [16, 100, 512, 1, 2048, 64, 300, 8000])
    q, k, v = inputs.make_qkv(B, H, N, d, seed=N + H)
    rows = None if N <= 1000 else np.unique(np.concatenate([np.arange(0, 300), np.arange(N - 300, N),
                                                            np.random.default_rng(5).integers(0, N, 300)]))
    log(f"per-head windows B={B} H={H} N={N} d={d}")
    check_per_head(q, k, v, s, e, inputs.default_scale(d), f"per-head windows {N}", rows=rows)


def test_per_head_mixed_ranges():
    """Per-head random multi-range rows with empty ranges."""
    B, H, N, d, K = 2, 3, 500, 128, 2
    rng = np.random.default_rng(71)
    s = np.empty((B, H, K, N), np.int32)
    e = np.empty((B, H, K, N), np.int32)
    for h in range(H):
        s[:, h], e[:, h] = inputs.random_multi_intervals(rng, B, K, N, empty_frac=0.2, max_width=80 * (h + 1))
    q, k, v = inputs.make_qkv(B, H, N, d, seed=71)
    check_per_head(q, k, v, s, e, inputs.default_scale(d), "per-head mixed")


@pytest.mark.parametrize("H,N", [(4, 2000), (16, 8192)])
def test_per_head_equal_sets_match_shared(H, N):
    """All heads given the same set: bit-identical to the shared-set call (small and large
    prep paths)."""
    B, d = 1, 128
    spec = inputs.make_intervals("doc_uniform", B, N, 9, lo=100, hi=1500)
    q, k, v = to_dev(*inputs.make_qkv(B, H, N, d, seed=9))
    sd, ed = to_dev(spec.col_start, spec.col_end)
    o1, l1 = fm.fm_attn_fwd(q, k, v, sd, ed, inputs.default_scale(d))
    sh = sd[:, None, None].expand(B, H, 1, N).contiguous()
    eh = ed[:, None, None].expand(B, H, 1, N).contiguous()
    o2, l2 = fm.fm_attn_fwd_per_head(q, k, v, sh, eh, inputs.default_scale(d))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("B,H,N,d", [(1, 3, 600, 128), (2, 8, 4096, 64)])
def test_per_head_backward(B, H, N, d):
    """Gradients with a different window per head against the oracle head by head;
    (2, 8, 4096) takes the preprocessor + ranked-segment paths."""
    s, e = window_per_head(B, H, N, [32, 300, 1, 1000, 64, 2048, 7, 4096])
    q, k, v = inputs.make_qkv(B, H, N, d, seed=N + 5)
    do = dout_for(q.shape, N)
    qd, kd, vd, dod = to_dev(q, k, v, do)
    sd, ed = to_dev(s, e)
    out, lse = fm.fm_attn_fwd_per_head(qd, kd, vd, sd, ed, inputs.default_scale(d))
    dq, dk, dv = fm.fm_attn_bwd_per_head(qd, kd, vd, out, dod, lse, sd, ed, inputs.default_scale(d))
    torch.cuda.synchronize()
    got = [g.cpu().numpy().astype(np.float64) for g in (dq, dk, dv)]
    qf, kf, vf, dof = (x.float().numpy() for x in (q, k, v, do))
    log(f"per-head backward B={B} H={H} N={N} d={d}")
    for h in range(H):
        ref = oracle.attention_bwd(qf[:, h:h + 1], kf[:, h:h + 1], vf[:, h:h + 1], dof[:, h:h + 1], s[:, h], e[:, h],
                                   inputs.default_scale(d))
        compare_grads([g[:, h:h + 1] for g in got], ref, f"per-head bwd h={h}")


def test_per_head_backward_equal_sets_match_shared():
    B, H, N, d = 1, 4, 1500, 128
    spec = inputs.make_intervals("doc_uniform", B, N, 11, lo=100, hi=700)
    q, k, v = to_dev(*inputs.make_qkv(B, H, N, d, seed=11))
    do = to_dev(dout_for((B, H, N, d), 11))[0]
    sd, ed = to_dev(spec.col_start, spec.col_end)
    out, lse = fm.fm_attn_fwd(q, k, v, sd, ed, inputs.default_scale(d))
    g1 = fm.fm_attn_bwd(q, k, v, out, do, lse, sd, ed, inputs.default_scale(d))
    sh = sd[:, None, None].expand(B, H, 1, N).contiguous()
    eh = ed[:, None, None].expand(B, H, 1, N).contiguous()
    g2 = fm.fm_attn_bwd_per_head(q, k, v, out, do, lse, sh, eh, inputs.default_scale(d))
    torch.cuda.synchronize()
    for a, b_ in zip(g1, g2):
        assert torch.equal(a, b_)


def test_per_head_segments_longer_than_one_sort_workgroup():
    """Two interval sets (one per head) of 20480 query blocks each (B = 5, N = 2^19): each
    segment of the launch order is longer than one workgroup sorts, so the order comes
    from the counting sort, segment by segment.  Sampled rows of both heads against the
    oracle (the order changes no result)."""
    B, H, N, d = 5, 2, 1 << 19, 64
    s = np.empty((B, H, 1, N), np.int32)
    e = np.empty((B, H, 1, N), np.int32)
    s[:, 0, 0], e[:, 0, 0] = inputs.sliding_window_intervals(N, 64)
    spec = inputs.make_intervals("doc_lognormal", B, N, 41, median=128, sigma=1.0, lo=1, hi=2048)
    s[:, 1, 0], e[:, 1, 0] = spec.col_start, spec.col_end
    assert B * (N // 128) > 16384
    q, k, v = inputs.make_qkv(B, H, N, d, seed=41)
    rng = np.random.default_rng(41)
    rows = np.unique(np.concatenate([[0, 1, 127, 128, N // 2, N - 1], rng.integers(0, N, 60)]))
    log("per-head, two long segments")
    check_per_head(q, k, v, s, e, inputs.default_scale(d), "per-head long segments", rows=rows)


def test_per_head_masks_from_specifications():
    """Heads with different mask kinds built by masks.head_intervals (padded to the sinks
    head's two ranges): causal, a window, sinks + window, packed documents, prefix-LM and
    full attention, each head against the oracle with its own intervals."""
    from masked_attention_fm_amd import masks as mk
    B, N, d = 2, 1500, 128
    specs = [mk.Causal(), mk.SlidingWindow(200), mk.SinksWindow(300, 4), mk.Documents([[700, 800], [1, 1499]]),
             mk.PrefixLM([400, 1100]), mk.Full()]
    s, e = mk.head_intervals(specs, B, N)
    assert s.shape == (B, len(specs), 2, N)
    q, k, v = inputs.make_qkv(B, len(specs), N, d, seed=61)
    log("per-head masks from specifications")
    check_per_head(q, k, v, s, e, inputs.default_scale(d), "per-head specs")
