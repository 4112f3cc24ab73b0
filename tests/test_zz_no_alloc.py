"""fm_attn_fwd_noalloc (the forward with a static device scratch array, no allocation)
against fm_attn_fwd_multi, which takes its workspace from the library's allocator: the
same kernels run in the same order, so the outputs must be bit-identical.  Two calls in
a row, the second smaller than the first (the array keeps the first call's contents),
then the path whose work order needs the counting sort's scratch, several ranges per
row, and a call between allocating calls on the same stream."""
import numpy as np
import pytest
import torch

import oracle
from masked_attention_fm_amd import flashmask as fm
from masked_attention_fm_amd import inputs

from test_gpu_parity import DEV, LSE_TOL, O_TOL, compare, log, to_dev

pytestmark = pytest.mark.gpu


def nan_outputs(q):
    out = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=q.device)
    return out, lse


def both(q, k, v, s, e, scale):
    """(noalloc out, lse), (allocating out, lse) for the same device inputs."""
    o1, l1 = nan_outputs(q)
    fm.fm_attn_fwd_noalloc(q, k, v, s, e, scale, out=o1, lse=l1)
    o2, l2 = nan_outputs(q)
    ss, ee = (s, e) if s.dim() == 3 else (s.unsqueeze(1).contiguous(), e.unsqueeze(1).contiguous())
    fm.fm_attn_fwd_multi(q, k, v, ss, ee, scale, out=o2, lse=l2)
    torch.cuda.synchronize()
    return (o1, l1), (o2, l2)


def assert_identical(a, b, what):
    (o1, l1), (o2, l2) = a, b
    assert not torch.isnan(o1).any() and not torch.isnan(l1).any(), f"{what}: unwritten output"
    assert torch.equal(o1, o2), f"{what}: O differs from fm_attn_fwd_multi"
    assert torch.equal(l1, l2), f"{what}: LSE differs from fm_attn_fwd_multi"
    log(f"{what}: bit-identical to fm_attn_fwd_multi")


def test_two_calls_second_smaller():
    """First call: 512 query blocks (preprocessor + one-workgroup sort); second call: a
    ragged 3000-row problem of 24 query blocks (one-launch prep) into the same array."""
    B, H, N, d = 1, 8, 1 << 16, 128
    spec = inputs.make_intervals("doc_uniform", B, N, 51, lo=256, hi=4096)
    qkv = to_dev(*inputs.make_qkv(B, H, N, d, seed=51))
    s, e = to_dev(spec.col_start, spec.col_end)
    scale = inputs.default_scale(d)
    log("noalloc call 1: B=1 H=8 N=65536")
    assert_identical(*both(*qkv, s, e, scale), "noalloc call 1")

    B, H, N, d = 2, 3, 3000, 64
    q, k, v = inputs.make_qkv(B, H, N, d, seed=52)
    spec = inputs.make_intervals("doc_uniform", B, N, 52, lo=50, hi=900)
    scale = inputs.default_scale(d)
    log("noalloc call 2: B=2 H=3 N=3000")
    a, b = both(*to_dev(q, k, v), *to_dev(spec.col_start, spec.col_end), scale)
    assert_identical(a, b, "noalloc call 2")
    O_ref, L_ref = oracle.attention(q.float().numpy(), k.float().numpy(), v.float().numpy(), spec.col_start,
                                    spec.col_end, scale)
    compare(a[0].double().cpu().numpy(), a[1].double().cpu().numpy(), O_ref, L_ref, "noalloc call 2 vs oracle")


def test_counting_sort_scratch_path():
    """24,576 query blocks in one segment (B = 3, N = 2^20): the work order is a counting sort
    whose scratch also lives in the static array."""
    B, H, N, d = 3, 1, 1 << 20, 64
    s_, e_ = inputs.sliding_window_intervals(N, 200)
    s = np.ascontiguousarray(np.tile(s_, (B, 1)))
    e = np.ascontiguousarray(np.tile(e_, (B, 1)))
    e[1, ::7] = s[1, ::7] - 1            # some empty rows, so the work varies
    qkv = to_dev(*inputs.make_qkv(B, H, N, d, seed=53))
    log("noalloc counting-sort path: B=3 N=2^20")
    assert_identical(*both(*qkv, *to_dev(s, e), inputs.default_scale(d)), "noalloc counting-sort path")


def test_several_ranges_and_interleaving():
    """Sinks plus a window (two ranges per row), called between allocating calls on one stream."""
    B, H, N, d = 1, 4, 5000, 128
    s, e = inputs.sinks_window_intervals(N, 700, 5)
    s, e = np.ascontiguousarray(s[None]), np.ascontiguousarray(e[None])
    qkv = to_dev(*inputs.make_qkv(B, H, N, d, seed=54))
    sd, ed = to_dev(s, e)
    scale = inputs.default_scale(d)
    log("noalloc two ranges")
    for i in range(2):
        assert_identical(*both(*qkv, sd, ed, scale), f"noalloc two ranges, round {i}")


def test_too_large_queues_nothing():
    B, H, N, d = 44, 1, 1 << 19, 64
    q = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=DEV)
    s = torch.zeros((B, N), dtype=torch.int32, device=DEV)
    out, lse = nan_outputs(q)
    with pytest.raises(fm.FlashMaskError) as ei:
        fm.fm_attn_fwd_noalloc(q, q, q, s, s, 0.125, out=out, lse=lse)
    assert ei.value.status == fm.FM_ERR_TOO_LARGE
    torch.cuda.synchronize()
    assert torch.isnan(lse).all()
