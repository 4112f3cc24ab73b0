"""The C-ABI library loads, exports every entry point the header declares, and
rejects bad arguments on the host before touching the GPU (CPU-only)."""
import ctypes
import os
import re
import subprocess

import pytest

from masked_attention_fm_amd import flashmask as fmb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flashmask.h")

# Pointers that are never dereferenced: every call below fails its host-side
# checks first.  They are 16-byte aligned unless a test says otherwise.
FAKE = 0x10000


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(fmb.LIB_PATH):
        from masked_attention_fm_amd import build
        build.build()
    return fmb.lib()


def header_functions():
    text = open(HEADER, encoding="utf-8").read()
    return re.findall(r"FM_API\s+[\w\s\*]+?\b(fm_\w+)\s*\(", text)


def test_header_lists_the_entry_points():
    names = header_functions()
    assert {"fm_classify_tiles", "fm_attn_fwd", "fm_attn_tile_shape"} <= set(names)
    assert set(names) == set(fmb.SIGNATURES)


def test_library_exports_every_declared_symbol(L):
    out = subprocess.run(["nm", "-D", "--defined-only", fmb.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in header_functions():
        assert name in exported, name
        assert getattr(L, name) is not None
    # nothing else with the fm_ prefix leaks out
    assert {n for n in exported if n.startswith("fm_")} == set(header_functions())


def attn(L, **kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, cs=FAKE, ce=FAKE, B=1, H=1, N=128, d=128, scale=0.125,
                out=FAKE, lse=FAKE)
    args.update(kw)
    return L.fm_attn_fwd(args["q"], args["k"], args["v"], args["cs"], args["ce"], args["B"], args["H"],
                         args["N"], args["d"], args["scale"], args["out"], args["lse"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), fmb.FM_ERR_INVALID_ARG),
    (dict(v=None), fmb.FM_ERR_INVALID_ARG),
    (dict(cs=None), fmb.FM_ERR_INVALID_ARG),
    (dict(lse=None), fmb.FM_ERR_INVALID_ARG),
    (dict(B=0), fmb.FM_ERR_INVALID_ARG),
    (dict(H=-1), fmb.FM_ERR_INVALID_ARG),
    (dict(N=0), fmb.FM_ERR_INVALID_ARG),
    (dict(N=(1 << 22) + 1), fmb.FM_ERR_INVALID_ARG),
    (dict(d=96), fmb.FM_ERR_UNSUPPORTED),
    (dict(d=256), fmb.FM_ERR_UNSUPPORTED),
    (dict(scale=0.0), fmb.FM_ERR_INVALID_ARG),
    (dict(scale=-0.1), fmb.FM_ERR_INVALID_ARG),
    (dict(scale=float("inf")), fmb.FM_ERR_INVALID_ARG),
    (dict(scale=float("nan")), fmb.FM_ERR_INVALID_ARG),
    (dict(q=FAKE + 8), fmb.FM_ERR_INVALID_ARG),
    (dict(out=FAKE + 2), fmb.FM_ERR_INVALID_ARG),
    (dict(lse=FAKE + 2), fmb.FM_ERR_INVALID_ARG),
    (dict(B=1 << 20, H=1 << 10, N=1 << 14), fmb.FM_ERR_INVALID_ARG),
])
def test_attn_fwd_rejects_bad_arguments(L, kw, status):
    assert attn(L, **kw) == status


@pytest.mark.parametrize("args,status", [
    ((None, FAKE, 100, 16, 16, FAKE), fmb.FM_ERR_INVALID_ARG),
    ((FAKE, FAKE, 100, 16, 16, None), fmb.FM_ERR_INVALID_ARG),
    ((FAKE, FAKE, 0, 16, 16, FAKE), fmb.FM_ERR_INVALID_ARG),
    ((FAKE, FAKE, 100, 0, 16, FAKE), fmb.FM_ERR_INVALID_ARG),
    ((FAKE, FAKE, 100, 16, -3, FAKE), fmb.FM_ERR_INVALID_ARG),
    ((FAKE + 2, FAKE, 100, 16, 16, FAKE), fmb.FM_ERR_INVALID_ARG),
])
def test_classify_rejects_bad_arguments(L, args, status):
    assert L.fm_classify_tiles(*args) == status


def test_schedule_rejects_bad_arguments(L):
    assert L.fm_tile_schedule(FAKE, FAKE, 1, 100, 96, FAKE, FAKE) == fmb.FM_ERR_UNSUPPORTED
    assert L.fm_tile_schedule(None, FAKE, 1, 100, 128, FAKE, FAKE) == fmb.FM_ERR_INVALID_ARG
    assert L.fm_tile_schedule(FAKE, FAKE, 0, 100, 128, FAKE, FAKE) == fmb.FM_ERR_INVALID_ARG


def test_tile_shape(L):
    for d in (64, 128):
        br, bc = fmb.fm_attn_tile_shape(d)
        assert br > 0 and bc > 0 and br % 32 == 0 and bc % 32 == 0
    with pytest.raises(fmb.FlashMaskError) as ei:
        fmb.fm_attn_tile_shape(80)
    assert ei.value.status == fmb.FM_ERR_UNSUPPORTED
    assert L.fm_attn_tile_shape(128, None, None) == fmb.FM_ERR_INVALID_ARG


def test_options_and_strings(L):
    assert L.fm_set_option(fmb.FM_OPT_SCHEDULE, 7) == fmb.FM_ERR_INVALID_ARG
    assert L.fm_set_option(999, 0) == fmb.FM_ERR_INVALID_ARG
    assert L.fm_set_option(fmb.FM_OPT_SCHEDULE, 0) == fmb.FM_OK
    assert L.fm_set_option(fmb.FM_OPT_BWD_SPLIT_CHUNKS, -1) == fmb.FM_ERR_INVALID_ARG
    assert L.fm_set_option(fmb.FM_OPT_BWD_SPLIT_CHUNKS, 32) == fmb.FM_OK
    assert L.fm_set_option(fmb.FM_OPT_SINGLE_LAUNCH, 2) == fmb.FM_ERR_INVALID_ARG
    assert L.fm_set_option(fmb.FM_OPT_SINGLE_LAUNCH, 1) == fmb.FM_OK
    assert L.fm_set_option(fmb.FM_OPT_SPLIT_KEYS, 2) == fmb.FM_ERR_INVALID_ARG
    assert L.fm_set_option(fmb.FM_OPT_SPLIT_KEYS, 1) == fmb.FM_OK
    assert L.fm_set_option(fmb.FM_OPT_ROW_SLICES, -1) == fmb.FM_ERR_INVALID_ARG
    assert L.fm_set_option(fmb.FM_OPT_ROW_SLICES, (1 << 20) + 1) == fmb.FM_ERR_INVALID_ARG
    assert L.fm_set_option(fmb.FM_OPT_ROW_SLICES, 512) == fmb.FM_OK
    assert L.fm_set_option(fmb.FM_OPT_BWD_FUSED_PREP, 2) == fmb.FM_ERR_INVALID_ARG
    assert L.fm_set_option(fmb.FM_OPT_BWD_FUSED_PREP, 1) == fmb.FM_OK
    for s in range(5):
        assert L.fm_status_string(s)
    assert b"unknown" in L.fm_status_string(42)
    assert L.fm_last_hip_error() == 0
    # nothing recorded: reading the kernel timer touches no GPU
    assert fmb.fm_profile_read() == (0.0, 0)


def test_binding_refuses_cpu_tensors(L):
    import torch
    x = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    s = torch.zeros(1, 8, dtype=torch.int32)
    with pytest.raises(ValueError):
        fmb.fm_attn_fwd(x, x, x, s, s)


def attn_multi(L, n_ranges, **kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, cs=FAKE, ce=FAKE, B=1, H=1, N=128, d=128, scale=0.125,
                out=FAKE, lse=FAKE)
    args.update(kw)
    return L.fm_attn_fwd_multi(args["q"], args["k"], args["v"], args["cs"], args["ce"], n_ranges, args["B"],
                               args["H"], args["N"], args["d"], args["scale"], args["out"], args["lse"],
                               None)


@pytest.mark.parametrize("n_ranges,kw,status", [
    (0, {}, fmb.FM_ERR_INVALID_ARG),
    (-1, {}, fmb.FM_ERR_INVALID_ARG),
    (fmb.FM_MAX_RANGES + 1, {}, fmb.FM_ERR_INVALID_ARG),
    (2, dict(q=None), fmb.FM_ERR_INVALID_ARG),
    (2, dict(ce=FAKE + 2), fmb.FM_ERR_INVALID_ARG),
    (2, dict(d=80), fmb.FM_ERR_UNSUPPORTED),
    (3, dict(scale=float("nan")), fmb.FM_ERR_INVALID_ARG),
    (4, dict(N=(1 << 22) + 1), fmb.FM_ERR_INVALID_ARG),
])
def test_attn_fwd_multi_rejects_bad_arguments(L, n_ranges, kw, status):
    assert attn_multi(L, n_ranges, **kw) == status


def test_classify_and_schedule_multi_reject_bad_arguments(L):
    assert L.fm_classify_tiles_multi(FAKE, FAKE, 0, 100, 16, 16, FAKE) == fmb.FM_ERR_INVALID_ARG
    assert L.fm_classify_tiles_multi(FAKE, FAKE, 5, 100, 16, 16, FAKE) == fmb.FM_ERR_INVALID_ARG
    assert L.fm_classify_tiles_multi(FAKE, FAKE, 2, 100, 0, 16, FAKE) == fmb.FM_ERR_INVALID_ARG
    assert L.fm_classify_tiles_multi(FAKE, None, 2, 100, 16, 16, FAKE) == fmb.FM_ERR_INVALID_ARG
    assert L.fm_tile_schedule_multi(FAKE, FAKE, 0, 1, 100, 128, FAKE, FAKE) == fmb.FM_ERR_INVALID_ARG
    assert L.fm_tile_schedule_multi(FAKE, FAKE, 2, 1, 100, 96, FAKE, FAKE) == fmb.FM_ERR_UNSUPPORTED


def test_header_range_limit_matches_binding():
    text = open(HEADER, encoding="utf-8").read()
    assert re.search(r"#define FM_MAX_RANGES (\d+)", text).group(1) == str(fmb.FM_MAX_RANGES)


def test_binding_multi_checks_shapes(L):
    import torch
    x = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    s = torch.zeros(1, 8, dtype=torch.int32)
    with pytest.raises(ValueError):
        fmb.fm_attn_fwd_multi(x, x, x, s, s)


def bwd(L, n_ranges=None, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, do=FAKE, lse=FAKE, cs=FAKE, ce=FAKE, B=1, H=1, N=128, d=128,
             scale=0.125, dq=FAKE, dk=FAKE, dv=FAKE)
    a.update(kw)
    head = [a["q"], a["k"], a["v"], a["out"], a["do"], a["lse"], a["cs"], a["ce"]]
    tail = [a["B"], a["H"], a["N"], a["d"], a["scale"], a["dq"], a["dk"], a["dv"], None]
    if n_ranges is None:
        return L.fm_attn_bwd(*head, *tail)
    return L.fm_attn_bwd_multi(*head, n_ranges, *tail)


@pytest.mark.parametrize("n_ranges", [None, 2])
@pytest.mark.parametrize("kw,status", [
    (dict(q=None), fmb.FM_ERR_INVALID_ARG),
    (dict(out=None), fmb.FM_ERR_INVALID_ARG),
    (dict(do=None), fmb.FM_ERR_INVALID_ARG),
    (dict(lse=None), fmb.FM_ERR_INVALID_ARG),
    (dict(dk=None), fmb.FM_ERR_INVALID_ARG),
    (dict(dv=FAKE + 4), fmb.FM_ERR_INVALID_ARG),
    (dict(do=FAKE + 2), fmb.FM_ERR_INVALID_ARG),
    (dict(N=0), fmb.FM_ERR_INVALID_ARG),
    (dict(N=(1 << 22) + 1), fmb.FM_ERR_INVALID_ARG),
    (dict(d=32), fmb.FM_ERR_UNSUPPORTED),
    (dict(scale=0.0), fmb.FM_ERR_INVALID_ARG),
    (dict(scale=float("inf")), fmb.FM_ERR_INVALID_ARG),
])
def test_attn_bwd_rejects_bad_arguments(L, n_ranges, kw, status):
    assert bwd(L, n_ranges, **kw) == status


def test_attn_bwd_multi_rejects_bad_range_count(L):
    assert bwd(L, 0) == fmb.FM_ERR_INVALID_ARG
    assert bwd(L, fmb.FM_MAX_RANGES + 1) == fmb.FM_ERR_INVALID_ARG


@pytest.mark.parametrize("scales,status", [
    ((0.0, 1.0, 1.0), fmb.FM_ERR_INVALID_ARG),
    ((1.0, -1.0, 1.0), fmb.FM_ERR_INVALID_ARG),
    ((1.0, 1.0, float("nan")), fmb.FM_ERR_INVALID_ARG),
    ((1.0, float("inf"), 1.0), fmb.FM_ERR_INVALID_ARG),
])
@pytest.mark.parametrize("mode", [fmb.FM_FP8_SCORES, fmb.FM_FP8_ALL])
def test_attn_fwd_fp8_rejects_bad_scales(L, scales, status, mode):
    assert L.fm_attn_fwd_fp8(FAKE, FAKE, FAKE, *scales, mode, FAKE, FAKE, 1, 1, 1, 128, 128, 0.125, FAKE, FAKE,
                             None) == status


@pytest.mark.parametrize("mode", [fmb.FM_FP8_SCORES, fmb.FM_FP8_ALL])
def test_attn_fwd_fp8_rejects_bad_arguments(L, mode):
    ok = (1.0, 1.0, 1.0, mode)
    assert L.fm_attn_fwd_fp8(None, FAKE, FAKE, *ok, FAKE, FAKE, 1, 1, 1, 128, 128, 0.125, FAKE, FAKE,
                             None) == fmb.FM_ERR_INVALID_ARG
    assert L.fm_attn_fwd_fp8(FAKE, FAKE, FAKE, *ok, FAKE, FAKE, 0, 1, 1, 128, 128, 0.125, FAKE, FAKE,
                             None) == fmb.FM_ERR_INVALID_ARG
    assert L.fm_attn_fwd_fp8(FAKE, FAKE, FAKE, *ok, FAKE, FAKE, 1, 1, 1, 128, 96, 0.125, FAKE, FAKE,
                             None) == fmb.FM_ERR_UNSUPPORTED
    assert L.fm_attn_fwd_fp8(FAKE + 8, FAKE, FAKE, *ok, FAKE, FAKE, 1, 1, 1, 128, 128, 0.125, FAKE, FAKE,
                             None) == fmb.FM_ERR_INVALID_ARG


def test_attn_fwd_fp8_rejects_bad_mode(L):
    for mode in (-1, 2):
        assert L.fm_attn_fwd_fp8(FAKE, FAKE, FAKE, 1.0, 1.0, 1.0, mode, FAKE, FAKE, 1, 1, 1, 128, 128, 0.125,
                                 FAKE, FAKE, None) == fmb.FM_ERR_INVALID_ARG


def test_header_options_match_binding():
    text = open(HEADER, encoding="utf-8").read()
    assert re.search(r"FM_OPT_SCHEDULE = (\d+)", text).group(1) == str(fmb.FM_OPT_SCHEDULE)
    assert re.search(r"FM_OPT_BWD_SPLIT_CHUNKS = (\d+)", text).group(1) == str(fmb.FM_OPT_BWD_SPLIT_CHUNKS)
    assert re.search(r"FM_OPT_SINGLE_LAUNCH = (\d+)", text).group(1) == str(fmb.FM_OPT_SINGLE_LAUNCH)


def test_header_fp8_modes_match_binding():
    text = open(HEADER, encoding="utf-8").read()
    assert re.search(r"#define FM_FP8_SCORES (\d+)", text).group(1) == str(fmb.FM_FP8_SCORES)
    assert re.search(r"#define FM_FP8_ALL (\d+)", text).group(1) == str(fmb.FM_FP8_ALL)


def test_attn_fwd_per_head_rejects_bad_arguments(L):
    args = [FAKE, FAKE, FAKE, FAKE, FAKE]
    assert L.fm_attn_fwd_per_head(*args, 0, 1, 2, 128, 128, 0.125, FAKE, FAKE, None) == fmb.FM_ERR_INVALID_ARG
    assert L.fm_attn_fwd_per_head(*args, 1, 1, 2, 128, 96, 0.125, FAKE, FAKE, None) == fmb.FM_ERR_UNSUPPORTED
    assert L.fm_attn_fwd_per_head(None, FAKE, FAKE, FAKE, FAKE, 1, 1, 2, 128, 128, 0.125, FAKE, FAKE,
                                  None) == fmb.FM_ERR_INVALID_ARG


def test_attn_bwd_per_head_rejects_bad_arguments(L):
    head = [FAKE] * 8
    tail = [1, 2, 128, 128, 0.125, FAKE, FAKE, FAKE, None]
    assert L.fm_attn_bwd_per_head(*head, 0, *tail) == fmb.FM_ERR_INVALID_ARG
    assert L.fm_attn_bwd_per_head(None, *head[1:], 1, *tail) == fmb.FM_ERR_INVALID_ARG
    bad_d = [1, 2, 128, 80, 0.125, FAKE, FAKE, FAKE, None]
    assert L.fm_attn_bwd_per_head(*head, 1, *bad_d) == fmb.FM_ERR_UNSUPPORTED


def noalloc(L, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, cs=FAKE, ce=FAKE, K=1, B=1, H=1, N=128, d=128, scale=0.125,
             out=FAKE, lse=FAKE)
    a.update(kw)
    return L.fm_attn_fwd_noalloc(a["q"], a["k"], a["v"], a["cs"], a["ce"], a["K"], a["B"], a["H"], a["N"],
                                 a["d"], a["scale"], a["out"], a["lse"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), fmb.FM_ERR_INVALID_ARG),
    (dict(K=0), fmb.FM_ERR_INVALID_ARG),
    (dict(K=5), fmb.FM_ERR_INVALID_ARG),
    (dict(d=96), fmb.FM_ERR_UNSUPPORTED),
    (dict(scale=0.0), fmb.FM_ERR_INVALID_ARG),
    (dict(out=FAKE + 8), fmb.FM_ERR_INVALID_ARG),
    # 64 x 2^22 rows: 2^21 query blocks, far beyond the 4 MiB scratch
    (dict(B=64, N=1 << 22), fmb.FM_ERR_TOO_LARGE),
    # 180,224 query blocks of one range (about 4.3 MB of records): just too large
    (dict(B=44, N=1 << 19), fmb.FM_ERR_TOO_LARGE),
    # four ranges per row: 65,536 query blocks need 6.3 MB
    (dict(B=2, N=1 << 22, K=4), fmb.FM_ERR_TOO_LARGE),
])
def test_noalloc_rejects_on_the_host(L, kw, status):
    """Every rejection happens before any HIP call (the pointers are never touched)."""
    assert noalloc(L, **kw) == status


def test_noalloc_limit_matches_the_workspace_plan():
    """The largest single-range problems that fit: 4 MiB holds 16 B of records plus two
    4-byte entries per query block (each part rounded to 256 B), plus the sort scratch
    above 16,384 query blocks in one segment."""
    per_block = 16 + 4 + 4
    assert (4 << 20) // per_block > 170_000
    assert fmb.FM_NOALLOC_SCRATCH_BYTES == 4 << 20
