"""Host-side logic of the product path that needs no GPU: the FLOP accounting and the
rocprofv3 counter summariser."""
import csv
import os

import numpy as np
import pytest

import oracle
from masked_attention_fm_amd import counters, inputs, metrics


@pytest.mark.parametrize("key", ["C1", "C2", "C3"])
def test_attended_pairs_equals_dense_count(key):
    cfg = inputs.CONFIGS[key]
    spec = inputs.config_intervals(cfg)
    for b in range(cfg.B):
        assert metrics.attended_pairs(spec.col_start[b], spec.col_end[b], cfg.N) == \
            oracle.unmasked_count(spec.col_start[b], spec.col_end[b], cfg.N)


def test_attended_pairs_general_intervals():
    rng = np.random.default_rng(4)
    N = 700
    s = rng.integers(-100, N + 100, size=N)
    e = s + rng.integers(-20, 300, size=N)
    assert metrics.attended_pairs(s, e, N) == oracle.unmasked_count(s, e, N)


@pytest.mark.parametrize("K", [1, 2, 3, 4])
def test_attended_pairs_union_equals_dense_count(K):
    rng = np.random.default_rng(40 + K)
    N = 500
    s, e = inputs.random_multi_intervals(rng, 2, K, N, empty_frac=0.2, max_width=120)
    s[:, 0, :50] -= 80                              # some ranges reach outside [0, N)
    e[:, -1, -50:] += 80
    assert metrics.attended_pairs_union(s, e, N) == sum(oracle.unmasked_count(s[b], e[b], N) for b in range(2))


def test_sinks_window_pairs_closed_form():
    """10 sinks and a window of 1024: rows up to 1033 see [0, i]; later rows 10 + 1024 keys."""
    cfg = inputs.CONFIGS["S1"]
    spec = inputs.config_intervals(cfg)
    n_join = cfg.param("window") + cfg.param("sinks")          # first row whose window leaves the sinks
    expect = n_join * (n_join + 1) // 2 + (cfg.N - n_join) * n_join
    assert metrics.spec_attended_pairs(spec.col_start, spec.col_end, cfg.N) == expect
    assert metrics.spec_attended_pairs(spec.col_start[:, :, :3000], spec.col_end[:, :, :3000], 3000) == \
        oracle.unmasked_count(spec.col_start[0, :, :3000], spec.col_end[0, :, :3000], 3000)


def test_effective_flops_c1_closed_form():
    cfg = inputs.CONFIGS["C1"]
    spec = inputs.config_intervals(cfg)
    # causal: N(N+1)/2 pairs per head, 4*d FLOPs each
    assert metrics.effective_flops(spec.col_start, spec.col_end, cfg.N, cfg.H, cfg.d) == \
        4 * 64 * 2 * (512 * 513 // 2)


def _write_run(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(["Kernel_Name", "Counter_Name", "Counter_Value"], r)))


def test_counter_summary_calibrates_with_the_copy(tmp_path):
    attn = "void fm::(anonymous namespace)::attn_fwd_kernel<128, 1, 0>(...)"
    fp8 = "void fm::(anonymous namespace)::attn_fwd_kernel<128, 1, 1>(...)"   # another kernel: never counted
    copy = "__amd_rocclr_copyBuffer"
    _write_run(tmp_path / "fetch", [(attn, "FETCH_SIZE", 1000.0), (attn, "FETCH_SIZE", 1200.0),
                                    (fp8, "FETCH_SIZE", 9e9), (copy, "FETCH_SIZE", 2.0),
                                    (copy, "FETCH_SIZE", 262144.0)])
    _write_run(tmp_path / "write", [(attn, "WRITE_SIZE", 300.0), (fp8, "WRITE_SIZE", 9e9),
                                    (copy, "WRITE_SIZE", 524288.0)])
    _write_run(tmp_path / "mfma", [(attn, "SQ_VALU_MFMA_BUSY_CYCLES", 400.0), (attn, "SQ_BUSY_CU_CYCLES", 200.0),
                                   (attn, "SQ_LDS_BANK_CONFLICT", 5.0), (attn, "SQ_LDS_IDX_ACTIVE", 50.0),
                                   (attn, "SQ_INSTS_MFMA", 3.0), (fp8, "SQ_INSTS_MFMA", 1e9)])
    rec = counters.summarise([tmp_path / "fetch", tmp_path / "write", tmp_path / "mfma"], copy_mib=512)
    assert rec["calibration"]["FETCH_SIZE"] == pytest.approx(2.0)     # the tiny helper copy is ignored
    assert rec["calibration"]["WRITE_SIZE"] == pytest.approx(1.0)
    assert rec["l2_miss_read_bytes_per_launch"] == pytest.approx(1024 * 1100 * 2.0)
    assert rec["write_bytes_per_launch"] == pytest.approx(1024 * 300)
    assert rec["l2_miss_bytes_per_launch"] == pytest.approx(1024 * (1100 * 2.0 + 300))
    assert rec["mfma_busy_per_cu_busy"] == pytest.approx(0.5)
    assert rec["lds_bank_conflict_per_lds_active"] == pytest.approx(0.1)
    assert rec["mfma_flops_per_launch"] == pytest.approx(3 * 32768)
    assert rec["dispatches"]["attention"]["FETCH_SIZE"] == 2
    assert rec["attn_source_sha256_16"] == counters.attn_source_hash()


def test_counter_kernel_filter():
    assert counters.kind_of("void fm::(anonymous namespace)::attn_fwd_kernel<64, 4, 0>(int)") == "attention"
    # the small-problem launches' instances (one or two wavefront groups) are the same kernel
    for prec in (3, 4):
        assert counters.kind_of(f"void fm::(anonymous namespace)::attn_fwd_kernel<128, 2, {prec}>(int)") == "attention"
    # and so is the 32-row slice kernel of the smallest problems
    assert counters.kind_of("void fm::(anonymous namespace)::attn_fwd_rows_kernel<64, 1>(int)") == "attention"
    for name in ("attn_fwd_kernel<128, 1, 1>", "attn_fwd_kernel<128, 2, 2>", "bwd_dq_kernel<128, 1>",
                 "prep_small_kernel<1>"):
        assert counters.kind_of(name) == ""


def test_counter_kernel_filter_backward(tmp_path):
    """--kernel bwd_dkdv / bwd_dq count only that backward kernel, hashed over the backward's
    launch sources."""
    dkdv = "void fm::(anonymous namespace)::bwd_dkdv_kernel<128, 1>(...)"
    dq = "void fm::(anonymous namespace)::bwd_dq_kernel<128, 1>(...)"
    fwd = "void fm::(anonymous namespace)::attn_fwd_kernel<128, 1, 0>(...)"
    assert counters.kind_of(dkdv, "bwd_dkdv") == "attention"
    assert counters.kind_of(dq, "bwd_dkdv") == ""
    assert counters.kind_of(fwd, "bwd_dkdv") == ""
    assert counters.kind_of(dq, "bwd_dq") == "attention"
    assert counters.kind_of(dkdv, "bwd_dq") == ""
    _write_run(tmp_path / "a", [(dkdv, "SQ_INSTS_MFMA", 10.0), (dq, "SQ_INSTS_MFMA", 99.0),
                                (fwd, "SQ_INSTS_MFMA", 7.0)])
    rec = counters.summarise([tmp_path / "a"], copy_mib=0, kernel="bwd_dkdv")
    assert rec["attention"]["SQ_INSTS_MFMA"] == 10.0 and rec["kernel"] == "bwd_dkdv"
    assert rec["attn_source_sha256_16"] == counters.source_hash("bwd_dkdv") != counters.attn_source_hash()


def test_code_hash_ignores_comments_and_whitespace():
    a = "int f(int x) {  // doubles\n    return 2 * x;\n}\n"
    b = "// f: twice x\nint f(int x) {\n\n  return 2 * x;   // twice\n}\n"
    c = "int f(int x) {\n    return 3 * x;\n}\n"
    assert counters.attn_source_hash([a]) == counters.attn_source_hash([b])
    assert counters.attn_source_hash([a]) != counters.attn_source_hash([c])


def _wave_mfma_brute(s, e, N, H, d, Br=128, Bc=64, R=32):
    """Wavefront by wavefront, key block by key block: computed when some row of the
    wavefront attends some key of the block through any of its ranges."""
    s = np.asarray(s); e = np.asarray(e)
    if s.ndim == 2:
        s, e = s[:, None], e[:, None]
    per_block = (d // 16) * (Bc // 32) + (Bc // 16) * (d // 32)
    n = 0
    for b in range(s.shape[0]):
        for w0 in range(0, N, R):
            rows = range(w0, min(w0 + R, N))
            for j in range(-(-N // Bc)):
                klo, khi = j * Bc, min(j * Bc + Bc, N) - 1
                if any(max(s[b, k, r], 0) <= min(e[b, k, r], N - 1) and max(s[b, k, r], 0) <= khi
                       and min(e[b, k, r], N - 1) >= klo
                       for r in rows for k in range(s.shape[1])):
                    n += per_block
    return n * H


@pytest.mark.parametrize("K,N,d", [(1, 300, 128), (1, 129, 64), (2, 500, 128), (3, 200, 64)])
def test_wave_mfma_count_matches_brute_force(K, N, d):
    """A wavefront computes a key block when one of its rows attends a key in it through
    one range: the count per wavefront is then the union of the ranges' block spans,
    which the vectorised count uses (valid and empty ranges, several per row)."""
    rng = np.random.default_rng(K * N + d)
    s, e = inputs.random_multi_intervals(rng, 2, K, N, empty_frac=0.2, max_width=N // 3)
    if K == 1:
        s, e = s[:, 0], e[:, 0]
    assert metrics.wave_mfma_instructions(s, e, N, 3, d) == _wave_mfma_brute(s, e, N, 3, d)
