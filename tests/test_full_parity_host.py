"""Host checks of the every-row comparison used by the full-size GPU parity tests: its
jobs cover every row once, it accepts the oracle's own output rounded to bf16, and it
names the (b, h, row) of a planted mistake.  CPU only: the "GPU output" here is made
from the oracle."""
import dataclasses

import numpy as np
import pytest
import torch

import full_parity
import oracle
from masked_attention_fm_amd import inputs


def tiny_cfg():
    return dataclasses.replace(inputs.CONFIGS["C2"], key="T", B=2, H=3, N=700, d=64,
                               params=(("lo", 50), ("hi", 300)))


def oracle_output(cfg, spec, scale):
    q, k, v = inputs.make_qkv(cfg.B, cfg.H, cfg.N, cfg.d, cfg.seed)
    O, L = oracle.attention(q.float().numpy(), k.float().numpy(), v.float().numpy(), spec.col_start,
                            spec.col_end, scale)
    return torch.from_numpy(O).to(torch.bfloat16), torch.from_numpy(L).float()


@pytest.mark.parametrize("threads", [1, 3, 16])
def test_jobs_cover_every_row_once(threads):
    for key in inputs.CONFIGS:
        cfg = inputs.CONFIGS[key]
        seen = {}
        for b, h, r0, r1 in full_parity.jobs_for(cfg, threads):
            assert r0 % 128 == 0 and r0 < r1 <= cfg.N
            seen.setdefault((b, h), []).append((r0, r1))
        assert len(seen) == cfg.B * cfg.H
        for ranges in seen.values():
            ranges.sort()
            assert ranges[0][0] == 0 and ranges[-1][1] == cfg.N
            assert all(a[1] == b[0] for a, b in zip(ranges, ranges[1:]))


def test_accepts_rounded_oracle_and_names_planted_mistakes():
    cfg = tiny_cfg()
    spec = inputs.config_intervals(cfg)
    scale = inputs.default_scale(cfg.d)
    out, lse = oracle_output(cfg, spec, scale)
    log = lambda m: None
    s = full_parity.compare_every_row(cfg, spec, out, lse, scale, 1e-2, 1e-3, log)
    assert s["rows_compared"] == cfg.B * cfg.H * cfg.N and s["max_dO"] <= 2 ** -8 * 8

    bad = out.clone()
    bad[1, 2, 517, 5] += 0.05
    with pytest.raises(AssertionError, match=r"b=1, h=2, row 517"):
        full_parity.compare_every_row(cfg, spec, bad, lse, scale, 1e-2, 1e-3, log)

    bad_l = lse.clone()
    bad_l[0, 1, 33] += 2e-3
    with pytest.raises(AssertionError, match=r"b=0, h=1, row 33"):
        full_parity.compare_every_row(cfg, spec, out, bad_l, scale, 1e-2, 1e-3, log)

    bad_l = lse.clone()
    bad_l[0, 0, 400] = -np.inf
    with pytest.raises(AssertionError, match=r"-inf LSE pattern"):
        full_parity.compare_every_row(cfg, spec, out, bad_l, scale, 1e-2, 1e-3, log)
