"""Every-row parity at full size: the float64 oracle on every row of every head of
a workload, compared element by element with the HIP path's output.

The oracle runs in a pool of threads inside the test process.  numpy's BLAS
calls and its large element-wise operations release the GIL, so the threads run
in parallel; BLAS itself is held to one thread per call so the pool does not
oversubscribe the cores.  No worker process is started: the test process holds
the GPU, and a process that has initialised the GPU is not forked.

With FM_PARITY_RECORD set to a file path, each comparison appends its worst
errors to that file as one JSON line.

Each job is one (b, h) head, or a range of its rows when a workload has fewer
heads than the pool has threads.  The query, key and value slices of a head are
regenerated from the workload seed inside the job (the same seeded draws the
GPU inputs came from), so no job holds more than one head's inputs.
"""
from __future__ import annotations

import json
import os
import time
from concurrent.futures import ThreadPoolExecutor
from typing import Callable, Dict, List, Tuple

import numpy as np
import torch
from threadpoolctl import threadpool_limits

import oracle
from masked_attention_fm_amd import inputs


def pool_threads() -> int:
    """Oracle threads: the host cores this process may run on, at most 16 (one GPU's
    share of a shared host)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def jobs_for(cfg, threads: int) -> List[Tuple[int, int, int, int]]:
    """(b, h, first row, end row) jobs: whole heads, or equal row ranges (multiples of
    128 rows) when there are fewer heads than twice the threads."""
    heads = cfg.B * cfg.H
    per_head = max(1, -(-2 * threads // heads))
    rows = -(-cfg.N // per_head)
    rows = -(-rows // 128) * 128
    return [(b, h, r0, min(r0 + rows, cfg.N))
            for b in range(cfg.B) for h in range(cfg.H) for r0 in range(0, cfg.N, rows)]


def _compare_rows(O_gpu, L_gpu, O_ref, L_ref, r0) -> Dict:
    """Element-by-element comparison of one job's rows; returns its worst errors and the
    absolute rows where they occur, plus the list of structural failures."""
    bad = []
    if not np.isfinite(O_gpu).all():
        bad.append("non-finite O")
    empty = np.isneginf(L_ref)
    if not np.array_equal(np.isneginf(L_gpu), empty):
        bad.append("-inf LSE pattern differs")
    if not np.all(O_gpu[empty] == 0.0):
        bad.append("a row that attends nothing has O != 0")
    dO_row = np.abs(O_gpu - O_ref).max(axis=1) if O_ref.size else np.zeros(0)
    dL_row = np.abs(np.where(empty, 0.0, L_gpu) - np.where(empty, 0.0, L_ref))
    iO = int(np.argmax(dO_row)) if dO_row.size else 0
    iL = int(np.argmax(dL_row)) if dL_row.size else 0
    return {"dO": float(dO_row[iO]) if dO_row.size else 0.0, "dO_row": r0 + iO,
            "dL": float(dL_row[iL]) if dL_row.size else 0.0, "dL_row": r0 + iL, "bad": bad,
            "rows": int(O_ref.shape[0])}


def compare_every_row(cfg, spec, out: torch.Tensor, lse: torch.Tensor, scale: float,
                      o_tol: float, lse_tol: float, log: Callable[[str], None]) -> Dict:
    """Compare out (bf16 [B, H, N, d]) and lse (fp32 [B, H, N]) with the oracle on every
    row of every head.  Intervals are spec's ([B, N] or [B, K, N]).  Returns the worst
    errors with where they occur; raises AssertionError naming every failing (b, h)."""
    out_c = out.cpu()
    lse_c = lse.cpu()
    threads = pool_threads()
    jobs = jobs_for(cfg, threads)

    def run(job):
        b, h, r0, r1 = job
        sl = [inputs.qkv_slice(cfg.seed, n, b, h, cfg.N, cfg.d).float().numpy()[None, None] for n in "qkv"]
        rows = np.arange(r0, r1)
        O_ref, L_ref = oracle.attention(*sl, spec.col_start[b:b + 1], spec.col_end[b:b + 1], scale, rows=rows)
        O_gpu = out_c[b, h, r0:r1].double().numpy()
        L_gpu = lse_c[b, h, r0:r1].double().numpy()
        res = _compare_rows(O_gpu, L_gpu, O_ref[0, 0], L_ref[0, 0], r0)
        res["job"] = job
        return res

    t0 = time.time()
    log(f"{cfg.key}: oracle on every row of {cfg.B * cfg.H} heads, {len(jobs)} jobs on {threads} threads")
    with threadpool_limits(1):
        with ThreadPoolExecutor(threads) as ex:
            results = list(ex.map(run, jobs))
    worst_O = max(results, key=lambda r: r["dO"])
    worst_L = max(results, key=lambda r: r["dL"])
    summary = {
        "rows_compared": sum(r["rows"] for r in results),
        "max_dO": worst_O["dO"], "max_dO_at": (worst_O["job"][0], worst_O["job"][1], worst_O["dO_row"]),
        "max_dLSE": worst_L["dL"], "max_dLSE_at": (worst_L["job"][0], worst_L["job"][1], worst_L["dL_row"]),
        "oracle_seconds": round(time.time() - t0, 1),
    }
    log(f"{cfg.key}: every row ({summary['rows_compared']} rows x {cfg.d}): worst max|dO|={summary['max_dO']:.3e} "
        f"at (b, h, row) {summary['max_dO_at']}, worst max|dLSE|={summary['max_dLSE']:.3e} at "
        f"{summary['max_dLSE_at']} ({summary['oracle_seconds']} s)")
    record = os.environ.get("FM_PARITY_RECORD")
    if record:                                   # optional JSON-lines record of the worst errors
        with open(record, "a") as f:
            f.write(json.dumps({"workload": cfg.key, **summary}) + "\n")
    failures = []
    for r in results:
        b, h = r["job"][:2]
        for what in r["bad"]:
            failures.append(f"(b={b}, h={h}, rows {r['job'][2]}..{r['job'][3] - 1}): {what}")
        if r["dO"] > o_tol:
            failures.append(f"(b={b}, h={h}, row {r['dO_row']}): max|dO| {r['dO']:.4e} > {o_tol}")
        if r["dL"] > lse_tol:
            failures.append(f"(b={b}, h={h}, row {r['dL_row']}): max|dLSE| {r['dL']:.4e} > {lse_tol}")
    assert not failures, f"{cfg.key}: " + "; ".join(failures[:20])
    return summary
