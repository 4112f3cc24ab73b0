"""Tile classes and unmasked-entry counts (oracle; test infrastructure only).

The FlashMask article ("FlashMask技术：大模型训练中的高效注意力掩码优化",
§2.2) decides, for every pair of a query block and a key/value block, one of
three cases: skip the block, compute it as a plain (full) GEMM, or compute it
with the per-row mask applied.  The printed code is garbled (it compares
only one row's start and never looks at the right-hand side), so the reading
used here is the plain one that the section's text and its "about half of
the causal work is skipped" claim support:

* SKIP    when the key block lies entirely left of every row's start or
          entirely right of every row's end:
              khi < min_r col_start[r]   or   klo > max_r col_end[r];
* FULL    when the key block lies inside every row's interval:
              klo >= max_r col_start[r]  and  khi <= min_r col_end[r];
* PARTIAL otherwise,

with klo = j*Bc, khi = min(klo + Bc, N) - 1 and r over the rows
[t*Br, min(t*Br + Br, N) - 1] of query block t.  Encoding (page order):
SKIP = 0, FULL = 1, PARTIAL = 2, table row-major [n_q][n_kv].

``classes_dense`` is a second, independent rule used to guard the first:
count the attended entries of the dense mask inside the tile (0 -> SKIP,
all -> FULL, else PARTIAL).
"""
from __future__ import annotations

import numpy as np

from .attention import dense_mask

SKIP, FULL, PARTIAL = 0, 1, 2


def classes_minmax(col_start, col_end, N: int, Br: int, Bc: int) -> np.ndarray:
    """Min/max rule over one sequence's valid intervals (0 <= s <= e <= N-1)."""
    s = [int(x) for x in col_start]
    e = [int(x) for x in col_end]
    n_q = -(-N // Br)
    n_kv = -(-N // Bc)
    out = np.empty((n_q, n_kv), dtype=np.uint8)
    for t in range(n_q):
        rows = range(t * Br, min(t * Br + Br, N))
        min_s = min(s[r] for r in rows)
        max_s = max(s[r] for r in rows)
        min_e = min(e[r] for r in rows)
        max_e = max(e[r] for r in rows)
        for j in range(n_kv):
            klo = j * Bc
            khi = min(klo + Bc, N) - 1
            if khi < min_s or klo > max_e:
                out[t, j] = SKIP
            elif klo >= max_s and khi <= min_e:
                out[t, j] = FULL
            else:
                out[t, j] = PARTIAL
    return out


def nonskip_counts(col_start, col_end, N: int, Br: int, Bc: int, blocks_per_pass: int = 64) -> np.ndarray:
    """Non-SKIP key blocks of every query block of one sequence (the row sums of the
    min/max rule's table, without building the table): for query block t, the number
    of key blocks j that are not SKIP, i.e. not (khi < min col_start or klo > max
    col_end) over the block's rows.  Valid intervals (0 <= s <= e <= N-1).  The rule
    is evaluated for every key block, a pass of `blocks_per_pass` query blocks at a
    time, so that long sequences (millions of rows) fit in memory."""
    s = np.asarray(col_start, dtype=np.int64)
    e = np.asarray(col_end, dtype=np.int64)
    n_q = -(-N // Br)
    n_kv = -(-N // Bc)
    klo = np.arange(n_kv, dtype=np.int64) * Bc
    khi = np.minimum(klo + Bc, N) - 1
    out = np.empty(n_q, dtype=np.int64)
    for t0 in range(0, n_q, blocks_per_pass):
        t1 = min(t0 + blocks_per_pass, n_q)
        min_s = np.array([s[t * Br:min(t * Br + Br, N)].min() for t in range(t0, t1)])
        max_e = np.array([e[t * Br:min(t * Br + Br, N)].max() for t in range(t0, t1)])
        skip = (khi[None, :] < min_s[:, None]) | (klo[None, :] > max_e[:, None])
        out[t0:t1] = (~skip).sum(axis=1)
    return out


def classes_dense(col_start, col_end, N: int, Br: int, Bc: int) -> np.ndarray:
    """Dense-exact rule: classify each tile by counting its attended entries."""
    n_q = -(-N // Br)
    n_kv = -(-N // Bc)
    out = np.empty((n_q, n_kv), dtype=np.uint8)
    for t in range(n_q):
        rows = np.arange(t * Br, min(t * Br + Br, N))
        M = dense_mask(col_start, col_end, N, rows)
        for j in range(n_kv):
            klo = j * Bc
            khi = min(klo + Bc, N) - 1
            block = M[:, klo:khi + 1]
            count = int(block.sum())
            if count == 0:
                out[t, j] = SKIP
            elif count == block.size:
                out[t, j] = FULL
            else:
                out[t, j] = PARTIAL
    return out


def classes_minmax_multi(col_start, col_end, N: int, Br: int, Bc: int) -> np.ndarray:
    """Rows with K ranges ([K, N] arrays, each range valid 0 <= s <= e <= N-1).

    Reading for the union: a tile is SKIP when every range alone would skip it,
    FULL when some single range covers it for every row of the block (a
    sufficient condition for the union to cover it), PARTIAL otherwise."""
    s_all = np.asarray(col_start)
    e_all = np.asarray(col_end)
    per_k = [classes_minmax(s_all[k], e_all[k], N, Br, Bc) for k in range(s_all.shape[0])]
    out = np.full(per_k[0].shape, SKIP, dtype=np.uint8)
    for tab in per_k:
        out = np.where((out == SKIP) & (tab != SKIP), PARTIAL, out)
    for tab in per_k:
        out = np.where(tab == FULL, FULL, out)
    return out


def unmasked_count(col_start, col_end, N: int) -> int:
    """Number of attended (query, key) pairs of one sequence, counted from the dense mask
    one row block at a time."""
    total = 0
    for r0 in range(0, N, 1024):
        rows = np.arange(r0, min(r0 + 1024, N))
        total += int(dense_mask(col_start, col_end, N, rows).sum())
    return total
