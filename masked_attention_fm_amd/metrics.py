"""Work accounting for the masked attention forward pass (host side).

The throughput metric counts 4*d floating-point operations per attended
(query, key) pair: 2*d for the score dot product and 2*d for the weighted
sum of values.  Masked pairs are not counted, so skipped work earns nothing.
"""
from __future__ import annotations

import numpy as np

# AMD's published dense (no sparsity) bf16 matrix peak of the MI355X, TFLOP/s.
MI355X_BF16_DENSE_TFLOPS = 2500.0
MI355X_HBM_TBPS = 8.0


def attended_pairs(col_start: np.ndarray, col_end: np.ndarray, N: int) -> int:
    """Number of attended (row, key) pairs over [B, N] intervals (keys limited to [0, N))."""
    s = np.maximum(np.asarray(col_start, np.int64), 0)
    e = np.minimum(np.asarray(col_end, np.int64), N - 1)
    return int(np.maximum(e - s + 1, 0).sum())


def attended_pairs_union(col_start: np.ndarray, col_end: np.ndarray, N: int) -> int:
    """Attended (row, key) pairs for rows with K ranges, arrays [..., K, N]: a key
    inside several ranges of a row counts once.  The ranges of each row are
    taken in increasing start order and each adds the keys past the furthest
    end seen so far."""
    s = np.maximum(np.asarray(col_start, np.int64), 0)
    e = np.minimum(np.asarray(col_end, np.int64), N - 1)
    empty = s > e
    s = np.where(empty, N, s)                       # empty ranges sort last and add nothing
    e = np.where(empty, -1, e)
    order = np.argsort(s, axis=-2, kind="stable")
    s = np.take_along_axis(s, order, axis=-2)
    e = np.take_along_axis(e, order, axis=-2)
    reach = np.full(s.shape[:-2] + s.shape[-1:], -1, np.int64)
    total = 0
    for k in range(s.shape[-2]):
        sk, ek = s[..., k, :], e[..., k, :]
        total += int(np.maximum(ek - np.maximum(sk, reach + 1) + 1, 0).sum())
        reach = np.maximum(reach, ek)
    return total


def spec_attended_pairs(col_start: np.ndarray, col_end: np.ndarray, N: int) -> int:
    """attended_pairs for [B, N] intervals, attended_pairs_union for [B, K, N]."""
    if np.ndim(col_start) == 3:
        return attended_pairs_union(col_start, col_end, N)
    return attended_pairs(col_start, col_end, N)


def effective_flops(col_start: np.ndarray, col_end: np.ndarray, N: int, H: int, d: int) -> int:
    return 4 * d * H * attended_pairs(col_start, col_end, N)


def algorithmic_bytes(B: int, H: int, N: int, d: int, n_ranges: int = 1) -> int:
    """Q, K, V read once, O written once (bf16), LSE written once (fp32), the intervals
    (start and end, int32, n_ranges per row) read once."""
    return 4 * B * H * N * d * 2 + B * H * N * 4 + 2 * B * n_ranges * N * 4
