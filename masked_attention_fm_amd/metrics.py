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


def wave_mfma_instructions(col_start: np.ndarray, col_end: np.ndarray, N: int, H: int, d: int,
                           Br: int = 128, Bc: int = 64, rows_per_wave: int = 32) -> int:
    """Matrix instructions the bf16 attention kernel issues in one launch.

    Each wavefront owns rows_per_wave rows of a query block and computes a key block
    of Bc keys unless none of its rows attends it through any range: for range k the
    wavefront's rows (those whose range holds a key of [0, N)) span key blocks
    floor(min start / Bc) .. floor(max end / Bc), and it computes the union of those
    spans over the ranges.  A computed key block costs (d/16)(Bc/32) score and
    (Bc/16)(d/32) output instructions of 32x32x16.  col_start / col_end are [B, N]
    or [B, K, N]; the count covers all H heads."""
    s = np.asarray(col_start, np.int64)
    e = np.asarray(col_end, np.int64)
    if s.ndim == 2:
        s, e = s[:, None], e[:, None]
    B, K, _ = s.shape
    per_block = (d // 16) * (Bc // 32) + (Bc // 16) * (d // 32)
    pad = (-N) % rows_per_wave
    total = 0
    for b in range(B):
        spans = []
        for k in range(K):
            sc = np.maximum(s[b, k], 0)
            ec = np.minimum(e[b, k], N - 1)
            live = sc <= ec
            lo = np.where(live, sc, np.iinfo(np.int64).max)
            hi = np.where(live, ec, -1)
            lo = np.concatenate([lo, np.full(pad, np.iinfo(np.int64).max)]).reshape(-1, rows_per_wave).min(1)
            hi = np.concatenate([hi, np.full(pad, -1)]).reshape(-1, rows_per_wave).max(1)
            any_row = hi >= 0
            spans.append((np.where(any_row, lo // Bc, 0), np.where(any_row, hi // Bc, -1)))
        # size of the union of the K spans [a_k, z_k] of every wavefront
        a = np.stack([sp[0] for sp in spans], 1)
        z = np.stack([sp[1] for sp in spans], 1)
        order = np.argsort(np.where(z >= a, a, np.iinfo(np.int64).max), axis=1, kind="stable")
        a = np.take_along_axis(a, order, 1)
        z = np.take_along_axis(z, order, 1)
        reach = np.full(a.shape[0], -1, np.int64)
        count = np.zeros(a.shape[0], np.int64)
        for k in range(K):
            ak, zk = a[:, k], z[:, k]
            ok = zk >= ak
            count += np.where(ok, np.maximum(zk - np.maximum(ak, reach + 1) + 1, 0), 0)
            reach = np.where(ok, np.maximum(reach, zk), reach)
        total += int(count.sum())
    return total * per_block * H
