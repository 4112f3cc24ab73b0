"""Dense-mask float64 softmax attention (oracle; test infrastructure only).

Definition followed (see the package docstring for the pages):

* mask      M[i, j] = col_start[i] <= j <= col_end[i] for key columns
            j in [0, N)  -- FlashMask article §1 (per-query key range) and
            §4.1 item 3 (both ends of the compare inclusive).  With several
            ranges per row (§6.1 item 1, several disjoint column ranges; §5.2
            item 4, attention sinks plus a window) M is their union;
* scores    S[i, j] = scale * (q_i . k_j), and -inf where M[i, j] is false
            -- FlashMask article §4.1 item 3 (mask added to the score);
* softmax   p[i, j] = exp(S[i, j] - max_j S[i, j]) / sum_j exp(...)
            -- FlashAttention article §2 item 2 (max-subtracted softmax);
* output    O[i, :] = sum_j p[i, j] v_j,
            LSE[i] = ln sum_{j : M[i,j]} exp(S[i, j]) = m_i + ln l_i;
* a row that attends nothing gives O = 0 and LSE = -inf.

Readings where the pages are silent: the scale is the float32 value the
kernel receives, promoted exactly to float64; LSE uses the natural log and
includes the scale.

Everything is float64 and unrounded; nothing is tiled.  To save time a row
block only multiplies against the key columns that its own dense mask marks
as attended by at least one of its rows; the other columns have weight
exactly 0 and contribute nothing.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np


def dense_mask(col_start: np.ndarray, col_end: np.ndarray, N: int,
               rows: Optional[np.ndarray] = None) -> np.ndarray:
    """Boolean [R, N] mask of one sequence: M[r, j] = s[r] <= j <= e[r].

    col_start / col_end are [N] (one range per row) or [K, N] (K ranges per
    row, united)."""
    s = np.asarray(col_start, dtype=np.int64)
    e = np.asarray(col_end, dtype=np.int64)
    if s.ndim == 1:
        s, e = s[None], e[None]
    if rows is not None:
        s = s[:, rows]
        e = e[:, rows]
    j = np.arange(N, dtype=np.int64)
    M = np.zeros((s.shape[1], N), dtype=bool)
    for k in range(s.shape[0]):
        M |= (j[None, :] >= s[k][:, None]) & (j[None, :] <= e[k][:, None])
    return M


def attention(q, k, v, col_start, col_end, scale: float,
              rows: Optional[np.ndarray] = None,
              row_block: int = 128) -> Tuple[np.ndarray, np.ndarray]:
    """Masked softmax attention of every (b, h) for the chosen query rows.

    q, k, v   : real arrays [B, H, N, d] (bfloat16 values held exactly in
                float32 or float64); slices are promoted to float64.
    col_start, col_end : integer arrays [B, N], shared by all heads, or
                [B, K, N] for K ranges per row (the row attends their union).
    scale     : the float32 scale value.
    rows      : query rows to evaluate (the same for every b); default all.

    Returns (O [B, H, R, d], LSE [B, H, R]) in float64.
    """
    B, H, N, d = q.shape
    scale64 = float(np.float32(scale))
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    R = rows.shape[0]
    O = np.zeros((B, H, R, d), dtype=np.float64)
    LSE = np.full((B, H, R), -np.inf, dtype=np.float64)
    for b in range(B):
        for r0 in range(0, R, row_block):
            rr = rows[r0:r0 + row_block]
            M = dense_mask(col_start[b], col_end[b], N, rr)
            support = np.flatnonzero(M.any(axis=0))
            if support.size == 0:
                continue                      # every row empty: O = 0, LSE = -inf
            Ms = M[:, support]
            attended = Ms.any(axis=1)         # rows with at least one key
            for h in range(H):
                qh = np.asarray(q[b, h][rr], dtype=np.float64)
                kh = np.asarray(k[b, h][support], dtype=np.float64)
                vh = np.asarray(v[b, h][support], dtype=np.float64)
                S = scale64 * (qh @ kh.T)
                S = np.where(Ms, S, -np.inf)
                m = S.max(axis=1)
                m_safe = np.where(attended, m, 0.0)
                p = np.exp(S - m_safe[:, None])          # exactly 0 where masked
                l = p.sum(axis=1)
                num = p @ vh
                ok = attended
                O[b, h, r0:r0 + len(rr)][ok] = num[ok] / l[ok][:, None]
                LSE[b, h, r0:r0 + len(rr)][ok] = m[ok] + np.log(l[ok])
    return O, LSE


def attention_weights(q, k, col_start, col_end, scale: float,
                      rows: Optional[np.ndarray] = None) -> np.ndarray:
    """Softmax weight matrix P [B, H, R, N] of the chosen query rows (default
    all: R = N; small N, or few rows, only)."""
    B, H, N, d = q.shape
    scale64 = float(np.float32(scale))
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    P = np.zeros((B, H, rows.shape[0], N), dtype=np.float64)
    for b in range(B):
        M = dense_mask(col_start[b], col_end[b], N, rows)
        attended = M.any(axis=1)
        for h in range(H):
            S = scale64 * (np.asarray(q[b, h][rows], np.float64) @ np.asarray(k[b, h], np.float64).T)
            S = np.where(M, S, -np.inf)
            m = np.where(attended, S.max(axis=1), 0.0)
            p = np.exp(S - m[:, None])
            l = p.sum(axis=1)
            P[b, h][attended] = p[attended] / l[attended][:, None]
    return P


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (ties to even), returned as float64.

    Used only to report the representability floor of a bfloat16 output:
    max |bf16(O_ref) - O_ref|.  Implemented on the bit pattern of the float32
    value nearest to x, then rounding its low 16 bits to even.
    """
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    rounded = ((u + 0x7FFF + lsb) >> 16) << 16
    out = rounded.astype(np.uint32).view(np.float32)
    # NaN and inf pass through unchanged.
    out = np.where(np.isfinite(f), out, f)
    return out.astype(np.float64)
