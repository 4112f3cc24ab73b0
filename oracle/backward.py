"""Gradients of masked softmax attention (oracle; test infrastructure only).

The pages give the method's forward pass only; they place it in training
(FlashMask abstract: fine-tuning and alignment runs), where the gradients of
Q, K and V are needed.  The gradient is fixed by the forward's definition
(see oracle.attention) and the chain rule.  For a loss L with dL/dO = dO:

    P      = softmax over the attended keys of S = scale * Q K^T   (0 elsewhere)
    dV     = P^T dO                       (O = P V)
    dP     = dO V^T
    dS_ij  = P_ij (dP_ij - sum_l P_il dP_il)    (softmax Jacobian, row i)
    dQ     = scale * dS K
    dK     = scale * dS^T Q

A row that attends nothing has P = 0 and contributes nothing.  Everything is
float64 and nothing is tiled; as in the forward oracle, a row block only
multiplies against the key columns its own dense mask marks, since every
other column has P = 0 and so dS = 0.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

from .attention import dense_mask


def attention_bwd(q, k, v, dout, col_start, col_end, scale: float,
                  row_block: int = 128) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """(dQ, dK, dV) float64 [B, H, N, d] for upstream gradient dout [B, H, N, d].

    q, k, v, dout : real arrays [B, H, N, d] (promoted to float64).
    col_start, col_end : [B, N] (one range per row) or [B, K, N] (union of K ranges).
    scale : the float32 scale value.
    """
    B, H, N, d = q.shape
    scale64 = float(np.float32(scale))
    dQ = np.zeros((B, H, N, d), dtype=np.float64)
    dK = np.zeros((B, H, N, d), dtype=np.float64)
    dV = np.zeros((B, H, N, d), dtype=np.float64)
    for b in range(B):
        for r0 in range(0, N, row_block):
            rr = np.arange(r0, min(r0 + row_block, N))
            M = dense_mask(col_start[b], col_end[b], N, rr)
            support = np.flatnonzero(M.any(axis=0))
            if support.size == 0:
                continue
            Ms = M[:, support]
            attended = Ms.any(axis=1)
            for h in range(H):
                qh = np.asarray(q[b, h][rr], dtype=np.float64)
                kh = np.asarray(k[b, h][support], dtype=np.float64)
                vh = np.asarray(v[b, h][support], dtype=np.float64)
                doh = np.asarray(dout[b, h][rr], dtype=np.float64)
                S = scale64 * (qh @ kh.T)
                S = np.where(Ms, S, -np.inf)
                m = np.where(attended, S.max(axis=1), 0.0)
                p = np.exp(S - m[:, None])                  # exactly 0 where masked
                l = p.sum(axis=1)
                P = np.zeros_like(p)
                P[attended] = p[attended] / l[attended][:, None]
                dV[b, h][support] += P.T @ doh
                dP = doh @ vh.T
                Dr = (P * dP).sum(axis=1)
                dS = P * (dP - Dr[:, None])
                dQ[b, h][rr] = scale64 * (dS @ kh)
                dK[b, h][support] += scale64 * (dS.T @ qh)
    return dQ, dK, dV
