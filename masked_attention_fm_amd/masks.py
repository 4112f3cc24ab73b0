"""Mask specifications -> interval arrays (host side, numpy).

The FlashMask article states every mask it supports as per-query-row inclusive
key ranges instead of an N x N matrix (§1; the interval vectors of §2.1; the
document-packing intervals of §3.3; several ranges per row, §6.1 item 1, as
attention sinks next to a window need, §5.2 item 4).  It also varies the mask
from layer to layer (§3.4 item 1, a window size per layer; §6.1 item 3, a mask
kind per layer).  This module writes such specifications down as the int32
arrays the C ABI takes:

* mask_intervals(spec, B, N)        -> [B][K][N]     (fm_attn_fwd_multi)
* head_intervals(specs, B, N)       -> [B][H][K][N]  (fm_attn_fwd_per_head,
                                                      fm_attn_bwd_per_head)
* layer_intervals(layers, B, N)     -> one array pair per layer

A row attends the union of its ranges.  Heads with fewer ranges than the
largest count K are padded with empty ranges (start 0, end -1), which attend
nothing, so the union is unchanged.  Nothing here runs attention; the arrays
go to the library as device tensors.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence, Tuple, Union

import numpy as np

Intervals = Tuple[np.ndarray, np.ndarray]


@dataclasses.dataclass(frozen=True)
class Full:
    """Every row attends every key: [0, N-1]."""


@dataclasses.dataclass(frozen=True)
class Causal:
    """Row i attends [0, i] (the article's §2.1 example)."""


@dataclasses.dataclass(frozen=True)
class SlidingWindow:
    """Row i attends the w keys ending at it: [max(0, i - w + 1), i]."""
    w: int


@dataclasses.dataclass(frozen=True)
class PrefixLM:
    """Rows i < p attend the whole prefix [0, p-1], later rows [0, i].  p is one length for
    every batch element or one per batch element."""
    p: Union[int, Sequence[int]]


@dataclasses.dataclass(frozen=True)
class Documents:
    """Packed documents, causal inside each and blind across them (§3.3): row i of the
    document starting at offset attends [offset, i].  lengths is one list for every batch
    element or one list per batch element; each list sums to N."""
    lengths: Union[Sequence[int], Sequence[Sequence[int]]]


@dataclasses.dataclass(frozen=True)
class SinksWindow:
    """Two ranges per row (§5.2 item 4): the first `sinks` keys, causally, and a causal
    window of w keys: [0, min(sinks-1, i)] and [max(0, i-w+1), i]."""
    w: int
    sinks: int


@dataclasses.dataclass(frozen=True)
class Ranges:
    """Explicit ranges: col_start, col_end of shape [N], [K, N] or [B, K, N]."""
    col_start: np.ndarray
    col_end: np.ndarray


Spec = Union[Full, Causal, SlidingWindow, PrefixLM, Documents, SinksWindow, Ranges]


def _per_batch(value, B: int, what: str) -> list:
    """One value shared by the batch (a number for p, a flat list for lengths) or a list
    of one value per batch element."""
    shared = np.isscalar(value) if what == "p" else all(np.isscalar(x) for x in value)
    if shared:
        return [value] * B
    if len(value) != B:
        raise ValueError(f"{what}: expected one entry per batch element ({B}), got {len(value)}")
    return list(value)


def mask_intervals(spec: Spec, B: int, N: int) -> Intervals:
    """int32 (col_start, col_end) of shape [B][K][N] for one mask specification."""
    if N < 1 or B < 1:
        raise ValueError("B and N must be >= 1")
    i = np.arange(N, dtype=np.int64)
    if isinstance(spec, Full):
        s, e = np.zeros((1, N), np.int64), np.full((1, N), N - 1, np.int64)
        return _batch(s, e, B)
    if isinstance(spec, Causal):
        return _batch(np.zeros((1, N), np.int64), i[None], B)
    if isinstance(spec, SlidingWindow):
        if spec.w < 1:
            raise ValueError("window must be >= 1")
        return _batch(np.maximum(0, i - spec.w + 1)[None], i[None], B)
    if isinstance(spec, SinksWindow):
        if spec.w < 1 or spec.sinks < 0:
            raise ValueError("window must be >= 1 and sinks >= 0")
        s = np.stack([np.zeros(N, np.int64), np.maximum(0, i - spec.w + 1)])
        e = np.stack([np.minimum(spec.sinks - 1, i), i])
        return _batch(s, e, B)
    if isinstance(spec, PrefixLM):
        ps = _per_batch(spec.p, B, "p")
        s = np.zeros((B, 1, N), np.int64)
        e = np.empty((B, 1, N), np.int64)
        for b, p in enumerate(ps):
            if not 0 <= int(p) <= N:
                raise ValueError("prefix length out of range")
            e[b, 0] = np.where(i < int(p), int(p) - 1, i)
        return s.astype(np.int32), e.astype(np.int32)
    if isinstance(spec, Documents):
        docs = _per_batch(spec.lengths, B, "lengths")
        s = np.empty((B, 1, N), np.int64)
        for b, lens in enumerate(docs):
            lens = [int(x) for x in lens]
            if min(lens) < 1 or sum(lens) != N:
                raise ValueError("document lengths must be >= 1 and sum to N")
            s[b, 0] = np.repeat(np.cumsum([0] + lens[:-1]), lens)
        return s.astype(np.int32), np.broadcast_to(i, (B, 1, N)).astype(np.int32)
    if isinstance(spec, Ranges):
        s = np.asarray(spec.col_start, np.int64)
        e = np.asarray(spec.col_end, np.int64)
        if s.shape != e.shape or s.shape[-1] != N or s.ndim not in (1, 2, 3):
            raise ValueError("explicit ranges must be [N], [K, N] or [B, K, N] with equal shapes")
        if s.ndim == 1:
            s, e = s[None], e[None]
        if s.ndim == 2:
            return _batch(s, e, B)
        if s.shape[0] != B:
            raise ValueError("explicit [B, K, N] ranges: wrong batch size")
        return s.astype(np.int32), e.astype(np.int32)
    raise TypeError(f"unknown mask specification {spec!r}")


def _batch(s: np.ndarray, e: np.ndarray, B: int) -> Intervals:
    """[K, N] ranges shared by the batch -> [B, K, N]."""
    return (np.ascontiguousarray(np.broadcast_to(s, (B,) + s.shape)).astype(np.int32),
            np.ascontiguousarray(np.broadcast_to(e, (B,) + e.shape)).astype(np.int32))


def head_intervals(specs: Sequence[Spec], B: int, N: int, n_ranges: Optional[int] = None) -> Intervals:
    """One specification per head -> int32 [B][H][K][N] arrays, K the largest range count
    (or n_ranges when given); a head with fewer ranges is padded with empty ones."""
    per_head = [mask_intervals(sp, B, N) for sp in specs]
    if not per_head:
        raise ValueError("at least one head")
    K = max(s.shape[1] for s, _ in per_head)
    if n_ranges is not None:
        if n_ranges < K:
            raise ValueError(f"a head needs {K} ranges, more than n_ranges = {n_ranges}")
        K = n_ranges
    H = len(per_head)
    s_out = np.zeros((B, H, K, N), np.int32)
    e_out = np.full((B, H, K, N), -1, np.int32)        # empty padding ranges: [0, -1]
    for h, (s, e) in enumerate(per_head):
        s_out[:, h, :s.shape[1]] = s
        e_out[:, h, :e.shape[1]] = e
    return s_out, e_out


def layer_intervals(layers: Sequence[Union[Spec, Sequence[Spec]]], B: int, N: int,
                    H: Optional[int] = None) -> List[Intervals]:
    """Per-layer masks (§3.4 item 1, §6.1 item 3): each layer is one specification for all
    of its heads ([B][K][N], for fm_attn_fwd_multi) or a list with one per head
    ([B][H][K][N], for the per-head calls; H, when given, must match its length)."""
    out = []
    for layer in layers:
        if isinstance(layer, (list, tuple)):
            if H is not None and len(layer) != H:
                raise ValueError(f"a layer lists {len(layer)} head masks, expected {H}")
            out.append(head_intervals(layer, B, N))
        else:
            out.append(mask_intervals(layer, B, N))
    return out
