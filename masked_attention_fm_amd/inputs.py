"""Seeded synthetic inputs for the FlashMask forward pass.

This module is shared by the kernel path, the tests and the oracle side.  It
only draws random numbers and writes down mask specifications as per-query
key intervals; it holds none of the attention arithmetic.

Mask families (FlashMask page, section 1 "FlashMask技术背景与核心价值", the
four listed mask kinds) are expressed as per-query inclusive key intervals
``[col_start[i], col_end[i]]`` (same page, section 2.1 and the fused compare in
section 4.1):

* causal            row i attends [0, i]                 (section 2.1 example)
* sliding window    row i attends [max(0, i-w+1), i]
* prefix-LM         rows i <  p attend [0, p-1]; rows i >= p attend [0, i]
* document packing  row i of the document starting at ``offset`` attends
                    [offset, i]                          (section 3.3 example)
* sinks + window    two ranges per row, united: the first ``sinks`` keys
                    (causally) and a causal window of w keys (section 5.2
                    item 4; several ranges per row: section 6.1 item 1)

Random draws
------------
* Document lengths and prefix lengths come from ``numpy.random.default_rng``
  (PCG64) seeded with the config seed.
* Q, K and V are i.i.d. N(0, 1) drawn in float32 and rounded to bfloat16
  (round-to-nearest-even).  Each (tensor, batch, head) slice has its own
  ``torch.Generator`` whose seed is derived with ``numpy.random.SeedSequence``
  from (config seed, tensor index, b, h), so any slice can be regenerated alone
  and slices can be drawn in parallel.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np
import torch

# --------------------------------------------------------------------------
# Interval constructors (int32 arrays of length N)
# --------------------------------------------------------------------------


def causal_intervals(N: int) -> Tuple[np.ndarray, np.ndarray]:
    """Row i attends keys [0, i]."""
    i = np.arange(N, dtype=np.int64)
    return np.zeros(N, np.int32), i.astype(np.int32)


def sliding_window_intervals(N: int, w: int) -> Tuple[np.ndarray, np.ndarray]:
    """Causal window of w keys ending at the query: [max(0, i-w+1), i]."""
    if w < 1:
        raise ValueError("window must be >= 1")
    i = np.arange(N, dtype=np.int64)
    return np.maximum(0, i - w + 1).astype(np.int32), i.astype(np.int32)


def prefix_lm_intervals(N: int, p: int) -> Tuple[np.ndarray, np.ndarray]:
    """Bidirectional prefix of length p, causal afterwards."""
    if not 0 <= p <= N:
        raise ValueError("prefix length out of range")
    i = np.arange(N, dtype=np.int64)
    end = np.where(i < p, p - 1, i)
    return np.zeros(N, np.int32), end.astype(np.int32)


def sinks_window_intervals(N: int, w: int, sinks: int) -> Tuple[np.ndarray, np.ndarray]:
    """Two ranges per row (FlashMask article §5.2 item 4): the first `sinks`
    tokens, causally, and a causal window of w keys: [0, min(sinks-1, i)] and
    [max(0, i-w+1), i].  Returned as [2, N] arrays."""
    if w < 1 or sinks < 0:
        raise ValueError("window must be >= 1 and sinks >= 0")
    i = np.arange(N, dtype=np.int64)
    s = np.stack([np.zeros(N, np.int64), np.maximum(0, i - w + 1)])
    e = np.stack([np.minimum(sinks - 1, i), i])
    return s.astype(np.int32), e.astype(np.int32)


def doc_causal_intervals(doc_lengths: Sequence[int]) -> Tuple[np.ndarray, np.ndarray]:
    """Packed documents, causal inside each document and blind across them."""
    starts: List[np.ndarray] = []
    ends: List[np.ndarray] = []
    offset = 0
    for length in doc_lengths:
        length = int(length)
        if length < 1:
            raise ValueError("document length must be >= 1")
        starts.append(np.full(length, offset, np.int64))
        ends.append(np.arange(offset, offset + length, dtype=np.int64))
        offset += length
    if not starts:
        return np.zeros(0, np.int32), np.zeros(0, np.int32)
    return (np.concatenate(starts).astype(np.int32),
            np.concatenate(ends).astype(np.int32))


# --------------------------------------------------------------------------
# Random length draws
# --------------------------------------------------------------------------


def uniform_doc_lengths(rng: np.random.Generator, N: int, lo: int, hi: int) -> List[int]:
    """Integer lengths uniform in [lo, hi] until they cover N; the last one is cut to fit."""
    out: List[int] = []
    total = 0
    while total < N:
        length = int(rng.integers(lo, hi + 1))
        length = min(length, N - total)
        out.append(length)
        total += length
    return out


def lognormal_doc_lengths(rng: np.random.Generator, N: int, median: float, sigma: float,
                          lo: int, hi: int) -> List[int]:
    """Lengths clip(rint(median * exp(sigma * z)), lo, hi), z ~ N(0,1), packed to N."""
    out: List[int] = []
    total = 0
    while total < N:
        z = rng.standard_normal()
        length = int(np.clip(np.rint(median * np.exp(sigma * z)), lo, hi))
        length = min(length, N - total)
        out.append(length)
        total += length
    return out


# --------------------------------------------------------------------------
# Workload configurations
# --------------------------------------------------------------------------


@dataclasses.dataclass(frozen=True)
class Config:
    key: str
    name: str
    B: int
    H: int
    N: int
    d: int
    mask: str
    seed: int
    params: Tuple[Tuple[str, float], ...] = ()

    def param(self, name: str):
        return dict(self.params)[name]

    def describe(self) -> str:
        extra = ",".join(f"{k}={v}" for k, v in self.params)
        return (f"{self.name}: B={self.B} H={self.H} N={self.N} d={self.d} mask={self.mask}"
                + (f" ({extra})" if extra else "") + f" seed={self.seed}")


# One fixed seed per workload, chosen before any kernel ran (seed = 1000 + index).
CONFIGS: Dict[str, Config] = {
    "C1": Config("C1", "causal_tiny", 1, 2, 512, 64, "causal", 1000),
    "C2": Config("C2", "doc_packed_causal", 1, 16, 8192, 128, "doc_uniform", 1001,
                 (("lo", 256), ("hi", 2048))),
    "C3": Config("C3", "sliding_window_causal", 1, 16, 32768, 128, "sliding", 1002,
                 (("window", 1024),)),
    "C4": Config("C4", "prefix_lm", 2, 32, 16384, 128, "prefix_lm", 1003),
    "C5": Config("C5", "long_context_packed", 1, 8, 131072, 128, "doc_lognormal", 1004,
                 (("median", 4096), ("sigma", 1.0), ("lo", 128), ("hi", 32768))),
    # Rows with two ranges: the article's sinks example (10 sink tokens, a
    # window of 1024 keys) at the sliding-window workload's shape.
    "S1": Config("S1", "sinks_plus_window", 1, 16, 32768, 128, "sinks_window", 1005,
                 (("window", 1024), ("sinks", 10))),
}


@dataclasses.dataclass
class MaskSpec:
    col_start: np.ndarray           # int32 [B, N], or [B, K, N] for K ranges per row
    col_end: np.ndarray             # same shape as col_start
    doc_lengths: Optional[List[List[int]]] = None   # per batch, for document masks
    prefix: Optional[List[int]] = None              # per batch, for prefix-LM


def make_intervals(mask: str, B: int, N: int, seed: int, **params) -> MaskSpec:
    """Build the [B, N] interval arrays of one mask family from a seed ([B, K, N]
    for the families with K ranges per row)."""
    rng = np.random.default_rng(seed)
    if mask == "sinks_window":
        s, e = sinks_window_intervals(N, int(params["window"]), int(params["sinks"]))
        return MaskSpec(np.ascontiguousarray(np.broadcast_to(s, (B,) + s.shape)),
                        np.ascontiguousarray(np.broadcast_to(e, (B,) + e.shape)))
    cs = np.empty((B, N), np.int32)
    ce = np.empty((B, N), np.int32)
    docs: Optional[List[List[int]]] = None
    prefix: Optional[List[int]] = None
    if mask == "causal":
        s, e = causal_intervals(N)
        cs[:], ce[:] = s, e
    elif mask == "sliding":
        s, e = sliding_window_intervals(N, int(params["window"]))
        cs[:], ce[:] = s, e
    elif mask == "prefix_lm":
        prefix = []
        lo = int(params.get("lo", N // 8))
        hi = int(params.get("hi", N // 2))
        for b in range(B):
            p = int(rng.integers(lo, hi + 1))
            prefix.append(p)
            cs[b], ce[b] = prefix_lm_intervals(N, p)
    elif mask in ("doc_uniform", "doc_lognormal"):
        docs = []
        for b in range(B):
            if mask == "doc_uniform":
                lens = uniform_doc_lengths(rng, N, int(params["lo"]), int(params["hi"]))
            else:
                lens = lognormal_doc_lengths(rng, N, float(params["median"]), float(params["sigma"]),
                                             int(params["lo"]), int(params["hi"]))
            docs.append(lens)
            cs[b], ce[b] = doc_causal_intervals(lens)
    else:
        raise ValueError(f"unknown mask family {mask!r}")
    return MaskSpec(cs, ce, docs, prefix)


def config_intervals(cfg: Config) -> MaskSpec:
    return make_intervals(cfg.mask, cfg.B, cfg.N, cfg.seed, **dict(cfg.params))


# --------------------------------------------------------------------------
# Q, K, V
# --------------------------------------------------------------------------

_TENSOR_INDEX = {"q": 0, "k": 1, "v": 2}


def _slice_seed(seed: int, tensor: int, b: int, h: int) -> int:
    return int(np.random.SeedSequence([seed, tensor, b, h]).generate_state(1)[0])


def qkv_slice(seed: int, tensor: str, b: int, h: int, N: int, d: int) -> torch.Tensor:
    """One [N, d] bfloat16 slice of q, k or v (CPU)."""
    g = torch.Generator().manual_seed(_slice_seed(seed, _TENSOR_INDEX[tensor], b, h))
    return torch.randn(N, d, generator=g, dtype=torch.float32).to(torch.bfloat16)


def make_qkv(B: int, H: int, N: int, d: int, seed: int,
             threads: Optional[int] = None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Q, K, V as contiguous bfloat16 [B, H, N, d] CPU tensors."""
    out = [torch.empty(B, H, N, d, dtype=torch.bfloat16) for _ in range(3)]
    jobs = [(t, b, h) for t in range(3) for b in range(B) for h in range(H)]
    names = ("q", "k", "v")

    def fill(job):
        t, b, h = job
        out[t][b, h] = qkv_slice(seed, names[t], b, h, N, d)

    if threads is None:
        threads = min(16, len(os.sched_getaffinity(0)))
    if threads <= 1 or len(jobs) == 1:
        for j in jobs:
            fill(j)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill, jobs))
    return out[0], out[1], out[2]


E4M3_MAX = 448.0        # largest finite OCP e4m3 ("e4m3fn") value


def quantize_e4m3(x: torch.Tensor) -> Tuple[torch.Tensor, float]:
    """Per-tensor FP8 quantization: (uint8 e4m3fn codes, scale) with scale = amax / 448 as a
    float32 value and codes = RNE(x / scale), so that scale * e4m3(code) approximates x."""
    xf = x.float()
    amax = float(xf.abs().max())
    scale = float(np.float32(amax / E4M3_MAX)) if amax > 0 else 1.0
    y = (xf / scale).clamp(-E4M3_MAX, E4M3_MAX)
    return y.to(torch.float8_e4m3fn).view(torch.uint8), scale


def dequantize_e4m3(codes: torch.Tensor, scale: float) -> np.ndarray:
    """float64 values scale * e4m3(code) (the decode is exact)."""
    return codes.view(torch.float8_e4m3fn).float().numpy().astype(np.float64) * float(np.float32(scale))


def make_qkv_fp8(B: int, H: int, N: int, d: int, seed: int, threads: Optional[int] = None):
    """The make_qkv draws (before their bf16 rounding), quantized per tensor to e4m3:
    ((q8, q_scale), (k8, k_scale), (v8, v_scale)) with uint8 codes [B, H, N, d]."""
    out = [torch.empty(B, H, N, d, dtype=torch.float32) for _ in range(3)]
    names = ("q", "k", "v")
    for t in range(3):
        for b in range(B):
            for h in range(H):
                g = torch.Generator().manual_seed(_slice_seed(seed, _TENSOR_INDEX[names[t]], b, h))
                out[t][b, h] = torch.randn(N, d, generator=g, dtype=torch.float32)
    return tuple(quantize_e4m3(x) for x in out)


def default_scale(d: int) -> float:
    """1/sqrt(d) rounded to float32 (the value a caller passes as a C float)."""
    return float(np.float32(1.0 / np.sqrt(np.float32(d))))


def random_multi_intervals(rng: np.random.Generator, B: int, K: int, N: int, empty_frac: float = 0.0,
                           max_width: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """K independent random ranges per row: [B, K, N] arrays."""
    cs = np.empty((B, K, N), np.int32)
    ce = np.empty((B, K, N), np.int32)
    for k in range(K):
        cs[:, k], ce[:, k] = random_intervals(rng, B, N, empty_frac, max_width)
    return cs, ce


def random_intervals(rng: np.random.Generator, B: int, N: int, empty_frac: float = 0.0,
                     max_width: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Unstructured valid intervals 0 <= s <= e <= N-1, optionally with empty rows (s > e)."""
    s = rng.integers(0, N, size=(B, N))
    if max_width is None:
        e = rng.integers(s, N)
    else:
        e = np.minimum(N - 1, s + rng.integers(0, max_width, size=(B, N)))
    if empty_frac > 0:
        empty = rng.random((B, N)) < empty_frac
        # An empty row: start one past the end.
        e = np.where(empty, s - 1, e)
    return s.astype(np.int32), e.astype(np.int32)
