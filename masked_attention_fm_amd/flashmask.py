"""ctypes binding of libflashmask (include/flashmask.h), argument marshalling only.

Every step of the computation runs in the library's HIP kernels; this module
only checks tensor metadata, passes device pointers and the current HIP
stream, and turns status codes into exceptions.  It never falls back to
another implementation: if the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libflashmask.so")

FM_OK, FM_ERR_INVALID_ARG, FM_ERR_UNSUPPORTED, FM_ERR_BAD_INTERVAL, FM_ERR_HIP, FM_ERR_TOO_LARGE = range(6)
FM_NOALLOC_SCRATCH_BYTES = 4 << 20
FM_TILE_SKIP, FM_TILE_FULL, FM_TILE_PARTIAL = 0, 1, 2
FM_OPT_SCHEDULE = 1
FM_OPT_BWD_SPLIT_CHUNKS = 2
FM_OPT_SINGLE_LAUNCH = 3
FM_OPT_SPLIT_KEYS = 4
FM_OPT_ROW_SLICES = 5
FM_OPT_BWD_FUSED_PREP = 6
FM_MAX_RANGES = 4
FM_FP8_SCORES, FM_FP8_ALL = 0, 1

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32

# name -> (restype, argtypes); the same names and argument order as the header.
SIGNATURES = {
    "fm_classify_tiles": (ctypes.c_int, [_P, _P, _I64, _I32, _I32, _P]),
    "fm_attn_fwd": (ctypes.c_int, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, ctypes.c_float,
                                   _P, _P, _P]),
    "fm_attn_tile_shape": (ctypes.c_int, [_I64, ctypes.POINTER(_I32), ctypes.POINTER(_I32)]),
    "fm_tile_schedule": (ctypes.c_int, [_P, _P, _I64, _I64, _I64, _P, _P]),
    "fm_attn_fwd_multi": (ctypes.c_int, [_P, _P, _P, _P, _P, _I32, _I64, _I64, _I64, _I64, ctypes.c_float,
                                         _P, _P, _P]),
    "fm_attn_fwd_noalloc": (ctypes.c_int, [_P, _P, _P, _P, _P, _I32, _I64, _I64, _I64, _I64, ctypes.c_float,
                                           _P, _P, _P]),
    "fm_classify_tiles_multi": (ctypes.c_int, [_P, _P, _I32, _I64, _I32, _I32, _P]),
    "fm_attn_fwd_per_head": (ctypes.c_int, [_P, _P, _P, _P, _P, _I32, _I64, _I64, _I64, _I64, ctypes.c_float,
                                            _P, _P, _P]),
    "fm_attn_fwd_fp8": (ctypes.c_int, [_P, _P, _P, ctypes.c_float, ctypes.c_float, ctypes.c_float, _I32, _P, _P,
                                       _I32, _I64, _I64, _I64, _I64, ctypes.c_float, _P, _P, _P]),
    "fm_attn_bwd": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, ctypes.c_float,
                                   _P, _P, _P, _P]),
    "fm_attn_bwd_per_head": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _I32, _I64, _I64, _I64, _I64,
                                            ctypes.c_float, _P, _P, _P, _P]),
    "fm_attn_bwd_multi": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _I32, _I64, _I64, _I64, _I64,
                                         ctypes.c_float, _P, _P, _P, _P]),
    "fm_tile_schedule_multi": (ctypes.c_int, [_P, _P, _I32, _I64, _I64, _I64, _P, _P]),
    "fm_set_option": (ctypes.c_int, [ctypes.c_int, _I64]),
    "fm_profile_enable": (ctypes.c_int, [ctypes.c_int]),
    "fm_profile_read": (ctypes.c_int, [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_I64)]),
    "fm_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "fm_last_hip_error": (ctypes.c_int, []),
}


class FlashMaskError(RuntimeError):
    def __init__(self, func: str, status: int, detail: str = ""):
        self.status = status
        super().__init__(f"{func} failed with status {status}{': ' + detail if detail else ''}")


_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m masked_attention_fm_amd.build` (needs hipcc)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _check(func: str, status: int):
    if status != FM_OK:
        L = lib()
        detail = L.fm_status_string(status).decode()
        if status == FM_ERR_HIP:
            detail += f" (hipError {L.fm_last_hip_error()})"
        raise FlashMaskError(func, status, detail)


def _stream_handle(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _require_scale(scale):
    """The score scale is the caller's (typically 1/sqrt(d) as a float32 value): the
    binding computes none, so every caller passes the exact value the oracle also uses."""
    if scale is None:
        raise ValueError("scale is required (the float32 value multiplying q.k, e.g. 1/sqrt(d))")


def _dev_tensor(x: torch.Tensor, name: str, dtype: torch.dtype):
    # (dtypes are singletons: `is` is the exact test and the cheapest one)
    if not isinstance(x, torch.Tensor) or not x.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if x.dtype is not dtype:
        raise ValueError(f"{name} must be {dtype}, got {x.dtype}")
    if not x.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def fm_attn_tile_shape(d: int) -> Tuple[int, int]:
    br, bc = _I32(), _I32()
    _check("fm_attn_tile_shape", lib().fm_attn_tile_shape(int(d), ctypes.byref(br), ctypes.byref(bc)))
    return br.value, bc.value


def _intervals(col_start: torch.Tensor, col_end: torch.Tensor, shape: Tuple[int, ...], what: str):
    _dev_tensor(col_start, "col_start", torch.int32)
    _dev_tensor(col_end, "col_end", torch.int32)
    if col_start.shape != shape or col_end.shape != shape:
        raise ValueError(f"col_start / col_end must be {what}, got {tuple(col_start.shape)} "
                         f"and {tuple(col_end.shape)}")


def _classify(func: str, col_start, col_end, n_ranges: Optional[int], Br: int, Bc: int, out):
    N = col_start.shape[-1]
    shape = (-(-N // Br), -(-N // Bc)) if Br > 0 and Bc > 0 else (0, 0)
    if out is None:
        out = torch.empty(shape, dtype=torch.uint8, device=col_start.device)
    else:
        _dev_tensor(out, "out", torch.uint8)
        if tuple(out.shape) != shape:
            raise ValueError(f"out must have shape {shape}")
    torch.cuda.current_stream(col_start.device).synchronize()
    L = lib()
    if n_ranges is None:
        status = L.fm_classify_tiles(col_start.data_ptr(), col_end.data_ptr(), N, int(Br), int(Bc),
                                     out.data_ptr())
    else:
        status = L.fm_classify_tiles_multi(col_start.data_ptr(), col_end.data_ptr(), n_ranges, N, int(Br),
                                           int(Bc), out.data_ptr())
    _check(func, status)
    return out


def fm_classify_tiles(col_start: torch.Tensor, col_end: torch.Tensor, Br: int, Bc: int,
                      out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """uint8 [ceil(N/Br), ceil(N/Bc)] class table of one sequence, intervals [N] (synchronous)."""
    if col_start.dim() != 1:
        raise ValueError("col_start / col_end must be 1-D of equal length")
    _intervals(col_start, col_end, tuple(col_start.shape), "[N]")
    return _classify("fm_classify_tiles", col_start, col_end, None, Br, Bc, out)


def fm_classify_tiles_multi(col_start: torch.Tensor, col_end: torch.Tensor, Br: int, Bc: int,
                            out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Class table of one sequence whose rows hold K ranges, intervals [K, N] (synchronous)."""
    if col_start.dim() != 2:
        raise ValueError("col_start / col_end must be [K, N]")
    _intervals(col_start, col_end, tuple(col_start.shape), "[K, N]")
    return _classify("fm_classify_tiles_multi", col_start, col_end, col_start.shape[0], Br, Bc, out)


def _schedule(func: str, col_start, col_end, n_ranges: Optional[int], d: int):
    B, N = col_start.shape[0], col_start.shape[-1]
    br, _ = fm_attn_tile_shape(d)
    M = B * (-(-N // br))
    work = torch.empty(M, dtype=torch.int32, device=col_start.device)
    order = torch.empty(M, dtype=torch.int32, device=col_start.device)
    torch.cuda.current_stream(col_start.device).synchronize()
    L = lib()
    if n_ranges is None:
        status = L.fm_tile_schedule(col_start.data_ptr(), col_end.data_ptr(), B, N, int(d), work.data_ptr(),
                                    order.data_ptr())
    else:
        status = L.fm_tile_schedule_multi(col_start.data_ptr(), col_end.data_ptr(), n_ranges, B, N, int(d),
                                          work.data_ptr(), order.data_ptr())
    _check(func, status)
    return work, order


def fm_tile_schedule(col_start: torch.Tensor, col_end: torch.Tensor, d: int):
    """(work, order) int32 [B * ceil(N/Br)] of the attention kernel's scheduler, intervals [B, N]
    (synchronous)."""
    if col_start.dim() != 2:
        raise ValueError("col_start / col_end must be [B, N]")
    _intervals(col_start, col_end, tuple(col_start.shape), "[B, N]")
    return _schedule("fm_tile_schedule", col_start, col_end, None, d)


def fm_tile_schedule_multi(col_start: torch.Tensor, col_end: torch.Tensor, d: int):
    """fm_tile_schedule for intervals [B, K, N] (synchronous)."""
    if col_start.dim() != 3:
        raise ValueError("col_start / col_end must be [B, K, N]")
    _intervals(col_start, col_end, tuple(col_start.shape), "[B, K, N]")
    return _schedule("fm_tile_schedule_multi", col_start, col_end, col_start.shape[1], d)


def _attn(func: str, q, k, v, col_start, col_end, n_ranges: Optional[int], scale, out, lse, stream):
    B, H, N, d = q.shape
    _require_scale(scale)
    if out is None:
        out = torch.empty_like(q)
    else:
        _dev_tensor(out, "out", torch.bfloat16)
        if out.shape != q.shape:
            raise ValueError("out must match q's shape")
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    else:
        _dev_tensor(lse, "lse", torch.float32)
        if lse.shape != (B, H, N):
            raise ValueError("lse must be [B, H, N]")
    L = _lib if _lib is not None else lib()
    if n_ranges is None:
        status = L.fm_attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), col_start.data_ptr(),
                               col_end.data_ptr(), B, H, N, d, float(scale), out.data_ptr(), lse.data_ptr(),
                               _stream_handle(stream))
    else:
        status = L.fm_attn_fwd_multi(q.data_ptr(), k.data_ptr(), v.data_ptr(), col_start.data_ptr(),
                                     col_end.data_ptr(), n_ranges, B, H, N, d, float(scale), out.data_ptr(),
                                     lse.data_ptr(), _stream_handle(stream))
    _check(func, status)
    return out, lse


def _qkv(q, k, v):
    _dev_tensor(q, "q", torch.bfloat16)
    _dev_tensor(k, "k", torch.bfloat16)
    _dev_tensor(v, "v", torch.bfloat16)
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one [B, H, N, d] shape")
    return q.shape


def fm_attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, col_start: torch.Tensor,
                col_end: torch.Tensor, scale: Optional[float] = None,
                out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Masked attention forward, intervals [B, N]; returns (out bf16 [B,H,N,d], lse fp32 [B,H,N]).
    Asynchronous."""
    B, H, N, d = _qkv(q, k, v)
    _intervals(col_start, col_end, (B, N), "[B, N]")
    return _attn("fm_attn_fwd", q, k, v, col_start, col_end, None, scale, out, lse, stream)


def fm_attn_fwd_multi(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, col_start: torch.Tensor,
                      col_end: torch.Tensor, scale: Optional[float] = None,
                      out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                      stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """fm_attn_fwd for rows with K ranges, intervals [B, K, N]; each row attends their union."""
    B, H, N, d = _qkv(q, k, v)
    if col_start.dim() != 3:
        raise ValueError("col_start / col_end must be [B, K, N]")
    _intervals(col_start, col_end, (B, col_start.shape[1], N), "[B, K, N]")
    return _attn("fm_attn_fwd_multi", q, k, v, col_start, col_end, col_start.shape[1], scale, out, lse,
                 stream)


def fm_attn_fwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, col_start: torch.Tensor,
                        col_end: torch.Tensor, scale: float, out: torch.Tensor, lse: torch.Tensor,
                        stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """fm_attn_fwd_multi into the caller's out and lse with the library's static scratch: the
    library allocates nothing.  Intervals [B, N] or [B, K, N].  Raises FlashMaskError with
    FM_ERR_TOO_LARGE when the problem needs more than FM_NOALLOC_SCRATCH_BYTES.  Calls that
    can overlap on one GPU share that scratch and race.  Asynchronous."""
    B, H, N, d = _qkv(q, k, v)
    if col_start.dim() == 2:
        col_start, col_end = col_start.unsqueeze(1), col_end.unsqueeze(1)
    if col_start.dim() != 3:
        raise ValueError("col_start / col_end must be [B, N] or [B, K, N]")
    _intervals(col_start, col_end, (B, col_start.shape[1], N), "[B, K, N]")
    _require_scale(scale)
    _dev_tensor(out, "out", torch.bfloat16)
    _dev_tensor(lse, "lse", torch.float32)
    if out.shape != q.shape or tuple(lse.shape) != (B, H, N):
        raise ValueError("out must match q's shape and lse must be [B, H, N]")
    status = lib().fm_attn_fwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), col_start.data_ptr(),
                                       col_end.data_ptr(), col_start.shape[1], B, H, N, d, float(scale),
                                       out.data_ptr(), lse.data_ptr(), _stream_handle(stream))
    _check("fm_attn_fwd_noalloc", status)
    return out, lse


def fm_attn_fwd_per_head(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, col_start: torch.Tensor,
                         col_end: torch.Tensor, scale: Optional[float] = None,
                         out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                         stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """fm_attn_fwd with one interval set per head: intervals [B, H, N] or [B, H, K, N]."""
    B, H, N, d = _qkv(q, k, v)
    if col_start.dim() == 3:
        col_start, col_end = col_start.unsqueeze(2), col_end.unsqueeze(2)
    if col_start.dim() != 4:
        raise ValueError("col_start / col_end must be [B, H, N] or [B, H, K, N]")
    _intervals(col_start, col_end, (B, H, col_start.shape[2], N), "[B, H, K, N]")
    if not (col_start.is_contiguous() and col_end.is_contiguous()):
        raise ValueError("col_start / col_end must be contiguous")
    _require_scale(scale)
    if out is None:
        out = torch.empty_like(q)
    else:
        _dev_tensor(out, "out", torch.bfloat16)
        if out.shape != q.shape:
            raise ValueError("out must match q's shape")
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    else:
        _dev_tensor(lse, "lse", torch.float32)
        if tuple(lse.shape) != (B, H, N):
            raise ValueError("lse must be [B, H, N]")
    status = lib().fm_attn_fwd_per_head(q.data_ptr(), k.data_ptr(), v.data_ptr(), col_start.data_ptr(),
                                        col_end.data_ptr(), col_start.shape[2], B, H, N, d, float(scale),
                                        out.data_ptr(), lse.data_ptr(), _stream_handle(stream))
    _check("fm_attn_fwd_per_head", status)
    return out, lse


def fm_attn_fwd_fp8(q8: torch.Tensor, k8: torch.Tensor, v8: torch.Tensor, q_scale: float, k_scale: float,
                    v_scale: float, col_start: torch.Tensor, col_end: torch.Tensor, scale: Optional[float] = None,
                    out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                    stream=None, mode: int = FM_FP8_SCORES) -> Tuple[torch.Tensor, torch.Tensor]:
    """Forward pass on e4m3 inputs (uint8 or torch.float8_e4m3fn tensors [B,H,N,d]) with per-tensor
    dequantization scales; intervals [B, N] or [B, K, N].  mode FM_FP8_SCORES keeps the weights and
    the PV product in bf16, FM_FP8_ALL rounds the weights to e4m3 for an FP8 PV product.  Returns
    (out bf16, lse fp32).  Asynchronous."""
    if mode not in (FM_FP8_SCORES, FM_FP8_ALL):
        raise ValueError("mode must be FM_FP8_SCORES or FM_FP8_ALL")
    codes = []
    for name, x in (("q8", q8), ("k8", k8), ("v8", v8)):
        if isinstance(x, torch.Tensor) and x.dtype == torch.float8_e4m3fn:
            x = x.view(torch.uint8)
        _dev_tensor(x, name, torch.uint8)
        codes.append(x)
    q8, k8, v8 = codes
    if q8.dim() != 4 or k8.shape != q8.shape or v8.shape != q8.shape:
        raise ValueError("q8, k8, v8 must share one [B, H, N, d] shape")
    B, H, N, d = q8.shape
    if col_start.dim() == 2:
        _intervals(col_start, col_end, (B, N), "[B, N]")
        n_ranges = 1
    else:
        if col_start.dim() != 3:
            raise ValueError("col_start / col_end must be [B, N] or [B, K, N]")
        _intervals(col_start, col_end, (B, col_start.shape[1], N), "[B, K, N]")
        n_ranges = col_start.shape[1]
    _require_scale(scale)
    if out is None:
        out = torch.empty(q8.shape, dtype=torch.bfloat16, device=q8.device)
    else:
        _dev_tensor(out, "out", torch.bfloat16)
        if out.shape != q8.shape:
            raise ValueError("out must match q8's shape")
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q8.device)
    else:
        _dev_tensor(lse, "lse", torch.float32)
        if tuple(lse.shape) != (B, H, N):
            raise ValueError("lse must be [B, H, N]")
    status = lib().fm_attn_fwd_fp8(q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), float(q_scale), float(k_scale),
                                   float(v_scale), int(mode), col_start.data_ptr(), col_end.data_ptr(), n_ranges,
                                   B, H, N, d,
                                   float(scale), out.data_ptr(), lse.data_ptr(), _stream_handle(stream))
    _check("fm_attn_fwd_fp8", status)
    return out, lse


def _bwd(func: str, q, k, v, out, dout, lse, col_start, col_end, n_ranges: Optional[int], scale,
         dq, dk, dv, stream):
    B, H, N, d = _qkv(q, k, v)
    for name, x in (("out", out), ("dout", dout)):
        _dev_tensor(x, name, torch.bfloat16)
        if x.shape != q.shape:
            raise ValueError(f"{name} must match q's shape")
    _dev_tensor(lse, "lse", torch.float32)
    if tuple(lse.shape) != (B, H, N):
        raise ValueError("lse must be [B, H, N]")
    _require_scale(scale)
    grads = []
    for name, g in (("dq", dq), ("dk", dk), ("dv", dv)):
        if g is None:
            g = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        else:
            _dev_tensor(g, name, torch.float32)
            if g.shape != q.shape:
                raise ValueError(f"{name} must match q's shape")
        grads.append(g)
    dq, dk, dv = grads
    L = lib()
    ptrs = [x.data_ptr() for x in (q, k, v, out, dout, lse, col_start, col_end)]
    tail = (B, H, N, d, float(scale), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), _stream_handle(stream))
    if n_ranges is None:
        status = L.fm_attn_bwd(*ptrs, *tail)
    elif func == "fm_attn_bwd_per_head":
        status = L.fm_attn_bwd_per_head(*ptrs, n_ranges, *tail)
    else:
        status = L.fm_attn_bwd_multi(*ptrs, n_ranges, *tail)
    _check(func, status)
    return dq, dk, dv


def fm_attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor, dout: torch.Tensor,
                lse: torch.Tensor, col_start: torch.Tensor, col_end: torch.Tensor, scale: Optional[float] = None,
                dq: Optional[torch.Tensor] = None, dk: Optional[torch.Tensor] = None,
                dv: Optional[torch.Tensor] = None, stream=None):
    """Gradients (dq, dk, dv) float32 [B,H,N,d] of fm_attn_fwd for upstream dout; intervals [B, N].
    Asynchronous."""
    B, H, N, d = _qkv(q, k, v)
    _intervals(col_start, col_end, (B, N), "[B, N]")
    return _bwd("fm_attn_bwd", q, k, v, out, dout, lse, col_start, col_end, None, scale, dq, dk, dv, stream)


def fm_attn_bwd_multi(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor, dout: torch.Tensor,
                      lse: torch.Tensor, col_start: torch.Tensor, col_end: torch.Tensor,
                      scale: Optional[float] = None, dq: Optional[torch.Tensor] = None,
                      dk: Optional[torch.Tensor] = None, dv: Optional[torch.Tensor] = None, stream=None):
    """fm_attn_bwd for intervals [B, K, N]."""
    B, H, N, d = _qkv(q, k, v)
    if col_start.dim() != 3:
        raise ValueError("col_start / col_end must be [B, K, N]")
    _intervals(col_start, col_end, (B, col_start.shape[1], N), "[B, K, N]")
    return _bwd("fm_attn_bwd_multi", q, k, v, out, dout, lse, col_start, col_end, col_start.shape[1], scale,
                dq, dk, dv, stream)


def fm_attn_bwd_per_head(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor,
                         dout: torch.Tensor, lse: torch.Tensor, col_start: torch.Tensor, col_end: torch.Tensor,
                         scale: Optional[float] = None, dq: Optional[torch.Tensor] = None,
                         dk: Optional[torch.Tensor] = None, dv: Optional[torch.Tensor] = None, stream=None):
    """fm_attn_bwd for one interval set per head: intervals [B, H, N] or [B, H, K, N]."""
    B, H, N, d = _qkv(q, k, v)
    if col_start.dim() == 3:
        col_start, col_end = col_start.unsqueeze(2).contiguous(), col_end.unsqueeze(2).contiguous()
    if col_start.dim() != 4:
        raise ValueError("col_start / col_end must be [B, H, N] or [B, H, K, N]")
    _intervals(col_start, col_end, (B, H, col_start.shape[2], N), "[B, H, K, N]")
    return _bwd("fm_attn_bwd_per_head", q, k, v, out, dout, lse, col_start, col_end, col_start.shape[2], scale,
                dq, dk, dv, stream)


def fm_set_option(option: int, value: int) -> None:
    _check("fm_set_option", lib().fm_set_option(int(option), int(value)))


def fm_profile_enable(enable: bool) -> None:
    _check("fm_profile_enable", lib().fm_profile_enable(1 if enable else 0))


def fm_profile_read() -> Tuple[float, int]:
    """(summed attention-kernel milliseconds, launches) since the last read."""
    ms, n = ctypes.c_double(), _I64()
    _check("fm_profile_read", lib().fm_profile_read(ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value
