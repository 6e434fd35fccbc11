"""Thin ctypes binding over libentmax.so (the C ABI of include/entmax.h).

Argument marshalling only: torch supplies device memory and the current HIP
stream; every step of the computation runs in the library's HIP kernels.
There is no fallback -- a missing library raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libentmax.so")

(OK, ERR_NULL, ERR_SHAPE, ERR_ALPHA, ERR_DTYPE, ERR_MASK, ERR_WORKSPACE, ERR_ALIGN, ERR_HIP, ERR_ARG,
 ERR_SCRATCH) = range(11)
MASK_NONE, MASK_CAUSAL, MASK_WINDOW_SINK = 0, 1, 2
F32, BF16 = 0, 1


class Options(ctypes.Structure):
    """entmax_options of include/entmax.h (per-call; all zero = defaults)."""
    _fields_ = [("candidate_cap", ctypes.c_int), ("row_plain_bracket", ctypes.c_int)]

_lib: Optional[ctypes.CDLL] = None


class EntmaxError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: status {status} ({status_str(status)})")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libentmax.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m adaptive_sparse_attention_row_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, i32, i64, f32, sz = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                            ctypes.c_float, ctypes.c_size_t)
    L.entmax_status_str.restype = ctypes.c_char_p
    L.entmax_status_str.argtypes = [i32]
    L.entmax_version.restype = i32
    L.entmax_version.argtypes = []
    L.entmax_tile_shape.restype = i32
    L.entmax_tile_shape.argtypes = [i32, i32, P, P]
    L.entmax_tau_rows.restype = i32
    L.entmax_tau_rows.argtypes = [P, P, P, i64, i64, i64, f32, P]
    L.entmax_attn_fwd_workspace.restype = sz
    L.entmax_attn_fwd_workspace.argtypes = [i32] * 7
    L.entmax_attn_fwd.restype = i32
    L.entmax_attn_fwd.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, f32, f32, i32,
                                  i32, i32, P, sz, P]
    L.entmax_attn_bwd_workspace.restype = sz
    L.entmax_attn_bwd_workspace.argtypes = [i32] * 7
    L.entmax_attn_bwd.restype = i32
    L.entmax_attn_bwd.argtypes = [P, P, P, P, P, P, P, P, P, i32, i32, i32, i32, f32, f32,
                                  i32, i32, i32, P, sz, P]
    L.entmax_attn_fwd_gv.restype = i32
    L.entmax_attn_fwd_gv.argtypes = [P, P, P, P, P, P, P, P, i32, i32, i32, i32, f32, f32, i32,
                                     i32, i32, P, sz, P]
    L.entmax_attn_bwd_gv.restype = i32
    L.entmax_attn_bwd_gv.argtypes = [P, P, P, P, P, P, P, P, P, P, P, i32, i32, i32, i32, f32, f32,
                                     i32, i32, i32, P, sz, P]
    L.entmax_attn_threshold.restype = i32
    L.entmax_attn_threshold.argtypes = [P, P, P, P, i32, i32, i32, i32, f32, f32, i32, i32, i32, P, sz, P]
    L.entmax_attn_threshold_workspace.restype = sz
    L.entmax_attn_threshold_workspace.argtypes = [i32] * 7
    L.entmax_attn_score_stats.restype = i32
    L.entmax_attn_score_stats.argtypes = [P, P, i32, i32, i32, i32, f32, f32, i32, i32, i32, P, sz, P]
    L.entmax_attn_output.restype = i32
    L.entmax_attn_output.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, f32, f32, i32, i32, i32, P]
    OP = ctypes.POINTER(Options)
    L.entmax_tau_rows_ex.restype = i32
    L.entmax_tau_rows_ex.argtypes = [P, P, P, i64, i64, i64, f32, OP, P]
    L.entmax_attn_fwd_ex.restype = i32
    L.entmax_attn_fwd_ex.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, f32, f32, i32,
                                     i32, i32, P, sz, OP, P]
    L.entmax_attn_threshold_ex.restype = i32
    L.entmax_attn_threshold_ex.argtypes = [P, P, P, P, i32, i32, i32, i32, f32, f32, i32, i32, i32, P, sz,
                                           OP, P]
    L.entmax_attn_decode_workspace.restype = sz
    L.entmax_attn_decode_workspace.argtypes = [i32] * 7
    L.entmax_attn_decode.restype = i32
    L.entmax_attn_decode.argtypes = [P, P, P, P, P, i32, i32, i32, i32, i32, f32, f32, i32, i32, i32,
                                     P, sz, P]
    L.entmax_attn_decode_noalloc.restype = i32
    L.entmax_attn_decode_noalloc.argtypes = [P, P, P, P, P, i32, i32, i32, i32, i32, f32, f32, i32, i32,
                                             i32, P]
    _lib = L
    return L


def status_str(status: int) -> str:
    return lib().entmax_status_str(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status != OK:
        raise EntmaxError(fn, status)


def _stream(device) -> int:
    import torch
    return torch.cuda.current_stream(device).cuda_stream


def _dev_ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def tile_shape(d: int, dtype: int = BF16) -> tuple[int, int]:
    br, bc = ctypes.c_int(0), ctypes.c_int(0)
    _check("entmax_tile_shape", lib().entmax_tile_shape(d, dtype, ctypes.byref(br), ctypes.byref(bc)))
    return br.value, bc.value


def _opts(candidate_cap: int = 0, row_plain_bracket: bool = False):
    """A per-call options struct, or None when every field is at its default."""
    if candidate_cap == 0 and not row_plain_bracket:
        return None
    return ctypes.byref(Options(int(candidate_cap), 1 if row_plain_bracket else 0))


def tau_rows(S, want_p: bool = True, P=None, tau=None, alpha: float = 1.5, row_plain_bracket: bool = False):
    """Row-wise alpha-entmax (alpha in (1, 2], default 1.5) of a [rows, cols]
    fp32 CUDA tensor (row stride may exceed cols).  Returns (tau [rows],
    P [rows, cols] or None).  row_plain_bracket: see entmax_options."""
    import torch
    if not S.is_cuda or S.dtype != torch.float32 or S.dim() != 2 or S.stride(1) != 1:
        raise ValueError("S must be a 2-D fp32 CUDA tensor with unit column stride")
    rows, cols = S.shape
    ld = S.stride(0) if rows > 1 else cols
    if want_p and P is None:
        P = torch.empty_strided((rows, cols), (ld, 1), device=S.device, dtype=torch.float32)
    if tau is None:
        tau = torch.empty(rows, device=S.device, dtype=torch.float32)
    if P is not None and P.stride() != (ld, 1) and rows > 1:
        raise ValueError("P must share S's row stride")
    st = lib().entmax_tau_rows_ex(S.data_ptr(), _dev_ptr(P), tau.data_ptr(), rows, cols, ld,
                                  float(alpha), _opts(0, row_plain_bracket), _stream(S.device))
    _check("entmax_tau_rows", st)
    return tau, P


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise ValueError(f"unsupported dtype {t.dtype}")


def mask_shape(B: int, H: int, L: int, d: int, dtype: int = BF16) -> tuple[int, int, int, int]:
    br, bc = tile_shape(d, dtype)
    tr, tc = -(-L // br), -(-L // bc)
    return (B, H, tr, -(-tc // 32))


def attn_fwd(q, k, v, scale: Optional[float] = None, mask: int = MASK_NONE, window: int = 0,
             want_block_mask: bool = True, out=None, alpha: float = 1.5, candidate_cap: int = 0):
    """alpha-entmax attention forward (alpha in (1, 2], default 1.5).  q, k,
    v: [B, H, L, d] CUDA tensors (bf16 or fp32, contiguous).  Returns (O fp32,
    tau fp32 [B, H, L], block_mask int32 view of the packed uint32 mask, or
    None).  candidate_cap: see entmax_options (0: the default)."""
    import torch
    B, H, L, d = q.shape
    for t in (q, k, v):
        if not t.is_cuda or not t.is_contiguous() or t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError("q, k, v must be contiguous CUDA tensors of one shape and dtype")
    dt = _dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    O = out if out is not None else torch.empty(B, H, L, d, device=q.device, dtype=torch.float32)
    tau = torch.empty(B, H, L, device=q.device, dtype=torch.float32)
    bm = None
    if want_block_mask:
        bm = torch.empty(mask_shape(B, H, L, d, dt), device=q.device, dtype=torch.int32)
    ws_bytes = lib().entmax_attn_fwd_workspace(B, H, L, d, dt, mask, window)
    ws = torch.empty(ws_bytes, device=q.device, dtype=torch.uint8)
    st = lib().entmax_attn_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), O.data_ptr(),
                                  tau.data_ptr(), _dev_ptr(bm), B, H, L, d, float(scale), float(alpha),
                                  dt, mask, window, _dev_ptr(ws), ws_bytes, _opts(candidate_cap),
                                  _stream(q.device))
    _check("entmax_attn_fwd", st)
    return O, tau, bm


def attn_threshold(q, k, scale: Optional[float] = None, mask: int = MASK_NONE, window: int = 0,
                   tau=None, block_mask=None, workspace=None, alpha: float = 1.5, candidate_cap: int = 0):
    """Phases 1-3 only: returns (tau fp32 [B, H, L], packed block mask)."""
    import torch
    B, H, L, d = q.shape
    dt = _dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if tau is None:
        tau = torch.empty(B, H, L, device=q.device, dtype=torch.float32)
    if block_mask is None:
        block_mask = torch.empty(mask_shape(B, H, L, d, dt), device=q.device, dtype=torch.int32)
    ws_bytes = lib().entmax_attn_threshold_workspace(B, H, L, d, dt, mask, window)
    if workspace is None:
        workspace = torch.empty(ws_bytes, device=q.device, dtype=torch.uint8)
    st = lib().entmax_attn_threshold_ex(q.data_ptr(), k.data_ptr(), tau.data_ptr(), block_mask.data_ptr(),
                                        B, H, L, d, float(scale), float(alpha), dt, mask, window,
                                        workspace.data_ptr(), workspace.numel(), _opts(candidate_cap),
                                        _stream(q.device))
    _check("entmax_attn_threshold", st)
    return tau, block_mask


def attn_output(q, k, v, tau, block_mask, scale: Optional[float] = None, mask: int = MASK_NONE,
                window: int = 0, out=None, alpha: float = 1.5):
    """Phase 4 only: O from a given tau and block mask."""
    import torch
    B, H, L, d = q.shape
    dt = _dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    O = out if out is not None else torch.empty(B, H, L, d, device=q.device, dtype=torch.float32)
    st = lib().entmax_attn_output(q.data_ptr(), k.data_ptr(), v.data_ptr(), tau.data_ptr(),
                                  block_mask.data_ptr(), O.data_ptr(), B, H, L, d, float(scale),
                                  float(alpha), dt, mask, window, _stream(q.device))
    _check("entmax_attn_output", st)
    return O


def attn_bwd(q, k, v, do, tau, block_mask, scale: Optional[float] = None,
             mask: int = MASK_NONE, window: int = 0, alpha: float = 1.5):
    """Backward of attn_fwd.  Returns (dQ, dK, dV), fp32 [B, H, L, d]."""
    import torch
    B, H, L, d = q.shape
    for t in (q, k, v, do):
        if not t.is_cuda or not t.is_contiguous() or t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError("q, k, v, do must be contiguous CUDA tensors of one shape and dtype")
    dt = _dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty(B, H, L, d, device=q.device, dtype=torch.float32)
    dk = torch.empty_like(dq)
    dv = torch.empty_like(dq)
    ws_bytes = lib().entmax_attn_bwd_workspace(B, H, L, d, dt, mask, window)
    ws = torch.empty(max(ws_bytes, 1), device=q.device, dtype=torch.uint8) if ws_bytes else None
    st = lib().entmax_attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), do.data_ptr(),
                               tau.data_ptr(), block_mask.data_ptr(), dq.data_ptr(),
                               dk.data_ptr(), dv.data_ptr(), B, H, L, d, float(scale), float(alpha),
                               dt, mask, window, _dev_ptr(ws), ws_bytes, _stream(q.device))
    _check("entmax_attn_bwd", st)
    return dq, dk, dv


def attn_fwd_gv(q, k, v, scale: Optional[float] = None, mask: int = MASK_NONE, window: int = 0,
                alpha: float = 1.5):
    """Forward for training (bf16, L <= 16384): returns (O, tau, block_mask,
    GV fp32 [B, H, L, d], gsum fp32 [B, H, L]) for attn_bwd_gv."""
    import torch
    B, H, L, d = q.shape
    for t in (q, k, v):
        if not t.is_cuda or not t.is_contiguous() or t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError("q, k, v must be contiguous CUDA tensors of one shape and dtype")
    dt = _dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    O = torch.empty(B, H, L, d, device=q.device, dtype=torch.float32)
    gv = torch.empty_like(O)
    tau = torch.empty(B, H, L, device=q.device, dtype=torch.float32)
    gsum = torch.empty_like(tau)
    bm = torch.empty(mask_shape(B, H, L, d, dt), device=q.device, dtype=torch.int32)
    ws_bytes = lib().entmax_attn_fwd_workspace(B, H, L, d, dt, mask, window)
    ws = torch.empty(ws_bytes, device=q.device, dtype=torch.uint8)
    st = lib().entmax_attn_fwd_gv(q.data_ptr(), k.data_ptr(), v.data_ptr(), O.data_ptr(), tau.data_ptr(),
                                  bm.data_ptr(), gv.data_ptr(), gsum.data_ptr(), B, H, L, d, float(scale),
                                  float(alpha), dt, mask, window, ws.data_ptr(), ws_bytes, _stream(q.device))
    _check("entmax_attn_fwd_gv", st)
    return O, tau, bm, gv, gsum


def attn_bwd_gv(q, k, v, do, tau, block_mask, gv, gsum, scale: Optional[float] = None,
                mask: int = MASK_NONE, window: int = 0, alpha: float = 1.5):
    """Backward of attn_fwd_gv.  Returns (dQ, dK, dV), fp32 [B, H, L, d]."""
    import torch
    B, H, L, d = q.shape
    for t in (q, k, v, do):
        if not t.is_cuda or not t.is_contiguous() or t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError("q, k, v, do must be contiguous CUDA tensors of one shape and dtype")
    dt = _dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty(B, H, L, d, device=q.device, dtype=torch.float32)
    dk = torch.empty_like(dq)
    dv = torch.empty_like(dq)
    ws_bytes = lib().entmax_attn_bwd_workspace(B, H, L, d, dt, mask, window)
    ws = torch.empty(max(ws_bytes, 1), device=q.device, dtype=torch.uint8)
    st = lib().entmax_attn_bwd_gv(q.data_ptr(), k.data_ptr(), v.data_ptr(), do.data_ptr(), tau.data_ptr(),
                                  block_mask.data_ptr(), gv.data_ptr(), gsum.data_ptr(), dq.data_ptr(),
                                  dk.data_ptr(), dv.data_ptr(), B, H, L, d, float(scale), float(alpha), dt,
                                  mask, window, ws.data_ptr(), ws_bytes, _stream(q.device))
    _check("entmax_attn_bwd_gv", st)
    return dq, dk, dv


def attn_decode(q, k_cache, v_cache, L: Optional[int] = None, scale: Optional[float] = None,
                mask: int = MASK_CAUSAL, window: int = 0, alpha: float = 1.5, out=None):
    """One decode step: q [B, H, d] is the query at position L - 1; k_cache and
    v_cache are [B, H, cache_len, d] (rows 0 .. L - 1 used; L defaults to
    cache_len).  Returns (o fp32 [B, H, d], tau fp32 [B, H])."""
    import torch
    B, H, Lc, d = k_cache.shape
    if L is None:
        L = Lc
    if q.shape != (B, H, d) or v_cache.shape != k_cache.shape:
        raise ValueError("q must be [B, H, d] and the caches [B, H, cache_len, d]")
    for t in (q, k_cache, v_cache):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != q.dtype:
            raise ValueError("q and the caches must be contiguous CUDA tensors of one dtype")
    dt = _dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = out if out is not None else torch.empty(B, H, d, device=q.device, dtype=torch.float32)
    tau = torch.empty(B, H, device=q.device, dtype=torch.float32)
    ws_bytes = lib().entmax_attn_decode_workspace(B, H, L, d, dt, mask, window)
    ws = torch.empty(max(ws_bytes, 4), device=q.device, dtype=torch.uint8)
    st = lib().entmax_attn_decode(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), o.data_ptr(),
                                  tau.data_ptr(), B, H, L, Lc, d, float(scale), float(alpha), dt, mask,
                                  window, ws.data_ptr(), ws.numel(), _stream(q.device))
    _check("entmax_attn_decode", st)
    return o, tau


def attn_decode_noalloc(q, k_cache, v_cache, L: Optional[int] = None, scale: Optional[float] = None,
                        mask: int = MASK_CAUSAL, window: int = 0, alpha: float = 1.5, out=None, tau=None):
    """attn_decode through the allocation-free entry point: no workspace; the
    library's static per-device scratch holds the scores (calls that overlap
    on one device race).  `out` and `tau` may be passed in so that the call
    itself allocates nothing."""
    import torch
    B, H, Lc, d = k_cache.shape
    if L is None:
        L = Lc
    if q.shape != (B, H, d) or v_cache.shape != k_cache.shape:
        raise ValueError("q must be [B, H, d] and the caches [B, H, cache_len, d]")
    for t in (q, k_cache, v_cache):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != q.dtype:
            raise ValueError("q and the caches must be contiguous CUDA tensors of one dtype")
    dt = _dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = out if out is not None else torch.empty(B, H, d, device=q.device, dtype=torch.float32)
    tau = tau if tau is not None else torch.empty(B, H, device=q.device, dtype=torch.float32)
    st = lib().entmax_attn_decode_noalloc(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), o.data_ptr(),
                                          tau.data_ptr(), B, H, L, Lc, d, float(scale), float(alpha), dt, mask,
                                          window, _stream(q.device))
    _check("entmax_attn_decode_noalloc", st)
    return o, tau
