"""Python entry points with the names of the C ABI.  They check tensor
placement and shapes, allocate outputs with torch, and pass raw pointers and
torch's current HIP stream to libfa.so."""
from __future__ import annotations

import ctypes

import torch

from . import _lib

DTYPE_CODES = {torch.float32: _lib.FA_F32, torch.float16: _lib.FA_F16, torch.bfloat16: _lib.FA_BF16}


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _check_qkv(*ts: torch.Tensor):
    ref = ts[0]
    if ref.dim() != 4:
        raise ValueError("expected [B, H, N, d] tensors")
    for t in ts:
        if t.device.type != "cuda":
            raise ValueError("tensors must be on a HIP device")
        if t.shape != ref.shape or t.dtype != ref.dtype or t.device != ref.device:
            raise ValueError("q, k, v (and o, dout) must share shape, dtype and device")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous [B, H, N, d]")
    if ref.dtype not in DTYPE_CODES:
        raise ValueError(f"unsupported dtype {ref.dtype}")


def fwd(q, k, v, scale: float, causal: bool, out=None, lse=None):
    """Fused forward: returns (O [B,H,N,d] in q.dtype, LSE float32 [B,H,N])."""
    _check_qkv(q, k, v)
    B, H, N, d = q.shape
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    st = _lib.load().fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, N, d,
                            float(scale), int(bool(causal)), DTYPE_CODES[q.dtype], _stream(q))
    _lib.check(st, "fa_fwd")
    return out, lse


def bwd(q, k, v, o, dout, lse, scale: float, causal: bool, delta=None, dq=None, dk=None, dv=None):
    """Backward: returns (dQ, dK, dV float32 [B,H,N,d], Delta float32 [B,H,N])."""
    _check_qkv(q, k, v, o, dout)
    B, H, N, d = q.shape
    f32 = dict(dtype=torch.float32, device=q.device)
    delta = torch.empty((B, H, N), **f32) if delta is None else delta
    dq = torch.empty((B, H, N, d), **f32) if dq is None else dq
    dk = torch.empty((B, H, N, d), **f32) if dk is None else dk
    dv = torch.empty((B, H, N, d), **f32) if dv is None else dv
    st = _lib.load().fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(), lse.data_ptr(),
                            delta.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d, float(scale),
                            int(bool(causal)), DTYPE_CODES[q.dtype], _stream(q))
    _lib.check(st, "fa_bwd")
    return dq, dk, dv, delta


def bwd_stage(stage: int, q, k, v, o, dout, lse, scale: float, causal: bool, delta, dq, dk, dv):
    """One of fa_bwd's three launches (1 Delta, 2 dK/dV, 3 dQ) into caller
    buffers; stages 1, 2, 3 in order equal one bwd() call."""
    _check_qkv(q, k, v, o, dout)
    B, H, N, d = q.shape
    st = _lib.load().fa_bwd_stage(int(stage), q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                  dout.data_ptr(), lse.data_ptr(), delta.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                  dv.data_ptr(), B, H, N, d, float(scale), int(bool(causal)), DTYPE_CODES[q.dtype],
                                  _stream(q))
    _lib.check(st, f"fa_bwd_stage({stage})")


def _check_gqa(q, k, v, *qlike):
    """q (and o, dout) [B,H,N,d]; k, v [B,Hkv,N,d] with Hkv dividing H."""
    _check_qkv(q, *qlike)
    _check_qkv(k, v)
    if k.dtype != q.dtype or k.device != q.device:
        raise ValueError("k, v must share q's dtype and device")
    B, H, N, d = q.shape
    if k.shape[0] != B or k.shape[2:] != q.shape[2:] or H % k.shape[1] != 0:
        raise ValueError(f"k, v shape {tuple(k.shape)} does not group q shape {tuple(q.shape)}")
    return B, H, k.shape[1], N, d


def fwd_gqa(q, k, v, scale: float, causal: bool, out=None, lse=None):
    """Grouped-query forward: q [B,H,N,d], k and v [B,Hkv,N,d]; query head h
    reads K/V head h // (H // Hkv).  Returns (O [B,H,N,d], LSE [B,H,N])."""
    B, H, Hkv, N, d = _check_gqa(q, k, v)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    st = _lib.load().fa_fwd_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H,
                                Hkv, N, d, float(scale), int(bool(causal)), DTYPE_CODES[q.dtype], _stream(q))
    _lib.check(st, "fa_fwd_gqa")
    return out, lse


def bwd_gqa(q, k, v, o, dout, lse, scale: float, causal: bool, delta=None, dq=None, dk=None, dv=None):
    """Backward of fwd_gqa: returns (dQ [B,H,N,d], dK and dV [B,Hkv,N,d],
    all float32, each dK/dV summed over its group, Delta [B,H,N])."""
    B, H, Hkv, N, d = _check_gqa(q, k, v, o, dout)
    f32 = dict(dtype=torch.float32, device=q.device)
    delta = torch.empty((B, H, N), **f32) if delta is None else delta
    dq = torch.empty((B, H, N, d), **f32) if dq is None else dq
    dk = torch.empty((B, Hkv, N, d), **f32) if dk is None else dk
    dv = torch.empty((B, Hkv, N, d), **f32) if dv is None else dv
    st = _lib.load().fa_bwd_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
                                lse.data_ptr(), delta.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H,
                                Hkv, N, d, float(scale), int(bool(causal)), DTYPE_CODES[q.dtype], _stream(q))
    _lib.check(st, "fa_bwd_gqa")
    return dq, dk, dv, delta


def kv_head(bh: int, H: int, Hkv: int) -> int:
    """The flat K/V head the flat query head bh reads (host copy of the
    kernels' map); -1 for invalid arguments."""
    return int(_lib.load().fa_kv_head(bh, H, Hkv))


def naive_workspace_bytes(B: int, H: int, N: int, dtype: torch.dtype) -> int:
    return int(_lib.load().fa_naive_workspace_bytes(B, H, N, DTYPE_CODES[dtype]))


def naive_fwd(q, k, v, scale: float, causal: bool, out=None, lse=None, s_ws=None, p_ws=None):
    """Three-kernel forward that writes S and P: returns (O, LSE, S, P)."""
    _check_qkv(q, k, v)
    B, H, N, d = q.shape
    ws_dtype = torch.float32 if q.dtype == torch.float32 else torch.float16
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if s_ws is None:
        s_ws = torch.empty((B, H, N, N), dtype=ws_dtype, device=q.device)
    if p_ws is None:
        p_ws = torch.empty((B, H, N, N), dtype=ws_dtype, device=q.device)
    st = _lib.load().fa_naive_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                  s_ws.data_ptr(), p_ws.data_ptr(), B, H, N, d, float(scale), int(bool(causal)),
                                  DTYPE_CODES[q.dtype], _stream(q))
    _lib.check(st, "fa_naive_fwd")
    return out, lse, s_ws, p_ws


def causal_stages(row0: int, row_end: int, bn: int, n: int):
    """The kernels' causal key-block plan for query rows [row0, row_end)."""
    a, b = ctypes.c_int(), ctypes.c_int()
    _lib.check(_lib.load().fa_causal_stages(row0, row_end, bn, n, ctypes.byref(a), ctypes.byref(b)),
               "fa_causal_stages")
    return a.value, b.value


def fwd_tile(d: int, dtype: torch.dtype):
    bm, bn, w = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    _lib.check(_lib.load().fa_fwd_tile(d, DTYPE_CODES[dtype], ctypes.byref(bm), ctypes.byref(bn), ctypes.byref(w)),
               "fa_fwd_tile")
    return bm.value, bn.value, w.value
