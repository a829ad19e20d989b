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


def _check_out(t, shape, dtype, device, name: str):
    """A caller-supplied output, workspace or auxiliary input must be exactly
    what the kernels address: the given shape and dtype, contiguous, on the
    inputs' device.  Anything smaller or strided would be written (or read)
    past its allocation or in the wrong order."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or t.device != device or not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous {dtype} tensor of shape {tuple(shape)} on {device}, got "
                         f"{t.dtype} {tuple(t.shape)} on {t.device}"
                         f"{'' if t.is_contiguous() else ' (not contiguous)'}")


def _check_bytes(t, nbytes: int, device, name: str):
    """A byte workspace: contiguous, on the device, at least nbytes long."""
    if t is None:
        return
    if t.device != device or not t.is_contiguous() or t.numel() * t.element_size() < nbytes:
        raise ValueError(f"{name}: expected a contiguous buffer of at least {nbytes} bytes on {device}")


def fwd(q, k, v, scale: float, causal: bool, out=None, lse=None):
    """Fused forward: returns (O [B,H,N,d] in q.dtype, LSE float32 [B,H,N])."""
    _check_qkv(q, k, v)
    B, H, N, d = q.shape
    _check_out(out, q.shape, q.dtype, q.device, "out")
    _check_out(lse, (B, H, N), torch.float32, q.device, "lse")
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    st = _lib.load().fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, N, d,
                            float(scale), int(bool(causal)), DTYPE_CODES[q.dtype], _stream(q))
    _lib.check(st, "fa_fwd")
    return out, lse


def _check_bwd_bufs(q, lse, delta, dq, dk, dv, kv_shape):
    B, H, N, d = q.shape
    if lse is None:
        raise ValueError("lse: the forward's LSE is required")
    _check_out(lse, (B, H, N), torch.float32, q.device, "lse")
    _check_out(delta, (B, H, N), torch.float32, q.device, "delta")
    _check_out(dq, (B, H, N, d), torch.float32, q.device, "dq")
    _check_out(dk, kv_shape, torch.float32, q.device, "dk")
    _check_out(dv, kv_shape, torch.float32, q.device, "dv")


def bwd(q, k, v, o, dout, lse, scale: float, causal: bool, delta=None, dq=None, dk=None, dv=None):
    """Backward: returns (dQ, dK, dV float32 [B,H,N,d], Delta float32 [B,H,N])."""
    _check_qkv(q, k, v, o, dout)
    B, H, N, d = q.shape
    _check_bwd_bufs(q, lse, delta, dq, dk, dv, (B, H, N, d))
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
    for name, t in (("delta", delta), ("dq", dq), ("dk", dk), ("dv", dv)):
        if t is None:
            raise ValueError(f"{name}: bwd_stage writes into caller buffers")
    _check_bwd_bufs(q, lse, delta, dq, dk, dv, (B, H, N, d))
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
    _check_out(out, q.shape, q.dtype, q.device, "out")
    _check_out(lse, (B, H, N), torch.float32, q.device, "lse")
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    st = _lib.load().fa_fwd_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H,
                                Hkv, N, d, float(scale), int(bool(causal)), DTYPE_CODES[q.dtype], _stream(q))
    _lib.check(st, "fa_fwd_gqa")
    return out, lse


def fwd_chunk(q, k, v, scale: float, causal: bool, out=None, lse=None):
    """Chunked prefill: q [B,H,Nq,d] are the last Nq of Nk positions, k and v
    [B,Hkv,Nk,d]; causal keeps key j for query i iff j <= i + Nk - Nq.
    Returns (O [B,H,Nq,d], LSE [B,H,Nq])."""
    _check_qkv(q)
    _check_qkv(k, v)
    if k.dtype != q.dtype or k.device != q.device:
        raise ValueError("k, v must share q's dtype and device")
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if k.shape[0] != B or k.shape[3] != d or H % Hkv != 0:
        raise ValueError(f"k, v shape {tuple(k.shape)} does not match q shape {tuple(q.shape)}")
    _check_out(out, q.shape, q.dtype, q.device, "out")
    _check_out(lse, (B, H, Nq), torch.float32, q.device, "lse")
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    st = _lib.load().fa_fwd_chunk(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H,
                                  Hkv, Nq, Nk, d, float(scale), int(bool(causal)), DTYPE_CODES[q.dtype], _stream(q))
    _lib.check(st, "fa_fwd_chunk")
    return out, lse


def bwd_gqa(q, k, v, o, dout, lse, scale: float, causal: bool, delta=None, dq=None, dk=None, dv=None):
    """Backward of fwd_gqa: returns (dQ [B,H,N,d], dK and dV [B,Hkv,N,d],
    all float32, each dK/dV summed over its group, Delta [B,H,N])."""
    B, H, Hkv, N, d = _check_gqa(q, k, v, o, dout)
    _check_bwd_bufs(q, lse, delta, dq, dk, dv, (B, Hkv, N, d))
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


def decode_plan(B: int, H: int, Hkv: int, Nkv: int, d: int) -> int:
    """The part count the library suggests for a decode step on the current
    device."""
    n = ctypes.c_int()
    _lib.check(_lib.load().fa_decode_plan(B, H, Hkv, Nkv, d, ctypes.byref(n)), "fa_decode_plan")
    return n.value


def decode_workspace_bytes(B: int, H: int, Hkv: int, d: int, n_parts: int) -> int:
    return int(_lib.load().fa_decode_workspace_bytes(B, H, Hkv, d, n_parts))


def decode(q, k_cache, v_cache, scale: float, kv_lens=None, n_parts=None, out=None, lse=None, ws=None):
    """One decode step: q [B,H,d] against the caches [B,Hkv,Nkv,d]; kv_lens
    an int32 device tensor [B] of valid cache rows (None: all Nkv).  Query
    head h reads K/V head h // (H // Hkv).  The batch's key tiles are shared
    among n_parts workgroups (None: the library's plan).  Returns (O [B,H,d]
    in q.dtype, LSE float32 [B,H]); with more than one part the workspace
    `ws` (allocated if None) holds the pieces of cut units afterwards."""
    if q.dim() != 3 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("expected q [B,H,d] and caches [B,Hkv,Nkv,d]")
    for t in (q, k_cache, v_cache):
        if t.device.type != "cuda" or not t.is_contiguous() or t.dtype != q.dtype or t.device != q.device:
            raise ValueError("q and the caches must be contiguous, on one HIP device, of one dtype")
    if q.dtype not in DTYPE_CODES:
        raise ValueError(f"unsupported dtype {q.dtype}")
    B, H, d = q.shape
    Hkv, Nkv = k_cache.shape[1], k_cache.shape[2]
    if k_cache.shape[0] != B or k_cache.shape[3] != d:
        raise ValueError(f"cache shape {tuple(k_cache.shape)} does not match q {tuple(q.shape)}")
    if kv_lens is not None and (kv_lens.dtype != torch.int32 or kv_lens.device != q.device
                                or kv_lens.numel() != B or not kv_lens.is_contiguous()):
        raise ValueError("kv_lens must be a contiguous int32 tensor of B values on q's device")
    if n_parts is None:
        n_parts = decode_plan(B, H, Hkv, Nkv, d)
    _check_out(out, q.shape, q.dtype, q.device, "out")
    _check_out(lse, (B, H), torch.float32, q.device, "lse")
    need = decode_workspace_bytes(B, H, Hkv, d, n_parts)
    _check_bytes(ws, need, q.device, "ws")
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    if ws is None and need:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    st = _lib.load().fa_decode(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                               kv_lens.data_ptr() if kv_lens is not None else None, out.data_ptr(),
                               lse.data_ptr(), ws.data_ptr() if ws is not None else None,
                               ws.numel() * ws.element_size() if ws is not None else 0, B, H, Hkv, Nkv, d,
                               float(scale), int(n_parts), DTYPE_CODES[q.dtype], _stream(q))
    _lib.check(st, "fa_decode")
    return out, lse


def decode_noalloc(q, k_cache, v_cache, scale: float, kv_lens=None, n_parts=None, out=None, lse=None):
    """decode() through fa_decode_noalloc: the pieces of cut units go to the
    library's fixed per-device scratch buffer instead of a workspace, so the
    library allocates nothing (out / lse are allocated here only if None).
    Calls that overlap on one device share that buffer and must not run
    concurrently."""
    if q.dim() != 3 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("expected q [B,H,d] and caches [B,Hkv,Nkv,d]")
    for t in (q, k_cache, v_cache):
        if t.device.type != "cuda" or not t.is_contiguous() or t.dtype != q.dtype or t.device != q.device:
            raise ValueError("q and the caches must be contiguous, on one HIP device, of one dtype")
    if q.dtype not in DTYPE_CODES:
        raise ValueError(f"unsupported dtype {q.dtype}")
    B, H, d = q.shape
    Hkv, Nkv = k_cache.shape[1], k_cache.shape[2]
    if k_cache.shape[0] != B or k_cache.shape[3] != d:
        raise ValueError(f"cache shape {tuple(k_cache.shape)} does not match q {tuple(q.shape)}")
    if kv_lens is not None and (kv_lens.dtype != torch.int32 or kv_lens.device != q.device
                                or kv_lens.numel() != B or not kv_lens.is_contiguous()):
        raise ValueError("kv_lens must be a contiguous int32 tensor of B values on q's device")
    if n_parts is None:
        n_parts = decode_plan(B, H, Hkv, Nkv, d)
    _check_out(out, q.shape, q.dtype, q.device, "out")
    _check_out(lse, (B, H), torch.float32, q.device, "lse")
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    st = _lib.load().fa_decode_noalloc(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                       kv_lens.data_ptr() if kv_lens is not None else None, out.data_ptr(),
                                       lse.data_ptr(), B, H, Hkv, Nkv, d, float(scale), int(n_parts),
                                       DTYPE_CODES[q.dtype], _stream(q))
    _lib.check(st, "fa_decode_noalloc")
    return out, lse


def decode_pieces(ws, B: int, H: int, Hkv: int, d: int, n_parts: int):
    """Views of a decode workspace after the call: (O [slots, 32, d], LSE
    [slots, 32]), both float32, slots = n_parts + units."""
    units = B * Hkv * ((H // Hkv + 31) // 32)
    slots = n_parts + units
    off = (slots * 32 * d * 4 + 255) // 256 * 256
    flat = ws.view(torch.uint8)
    o = flat[:slots * 32 * d * 4].view(torch.float32).view(slots, 32, d)
    l = flat[off:off + slots * 32 * 4].view(torch.float32).view(slots, 32)
    return o, l


def fwd_fp8(q8, k8, v8, descales, scale: float, causal: bool, out=None, lse=None):
    """FP8 forward: q8 [B,H,N,d], k8 and v8 [B,Hkv,N,d] hold OCP E4M3 codes
    (uint8 or torch.float8_e4m3fn), descales = (q, k, v) factors with value =
    code * factor.  Returns (O bf16 [B,H,N,d], LSE float32 [B,H,N])."""
    ts = [t.view(torch.uint8) if t.dtype == torch.float8_e4m3fn else t for t in (q8, k8, v8)]
    for t in ts:
        if t.dtype != torch.uint8 or t.dim() != 4 or t.device.type != "cuda" or not t.is_contiguous():
            raise ValueError("fp8 inputs must be contiguous 4-d uint8 / float8_e4m3fn tensors on a HIP device")
    q8, k8, v8 = ts
    B, H, N, d = q8.shape
    Hkv = k8.shape[1]
    if k8.shape != v8.shape or k8.shape[0] != B or k8.shape[2:] != q8.shape[2:] or H % Hkv != 0:
        raise ValueError(f"k, v shape {tuple(k8.shape)} does not group q shape {tuple(q8.shape)}")
    _check_out(out, (B, H, N, d), torch.bfloat16, q8.device, "out")
    _check_out(lse, (B, H, N), torch.float32, q8.device, "lse")
    if out is None:
        out = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=q8.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q8.device)
    dq, dk, dv = (float(x) for x in descales)
    st = _lib.load().fa_fwd_fp8(q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H,
                                Hkv, N, d, float(scale), dq, dk, dv, int(bool(causal)), _stream(q8))
    _lib.check(st, "fa_fwd_fp8")
    return out, lse


def fa1_workspace_bytes(B: int, H: int, N: int, d: int) -> int:
    return int(_lib.load().fa_fa1_workspace_bytes(B, H, N, d))


def fwd_fa1(q, k, v, scale: float, causal: bool, out=None, lse=None, ws=None):
    """The FlashAttention-1 loop order (K/V outer, running O/l/m in global
    memory): returns (O, LSE) like fwd(); `ws` (allocated if None) holds the
    final running state afterwards."""
    _check_qkv(q, k, v)
    B, H, N, d = q.shape
    _check_out(out, q.shape, q.dtype, q.device, "out")
    _check_out(lse, (B, H, N), torch.float32, q.device, "lse")
    _check_bytes(ws, fa1_workspace_bytes(B, H, N, d), q.device, "ws")
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if ws is None:
        ws = torch.empty(fa1_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=q.device)
    st = _lib.load().fa_fwd_fa1(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                ws.data_ptr(), ws.numel() * ws.element_size(), B, H, N, d, float(scale),
                                int(bool(causal)), DTYPE_CODES[q.dtype], _stream(q))
    _lib.check(st, "fa_fwd_fa1")
    return out, lse


def fa1_state(ws, B: int, H: int, N: int, d: int):
    """Views of an fwd_fa1 workspace: (O [B,H,N,d], m [B,H,N] log2 units, l)."""
    rows = B * H * N
    a = (rows * d * 4 + 255) // 256 * 256
    b = (rows * 4 + 255) // 256 * 256
    flat = ws.view(torch.uint8)
    o = flat[:rows * d * 4].view(torch.float32).view(B, H, N, d)
    m = flat[a:a + rows * 4].view(torch.float32).view(B, H, N)
    l = flat[a + b:a + b + rows * 4].view(torch.float32).view(B, H, N)
    return o, m, l


def naive_workspace_bytes(B: int, H: int, N: int, dtype: torch.dtype) -> int:
    return int(_lib.load().fa_naive_workspace_bytes(B, H, N, DTYPE_CODES[dtype]))


def naive_fwd(q, k, v, scale: float, causal: bool, out=None, lse=None, s_ws=None, p_ws=None):
    """Three-kernel forward that writes S and P: returns (O, LSE, S, P)."""
    _check_qkv(q, k, v)
    B, H, N, d = q.shape
    ws_dtype = torch.float32 if q.dtype == torch.float32 else torch.float16
    _check_out(out, q.shape, q.dtype, q.device, "out")
    _check_out(lse, (B, H, N), torch.float32, q.device, "lse")
    _check_out(s_ws, (B, H, N, N), ws_dtype, q.device, "s_ws")
    _check_out(p_ws, (B, H, N, N), ws_dtype, q.device, "p_ws")
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


# ---------------------------------------------------------------------------
# Measured ceilings of the chip (no attention arithmetic).
# ---------------------------------------------------------------------------
def ceiling_mfma(workgroups: int, waves: int, iters: int, device="cuda", clocks: bool = False):
    """Launch the matrix-core-only loop; returns (sink, clocks or None).  The
    launch performs workgroups * waves * iters * 8 * 32768 flops."""
    sink = torch.empty(workgroups * waves * 64, dtype=torch.float32, device=device)
    clk = torch.empty(2 * workgroups, dtype=torch.int64, device=device) if clocks else None
    st = _lib.load().fa_ceiling_mfma(sink.data_ptr(), clk.data_ptr() if clk is not None else None, workgroups,
                                     waves, iters, _stream(sink))
    _lib.check(st, "fa_ceiling_mfma")
    return sink, clk


def ceiling_mfma_flops(workgroups: int, waves: int, iters: int) -> float:
    return float(workgroups) * waves * iters * 8 * 32768


def ceiling_copy(src, dst):
    """Copy src into dst (same byte size, a multiple of 16) with the
    streaming-copy kernel; HBM traffic 2 x bytes."""
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes or not src.is_contiguous() or not dst.is_contiguous():
        raise ValueError("src and dst must be contiguous and of equal byte size")
    _lib.check(_lib.load().fa_ceiling_copy(src.data_ptr(), dst.data_ptr(), nbytes, _stream(src)), "fa_ceiling_copy")


def ceiling_valu(mode: int, iters: int, device="cuda") -> float:
    """Shader-clock cycles per loop iteration of the vector-issue loop (mode
    0: 32 exp + 32 mul, 1: 96 fma, 2: both; one wavefront).  Synchronises."""
    sink = torch.empty(64, dtype=torch.float32, device=device)
    cyc = torch.zeros(1, dtype=torch.int64, device=device)
    _lib.check(_lib.load().fa_ceiling_valu(int(mode), sink.data_ptr(), cyc.data_ptr(), int(iters), _stream(sink)),
               "fa_ceiling_valu")
    return cyc.item() / iters


def ceiling_mix(mode: int, workgroups: int, iters: int, device="cuda", clocks: bool = False):
    """Launch the forward-step instruction-mix loop (mode 0: operands in
    registers, 1: operands read from LDS, 2: plus a barrier every two steps);
    returns (sink, clocks or None).  The launch performs
    ceiling_mix_flops(...) matrix flops."""
    sink = torch.empty(workgroups * 512, dtype=torch.float32, device=device)
    clk = torch.empty(2 * workgroups, dtype=torch.int64, device=device) if clocks else None
    _lib.check(_lib.load().fa_ceiling_mix(int(mode), sink.data_ptr(), clk.data_ptr() if clk is not None else None,
                                          int(workgroups), int(iters), _stream(sink)), "fa_ceiling_mix")
    return sink, clk


def ceiling_mix_flops(workgroups: int, iters: int) -> float:
    return float(workgroups) * 8 * iters * 32 * 32768


def ceiling_read(src, sink=None):
    """Read every byte of src once (streaming-read kernel); returns the sink."""
    nbytes = src.numel() * src.element_size()
    if sink is None:
        sink = torch.empty(int(_lib.load().fa_ceiling_read_sink_bytes()), dtype=torch.uint8, device=src.device)
    _lib.check(_lib.load().fa_ceiling_read(src.data_ptr(), nbytes, sink.data_ptr(), _stream(src)), "fa_ceiling_read")
    return sink
