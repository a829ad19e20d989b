"""Grouped-query attention in fp64 (test infrastructure only).

[essay] "Flash Attention: IO-awareness principle", section on serving, names
models whose query heads share fewer K/V heads (GQA, and MQA with a single
K/V head).  The pages fix no head map; the reading used here, and by the
library, is the usual one: with H query heads and Hkv K/V heads per batch,
G = H / Hkv consecutive query heads share one K/V head, so query head h
reads K/V head h // G.

Forward: each query head is standard attention ([review] Algorithm 0) with
its group's K and V, so it is written as attn_fwd on those slices.
Backward: K and V of a group feed G query heads, so by the chain rule their
gradients are the sums of the G per-head gradients; dQ is per head.
"""
from __future__ import annotations

import numpy as np

from .attention import attn_bwd, attn_fwd, attn_fwd_rows


def _group(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or k.shape != v.shape[:3] + (k.shape[3],) or v.shape[:3] != k.shape[:3]:
        raise ValueError(f"need q [B,H,N,d] and k, v [B,Hkv,N,d], got {q.shape} {k.shape} {v.shape}")
    B, H, N, _ = q.shape
    if k.shape[0] != B or k.shape[2] != N or H % k.shape[1] != 0:
        raise ValueError(f"K/V heads {k.shape[1]} do not divide query heads {H}")
    return H // k.shape[1]


def attn_fwd_gqa(q, k, v, scale: float, causal: bool):
    """q [B,H,N,d]; k, v [B,Hkv,N,d].  Query head h attends over K/V head
    h // (H // Hkv).  Returns (O [B,H,N,d], LSE [B,H,N]) in float64."""
    G = _group(q, k, v)
    B, H, N, _ = q.shape
    out = np.empty(q.shape[:3] + (v.shape[3],))
    lse = np.empty((B, H, N))
    for h in range(H):
        g = h // G
        o_h, l_h = attn_fwd(q[:, h:h + 1], k[:, g:g + 1], v[:, g:g + 1], scale, causal)
        out[:, h] = o_h[:, 0]
        lse[:, h] = l_h[:, 0]
    return out, lse


def attn_fwd_rows_gqa(q, k, v, scale: float, causal: bool, rows):
    """O and LSE of selected (b, h, i) query rows under the same head map."""
    G = _group(q, k, v)
    rows = list(rows)
    o = np.empty((len(rows), v.shape[3]))
    lse = np.empty(len(rows))
    for n, (b, h, i) in enumerate(rows):
        g = h // G
        o_r, l_r = attn_fwd_rows(q[b:b + 1, h:h + 1], k[b:b + 1, g:g + 1], v[b:b + 1, g:g + 1], scale, causal,
                                 [(0, 0, i)])
        o[n] = o_r[0]
        lse[n] = l_r[0]
    return o, lse


def attn_bwd_gqa(q, k, v, dout, scale: float, causal: bool):
    """Gradients of attn_fwd_gqa: dQ [B,H,N,d] per query head; dK, dV
    [B,Hkv,N,d], each the sum over the G query heads that read that K/V head.
    Returns (dQ, dK, dV, Delta [B,H,N])."""
    G = _group(q, k, v)
    B, H, N, _ = q.shape
    dq = np.empty_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    delta = np.empty((B, H, N))
    for h in range(H):
        g = h // G
        dq_h, dk_h, dv_h, de_h = attn_bwd(q[:, h:h + 1], k[:, g:g + 1], v[:, g:g + 1], dout[:, h:h + 1], scale,
                                          causal)
        dq[:, h] = dq_h[:, 0]
        dk[:, g] += dk_h[:, 0]
        dv[:, g] += dv_h[:, 0]
        delta[:, h] = de_h[:, 0]
    return dq, dk, dv, delta
