"""Chunked prefill: a block of Nq new queries against Nk keys (test
infrastructure only).

[essay], section on PagedAttention and chunked prefill: serving systems feed
the attention kernel a chunk of the prompt at a time, and each chunk
attends to every key before it (the cached ones and its own).  The chunk's
queries are the last Nq of Nk positions, so with the causal mask query i
(0-based within the chunk) keeps key j iff j <= i + (Nk - Nq): the square
mask of [triton] "Improvement 3" aligned at the bottom-right corner.  That
alignment is the reading taken; the pages draw no picture of it.  Without
the mask every query sees all Nk keys.  K/V heads are shared as in
oracle/gqa.py (query head h reads K/V head h // (H // Hkv)).
"""
from __future__ import annotations

import math

import numpy as np


def attn_fwd_chunk(q, k, v, scale: float, causal: bool):
    """q [B,H,Nq,d]; k, v [B,Hkv,Nk,d].  The definition ([review] Algorithm
    0) with the bottom-right causal mask.  Returns (O [B,H,Nq,d], LSE
    [B,H,Nq]) in float64."""
    if q.ndim != 4 or k.ndim != 4 or v.shape[:3] != k.shape[:3]:
        raise ValueError(f"need q [B,H,Nq,d], k and v [B,Hkv,Nk,d]; got {q.shape} {k.shape} {v.shape}")
    B, H, Nq, _ = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if k.shape[0] != B or H % Hkv != 0 or (causal and Nq > Nk):
        raise ValueError("bad grouping, or a causal chunk longer than its keys")
    G = H // Hkv
    off = Nk - Nq
    out = np.empty((B, H, Nq, v.shape[3]))
    lse = np.empty((B, H, Nq))
    for b in range(B):
        for h in range(H):
            g = h // G
            s = scale * (q[b, h] @ k[b, g].T)
            if causal:
                s[np.arange(Nk)[None, :] > np.arange(Nq)[:, None] + off] = -np.inf
            m = s.max(axis=1, keepdims=True)
            f = np.exp(s - m)
            l = f.sum(axis=1, keepdims=True)
            out[b, h] = (f / l) @ v[b, g]
            lse[b, h] = (m + np.log(l))[:, 0]
    return out, lse


def attn_fwd_chunk_rows(q, k, v, scale: float, causal: bool, rows):
    """O and LSE of selected (b, h, i) rows, one at a time (for full-size
    sampled checks)."""
    B, H, Nq, _ = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    G = H // Hkv
    rows = list(rows)
    o = np.empty((len(rows), v.shape[3]))
    lse = np.empty(len(rows))
    for n, (b, h, i) in enumerate(rows):
        g = h // G
        n_keys = i + (Nk - Nq) + 1 if causal else Nk
        s = scale * (k[b, g, :n_keys] @ q[b, h, i])
        m = s.max()
        f = np.exp(s - m)
        o[n] = (f / f.sum()) @ v[b, g, :n_keys]
        lse[n] = m + math.log(f.sum())
    return o, lse
