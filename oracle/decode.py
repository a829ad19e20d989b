"""Decode attention (one new query per head over a K/V cache) in fp64, and
an executable model of the split-K/V algorithm (test infrastructure only).

[lesson] "LLM-serving translation" and [essay]'s section on serving: in
decoding the sequence length of Q is 1 -- the newest token attends to every
cached key -- and with few K/V heads (GQA) and batch 1 the work splits into
too few tiles, which is why decoding kernels split the keys.  The pages give
no algorithm for that split; its merge step is the softmax decomposition of
[review] ("Tiling": the max and the normaliser of a concatenation follow
from those of the parts), written in log-sum-exp form.

Conventions.  q is [B, H, d] (the query of each head); k and v are the
caches [B, Hkv, Nkv, d] with query head h reading K/V head h // (H // Hkv);
kv_lens[b] (default Nkv) is the number of valid keys of batch b, the first
kv_lens[b] rows of its cache.  A batch with no valid key has no softmax:
the reading taken is the empty sum, O = 0 and LSE = -inf.
"""
from __future__ import annotations

import math

import numpy as np


def _shapes(q, k, v, kv_lens):
    if q.ndim != 3 or k.ndim != 4 or v.shape != k.shape:
        raise ValueError(f"need q [B,H,d], k and v [B,Hkv,Nkv,d]; got {q.shape} {k.shape} {v.shape}")
    B, H, d = q.shape
    if k.shape[0] != B or k.shape[3] != d or H % k.shape[1] != 0:
        raise ValueError(f"K/V cache {k.shape} does not match q {q.shape}")
    Nkv = k.shape[2]
    lens = [Nkv] * B if kv_lens is None else [int(x) for x in kv_lens]
    if len(lens) != B or any(x < 0 or x > Nkv for x in lens):
        raise ValueError(f"kv_lens must hold B values in [0, {Nkv}]")
    return B, H, H // k.shape[1], lens


def attn_decode(q, k, v, scale: float, kv_lens=None):
    """The definition ([review] Algorithm 0 for a single query row): for
    each (b, h), s = scale * K[:len] q over the valid keys of K/V head
    h // G, O = softmax(s) V[:len], LSE = ln sum exp(s).
    Returns (O [B,H,d], LSE [B,H]) in float64."""
    B, H, G, lens = _shapes(q, k, v, kv_lens)
    o = np.zeros((B, H, v.shape[3]))
    lse = np.full((B, H), -np.inf)
    for b in range(B):
        n = lens[b]
        if n == 0:
            continue
        for h in range(H):
            g = h // G
            s = scale * (k[b, g, :n] @ q[b, h])
            m = s.max()
            f = np.exp(s - m)
            l = f.sum()
            o[b, h] = (f / l) @ v[b, g, :n]
            lse[b, h] = m + math.log(l)
    return o, lse


def split_bounds(length: int, n_splits: int, chunk: int):
    """Key ranges of the splits: split s covers [s * chunk, (s + 1) * chunk)
    clipped to [0, length); a split past the end is empty."""
    return [(min(s * chunk, length), min((s + 1) * chunk, length)) for s in range(n_splits)]


def decode_partials(q, k, v, scale: float, n_splits: int, chunk: int, kv_lens=None):
    """First step of the split algorithm: attention of each query over each
    split's keys alone.  Returns (O_s [B,H,S,d] normalised within the split,
    LSE_s [B,H,S]); an empty split gives O_s = 0, LSE_s = -inf."""
    B, H, G, lens = _shapes(q, k, v, kv_lens)
    if n_splits < 1 or chunk < 1 or n_splits * chunk < k.shape[2]:
        raise ValueError("the splits must cover the cache")
    o = np.zeros((B, H, n_splits, v.shape[3]))
    lse = np.full((B, H, n_splits), -np.inf)
    for b in range(B):
        for s, (k0, k1) in enumerate(split_bounds(lens[b], n_splits, chunk)):
            if k1 <= k0:
                continue
            for h in range(H):
                g = h // G
                sc = scale * (k[b, g, k0:k1] @ q[b, h])
                m = sc.max()
                f = np.exp(sc - m)
                l = f.sum()
                o[b, h, s] = (f / l) @ v[b, g, k0:k1]
                lse[b, h, s] = m + math.log(l)
    return o, lse


def merge_partials(o_s, lse_s):
    """Second step: [review]'s decomposition across the splits.  With
    M = max_s LSE_s, w_s = exp(LSE_s - M): LSE = M + ln sum_s w_s and
    O = sum_s w_s O_s / sum_s w_s.  All splits empty: O = 0, LSE = -inf."""
    B, H, S, d = o_s.shape
    o = np.zeros((B, H, d))
    lse = np.full((B, H), -np.inf)
    for b in range(B):
        for h in range(H):
            m = lse_s[b, h].max()
            if m == -np.inf:
                continue
            w = np.exp(lse_s[b, h] - m)
            o[b, h] = (w @ o_s[b, h]) / w.sum()
            lse[b, h] = m + math.log(w.sum())
    return o, lse


def decode_split_merge(q, k, v, scale: float, n_splits: int, chunk: int, kv_lens=None):
    """The whole split algorithm: partials, then the merge."""
    return merge_partials(*decode_partials(q, k, v, scale, n_splits, chunk, kv_lens))
