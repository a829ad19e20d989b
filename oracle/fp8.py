"""FP8 forward (test infrastructure only): the E4M3 code book, attention of
the dequantised inputs, and a bound on the error that rounding the weights
P to E4M3 before the P V product may add.

[essay] section "FA2/FA3": FA3 has an FP8 mode.  The pages give no number
format, scaling or error statement for it; the readings taken here are
OCP E4M3 codes for Q, K and V with one dequantisation factor per tensor
(value = code value * descale), scores and softmax in fp32, and P rounded
to E4M3 (after a power-of-two scale) for the second product only, so the
row sums and the LSE come from unrounded P.
"""
from __future__ import annotations

import math

import numpy as np

from .gqa import attn_fwd_gqa


def e4m3_decode(codes) -> np.ndarray:
    """OCP E4M3 (no infinities): sign, 4 exponent bits (bias 7), 3 mantissa
    bits; exponent 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    val = np.where((c & 0x7F) == 0x7F, np.nan, val)
    return sign * val


def dequantize(codes, descale: float) -> np.ndarray:
    return e4m3_decode(codes) * float(descale)


def attn_fwd_fp8(q8, k8, v8, descales, scale: float, causal: bool):
    """Attention ([review] Algorithm 0, grouped K/V heads as in
    oracle/gqa.py) of the dequantised inputs, in float64: the value the FP8
    kernel approximates.  q8 [B,H,N,d], k8 and v8 [B,Hkv,N,d] hold codes."""
    dq, dk, dv = descales
    return attn_fwd_gqa(dequantize(q8, dq), dequantize(k8, dk), dequantize(v8, dv), scale, causal)


def p_rounding_bound(q8, k8, v8, descales, scale: float, causal: bool):
    """Per-element bound on |O - O_exact| from rounding each weight.

    Let P_j = exp(s_j - m) with m the row max and l = sum_j P_j.  A kernel
    that rounds a * 2^8 * P_j to E4M3 and multiplies back exactly, with a
    reference that lies at most 2 log2 units above the row max (a >= 2^-2;
    a reference below the max, a > 1, only helps), changes P_j by at most
    2^-4 P_j (half the 3-bit mantissa spacing) or, below the normal range
    (2^-6), by at most 2^-10 / (2^8 a) <= 2^-16.  With O computed as
    sum_j P~_j V_j / l, the error in column c is at most
    (2^-4 sum_j P_j |V_jc| + 2^-16 sum_j |V_jc|) / l.  Returns that array
    [B,H,N,d]."""
    dq, dk, dv = descales
    q, k, v = dequantize(q8, dq), dequantize(k8, dk), dequantize(v8, dv)
    B, H, N, _ = q.shape
    G = H // k.shape[1]
    out = np.empty(q.shape[:3] + (v.shape[3],))
    for b in range(B):
        for h in range(H):
            g = h // G
            s = scale * (q[b, h] @ k[b, g].T)
            if causal:
                s[np.arange(N)[None, :] > np.arange(N)[:, None]] = -np.inf
            p = np.exp(s - s.max(axis=1, keepdims=True))
            l = p.sum(axis=1, keepdims=True)
            av = np.abs(v[b, g])
            vis = np.isfinite(s).astype(np.float64)
            out[b, h] = (2.0 ** -4 * (p @ av) + 2.0 ** -16 * (vis @ av)) / l
    return out


def e4m3_round(x) -> np.ndarray:
    """Round to the nearest E4M3 value, ties to even mantissa, in float64
    (no saturation: |x| must stay below 464)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -6.0)           # subnormals share the 2^-6 spacing rule
    step = np.exp2(e - 3.0)           # 3 mantissa bits
    r = a / step
    fl = np.floor(r)
    frac = r - fl
    up = (frac > 0.5) | ((frac == 0.5) & (np.mod(fl, 2.0) == 1.0))
    return np.sign(x) * (fl + up) * step


def attn_fwd_fp8_model(q8, k8, v8, descales, scale: float, causal: bool, p_scale: float = 256.0):
    """The FP8 algorithm with P rounded relative to the exact row max:
    O = sum_j round(p_scale P_j) / p_scale V_j / sum_j P_j.  Used only to
    pin p_rounding_bound (a kernel's reference max may differ)."""
    dq, dk, dv = descales
    q, k, v = dequantize(q8, dq), dequantize(k8, dk), dequantize(v8, dv)
    B, H, N, _ = q.shape
    G = H // k.shape[1]
    out = np.empty(q.shape[:3] + (v.shape[3],))
    for b in range(B):
        for h in range(H):
            g = h // G
            s = scale * (q[b, h] @ k[b, g].T)
            if causal:
                s[np.arange(N)[None, :] > np.arange(N)[:, None]] = -np.inf
            p = np.exp(s - s.max(axis=1, keepdims=True))
            pq = e4m3_round(p * p_scale) / p_scale
            out[b, h] = (pq @ v[b, g]) / p.sum(axis=1, keepdims=True)
    return out


def attn_fwd_fp8_rows(q8, k8, v8, descales, scale: float, causal: bool, rows):
    """O, LSE and the P-rounding bound of selected (b, h, i) rows, one at a
    time (full-size sampled checks); same definitions as attn_fwd_fp8 and
    p_rounding_bound."""
    dq, dk, dv = descales
    H, Hkv = q8.shape[1], k8.shape[1]
    G = H // Hkv
    rows = list(rows)
    d = v8.shape[3]
    o, lse, bnd = np.empty((len(rows), d)), np.empty(len(rows)), np.empty((len(rows), d))
    for n, (b, h, i) in enumerate(rows):
        g = h // G
        n_keys = i + 1 if causal else k8.shape[2]
        q = dequantize(q8[b, h, i], dq)
        k = dequantize(k8[b, g, :n_keys], dk)
        v = dequantize(v8[b, g, :n_keys], dv)
        s = scale * (k @ q)
        m = s.max()
        p = np.exp(s - m)
        l = p.sum()
        o[n] = (p @ v) / l
        lse[n] = m + math.log(l)
        bnd[n] = (2.0 ** -4 * (p @ np.abs(v)) + 2.0 ** -16 * np.abs(v).sum(axis=0)) / l
    return o, lse, bnd
