"""Plain fp64 definitions of exact attention (test infrastructure only).

Tensor convention everywhere: float64 NumPy arrays of shape [B, H, N, d]
(batch, head, sequence, head dim), row-major.  ``scale`` multiplies QK^T.
``causal`` keeps key j for query i iff j <= i (square, top-left aligned,
diagonal kept) -- the mask of [triton] "Improvement 3", which keeps the
positions where the query offset is at least the key offset.

Nothing here is blocked, fused or reordered beyond what the cited definition
or algorithm states; BLAS matmul and NumPy exp are the only library steps.
See the package docstring for the page tags [essay], [lesson], [triton],
[review].
"""
from __future__ import annotations

import math

import numpy as np

LOG2E = 1.0 / math.log(2.0)

# Rows of S held at once by attn_fwd/attn_bwd: bounds memory to
# ROW_CHUNK * N float64 per temporary, nothing more.
ROW_CHUNK = 512


def _check(q, k, v):
    """q and k are [B,H,N,d]; v is [B,H,N,d_v] with any d_v (Algorithm 0
    only needs V to have one row per key)."""
    if q.ndim != 4 or q.shape != k.shape or v.ndim != 4 or v.shape[:3] != q.shape[:3]:
        raise ValueError(f"need q, k [B,H,N,d] and v [B,H,N,d_v], got {q.shape} {k.shape} {v.shape}")
    for t in (q, k, v):
        if t.dtype != np.float64:
            raise TypeError("the oracle computes in float64; upcast the inputs first")


def _causal_mask(rows: np.ndarray, n_keys: int) -> np.ndarray:
    """True where key j is *not* allowed for query i (j > i)."""
    return np.arange(n_keys)[None, :] > rows[:, None]


def attn_fwd(q, k, v, scale: float, causal: bool):
    """Standard attention, [review] Algorithm 0, with the 1/sqrt(d)-style scale
    of [essay] "Standard Attention's real bottleneck" taken as an argument.

    S = scale * Q K^T (masked to -inf above the diagonal when causal);
    P = softmax(S) row-wise in the safe form of [review] "Tiling"
    (m = max, f = exp(x - m), l = sum f, softmax = f / l); O = P V.
    LSE_i = m_i + ln l_i, natural log (the value [triton] "Improvement 2"
    returns after converting its base-2 statistic).

    Returns (O [B,H,N,d], LSE [B,H,N]) in float64.
    """
    _check(q, k, v)
    B, H, N, d = q.shape
    out = np.empty((B, H, N, v.shape[3]), dtype=np.float64)
    lse = np.empty((B, H, N), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            for r0 in range(0, N, ROW_CHUNK):
                r1 = min(N, r0 + ROW_CHUNK)
                s = scale * (q[b, h, r0:r1] @ k[b, h].T)
                if causal:
                    s[_causal_mask(np.arange(r0, r1), N)] = -np.inf
                m = s.max(axis=1, keepdims=True)
                f = np.exp(s - m)
                l = f.sum(axis=1, keepdims=True)
                out[b, h, r0:r1] = (f / l) @ v[b, h]
                lse[b, h, r0:r1] = (m + np.log(l))[:, 0]
    return out, lse


def attn_fwd_rows(q, k, v, scale: float, causal: bool, rows):
    """O and LSE for selected query rows only, one row at a time.

    ``rows`` is an iterable of (b, h, i).  Same definition as attn_fwd; used to
    check full-size GPU results on a sample where the full N x N is too big.
    Returns (O rows [len, d], LSE [len]).
    """
    rows = list(rows)
    o = np.empty((len(rows), v.shape[-1]), dtype=np.float64)
    lse = np.empty(len(rows), dtype=np.float64)
    for n, (b, h, i) in enumerate(rows):
        n_keys = i + 1 if causal else q.shape[2]
        s = scale * (k[b, h, :n_keys] @ q[b, h, i])
        m = s.max()
        f = np.exp(s - m)
        l = f.sum()
        o[n] = (f / l) @ v[b, h, :n_keys]
        lse[n] = m + math.log(l)
    return o, lse


def attn_bwd(q, k, v, dout, scale: float, causal: bool):
    """Analytic gradients of attention through the textbook softmax Jacobian.

    With S, P as in attn_fwd and upstream gradient dO:
      dV = P^T dO,  dP = dO V^T,
      dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik),
      dQ = scale * dS K,  dK = scale * dS^T Q.
    This deliberately does *not* use the shortcut Delta_i = rowsum(dO_i * O_i)
    of [triton] "Backward"; it returns Delta_i := sum_k P_ik dP_ik so that a
    test can check the shortcut against it.

    Returns (dQ, dK, dV [B,H,N,d], Delta [B,H,N]) in float64.
    """
    _check(q, k, v)
    if dout.shape != q.shape or dout.dtype != np.float64:
        raise ValueError("dout must be float64 with q's shape")
    B, H, N, d = q.shape
    dq = np.empty_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    delta = np.empty((B, H, N), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            for r0 in range(0, N, ROW_CHUNK):
                r1 = min(N, r0 + ROW_CHUNK)
                s = scale * (q[b, h, r0:r1] @ k[b, h].T)
                if causal:
                    s[_causal_mask(np.arange(r0, r1), N)] = -np.inf
                m = s.max(axis=1, keepdims=True)
                f = np.exp(s - m)
                p = f / f.sum(axis=1, keepdims=True)
                dp = dout[b, h, r0:r1] @ v[b, h].T
                dl = (p * dp).sum(axis=1)
                ds = p * (dp - dl[:, None])
                dq[b, h, r0:r1] = scale * (ds @ k[b, h])
                dk[b, h] += scale * (ds.T @ q[b, h, r0:r1])
                dv[b, h] += p.T @ dout[b, h, r0:r1]
                delta[b, h, r0:r1] = dl
    return dq, dk, dv, delta


def loss(o, dout) -> float:
    """Scalar L = sum(dO * O); its gradient w.r.t. O is dO (used for finite
    differences of the backward)."""
    return float(np.sum(dout * o))


# ---------------------------------------------------------------------------
# Brute force: explicit sums with math.exp, for N <= 16.  Independent of BLAS
# and of the vectorised code above.
# ---------------------------------------------------------------------------

def _bf_probs(qh, kh, scale, causal, i):
    n = len(kh)
    d = len(qh[0])
    allowed = [j for j in range(n) if (not causal) or j <= i]
    s = {j: scale * sum(qh[i][c] * kh[j][c] for c in range(d)) for j in allowed}
    mx = max(s.values())
    e = {j: math.exp(s[j] - mx) for j in allowed}
    tot = sum(e.values())
    return {j: e[j] / tot for j in allowed}, mx + math.log(tot)


def attn_fwd_bruteforce(q, k, v, scale: float, causal: bool):
    """O and LSE by explicit loops (tiny N only)."""
    B, H, N, d = q.shape
    if N > 16:
        raise ValueError("brute force is for N <= 16")
    o = np.zeros_like(q)
    lse = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            qh, kh, vh = q[b, h].tolist(), k[b, h].tolist(), v[b, h].tolist()
            for i in range(N):
                p, l = _bf_probs(qh, kh, scale, causal, i)
                lse[b, h, i] = l
                for c in range(d):
                    o[b, h, i, c] = sum(p[j] * vh[j][c] for j in p)
    return o, lse


def attn_bwd_bruteforce(q, k, v, dout, scale: float, causal: bool):
    """dQ, dK, dV by explicit chain rule through each softmax row (tiny N)."""
    B, H, N, d = q.shape
    if N > 16:
        raise ValueError("brute force is for N <= 16")
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            qh, kh, vh, gh = (t[b, h].tolist() for t in (q, k, v, dout))
            for i in range(N):
                p, _ = _bf_probs(qh, kh, scale, causal, i)
                # dL/dP_ij = dO_i . V_j
                g = {j: sum(gh[i][c] * vh[j][c] for c in range(d)) for j in p}
                for j in p:
                    for c in range(d):
                        dv[b, h, j, c] += p[j] * gh[i][c]
                # softmax Jacobian: dS_ij = sum_k g_k * P_k (delta_jk - P_j)
                for j in p:
                    dsij = sum(g[kk] * p[kk] * ((1.0 if kk == j else 0.0) - p[j]) for kk in p)
                    for c in range(d):
                        dq[b, h, i, c] += scale * dsij * kh[j][c]
                        dk[b, h, j, c] += scale * dsij * qh[i][c]
    return dq, dk, dv


# ---------------------------------------------------------------------------
# Executable models of the tiled algorithms (fp64, tiny N).  They follow the
# pages' steps in the pages' order; tests show they equal attn_fwd.
# ---------------------------------------------------------------------------

def _exp_sub(a, b, exp=np.exp):
    """exp(a - b) with the convention that a = -inf contributes 0 (also when
    b = -inf, where a - b would be NaN).  Needed where a causal block holds
    no allowed key for some row."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    safe_b = np.where(np.isneginf(b), 0.0, b)
    return np.where(np.isneginf(a), 0.0, exp(a - safe_b))


def fa1_block_sizes(sram_elems: int, d: int):
    """Block sizes of [review] Algorithm 1 step 1: B_c = ceil(M / 4d),
    B_r = min(ceil(M / 4d), d).  (The printed bracket is misplaced; this is
    the reading where the min compares ceil(M/4d) with d.)"""
    bc = -(-sram_elems // (4 * d))
    return min(bc, d), bc


def online_fa1(q, k, v, scale: float, causal: bool, br: int, bc: int, trace=None):
    """[review] Algorithm 1: K/V blocks in the outer loop, Q blocks inside,
    O_i, l_i, m_i kept in 'HBM' arrays and rewritten every (i, j) step with
    the normalised update of [essay] "Tiling":

      m~ = rowmax(S_ij), P~ = exp(S_ij - m~), l~ = rowsum(P~)
      m_new = max(m_i, m~),  l_new = e^{m_i - m_new} l_i + e^{m~ - m_new} l~
      O_i <- diag(l_new)^-1 (diag(l_i) e^{m_i - m_new} O_i + e^{m~ - m_new} P~ V_j)

    The printed algorithm has no scale; S_ij here is scale * Q_i K_j^T.
    ``trace``, if a list, receives (i, j, m_i, l_i) after every step.
    Returns (O, LSE) with LSE = m + ln l.
    """
    _check(q, k, v)
    B, H, N, d = q.shape
    out = np.zeros_like(q)
    lse = np.zeros((B, H, N))
    tr = -(-N // br)
    tc = -(-N // bc)
    for b in range(B):
        for h in range(H):
            o = np.zeros((N, d))
            l = np.zeros(N)
            m = np.full(N, -np.inf)
            for j in range(tc):
                kj = k[b, h, j * bc:(j + 1) * bc]
                vj = v[b, h, j * bc:(j + 1) * bc]
                cols = np.arange(j * bc, j * bc + len(kj))
                for i in range(tr):
                    rows = np.arange(i * br, min(N, (i + 1) * br))
                    s = scale * (q[b, h, rows] @ kj.T)
                    if causal:
                        s[cols[None, :] > rows[:, None]] = -np.inf
                    mt = s.max(axis=1)
                    pt = _exp_sub(s, mt[:, None])
                    lt = pt.sum(axis=1)
                    mi, li, oi = m[rows], l[rows], o[rows]
                    mn = np.maximum(mi, mt)
                    a_old = _exp_sub(mi, mn)
                    a_new = _exp_sub(mt, mn)
                    ln = a_old * li + a_new * lt
                    num = (li * a_old)[:, None] * oi + a_new[:, None] * (pt @ vj)
                    with np.errstate(invalid="ignore", divide="ignore"):
                        o[rows] = np.where(ln[:, None] > 0, num / np.where(ln > 0, ln, 1.0)[:, None], 0.0)
                    l[rows] = ln
                    m[rows] = mn
                    if trace is not None:
                        trace.append((i, j, mn.copy(), ln.copy()))
            out[b, h] = o
            lse[b, h] = m + np.log(l)
    return out, lse


def causal_stage_ranges(i: int, bm: int, bn: int, n: int):
    """Key-block ranges for query block i under the causal 2-stage split of
    [triton] "Improvement 3".

    Query block i holds rows [i*bm, min((i+1)*bm, n)).  Key block j holds keys
    [j*bn, (j+1)*bn).  Stage 1 (no mask) takes every block lying entirely at or
    left of the block's first row: (j+1)*bn <= i*bm.  Stage 2 (masked) takes the
    blocks from there up to the one holding the block's last row.  Blocks after
    that are all in the future for every row and are skipped.

    The page's own test compares the block's first key with the first row;
    that equals "entirely left" only when bm is a multiple of bn.  The form
    above is correct for any bm, bn.

    Returns ((0, s1_end), (s1_end, s2_end)) as half-open ranges of j.
    """
    if not (0 <= i and i * bm < n):
        raise ValueError("query block out of range")
    s1_end = (i * bm) // bn
    last_row = min((i + 1) * bm, n) - 1
    s2_end = last_row // bn + 1
    return (0, s1_end), (s1_end, s2_end)


def online_fa2(q, k, v, scale: float, causal: bool, bm: int, bn: int, trace=None):
    """The FlashAttention-2 forward as [triton] describes it: Q blocks in the
    outer loop, K/V blocks inside; the accumulator is kept un-scaled and
    corrected by alpha = exp2(m_old - m_new) each block, with one divide by l
    at the end ("Improvement 1"); exp2 with qk_scale = scale * log2(e) folded
    in before the loop and a base-2 LSE = m + log2(l) converted to natural log
    on return ("Improvement 2"); l starts at 1.0, which the first alpha = 0
    cancels; causal runs stage 1 (no mask) then stage 2 (diagonal, masked),
    non-causal runs every block unmasked ("Improvement 3").

    ``trace``, if a list, receives (i, j, stage, m, l) after every block.
    Returns (O, LSE natural).
    """
    _check(q, k, v)
    B, H, N, d = q.shape
    qk_scale = scale * LOG2E
    out = np.zeros_like(q)
    lse = np.zeros((B, H, N))
    exp2 = np.exp2
    for b in range(B):
        for h in range(H):
            for i in range(-(-N // bm)):
                rows = np.arange(i * bm, min(N, (i + 1) * bm))
                qi = q[b, h, rows]
                acc = np.zeros((len(rows), d))
                m = np.full(len(rows), -np.inf)
                l = np.ones(len(rows))
                if causal:
                    (a1, b1), (a2, b2) = causal_stage_ranges(i, bm, bn, N)
                    plan = [(j, 1) for j in range(a1, b1)] + [(j, 2) for j in range(a2, b2)]
                else:
                    plan = [(j, 3) for j in range(-(-N // bn))]
                for j, stage in plan:
                    cols = np.arange(j * bn, min(N, (j + 1) * bn))
                    t = (qi @ k[b, h, cols].T) * qk_scale
                    if stage == 2:
                        t[cols[None, :] > rows[:, None]] = -np.inf
                    mn = np.maximum(m, t.max(axis=1))
                    alpha = _exp_sub(m, mn, exp2)
                    p = _exp_sub(t, mn[:, None], exp2)
                    l = l * alpha + p.sum(axis=1)
                    acc = acc * alpha[:, None] + p @ v[b, h, cols]
                    m = mn
                    if trace is not None:
                        trace.append((i, j, stage, m.copy(), l.copy()))
                out[b, h, rows] = acc / l[:, None]
                lse[b, h, rows] = (m + np.log2(l)) / LOG2E
    return out, lse
