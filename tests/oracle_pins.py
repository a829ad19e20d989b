"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each ``pin_*`` takes the implementation under test as an argument and raises
AssertionError when it disagrees with something *other* than itself: a closed
form, an invariant, calculus (finite differences), brute-force sums, or an
independent library routine (torch's float64 scaled_dot_product_attention and
autograd, scipy's logsumexp).  ``tests/test_oracle.py`` runs them on the
oracle; ``tests/test_oracle_mutants.py`` runs them on copies of the oracle
with planted mistakes and requires that every mistake fails at least one pin.

Page tags: [essay] "Flash Attention: IO-awareness principle" (hrletsgo.me);
[triton] "Triton 06: Flash Attention v2" (wonbeomjang.kr); [review] "Paper
review: FlashAttention ... with IO-Awareness" (osehyeon.github.io).
"""
from __future__ import annotations

import math

import numpy as np
import torch
from scipy.special import logsumexp

RNG = np.random.default_rng


def rand(shape, seed, sigma=1.0):
    return RNG(seed).standard_normal(shape) * sigma


def _close(a, b, tol, what):
    err = float(np.max(np.abs(np.asarray(a) - np.asarray(b)))) if np.size(a) else 0.0
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"


# ----------------------------------------------------------------------------
# forward pins
# ----------------------------------------------------------------------------

def pin_rows_are_distributions(fwd):
    """With V = I (d = N) the output is P itself: every row sums to 1, is
    non-negative, and is zero above the diagonal when causal ([review] the
    softmax definition under 'Tiling')."""
    for causal in (False, True):
        for n in (1, 5, 12):
            q = rand((1, 2, n, n), 1 + n)
            k = rand((1, 2, n, n), 2 + n)
            v = np.broadcast_to(np.eye(n), (1, 2, n, n)).copy()
            o, _ = fwd(q, k, v, 0.7, causal)
            _close(o.sum(-1), 1.0, 1e-12, "row sums")
            assert np.all(o >= 0), "negative probability"
            if causal:
                _close(np.triu(o[0, 0], 1), 0.0, 0.0, "future keys")
                _close(np.triu(o[0, 1], 1), 0.0, 0.0, "future keys")


def pin_constant_v(fwd):
    """Every V row equal to c gives O_i = c (a convex combination of equal rows)."""
    for causal in (False, True):
        q = rand((2, 2, 9, 4), 11)
        k = rand((2, 2, 9, 4), 12)
        c = np.array([0.5, -1.25, 3.0, 7.0])
        v = np.broadcast_to(c, (2, 2, 9, 4)).copy()
        o, _ = fwd(q, k, v, 0.9, causal)
        _close(o, np.broadcast_to(c, o.shape), 1e-12, "constant V")


def pin_zero_q(fwd):
    """Q = 0 makes every logit 0: O_i is the plain mean of the allowed V rows
    and LSE_i = ln(#allowed keys), for any scale."""
    n, d = 13, 5
    v = rand((1, 3, n, d), 21)
    k = rand((1, 3, n, d), 22)
    q = np.zeros((1, 3, n, d))
    o, lse = fwd(q, k, v, 2.5, False)
    _close(o, np.broadcast_to(v.mean(axis=2, keepdims=True), o.shape), 1e-12, "Q=0 mean")
    _close(lse, math.log(n), 1e-12, "Q=0 LSE")
    o, lse = fwd(q, k, v, 2.5, True)
    pref = np.cumsum(v, axis=2) / np.arange(1, n + 1)[None, None, :, None]
    _close(o, pref, 1e-12, "Q=0 causal prefix mean")
    _close(lse, np.broadcast_to(np.log(np.arange(1, n + 1)), lse.shape), 1e-12, "Q=0 causal LSE")


def pin_single_key(fwd):
    """N = 1: O = V and LSE = scale * q.k.  Causal row 0 sees only key 0:
    O_0 = V_0 and LSE_0 = scale * q_0.k_0."""
    q, k, v = rand((2, 1, 1, 6), 31), rand((2, 1, 1, 6), 32), rand((2, 1, 1, 6), 33)
    o, lse = fwd(q, k, v, 0.3, False)
    _close(o, v, 1e-12, "N=1 O")
    _close(lse, 0.3 * np.sum(q * k, -1), 1e-12, "N=1 LSE")
    q, k, v = rand((1, 2, 7, 6), 34), rand((1, 2, 7, 6), 35), rand((1, 2, 7, 6), 36)
    o, lse = fwd(q, k, v, 0.3, True)
    _close(o[:, :, 0], v[:, :, 0], 1e-12, "causal row 0 O")
    _close(lse[:, :, 0], 0.3 * np.sum(q[:, :, 0] * k[:, :, 0], -1), 1e-12, "causal row 0 LSE")


def pin_shift_invariance(fwd):
    """Adding u to every key adds scale*q_i.u to every logit of row i: softmax
    is unchanged, LSE_i grows by scale*q_i.u."""
    for causal in (False, True):
        q, k, v = rand((1, 2, 10, 4), 41), rand((1, 2, 10, 4), 42), rand((1, 2, 10, 4), 43)
        u = np.array([0.3, -2.0, 1.1, 0.05])
        o1, l1 = fwd(q, k, v, 0.8, causal)
        o2, l2 = fwd(q, k + u, v, 0.8, causal)
        _close(o2, o1, 1e-10, "shift O")
        _close(l2 - l1, 0.8 * (q @ u), 1e-10, "shift LSE")


def pin_key_permutation(fwd):
    """Non-causal attention is a function of the *set* of (k_j, v_j) pairs."""
    q, k, v = rand((2, 1, 11, 3), 51), rand((2, 1, 11, 3), 52), rand((2, 1, 11, 3), 53)
    perm = RNG(54).permutation(11)
    o1, l1 = fwd(q, k, v, 1.3, False)
    o2, l2 = fwd(q, k[:, :, perm], v[:, :, perm], 1.3, False)
    _close(o2, o1, 1e-12, "perm O")
    _close(l2, l1, 1e-12, "perm LSE")


def pin_huge_logits(fwd):
    """Logits ~1e3 stay finite (max subtraction), and when one key dominates
    every row by a margin of hundreds, O_i equals that key's V row."""
    n, d = 8, 4
    q = rand((1, 1, n, d), 61)
    k = rand((1, 1, n, d), 62)
    v = rand((1, 1, n, d), 63)
    o, lse = fwd(q, k, v, 40.0, False)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse)), "huge logits overflowed"
    # a construction with one dominant key for every row
    q = np.ones((1, 1, n, d))
    k = np.zeros((1, 1, n, d))
    k[0, 0, 3] = 10.0
    o, lse = fwd(q, k, v, 25.0, False)  # logit 1000 vs 0
    _close(o[0, 0], np.broadcast_to(v[0, 0, 3], (n, d)), 1e-12, "dominant key")
    _close(lse, 1000.0, 1e-12, "dominant LSE")


def pin_bruteforce_fwd(fwd, brute):
    """Vectorised result equals explicit-loop sums on tiny inputs."""
    for causal in (False, True):
        for n in (1, 3, 7):
            q, k, v = rand((2, 2, n, 3), 71 + n), rand((2, 2, n, 3), 72 + n), rand((2, 2, n, 3), 73 + n)
            o1, l1 = fwd(q, k, v, 0.6, causal)
            o2, l2 = brute(q, k, v, 0.6, causal)
            _close(o1, o2, 1e-12, "brute O")
            _close(l1, l2, 1e-12, "brute LSE")


def pin_torch_sdpa(fwd):
    """Independent library: torch's float64 CPU scaled_dot_product_attention
    (is_causal is the lower-triangular, diagonal-kept mask) and scipy's
    logsumexp of the scaled, masked logits."""
    for causal in (False, True):
        for n, d in ((1, 8), (33, 16), (70, 8)):
            q, k, v = rand((2, 3, n, d), 81), rand((2, 3, n, d), 82), rand((2, 3, n, d), 83)
            o, lse = fwd(q, k, v, 0.25, causal)
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), is_causal=causal, scale=0.25)
            _close(o, ref.numpy(), 1e-12, "SDPA O")
            s = 0.25 * np.einsum("bhid,bhjd->bhij", q, k)
            if causal:
                s = np.where(np.tril(np.ones((n, n), bool)), s, -np.inf)
            _close(lse, logsumexp(s, axis=-1), 1e-12, "logsumexp LSE")


def pin_rows_helper(fwd, rows_fn):
    """The per-row helper equals the full forward at sampled rows."""
    for causal in (False, True):
        q, k, v = rand((2, 2, 40, 8), 91), rand((2, 2, 40, 8), 92), rand((2, 2, 40, 8), 93)
        o, lse = fwd(q, k, v, 0.4, causal)
        rows = [(0, 0, 0), (1, 1, 39), (0, 1, 17), (1, 0, 5)]
        ro, rl = rows_fn(q, k, v, 0.4, causal, rows)
        for n, (b, h, i) in enumerate(rows):
            _close(ro[n], o[b, h, i], 1e-12, "row helper O")
            _close(rl[n], lse[b, h, i], 1e-12, "row helper LSE")


# ----------------------------------------------------------------------------
# backward pins
# ----------------------------------------------------------------------------

def pin_finite_differences(fwd, bwd):
    """Central differences of L = sum(dO * O) (h = 1e-6) match the analytic
    dQ, dK, dV to 1e-6 relative, at N <= 16, d <= 8."""
    for causal in (False, True):
        n, d = 6, 3
        q, k, v, g = (rand((1, 1, n, d), s) for s in (101, 102, 103, 104))
        dq, dk, dv, _ = bwd(q, k, v, g, 0.9, causal)
        h = 1e-6
        for name, x, dx in (("Q", q, dq), ("K", k, dk), ("V", v, dv)):
            fd = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                old = x[idx]
                x[idx] = old + h
                lp = float(np.sum(g * fwd(q, k, v, 0.9, causal)[0]))
                x[idx] = old - h
                lm = float(np.sum(g * fwd(q, k, v, 0.9, causal)[0]))
                x[idx] = old
                fd[idx] = (lp - lm) / (2 * h)
            scale = max(1.0, float(np.max(np.abs(dx))))
            _close(fd / scale, dx / scale, 1e-6, f"finite differences d{name}")


def pin_delta_identity(fwd, bwd):
    """The Jacobian-form Delta_i = sum_k P_ik dP_ik equals rowsum(dO_i * O_i),
    the preprocessing step of [triton] 'Backward' (because O = P V)."""
    for causal in (False, True):
        q, k, v, g = (rand((2, 2, 21, 5), s) for s in (111, 112, 113, 114))
        o, _ = fwd(q, k, v, 0.7, causal)
        _, _, _, delta = bwd(q, k, v, g, 0.7, causal)
        _close(delta, np.sum(g * o, -1), 1e-10, "Delta identity")


def pin_gradient_sums(bwd):
    """sum_j dS_ij = 0 for every row gives sum_j dK_j = 0; sum_j P_ij = 1 gives
    sum_j dV_j = sum_i dO_i."""
    for causal in (False, True):
        q, k, v, g = (rand((2, 2, 19, 4), s) for s in (121, 122, 123, 124))
        _, dk, dv, _ = bwd(q, k, v, g, 1.1, causal)
        _close(dk.sum(axis=2), 0.0, 1e-9, "sum dK")
        _close(dv.sum(axis=2), g.sum(axis=2), 1e-9, "sum dV")


def pin_torch_autograd(bwd):
    """Independent library: torch float64 autograd through SDPA."""
    for causal in (False, True):
        n, d = 37, 8
        q, k, v, g = (rand((2, 2, n, d), s) for s in (131, 132, 133, 134))
        tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_(True) for x in (q, k, v))
        out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=0.35)
        out.backward(torch.from_numpy(g))
        dq, dk, dv, _ = bwd(q, k, v, g, 0.35, causal)
        _close(dq, tq.grad.numpy(), 1e-11, "autograd dQ")
        _close(dk, tk.grad.numpy(), 1e-11, "autograd dK")
        _close(dv, tv.grad.numpy(), 1e-11, "autograd dV")


def pin_bruteforce_bwd(bwd, brute):
    for causal in (False, True):
        q, k, v, g = (rand((1, 2, 5, 3), s) for s in (141, 142, 143, 144))
        a = bwd(q, k, v, g, 0.8, causal)[:3]
        b = brute(q, k, v, g, 0.8, causal)
        for x, y, nm in zip(a, b, ("dQ", "dK", "dV")):
            _close(x, y, 1e-12, f"brute {nm}")


FWD_PINS = (pin_rows_are_distributions, pin_constant_v, pin_zero_q, pin_single_key,
            pin_shift_invariance, pin_key_permutation, pin_huge_logits, pin_torch_sdpa)


# ----------------------------------------------------------------------------
# grouped-query attention pins ([essay], section on serving: GQA / MQA).  The
# head map (query head h reads K/V head h // (H // Hkv)) is the reading the
# oracle states; torch's enable_gqa uses the same one and is independent code.
# ----------------------------------------------------------------------------

GQA_SHAPES = ((2, 8, 2), (1, 4, 1), (1, 3, 3), (2, 6, 3))  # (B, H, Hkv): G = 4, MQA, G = 1, G = 2


def _gqa_inputs(B, H, Hkv, n, d, seed):
    q, dout = rand((B, H, n, d), seed), rand((B, H, n, d), seed + 1)
    k, v = rand((B, Hkv, n, d), seed + 2), rand((B, Hkv, n, d), seed + 3)
    return q, k, v, dout


def pin_gqa_torch_sdpa(fwd_gqa):
    """O equals torch float64 SDPA with enable_gqa; LSE equals scipy's
    logsumexp of the explicitly masked logits of K/V head h // G."""
    for causal in (False, True):
        for B, H, Hkv in GQA_SHAPES:
            q, k, v, _ = _gqa_inputs(B, H, Hkv, 23, 5, 300 + H)
            o, lse = fwd_gqa(q, k, v, 0.6, causal)
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), is_causal=causal, scale=0.6,
                enable_gqa=True).numpy()
            _close(o, ref, 1e-12, f"gqa sdpa O {B, H, Hkv}")
            G = H // Hkv
            for b in range(B):
                for h in range(H):
                    s = 0.6 * (q[b, h] @ k[b, h // G].T)
                    if causal:
                        s[np.triu_indices(23, 1)] = -np.inf
                    _close(lse[b, h], logsumexp(s, axis=1), 1e-12, "gqa LSE")


def pin_gqa_bruteforce(fwd_gqa, brute):
    """Brute-force MHA (explicit sums) on K/V heads repeated G times in head
    order 0,0,..,1,1,.. gives the same O and LSE."""
    for causal in (False, True):
        q, k, v, _ = _gqa_inputs(1, 6, 2, 7, 3, 320)
        o, lse = fwd_gqa(q, k, v, 0.8, causal)
        ob, lb = brute(q, np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1), 0.8, causal)
        _close(o, ob, 1e-12, "gqa brute O")
        _close(lse, lb, 1e-12, "gqa brute LSE")


def pin_gqa_autograd(bwd_gqa):
    """dQ, dK, dV equal torch float64 autograd through SDPA with enable_gqa
    (which sums the shared K/V heads' gradients itself)."""
    for causal in (False, True):
        for B, H, Hkv in GQA_SHAPES:
            q, k, v, g = _gqa_inputs(B, H, Hkv, 19, 4, 340 + H)
            tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_(True) for x in (q, k, v))
            out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=0.45,
                                                                   enable_gqa=True)
            out.backward(torch.from_numpy(g))
            dq, dk, dv, _ = bwd_gqa(q, k, v, g, 0.45, causal)
            _close(dq, tq.grad.numpy(), 1e-11, f"gqa autograd dQ {B, H, Hkv}")
            _close(dk, tk.grad.numpy(), 1e-11, f"gqa autograd dK {B, H, Hkv}")
            _close(dv, tv.grad.numpy(), 1e-11, f"gqa autograd dV {B, H, Hkv}")


def pin_gqa_finite_differences(fwd_gqa, bwd_gqa):
    """Central differences of L = sum(dO * O) with respect to the shared K
    and V (h = 1e-6) match the analytic dK, dV: a K/V head's gradient is the
    sum over the query heads that read it."""
    for causal in (False, True):
        q, k, v, g = _gqa_inputs(1, 4, 2, 5, 3, 360)
        _, dk, dv, _ = bwd_gqa(q, k, v, g, 0.9, causal)
        h = 1e-6
        for name, x, dx in (("K", k, dk), ("V", v, dv)):
            fd = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                old = x[idx]
                x[idx] = old + h
                lp = float(np.sum(g * fwd_gqa(q, k, v, 0.9, causal)[0]))
                x[idx] = old - h
                lm = float(np.sum(g * fwd_gqa(q, k, v, 0.9, causal)[0]))
                x[idx] = old
                fd[idx] = (lp - lm) / (2 * h)
            scale = max(1.0, float(np.max(np.abs(dx))))
            _close(fd / scale, dx / scale, 1e-6, f"gqa finite differences d{name}")


def pin_gqa_identical_heads(bwd_gqa):
    """Closed form: when every query head of a group carries the same Q and dO,
    the group's dK and dV are G times one head's, and all its dQ are equal."""
    for causal in (False, True):
        q1, k, v, g1 = _gqa_inputs(1, 1, 1, 11, 4, 380)
        G = 4
        q, g = np.repeat(q1, G, axis=1), np.repeat(g1, G, axis=1)
        dq, dk, dv, _ = bwd_gqa(q, k, v, g, 0.7, causal)
        dq1, dk1, dv1, _ = bwd_gqa(q1, k, v, g1, 0.7, causal)
        _close(dk, G * dk1, 1e-12, "identical heads dK")
        _close(dv, G * dv1, 1e-12, "identical heads dV")
        _close(dq, np.repeat(dq1, G, axis=1), 1e-12, "identical heads dQ")


# ----------------------------------------------------------------------------
# decode pins ([lesson] "LLM-serving translation": decoding has one query per
# head; [review]'s softmax decomposition merges the split partials)
# ----------------------------------------------------------------------------

def _decode_inputs(B, H, Hkv, nkv, d, seed, sigma=1.0):
    q = rand((B, H, d), seed, sigma)
    k, v = rand((B, Hkv, nkv, d), seed + 1, sigma), rand((B, Hkv, nkv, d), seed + 2)
    return q, k, v


def pin_decode_is_last_causal_row(decode, fwd_gqa):
    """Decoding the newest token equals the last row of causal grouped-query
    attention over a sequence whose last query is that token."""
    q, k, v = _decode_inputs(3, 6, 2, 19, 4, 400)
    lens = [19, 7, 1]
    o, lse = decode(q, k, v, 0.7, lens)
    for b, n in enumerate(lens):
        qs = rand((1, 6, n, 4), 410 + b)
        qs[0, :, n - 1] = q[b]
        of, lf = fwd_gqa(qs, k[b:b + 1, :, :n], v[b:b + 1, :, :n], 0.7, True)
        _close(o[b], of[0, :, n - 1], 1e-12, "decode vs last causal row O")
        _close(lse[b], lf[0, :, n - 1], 1e-12, "decode vs last causal row LSE")


def pin_decode_torch_sdpa(decode):
    """Independent library: torch float64 SDPA with enable_gqa on one query
    over each batch's valid keys; LSE from scipy's logsumexp."""
    for (B, H, Hkv) in ((2, 8, 2), (1, 4, 1), (2, 3, 3)):
        q, k, v = _decode_inputs(B, H, Hkv, 41, 8, 420 + H)
        lens = [41, 13][:B]
        o, lse = decode(q, k, v, 0.35, lens)
        G = H // Hkv
        for b, n in enumerate(lens):
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(q[b][:, None].copy()), torch.from_numpy(k[b, :, :n].copy()),
                torch.from_numpy(v[b, :, :n].copy()), scale=0.35, enable_gqa=True).numpy()[:, 0]
            _close(o[b], ref, 1e-12, f"decode sdpa O {B, H, Hkv}")
            for h in range(H):
                _close(lse[b, h], logsumexp(0.35 * (k[b, h // G, :n] @ q[b, h])), 1e-12, "decode LSE")


def pin_decode_closed_forms(decode):
    """One valid key: O = v_0 and LSE = scale q.k_0.  No valid key: O = 0 and
    LSE = -inf (the empty sum).  Logits near 1000 stay finite."""
    q, k, v = _decode_inputs(2, 4, 2, 5, 3, 430)
    o, lse = decode(q, k, v, 0.9, [1, 0])
    for h in range(4):
        _close(o[0, h], v[0, h // 2, 0], 1e-15, "decode single key O")
        _close(lse[0, h], 0.9 * float(q[0, h] @ k[0, h // 2, 0]), 1e-13, "decode single key LSE")
    assert np.all(o[1] == 0.0) and np.all(np.isneginf(lse[1])), "decode with no key"
    q, k, v = _decode_inputs(1, 2, 1, 9, 4, 440, sigma=20.0)
    o, lse = decode(q, k, v, 1.0, None)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse)), "decode huge logits"
    for h in range(2):
        _close(lse[0, h], logsumexp(k[0, 0] @ q[0, h]), 1e-9, "decode huge logits LSE")


def pin_split_merge(split_merge, decode):
    """The split algorithm reproduces the definition for any split count and
    chunk that cover the cache: splits past the valid keys, splits of one
    key, one split, ragged lengths, empty batches and huge logits."""
    for sigma, scale in ((1.0, 0.5), (15.0, 1.0)):
        q, k, v = _decode_inputs(3, 4, 2, 37, 5, 450, sigma)
        lens = [37, 10, 0]
        ref_o, ref_l = decode(q, k, v, scale, lens)
        for n_splits, chunk in ((1, 37), (2, 19), (3, 16), (5, 8), (37, 1), (40, 1), (4, 128)):
            o, lse = split_merge(q, k, v, scale, n_splits, chunk, lens)
            _close(o, ref_o, 1e-12 * max(1.0, sigma), f"split/merge O S={n_splits} C={chunk}")
            assert np.array_equal(np.isneginf(lse), np.isneginf(ref_l)), "split/merge empty rows"
            fin = np.isfinite(ref_l)
            _close(lse[fin], ref_l[fin], 1e-11 * max(1.0, sigma ** 2), f"split/merge LSE S={n_splits}")


def pin_partials_torch(partials):
    """Each split's partial is attention over that split's keys alone
    (torch float64 SDPA), with its own LSE (scipy); empty splits are
    (0, -inf)."""
    q, k, v = _decode_inputs(2, 4, 4, 30, 6, 460)
    lens = [30, 9]
    o_s, lse_s = partials(q, k, v, 0.6, 4, 8, lens)
    for b, n in enumerate(lens):
        for s in range(4):
            k0, k1 = min(8 * s, n), min(8 * s + 8, n)
            if k1 <= k0:
                assert np.all(o_s[b, :, s] == 0) and np.all(np.isneginf(lse_s[b, :, s])), "empty split"
                continue
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(q[b][:, None].copy()), torch.from_numpy(k[b, :, k0:k1].copy()),
                torch.from_numpy(v[b, :, k0:k1].copy()), scale=0.6).numpy()[:, 0]
            _close(o_s[b, :, s], ref, 1e-12, "partial O")
            for h in range(4):
                _close(lse_s[b, h, s], logsumexp(0.6 * (k[b, h, k0:k1] @ q[b, h])), 1e-12, "partial LSE")


# ----------------------------------------------------------------------------
# chunked prefill pins ([essay], section on PagedAttention and chunked
# prefill): Nq queries, the last Nq of Nk positions
# ----------------------------------------------------------------------------

def _chunk_inputs(B, H, Hkv, nq, nk, d, seed):
    return (rand((B, H, nq, d), seed), rand((B, Hkv, nk, d), seed + 1), rand((B, Hkv, nk, d), seed + 2))


def pin_chunk_is_suffix_of_causal(chunk_fwd, fwd_gqa):
    """A chunk's rows equal the last Nq rows of causal grouped-query attention
    over the whole sequence (earlier query rows arbitrary)."""
    for nq, nk in ((5, 19), (1, 7), (19, 19), (32, 70)):
        q, k, v = _chunk_inputs(2, 4, 2, nq, nk, 3, 500 + nk)
        qfull = rand((2, 4, nk, 3), 510 + nk)
        qfull[:, :, nk - nq:] = q
        of, lf = fwd_gqa(qfull, k, v, 0.6, True)
        o, lse = chunk_fwd(q, k, v, 0.6, True)
        _close(o, of[:, :, nk - nq:], 1e-12, f"chunk suffix O {nq}/{nk}")
        _close(lse, lf[:, :, nk - nq:], 1e-12, f"chunk suffix LSE {nq}/{nk}")


def pin_chunk_torch_sdpa(chunk_fwd):
    """Independent library: torch float64 SDPA with an explicit boolean mask
    (key j allowed for query i iff j <= i + Nk - Nq) and enable_gqa; without
    the mask, plain SDPA.  LSE from scipy's logsumexp."""
    for causal in (False, True):
        for nq, nk in ((7, 23), (23, 23), (1, 9)):
            q, k, v = _chunk_inputs(1, 6, 3, nq, nk, 5, 520 + nq)
            o, lse = chunk_fwd(q, k, v, 0.45, causal)
            mask = None
            if causal:
                mask = torch.from_numpy(np.arange(nk)[None, :] <= np.arange(nq)[:, None] + (nk - nq))
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), attn_mask=mask, scale=0.45,
                enable_gqa=True).numpy()
            _close(o, ref, 1e-12, f"chunk sdpa O causal={causal} {nq}/{nk}")
            for h in range(6):
                s = 0.45 * (q[0, h] @ k[0, h // 2].T)
                if causal:
                    s[~mask.numpy()] = -np.inf
                _close(lse[0, h], logsumexp(s, axis=1), 1e-12, "chunk LSE")


def pin_chunked_prefill_reassembles(chunk_fwd, fwd_gqa):
    """Prefill done chunk by chunk (each chunk against every key up to its
    end) reassembles causal attention over the whole prompt."""
    n = 41
    q, k, v = _chunk_inputs(1, 2, 1, n, n, 4, 530)
    full_o, full_l = fwd_gqa(q, k, v, 0.8, True)
    for cuts in ((0, 16, 32, 41), (0, 1, 40, 41), (0, 41)):
        for c0, c1 in zip(cuts[:-1], cuts[1:]):
            o, lse = chunk_fwd(q[:, :, c0:c1], k[:, :, :c1], v[:, :, :c1], 0.8, True)
            _close(o, full_o[:, :, c0:c1], 1e-12, f"chunk [{c0},{c1})")
            _close(lse, full_l[:, :, c0:c1], 1e-12, f"chunk LSE [{c0},{c1})")


# ----------------------------------------------------------------------------
# FP8 pins ([essay] section "FA2/FA3": FA3's FP8 mode).  The code book is
# OCP E4M3; torch's float8_e4m3fn is the independent implementation.
# ----------------------------------------------------------------------------

def pin_e4m3_codebook(decode):
    """All 256 codes against torch.float8_e4m3fn, plus closed forms: 0x38 = 1,
    0x7E = 448 (largest), 0x08 = 2^-6 (smallest normal), 0x01 = 2^-9
    (smallest subnormal), 0x80 = -0, 0x7F and 0xFF = NaN."""
    got = decode(np.arange(256))
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(got), np.isnan(ref)), "E4M3 NaN codes"
    fin = ~np.isnan(ref)
    _close(got[fin], ref[fin], 0.0, "E4M3 code book")
    assert got[0x38] == 1.0 and got[0x7E] == 448.0 and got[0x08] == 2.0 ** -6 and got[0x01] == 2.0 ** -9
    assert got[0x80] == 0.0 and np.signbit(got[0x80]) and np.isnan(got[0x7F]) and np.isnan(got[0xFF])


def pin_e4m3_round(rnd, decode):
    """Round-to-nearest-even onto the code book: random values, exact
    midpoints between neighbouring codes (ties go to the even mantissa) and
    subnormals, against torch's conversion."""
    vals = decode(np.arange(0x7F))  # non-negative finite codes, ascending
    mids = (vals[:-1] + vals[1:]) / 2
    x = np.concatenate([RNG(600).standard_normal(4000) * 40, RNG(601).standard_normal(1000) * 0.01,
                        mids, -mids, vals])
    x = np.clip(x, -448, 448)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).double().numpy()
    _close(rnd(x), ref, 0.0, "E4M3 rounding")


def _fp8_inputs(B, H, Hkv, n, d, seed, sigma=1.0):
    """Codes via torch's conversion after a per-tensor scale amax / 448."""
    out, scales = [], []
    for i, heads in enumerate((H, Hkv, Hkv)):
        x = torch.from_numpy(rand((B, heads, n, d), seed + i, sigma))
        ds = float(x.abs().max()) / 448.0
        out.append((x / ds).to(torch.float8_e4m3fn).view(torch.uint8).numpy())
        scales.append(ds)
    return out[0], out[1], out[2], tuple(scales)


def pin_fp8_attention(attn_fp8, fwd_gqa):
    """The FP8 reference is grouped-query attention of the dequantised codes
    (dequantised here with torch, independently of the oracle's decoder)."""
    for causal in (False, True):
        q8, k8, v8, ds = _fp8_inputs(2, 4, 2, 21, 8, 610)
        deq = [torch.from_numpy(c).view(torch.float8_e4m3fn).double().numpy() * s for c, s in zip((q8, k8, v8), ds)]
        o, lse = attn_fp8(q8, k8, v8, ds, 0.4, causal)
        ro, rl = fwd_gqa(*deq, 0.4, causal)
        _close(o, ro, 1e-13, "fp8 attention O")
        _close(lse, rl, 1e-13, "fp8 attention LSE")


def pin_p_rounding_bound(bound, model, attn_fp8):
    """Simulating the rounding of P (E4M3, ties to even, relative to the
    exact row max, with pre-scales 2^8 and 2^6 -- a reference 2 log2 units
    above the max) stays within the bound, and the bound is not vacuous:
    some element uses at least a tenth of it, and it never exceeds
    2^-4 max|V| + N 2^-16 max|V|."""
    for causal in (False, True):
        for sigma in (1.0, 3.0):
            q8, k8, v8, ds = _fp8_inputs(1, 2, 2, 150, 16, 620 + int(sigma), sigma)
            exact, _ = attn_fp8(q8, k8, v8, ds, 0.3, causal)
            bnd = bound(q8, k8, v8, ds, 0.3, causal)
            vmax = float(np.abs(torch.from_numpy(v8).view(torch.float8_e4m3fn).double().numpy()).max()) * ds[2]
            assert bnd.max() <= (2.0 ** -4 + 150 * 2.0 ** -16) * vmax * (1 + 1e-12), "bound above its ceiling"
            for p_scale in (256.0, 64.0):
                err = np.abs(model(q8, k8, v8, ds, 0.3, causal, p_scale) - exact)
                assert np.all(err <= bnd * (1 + 1e-9) + 1e-15), f"rounding exceeds the bound ({p_scale})"
                assert (err / bnd).max() >= 0.1, "bound vacuous"
