"""Planted mistakes in copies of the oracle must each fail a pin (CPU only).

The mutants below are the oracle's forward/backward with one plausible slip
each: a dropped scale, a mask that points the wrong way or drops the
diagonal, a transposed or swapped operand, a wrong log base, no max
subtraction, a dropped term of the softmax Jacobian, a missing scale in one
gradient.  If a mutant passed every pin, the pins would not be strong enough
to trust the oracle; this test fails in that case.
"""
import numpy as np
import pytest

import oracle
from tests import oracle_pins as P


def _fwd_variant(q, k, v, scale, causal, mut):
    B, H, N, d = q.shape
    o = np.empty_like(q)
    lse = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            s = (1.0 if mut == "no_scale" else scale) * (q[b, h] @ k[b, h].T)
            if causal:
                i = np.arange(N)[:, None]
                j = np.arange(N)[None, :]
                bad = {"mask_reversed": j < i, "mask_no_diag": j >= i}.get(mut, j > i)
                s = np.where(bad, -np.inf, s)
            m = 0.0 if mut == "no_max_sub" else s.max(1, keepdims=True)
            with np.errstate(over="ignore", invalid="ignore"):
                f = np.exp(s - m)
                l = f.sum(1, keepdims=True)
                p = f / l
            if mut == "p_transposed":
                p = p.T
            o[b, h] = p @ (k[b, h] if mut == "uses_k_not_v" else v[b, h])
            with np.errstate(divide="ignore", invalid="ignore"):
                ll = (m + np.log(l))[:, 0]
            lse[b, h] = ll / np.log(2) if mut == "lse_base2" else ll
    return o, lse


FWD_MUTANTS = ["no_scale", "mask_reversed", "mask_no_diag", "no_max_sub", "p_transposed",
               "uses_k_not_v", "lse_base2"]


def _bwd_variant(q, k, v, g, scale, causal, mut):
    B, H, N, d = q.shape
    dq, dk, dv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
    delta = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            s = scale * (q[b, h] @ k[b, h].T)
            if causal:
                s = np.where(np.arange(N)[None, :] > np.arange(N)[:, None], -np.inf, s)
            p = np.exp(s - s.max(1, keepdims=True))
            p /= p.sum(1, keepdims=True)
            dp = g[b, h] @ v[b, h].T
            dl = (p * dp).sum(1)
            ds = p * dp if mut == "no_delta_term" else p * (dp - dl[:, None])
            dq[b, h] = scale * ds @ k[b, h]
            dk[b, h] = (1.0 if mut == "dk_no_scale" else scale) * ds.T @ q[b, h]
            dv[b, h] = (p @ g[b, h]) if mut == "dv_no_transpose" else p.T @ g[b, h]
            if mut == "dq_uses_q":
                dq[b, h] = scale * ds @ q[b, h]
            delta[b, h] = dl
    return dq, dk, dv, delta


BWD_MUTANTS = ["no_delta_term", "dk_no_scale", "dv_no_transpose", "dq_uses_q"]


def _fails_some(pins):
    failed = []
    for name, run in pins:
        try:
            run()
        except (AssertionError, ValueError, FloatingPointError):
            failed.append(name)
    return failed


def test_unmutated_variants_pass():
    fwd = lambda q, k, v, s, c: _fwd_variant(q, k, v, s, c, None)  # noqa: E731
    bwd = lambda q, k, v, g, s, c: _bwd_variant(q, k, v, g, s, c, None)  # noqa: E731
    for pin in P.FWD_PINS:
        pin(fwd)
    P.pin_finite_differences(oracle.attn_fwd, bwd)
    P.pin_gradient_sums(bwd)
    P.pin_torch_autograd(bwd)


@pytest.mark.parametrize("mut", FWD_MUTANTS)
def test_forward_mutant_is_caught(mut):
    fwd = lambda q, k, v, s, c: _fwd_variant(q, k, v, s, c, mut)  # noqa: E731
    pins = [(p.__name__, (lambda p=p: p(fwd))) for p in P.FWD_PINS]
    pins.append(("bruteforce", lambda: P.pin_bruteforce_fwd(fwd, oracle.attn_fwd_bruteforce)))
    assert _fails_some(pins), f"mutant {mut} passed every forward pin"


@pytest.mark.parametrize("mut", BWD_MUTANTS)
def test_backward_mutant_is_caught(mut):
    bwd = lambda q, k, v, g, s, c: _bwd_variant(q, k, v, g, s, c, mut)  # noqa: E731
    pins = [
        ("fd", lambda: P.pin_finite_differences(oracle.attn_fwd, bwd)),
        ("sums", lambda: P.pin_gradient_sums(bwd)),
        ("autograd", lambda: P.pin_torch_autograd(bwd)),
    ]
    assert _fails_some(pins), f"mutant {mut} passed every backward pin"


def test_fd_alone_catches_every_backward_mutant():
    """Calculus alone (no library) already rejects each backward mutant."""
    for mut in BWD_MUTANTS:
        bwd = lambda q, k, v, g, s, c, mut=mut: _bwd_variant(q, k, v, g, s, c, mut)  # noqa: E731
        with pytest.raises(AssertionError):
            P.pin_finite_differences(oracle.attn_fwd, bwd)


# ---------------------------------------------------------------------------
# grouped-query attention: plausible mistakes in the head map or the group sum
# ---------------------------------------------------------------------------

def _gqa_variant(mut):
    """(fwd, bwd) of grouped-query attention built on the MHA oracle, with one
    planted mistake."""
    def kv_of(h, H, Hkv):
        return h % Hkv if mut == "head_map_modulo" else h // (H // Hkv)

    def fwd(q, k, v, s, c):
        B, H, N, _ = q.shape
        o, lse = np.empty_like(q), np.empty((B, H, N))
        for h in range(H):
            g = kv_of(h, H, k.shape[1])
            oh, lh = oracle.attn_fwd(q[:, h:h + 1], k[:, g:g + 1], v[:, g:g + 1], s, c)
            o[:, h], lse[:, h] = oh[:, 0], lh[:, 0]
        return o, lse

    def bwd(q, k, v, go, s, c):
        B, H, N, _ = q.shape
        dq, dk, dv, de = np.empty_like(q), np.zeros_like(k), np.zeros_like(v), np.empty((B, H, N))
        for h in range(H):
            g = kv_of(h, H, k.shape[1])
            a, b, cc, e = oracle.attn_bwd(q[:, h:h + 1], k[:, g:g + 1], v[:, g:g + 1], go[:, h:h + 1], s, c)
            dq[:, h], de[:, h] = a[:, 0], e[:, 0]
            if mut == "group_last_head_only":
                dk[:, g], dv[:, g] = b[:, 0], cc[:, 0]
            elif mut == "group_mean":
                G = H // k.shape[1]
                dk[:, g] += b[:, 0] / G
                dv[:, g] += cc[:, 0] / G
            else:
                dk[:, g] += b[:, 0]
                dv[:, g] += cc[:, 0]
        return dq, dk, dv, de
    return fwd, bwd


GQA_MUTANTS = ["head_map_modulo", "group_last_head_only", "group_mean"]


def test_gqa_unmutated_variant_passes():
    fwd, bwd = _gqa_variant(None)
    P.pin_gqa_torch_sdpa(fwd)
    P.pin_gqa_bruteforce(fwd, oracle.attn_fwd_bruteforce)
    P.pin_gqa_autograd(bwd)
    P.pin_gqa_identical_heads(bwd)


@pytest.mark.parametrize("mut", GQA_MUTANTS)
def test_gqa_mutant_is_caught(mut):
    fwd, bwd = _gqa_variant(mut)
    pins = [("sdpa", lambda: P.pin_gqa_torch_sdpa(fwd)),
            ("brute", lambda: P.pin_gqa_bruteforce(fwd, oracle.attn_fwd_bruteforce)),
            ("autograd", lambda: P.pin_gqa_autograd(bwd)),
            ("fd", lambda: P.pin_gqa_finite_differences(fwd, bwd)),
            ("identical", lambda: P.pin_gqa_identical_heads(bwd))]
    assert _fails_some(pins), f"mutant {mut} passed every GQA pin"


# ---------------------------------------------------------------------------
# decode and the split merge
# ---------------------------------------------------------------------------

def _decode_variant(mut):
    from oracle import decode as D

    def decode(q, k, v, scale, kv_lens=None):
        lens = None if mut == "lens_ignored" else kv_lens
        if mut == "head_map_modulo":
            B, H, d = q.shape
            Hkv = k.shape[1]
            o, lse = np.zeros((B, H, d)), np.full((B, H), -np.inf)
            for h in range(H):
                oh, lh = D.attn_decode(q[:, h:h + 1], k[:, h % Hkv:h % Hkv + 1], v[:, h % Hkv:h % Hkv + 1],
                                       scale, lens)
                o[:, h], lse[:, h] = oh[:, 0], lh[:, 0]
            return o, lse
        return D.attn_decode(q, k, v, scale, lens)

    def merge(o_s, lse_s):
        B, H, S, d = o_s.shape
        o, lse = np.zeros((B, H, d)), np.full((B, H), -np.inf)
        for b in range(B):
            for h in range(H):
                live = np.isfinite(lse_s[b, h])
                if not live.any():
                    continue
                if mut == "merge_unweighted":
                    o[b, h] = o_s[b, h, live].mean(axis=0)
                    lse[b, h] = np.log(np.exp(lse_s[b, h, live]).sum())
                elif mut == "merge_no_max":
                    w = np.exp(lse_s[b, h])
                    o[b, h] = (w @ o_s[b, h]) / w.sum()
                    lse[b, h] = np.log(w.sum())
                elif mut == "merge_lse_is_max":
                    m = lse_s[b, h].max()
                    w = np.exp(lse_s[b, h] - m)
                    o[b, h] = (w @ o_s[b, h]) / w.sum()
                    lse[b, h] = m
                else:
                    return D.merge_partials(o_s, lse_s)
        return o, lse

    def split_merge(q, k, v, scale, n_splits, chunk, kv_lens=None):
        return merge(*D.decode_partials(q, k, v, scale, n_splits, chunk, kv_lens))
    return decode, split_merge


DECODE_MUTANTS = ["lens_ignored", "head_map_modulo", "merge_unweighted", "merge_no_max", "merge_lse_is_max"]


def test_decode_unmutated_variant_passes():
    decode, split_merge = _decode_variant(None)
    P.pin_decode_is_last_causal_row(decode, oracle.attn_fwd_gqa)
    P.pin_decode_torch_sdpa(decode)
    P.pin_decode_closed_forms(decode)
    P.pin_split_merge(split_merge, oracle.attn_decode)


@pytest.mark.parametrize("mut", DECODE_MUTANTS)
def test_decode_mutant_is_caught(mut):
    decode, split_merge = _decode_variant(mut)
    pins = [("last_row", lambda: P.pin_decode_is_last_causal_row(decode, oracle.attn_fwd_gqa)),
            ("sdpa", lambda: P.pin_decode_torch_sdpa(decode)),
            ("closed", lambda: P.pin_decode_closed_forms(decode)),
            ("split", lambda: P.pin_split_merge(split_merge, oracle.attn_decode))]
    with np.errstate(over="ignore", invalid="ignore"):
        assert _fails_some(pins), f"mutant {mut} passed every decode pin"


# ---------------------------------------------------------------------------
# chunked prefill: the alignment of the causal mask
# ---------------------------------------------------------------------------

def _chunk_variant(mut):
    def fwd(q, k, v, scale, causal):
        B, H, Nq, _ = q.shape
        Hkv, Nk = k.shape[1], k.shape[2]
        off = {"top_left": 0, "offset_sign": -(Nk - Nq), "off_by_one": Nk - Nq - 1}.get(mut, Nk - Nq)
        o, lse = np.empty(q.shape[:3] + (v.shape[3],)), np.empty(q.shape[:3])
        for b in range(B):
            for h in range(H):
                g = h // (H // Hkv)
                s = scale * (q[b, h] @ k[b, g].T)
                if causal:
                    s[np.arange(Nk)[None, :] > np.arange(Nq)[:, None] + off] = -np.inf
                m = s.max(1, keepdims=True)
                f = np.exp(s - m)
                o[b, h] = (f / f.sum(1, keepdims=True)) @ v[b, g]
                lse[b, h] = (m + np.log(f.sum(1, keepdims=True)))[:, 0]
        return o, lse
    return fwd


CHUNK_MUTANTS = ["top_left", "offset_sign", "off_by_one"]


def test_chunk_unmutated_variant_passes():
    fwd = _chunk_variant(None)
    P.pin_chunk_is_suffix_of_causal(fwd, oracle.attn_fwd_gqa)
    P.pin_chunk_torch_sdpa(fwd)
    P.pin_chunked_prefill_reassembles(fwd, oracle.attn_fwd_gqa)


@pytest.mark.parametrize("mut", CHUNK_MUTANTS)
def test_chunk_mutant_is_caught(mut):
    fwd = _chunk_variant(mut)
    pins = [("suffix", lambda: P.pin_chunk_is_suffix_of_causal(fwd, oracle.attn_fwd_gqa)),
            ("sdpa", lambda: P.pin_chunk_torch_sdpa(fwd)),
            ("reassemble", lambda: P.pin_chunked_prefill_reassembles(fwd, oracle.attn_fwd_gqa))]
    with np.errstate(invalid="ignore"):
        assert _fails_some(pins), f"mutant {mut} passed every chunk pin"


# ---------------------------------------------------------------------------
# FP8 code book and rounding
# ---------------------------------------------------------------------------

def _e4m3_variant(mut):
    from oracle import fp8 as F

    def decode(codes):
        c = np.asarray(codes, dtype=np.int64)
        sign = np.where(c & 0x80, -1.0, 1.0)
        e = (c >> 3) & 15
        m = (c & 7).astype(np.float64)
        bias = 8.0 if mut == "bias_8" else 7.0
        sub = (1.0 + m / 8.0) * 2.0 ** (1 - bias) if mut == "no_subnormal" else m / 8.0 * 2.0 ** (1 - bias)
        val = np.where(e == 0, sub, (1.0 + m / 8.0) * np.exp2(e - bias))
        val = np.where((c & 0x7F) == 0x7F, np.nan, val)
        return sign * val

    def rnd(x):
        if mut == "ties_away":
            x = np.asarray(x, dtype=np.float64)
            a = np.abs(x)
            e = np.maximum(np.floor(np.log2(np.where(a > 0, a, 1.0))), -6.0)
            step = np.exp2(e - 3.0)
            return np.sign(x) * np.floor(a / step + 0.5) * step
        return F.e4m3_round(x)
    return decode, rnd


E4M3_MUTANTS = ["bias_8", "no_subnormal", "ties_away"]


@pytest.mark.parametrize("mut", E4M3_MUTANTS)
def test_e4m3_mutant_is_caught(mut):
    decode, rnd = _e4m3_variant(mut)
    pins = [("codebook", lambda: P.pin_e4m3_codebook(decode)),
            ("round", lambda: P.pin_e4m3_round(rnd, oracle.e4m3_decode))]
    assert _fails_some(pins), f"mutant {mut} passed every E4M3 pin"
