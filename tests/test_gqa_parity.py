"""fa_fwd_gqa / fa_bwd_gqa (through the C ABI) against the fp64 oracle's
grouped-query attention, element by element, plus identities at full size.

Grouped-query attention is the head sharing that "Flash Attention:
IO-awareness principle" names in its section on serving: H query heads per
batch share Hkv K/V heads, query head h reading K/V head h // (H // Hkv).
"""
import math

import numpy as np
import pytest
import torch

import fa_synth
import oracle
from tests import parity as P
from tests.test_bwd_parity import grad_tol

pytestmark = pytest.mark.gpu


def _fa():
    import io_aware_exact_03_amd as fa
    return fa


def _inputs(B, H, Hkv, N, d, dtype, seed, with_dout=True):
    return fa_synth.make_inputs(B, H, N, d, dtype, seed=seed, with_dout=with_dout, Hkv=Hkv)


# (B, H, Hkv): groups of 2 and 4, MQA (one K/V head), and G = 1 through the
# grouped entry points.
GROUPS = [(2, 4, 2), (1, 8, 2), (1, 4, 1), (2, 3, 3)]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 17, 130, 300])
@pytest.mark.parametrize("grp", GROUPS, ids=lambda g: f"B{g[0]}H{g[1]}Hkv{g[2]}")
def test_small_shapes(grp, N, causal, d, dtype):
    fa = _fa()
    B, H, Hkv = grp
    scale = 1 / math.sqrt(d)
    ctx = f"B={B} H={H} Hkv={Hkv} N={N} d={d} causal={causal} {dtype}"
    q, k, v, do = _inputs(B, H, Hkv, N, d, dtype, 9500 + N + d + H + Hkv)
    qd, kd, vd, dod = P.to_dev(q, k, v, do)
    o, lse = fa.fwd_gqa(qd, kd, vd, scale, causal)
    dq, dk, dv, delta = fa.bwd_gqa(qd, kd, vd, o, dod, lse, scale, causal)
    torch.cuda.synchronize()
    assert dk.shape == k.shape and dv.shape == v.shape and dq.shape == q.shape
    qq, kk, vv, gg = (P.f64(t) for t in (q, k, v, do))
    ro, rl = oracle.attn_fwd_gqa(qq, kk, vv, scale, causal)
    P.compare("O", P.f64(o), ro, P.TOL_OUT[dtype], dtype, ctx)
    P.compare("LSE", P.f64(lse), rl, P.TOL_LSE, dtype, ctx)
    rdq, rdk, rdv, _ = oracle.attn_bwd_gqa(qq, kk, vv, gg, scale, causal)
    # dK and dV sum G heads' contributions, so their rounding grows with G.
    G = H // Hkv
    tol = grad_tol(scale, d)
    P.compare("dQ", P.f64(dq), rdq, tol, "f32", ctx)
    P.compare("dK", P.f64(dk), rdk, tol * math.sqrt(G), "f32", ctx)
    P.compare("dV", P.f64(dv), rdv, tol * math.sqrt(G), "f32", ctx)


@pytest.mark.parametrize("causal", [False, True])
def test_f32_forward(causal):
    fa = _fa()
    q, k, v = _inputs(1, 6, 2, 150, 64, "f32", 9600, with_dout=False)
    o, lse = fa.fwd_gqa(*P.to_dev(q, k, v), 0.125, causal)
    torch.cuda.synchronize()
    ro, rl = oracle.attn_fwd_gqa(P.f64(q), P.f64(k), P.f64(v), 0.125, causal)
    P.compare("O", P.f64(o), ro, P.out_tol("f32", q, k, 0.125), "f32", f"f32 causal={causal}")
    P.compare("LSE", P.f64(lse), rl, P.TOL_LSE, "f32", f"f32 causal={causal}")


def _repeat(t, G):
    return t.repeat_interleave(G, dim=1).contiguous()


def test_matches_mha_on_repeated_heads():
    """Forward O, LSE and the backward's dQ, Delta are bitwise those of the
    one-K/V-head-per-query-head path run on K, V repeated G times; dK and dV
    equal the group sums of that path's per-head gradients to fp32 rounding."""
    fa = _fa()
    B, H, Hkv, N, d = 2, 8, 2, 517, 128
    G = H // Hkv
    q, k, v, do = P.to_dev(*_inputs(B, H, Hkv, N, d, "bf16", 9700))
    for causal in (False, True):
        o, lse = fa.fwd_gqa(q, k, v, 0.09, causal)
        dq, dk, dv, delta = fa.bwd_gqa(q, k, v, o, do, lse, 0.09, causal)
        kr, vr = _repeat(k, G), _repeat(v, G)
        o2, lse2 = fa.fwd(q, kr, vr, 0.09, causal)
        dq2, dk2, dv2, delta2 = fa.bwd(q, kr, vr, o2, do, lse2, 0.09, causal)
        torch.cuda.synchronize()
        assert torch.equal(o, o2) and torch.equal(lse, lse2)
        assert torch.equal(dq, dq2) and torch.equal(delta, delta2)
        dk_sum = dk2.view(B, Hkv, G, N, d).sum(2)
        dv_sum = dv2.view(B, Hkv, G, N, d).sum(2)
        for name, a, b in (("dK", dk, dk_sum), ("dV", dv, dv_sum)):
            err = float((a - b).abs().max())
            ref = float(b.abs().max())
            assert err <= 1e-4 * max(1.0, ref), f"{name} causal={causal}: {err:.3e} vs group sum (max {ref:.3e})"


def test_full_size_prefill():
    """The grouped-query prefill workload at full size (64 query heads on 8
    K/V heads, N = 8192, d = 128, causal bf16), in the launch configuration
    the bench times: forward rows sampled against the oracle; dQ of the
    first 1200 rows of one head against the oracle; dK and dV through
    identities that hold at any size (sum_j dK_j = 0; sum_j dV_j = the sum of
    dO over the group's query heads and rows) and against the group sums of
    the per-head path run on repeated K/V."""
    fa = _fa()
    w = fa_synth.GQA_PREFILL
    q, k, v, do = fa_synth.workload_inputs(w)
    qd, kd, vd, dod = P.to_dev(q, k, v, do)
    o, lse = fa.fwd_gqa(qd, kd, vd, w.scale, w.causal)
    dq, dk, dv, _ = fa.bwd_gqa(qd, kd, vd, o, dod, lse, w.scale, w.causal)
    torch.cuda.synchronize()
    G = w.H // w.kv_heads
    heads = P.heads_to_check(w.B, w.H, 3, seed=w.seed)
    rows = P.sample_rows(w.N, 24, seed=w.seed)
    qq, kk, vv, gg = (P.f64(t) for t in (q, k, v, do))
    for (b, h) in heads:
        sel = [(b, h, i) for i in rows]
        ro, rl = oracle.attn_fwd_rows_gqa(qq, kk, vv, w.scale, w.causal, sel)
        ctx = f"{w.name} head ({b},{h})"
        P.compare("O", P.f64(o[b, h, rows]), ro, P.TOL_OUT[w.dtype], w.dtype, ctx)
        P.compare("LSE", P.f64(lse[b, h, rows]), rl, P.TOL_LSE, w.dtype, ctx)
    # dQ rows: the oracle's gradient on the query head, restricted to rows.
    b, h = heads[0]
    g = h // G
    sub = slice(0, 1200)  # causal: rows < 1200 see keys < 1200 only
    rdq, _, _, _ = oracle.attn_bwd(qq[b:b + 1, h:h + 1, sub], kk[b:b + 1, g:g + 1, sub], vv[b:b + 1, g:g + 1, sub],
                                   gg[b:b + 1, h:h + 1, sub], w.scale, w.causal)
    P.compare("dQ rows < 1200", P.f64(dq[b:b + 1, h:h + 1, sub]), rdq, grad_tol(w.scale, w.d), "f32", w.name)
    dk_sum = P.f64(dk).sum(axis=2)
    dv_sum = P.f64(dv).sum(axis=2)
    do_sum = gg.sum(axis=2).reshape(w.B, w.kv_heads, G, w.d).sum(axis=2)
    assert np.abs(dk_sum).max() <= 2e-2 * math.sqrt(w.N * G), f"sum_j dK_j: {np.abs(dk_sum).max():.3e}"
    assert np.abs(dv_sum - do_sum).max() <= 2e-2 * math.sqrt(w.N * G), \
        f"sum_j dV_j - sum dO: {np.abs(dv_sum - do_sum).max():.3e}"
    # dK, dV against the group sums of the per-head path on repeated K/V
    # (that path is checked against the oracle on its own tests).
    del qq, kk, vv, gg
    kr, vr = _repeat(kd, G), _repeat(vd, G)
    o2, lse2 = fa.fwd(qd, kr, vr, w.scale, w.causal)
    _, dk2, dv2, _ = fa.bwd(qd, kr, vr, o2, dod, lse2, w.scale, w.causal)
    torch.cuda.synchronize()
    for name, a, b2 in (("dK", dk, dk2), ("dV", dv, dv2)):
        ref = b2.view(w.B, w.kv_heads, G, w.N, w.d).sum(2)
        err = float((a - ref).abs().max())
        assert err <= 1e-4 * max(1.0, float(ref.abs().max())), f"{name} vs group sum: {err:.3e}"


def _whole_kv_head(B, H, Hkv, N, d, causal, seed, b, g, context):
    """fwd_gqa + bwd_gqa on the whole problem; one whole K/V head's dK, dV
    and its G query heads' dQ against oracle.attn_bwd_gqa on that slice."""
    fa = _fa()
    q, k, v, do = _inputs(B, H, Hkv, N, d, "bf16", seed)
    qd, kd, vd, dod = P.to_dev(q, k, v, do)
    scale = 1 / math.sqrt(d)
    o, lse = fa.fwd_gqa(qd, kd, vd, scale, causal)
    dq, dk, dv, _ = fa.bwd_gqa(qd, kd, vd, o, dod, lse, scale, causal)
    torch.cuda.synchronize()
    G = H // Hkv
    hs = slice(g * G, (g + 1) * G)
    sl_q = (slice(b, b + 1), hs)
    sl_k = (slice(b, b + 1), slice(g, g + 1))
    rdq, rdk, rdv, _ = oracle.attn_bwd_gqa(P.f64(q[sl_q]), P.f64(k[sl_k]), P.f64(v[sl_k]), P.f64(do[sl_q]), scale,
                                           causal)
    tol = grad_tol(scale, d)
    P.compare("dK", P.f64(dk[sl_k]), rdk, tol * math.sqrt(G), "f32", context)
    P.compare("dV", P.f64(dv[sl_k]), rdv, tol * math.sqrt(G), "f32", context)
    P.compare("dQ", P.f64(dq[sl_q]), rdq, tol, "f32", context)
    ro, rl = oracle.attn_fwd_gqa(P.f64(q[sl_q]), P.f64(k[sl_k]), P.f64(v[sl_k]), scale, causal)
    P.compare("O", P.f64(o[sl_q]), ro, P.TOL_OUT["bf16"], "bf16", context)
    P.compare("LSE", P.f64(lse[sl_q]), rl, P.TOL_LSE, "bf16", context)


def test_whole_kv_head_many_segments():
    """Eight query heads per K/V head at N = 2048 (causal): each dK/dV work
    item walks eight segments back to back, with the next segment's Q/dO
    loads issued across the segment boundary."""
    _whole_kv_head(1, 16, 2, 2048, 128, True, 9700, 0, 1, "B1 H16 Hkv2 N2048 causal, K/V head 1")


def test_whole_kv_head_many_items():
    """More grouped dK/dV work items than CUs (128 K/V heads x 4 pair items
    at N = 1024), so every workgroup walks two items; the last K/V head is
    compared whole."""
    _whole_kv_head(16, 32, 8, 1024, 128, True, 9710, 15, 7, "B16 H32 Hkv8 N1024 causal, K/V head (15, 7)")


def test_deterministic():
    fa = _fa()
    q, k, v, do = P.to_dev(*_inputs(1, 8, 2, 1000, 128, "bf16", 9800))
    o, lse = fa.fwd_gqa(q, k, v, 0.09, True)
    a = fa.bwd_gqa(q, k, v, o, do, lse, 0.09, True)
    b = fa.bwd_gqa(q, k, v, o, do, lse, 0.09, True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
