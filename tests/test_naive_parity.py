"""fa_naive_fwd (three kernels, S and P in memory) against the fp64 oracle.

Besides O and LSE, the stored S and P are checked against the definition:
S = scale * Q K^T (rounded to the workspace dtype) and P = softmax(S) with
causal zeros."""
import math

import numpy as np
import pytest
import torch

import fa_synth
import oracle
from tests import parity as P

pytestmark = pytest.mark.gpu


def _fa():
    import io_aware_exact_03_amd as fa
    return fa


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 7, 64, 65, 200, 513])
def test_small(N, causal, d, dtype):
    fa = _fa()
    q, k, v = fa_synth.make_inputs(2, 2, N, d, dtype, seed=8000 + N)
    scale = 1 / math.sqrt(d)
    o, lse, s, p = fa.naive_fwd(*P.to_dev(q, k, v), scale, causal)
    torch.cuda.synchronize()
    ctx = f"naive N={N} d={d} causal={causal} {dtype}"
    P.check_fwd_full(q, k, v, o, lse, scale, causal, dtype, ctx, lse_tol=P.naive_lse_tol(q, k, scale, dtype))
    qq, kk = P.f64(q), P.f64(k)
    s_ref = scale * np.einsum("bhid,bhjd->bhij", qq, kk)
    ws = "f32" if dtype == "f32" else "f16"
    P.compare("S", P.f64(s), s_ref, max(1e-5, 2 * P.half_ulp(np.abs(s_ref).max(), ws)), ws, ctx)
    # P against the oracle's own O with V = I: the oracle's probabilities
    eye = np.broadcast_to(np.eye(N), (2, 2, N, N)).copy()
    p_ref, _ = oracle.attn_fwd(qq, kk, eye, scale, causal)
    P.compare("P", P.f64(p), p_ref, 1e-5 if dtype == "f32" else 2e-3, ws, ctx)
    if causal:
        assert float(torch.triu(p.float(), 1).abs().max()) == 0.0


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1000, 2056])
def test_vector_paths(N, causal, d, dtype):
    """Row lengths that are multiples of eight take the 16-byte kernels: the
    staged S writer (tiles of 128 x 128, here with a partial last tile), the
    vector softmax with a wave per row (N <= 2048) or the workgroup per row
    (N > 2048).  O, LSE and S are compared element by element; P through
    the oracle's probabilities where the V = I product stays small."""
    fa = _fa()
    q, k, v = fa_synth.make_inputs(1, 2, N, d, dtype, seed=8100 + N + d)
    scale = 1 / math.sqrt(d)
    o, lse, s, p = fa.naive_fwd(*P.to_dev(q, k, v), scale, causal)
    torch.cuda.synchronize()
    ctx = f"naive vector N={N} d={d} causal={causal} {dtype}"
    P.check_fwd_full(q, k, v, o, lse, scale, causal, dtype, ctx, lse_tol=P.naive_lse_tol(q, k, scale, dtype))
    qq, kk = P.f64(q), P.f64(k)
    s_ref = scale * np.einsum("bhid,bhjd->bhij", qq, kk)
    P.compare("S", P.f64(s), s_ref, max(1e-5, 2 * P.half_ulp(np.abs(s_ref).max(), "f16")), "f16", ctx)
    if N <= 1000:
        eye = np.broadcast_to(np.eye(N), (1, 2, N, N)).copy()
        p_ref, _ = oracle.attn_fwd(qq, kk, eye, scale, causal)
        P.compare("P", P.f64(p), p_ref, 2e-3, "f16", ctx)
    if causal:
        assert float(torch.triu(p.float(), 1).abs().max()) == 0.0
    rows = torch.isfinite(p.float()).all()
    assert bool(rows)


@pytest.mark.parametrize("w", fa_synth.NONCAUSAL_SWEEP + (fa_synth.LONG_CAUSAL,), ids=lambda w: w.name)
def test_full_size_sampled(w):
    fa = _fa()
    q, k, v = fa_synth.workload_inputs(w, with_dout=False)
    o, lse, s, p = fa.naive_fwd(*P.to_dev(q, k, v), w.scale, w.causal)
    torch.cuda.synchronize()
    del s, p
    assert bool(torch.isfinite(o).all())
    o, lse = o.cpu(), lse.cpu()
    heads = P.heads_to_check(w.B, w.H, 2, seed=w.seed)
    rows = P.sample_rows(w.N, 32, seed=w.seed)
    P.check_fwd_sampled(q, k, v, o, lse, w.scale, w.causal, w.dtype, heads, rows, "naive " + w.name,
                        lse_tol=P.naive_lse_tol(q, k, w.scale, w.dtype, heads, rows))
