"""fa_bwd (through the C ABI) against the fp64 oracle's textbook-Jacobian
gradients, element by element.

The forward output O and LSE fed to fa_bwd come from fa_fwd (as in
training); the oracle differentiates the exact attention of the same rounded
inputs.  Delta is checked twice: against the oracle's Jacobian-form value
(which tests the rowsum(dO * O) shortcut end to end) and against rowsum of
the very O the kernel read (which isolates the preprocessing kernel).
"""
import math

import numpy as np
import pytest
import torch

import fa_synth
import oracle
from tests import parity as P

pytestmark = pytest.mark.gpu

TOL_GRAD = 2e-2
U_REL = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11}  # relative half-ulp bound of the dtype


def grad_tol(scale: float, d: int) -> float:
    """2e-2 at the workload scale 1/sqrt(d).  The dominant rounding is dS
    (and P) cast to the input dtype before the dQ/dK (dV) products; its
    effect on dQ = scale * dS K is about u * |scale| * |dP| * |K| with |dP|
    growing like sqrt(d), so the bound grows with |scale| * sqrt(d) beyond 1."""
    return TOL_GRAD * max(1.0, abs(scale) * math.sqrt(d) * (1 + 1e-6))


def delta_tol(do, o, dtype):
    """Per-row bound for Delta = rowsum(dO * O) against the exact value: O is
    stored rounded to the dtype, each element off by at most u |O|, so the
    row sum is off by at most u * sum_c |dO_c O_c| (plus fp32 summation)."""
    return U_REL[dtype] * np.abs(P.f64(do) * P.f64(o)).sum(-1) + 1e-3


def _fa():
    import io_aware_exact_03_amd as fa
    return fa


def run_and_check(B, H, N, d, dtype, causal, scale, seed, context, heads=None):
    fa = _fa()
    q, k, v, do = fa_synth.make_inputs(B, H, N, d, dtype, seed=seed, with_dout=True)
    qd, kd, vd, dod = P.to_dev(q, k, v, do)
    o, lse = fa.fwd(qd, kd, vd, scale, causal)
    dq, dk, dv, delta = fa.bwd(qd, kd, vd, o, dod, lse, scale, causal)
    torch.cuda.synchronize()
    for name, t in (("dQ", dq), ("dK", dk), ("dV", dv), ("Delta", delta)):
        assert bool(torch.isfinite(t).all()), f"{context}: non-finite {name}"
    # Delta of the kernel vs rowsum(dO * O) of the O it read
    d_direct = (P.f64(do) * P.f64(o)).sum(-1)
    P.compare("Delta(kernel)", P.f64(delta), d_direct, 1e-4 * max(1.0, float(np.abs(d_direct).max())), "f32", context)
    heads = heads or [(b, h) for b in range(B) for h in range(H)]
    tol = grad_tol(scale, d)
    dtol = delta_tol(do, o.cpu(), dtype)
    for (b, h) in heads:
        sl = (slice(b, b + 1), slice(h, h + 1))
        rdq, rdk, rdv, rdl = oracle.attn_bwd(*(P.f64(t[sl]) for t in (q, k, v, do)), scale, causal)
        ctx = f"{context} head ({b},{h})"
        P.compare("dQ", P.f64(dq[sl]), rdq, tol, "f32", ctx)
        P.compare("dK", P.f64(dk[sl]), rdk, tol, "f32", ctx)
        P.compare("dV", P.f64(dv[sl]), rdv, tol, "f32", ctx)
        err = np.abs(P.f64(delta[sl]) - rdl)
        bad = err > dtol[sl]
        assert not bad.any(), (f"{ctx} Delta(oracle): {int(bad.sum())} rows above the O-rounding bound, "
                               f"worst err {float(err.max()):.3e}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 2, 17, 63, 64, 65, 127, 128, 129, 200, 300, 513])
def test_small_shapes(N, causal, d, dtype):
    run_and_check(2, 2, N, d, dtype, causal, 1 / math.sqrt(d), 9000 + N + d, f"N={N} d={d} causal={causal} {dtype}")


# 0.2 is 2.3x the 1/sqrt(128) scale; far sharper softmaxes make the bf16
# rounding of dS (|dS| ~ sqrt(d)) the whole error, which grad_tol models only
# roughly.
@pytest.mark.parametrize("scale", [-0.2, 0.0, 0.2])
@pytest.mark.parametrize("causal", [False, True])
def test_scale_values(scale, causal):
    run_and_check(1, 3, 333, 128, "bf16", causal, scale, 9100, f"scale={scale} causal={causal}")


def test_many_heads():
    run_and_check(3, 5, 700, 64, "f16", True, 0.125, 9200, "B3 H5 N700")


def test_noncausal_many_items():
    """Non-causal forward and backward with more work items than CUs (B8 H64
    N512 d128: 1024 forward and dQ items, 2048 dK/dV items over the
    persistent grids), so workgroups walk several items and change K/V (or
    query) block between them; sampled whole heads against the oracle."""
    run_and_check(8, 64, 512, 128, "bf16", False, 1 / math.sqrt(128), 9250, "B8 H64 N512 non-causal",
                  heads=P.heads_to_check(8, 64, 4, seed=9250))


def test_deterministic():
    fa = _fa()
    q, k, v, do = P.to_dev(*fa_synth.make_inputs(2, 4, 1000, 128, "bf16", seed=9300, with_dout=True))
    o, lse = fa.fwd(q, k, v, 0.09, True)
    a = fa.bwd(q, k, v, o, do, lse, 0.09, True)
    b = fa.bwd(q, k, v, o, do, lse, 0.09, True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_fp32_rejected():
    fa = _fa()
    from io_aware_exact_03_amd import _lib
    q, k, v, do = P.to_dev(*fa_synth.make_inputs(1, 1, 64, 64, "f32", seed=1, with_dout=True))
    o, lse = fa.fwd(q, k, v, 0.125, False)
    with pytest.raises(_lib.FaError) as e:
        fa.bwd(q, k, v, o, do, lse, 0.125, False)
    assert e.value.status == 2


def test_train_step_full_size():
    """The causal training-step workload at full size, in the launch
    configuration the bench times; two whole heads against the oracle."""
    w = fa_synth.TRAIN_STEP
    run_and_check(w.B, w.H, w.N, w.d, w.dtype, w.causal, w.scale, w.seed, w.name,
                  heads=P.heads_to_check(w.B, w.H, 2, seed=w.seed))


def test_stages_equal_full_backward():
    """fa_bwd_stage 1, 2, 3 in order reproduce fa_bwd bitwise (the bench
    times the stages one by one)."""
    fa = _fa()
    q, k, v, do = P.to_dev(*fa_synth.make_inputs(1, 3, 777, 128, "bf16", seed=9400, with_dout=True))
    o, lse = fa.fwd(q, k, v, 0.088, True)
    ref = fa.bwd(q, k, v, o, do, lse, 0.088, True)
    outs = [torch.full_like(t, float("nan")) for t in ref]
    dq, dk, dv, delta = outs
    for s in (1, 2, 3):
        fa.bwd_stage(s, q, k, v, o, do, lse, 0.088, True, delta, dq, dk, dv)
    torch.cuda.synchronize()
    for a, b in zip(ref, outs):
        assert torch.equal(a, b)
