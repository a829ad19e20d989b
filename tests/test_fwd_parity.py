"""fa_fwd (through the C ABI) against the fp64 oracle, element by element.

Small shapes span several tiles with ragged tails and are compared in full;
the full-size workloads (the shapes the bench times) are compared on sampled
heads and rows, which the oracle computes one row at a time.
"""
import math

import numpy as np
import pytest
import torch

import fa_synth
from tests import parity as P

pytestmark = pytest.mark.gpu

DTYPES = ["f32", "f16", "bf16"]
SMALL_N = [1, 2, 3, 15, 16, 17, 31, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257, 300, 513, 1000]


def _fa():
    import io_aware_exact_03_amd as fa
    return fa


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", SMALL_N)
def test_small_shapes(N, causal, d, dtype):
    fa = _fa()
    q, k, v = fa_synth.make_inputs(2, 2, N, d, dtype, seed=7000 + N + d)
    scale = 1.0 / math.sqrt(d)
    o, lse = fa.fwd(*P.to_dev(q, k, v), scale, causal)
    torch.cuda.synchronize()
    P.check_fwd_full(q, k, v, o, lse, scale, causal, dtype, f"N={N} d={d} causal={causal} {dtype}")


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 17, 65, 129, 300, 513])
def test_small_shapes_persistent_kernel(N, causal, d, dtype):
    """Short sequences with enough heads (B2 H128) that the 256-query
    persistent kernel (16-bit) or the 128-query fp32 kernel has at least one
    work item per CU and serves them (with fewer heads the key-split kernels
    do): ragged tails, the masked sub-block, several heads per workgroup;
    sampled whole heads."""
    fa = _fa()
    q, k, v = fa_synth.make_inputs(2, 128, N, d, dtype, seed=7050 + N + d)
    scale = 1.0 / math.sqrt(d)
    o, lse = fa.fwd(*P.to_dev(q, k, v), scale, causal)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    for (b, h) in P.heads_to_check(2, 128, 3, seed=7050 + N):
        sl = (slice(b, b + 1), slice(h, h + 1))
        P.check_fwd_full(q[sl], k[sl], v[sl], o[sl], lse[sl], scale, causal, dtype,
                         f"B2 H128 head ({b},{h}) N={N} d={d} causal={causal} {dtype}")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("causal", [False, True])
def test_many_heads_grid_order(dtype, causal):
    """B*H not a multiple of 8 and several query blocks per head: every
    workgroup renumbering lands on a distinct (head, block)."""
    fa = _fa()
    q, k, v = fa_synth.make_inputs(3, 5, 700, 64, dtype, seed=7101)
    o, lse = fa.fwd(*P.to_dev(q, k, v), 0.125, causal)
    torch.cuda.synchronize()
    P.check_fwd_full(q, k, v, o, lse, 0.125, causal, dtype, f"B3 H5 N700 {dtype}")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("scale", [-0.3, 0.0, 2.0])
@pytest.mark.parametrize("d,N", [(128, 333), (64, 333), (128, 200)])
def test_scale_values(dtype, scale, d, N):
    """Negative scale (folded into the sign of Q), zero scale (uniform
    weights) and a large scale (sharp softmax); with two heads, d = 128 at
    N = 333 runs the persistent kernel and the other two shapes the
    key-split one (16-bit types)."""
    fa = _fa()
    for causal in (False, True):
        q, k, v = fa_synth.make_inputs(1, 2, N, d, dtype, seed=7200)
        o, lse = fa.fwd(*P.to_dev(q, k, v), scale, causal)
        torch.cuda.synchronize()
        P.check_fwd_full(q, k, v, o, lse, scale, causal, dtype, f"scale={scale} d={d} N={N} causal={causal} {dtype}")


@pytest.mark.parametrize("dtype", DTYPES)
def test_closed_forms(dtype):
    """Closed forms on the GPU: constant V gives O = c; Q = 0 gives the mean
    of the allowed V rows with LSE = ln(#keys); one dominant key gives its V
    row (logits near 1e3 must not overflow)."""
    fa = _fa()
    N, d = 200, 64
    dt = fa_synth.DTYPES[dtype]
    q, k, v = fa_synth.make_inputs(1, 2, N, d, dtype, seed=7300)
    c = torch.linspace(-3, 3, d).to(dt)
    vc = c.expand(1, 2, N, d).contiguous()
    for causal in (False, True):
        o, lse = fa.fwd(*P.to_dev(q, k, vc), 0.125, causal)
        torch.cuda.synchronize()
        P.compare("O(const V)", P.f64(o), np.broadcast_to(P.f64(c), (1, 2, N, d)), P.TOL_OUT[dtype], dtype)
        qz = torch.zeros_like(q)
        o, lse = fa.fwd(*P.to_dev(qz, k, v), 0.125, causal)
        torch.cuda.synchronize()
        vv = P.f64(v)
        if causal:
            ref = np.cumsum(vv, axis=2) / np.arange(1, N + 1)[None, None, :, None]
            rl = np.broadcast_to(np.log(np.arange(1, N + 1)), (1, 2, N))
        else:
            ref = np.broadcast_to(vv.mean(axis=2, keepdims=True), vv.shape)
            rl = np.full((1, 2, N), math.log(N))
        P.compare("O(Q=0)", P.f64(o), ref, P.TOL_OUT[dtype], dtype)
        P.compare("LSE(Q=0)", P.f64(lse), rl, P.TOL_LSE, dtype)
    # one dominant key: logits 1000 vs 0
    qo = torch.ones(1, 1, 64, d).to(dt)
    ko = torch.zeros(1, 1, 64, d).to(dt)
    ko[0, 0, 5] = 1.0
    vo = fa_synth.make_inputs(1, 1, 64, d, dtype, seed=7301)[2]
    o, lse = fa.fwd(*P.to_dev(qo, ko, vo), 1000.0 / d, False)
    torch.cuda.synchronize()
    P.compare("O(dominant)", P.f64(o)[0, 0], np.broadcast_to(P.f64(vo)[0, 0, 5], (64, d)), P.TOL_OUT[dtype], dtype)
    P.compare("LSE(dominant)", P.f64(lse), np.full((1, 1, 64), 1000.0), P.TOL_LSE, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_deterministic(dtype):
    """Two runs give bitwise-equal O and LSE (no atomics, fixed order)."""
    fa = _fa()
    q, k, v = P.to_dev(*fa_synth.make_inputs(2, 4, 1500, 128, dtype, seed=7400))
    o1, l1 = fa.fwd(q, k, v, 0.09, True)
    o2, l2 = fa.fwd(q, k, v, 0.09, True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_single_head_f32_full():
    """The fp32 single-head workload, compared in full at 1e-5."""
    fa = _fa()
    w = fa_synth.SINGLE_HEAD_F32
    q, k, v = fa_synth.workload_inputs(w)
    o, lse = fa.fwd(*P.to_dev(q, k, v), w.scale, w.causal)
    torch.cuda.synchronize()
    P.check_fwd_full(q, k, v, o, lse, w.scale, w.causal, w.dtype, w.name)


@pytest.mark.parametrize("w", fa_synth.NONCAUSAL_SWEEP + (fa_synth.CAUSAL_PREFILL, fa_synth.LONG_CAUSAL,
                                                          fa_synth.TRAIN_STEP, fa_synth.NONCAUSAL_PREFILL,
                                                          fa_synth.NONCAUSAL_LONG), ids=lambda w: w.name)
def test_full_size_sampled(w):
    """Full-size workloads in the launch configuration the bench times:
    sampled heads and rows against the oracle, and every output finite."""
    fa = _fa()
    q, k, v = fa_synth.workload_inputs(w, with_dout=False)
    qd, kd, vd = P.to_dev(q, k, v)
    o, lse = fa.fwd(qd, kd, vd, w.scale, w.causal)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    o, lse = o.cpu(), lse.cpu()
    heads = P.heads_to_check(w.B, w.H, 3, seed=w.seed)
    rows = P.sample_rows(w.N, 48, seed=w.seed, extra=(w.N - 2, 4095, 4096, 8191, 8192))
    P.check_fwd_sampled(q, k, v, o, lse, w.scale, w.causal, w.dtype, heads, rows, w.name)
