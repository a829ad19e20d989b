"""fa_fwd_fp8 (E4M3 inputs, through the C ABI) against the fp64 oracle:
attention of the dequantised codes, with O allowed the error that rounding
the weights to E4M3 can add (a per-element bound the oracle computes and
its own pins check) plus the bf16 output rounding; LSE uses unrounded
weights and keeps the 16-bit paths' 1e-3.
"""
import math

import numpy as np
import pytest
import torch

import fa_synth
import oracle
from tests import parity as P

pytestmark = pytest.mark.gpu

OUT_REL = 2.0 ** -8   # bf16 output rounding (half an ulp is 2^-9) with slack
OUT_ABS = 1e-4        # fp32 accumulation


def _fa():
    import io_aware_exact_03_amd as fa
    return fa


def _np(t):
    return t.numpy()


def lse_tol(q8, k8, ds, scale):
    """1e-3, widened for large logits: each score is an fp32 sum of d exact
    products (E4M3 x E4M3 is exact in fp32), off by at most about
    d 2^-24 sum_c |q_c k_c|, times |scale|; the LSE is 1-Lipschitz in the
    scores."""
    q = np.abs(oracle.dequantize(q8, ds[0]))
    k = np.abs(oracle.dequantize(k8, ds[1]))
    d = q.shape[-1]
    qa = q.max(axis=(0, 1))  # [N, d] envelope over heads
    ka = k.max(axis=(0, 1))
    return P.TOL_LSE + abs(scale) * float((qa @ ka.T).max()) * d * 2.0 ** -24


def check(o, lse, ro, rl, bnd, ctx, ltol=P.TOL_LSE):
    go = P.f64(o)
    err = np.abs(go - ro)
    allowed = bnd + OUT_REL * np.abs(ro) + OUT_ABS
    bad = err > allowed
    if bad.any():
        idx = np.unravel_index(int(np.argmax(err - allowed)), err.shape)
        raise AssertionError(f"{ctx}: {int(bad.sum())} elements beyond the E4M3 bound; worst at {idx}: gpu "
                             f"{go[idx]:.6g} oracle {ro[idx]:.6g} err {err[idx]:.3e} allowed {allowed[idx]:.3e}")
    P.compare("LSE", P.f64(lse), rl, ltol, "f32", ctx)
    return float((err / allowed).max())


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 17, 64, 65, 128, 129, 300, 513])
def test_small_shapes(N, causal, d):
    fa = _fa()
    B, H, Hkv = 2, 4, 2
    scale = 1 / math.sqrt(d)
    q8, k8, v8, ds = fa_synth.make_fp8_inputs(B, H, Hkv, N, d, seed=9900 + N + d)
    o, lse = fa.fwd_fp8(*P.to_dev(q8, k8, v8), ds, scale, causal)
    torch.cuda.synchronize()
    a = (_np(q8), _np(k8), _np(v8), ds, scale, causal)
    ro, rl = oracle.attn_fwd_fp8(*a)
    check(o, lse, ro, rl, oracle.p_rounding_bound(*a), f"N={N} causal={causal} d={d}",
          lse_tol(_np(q8), _np(k8), ds, scale))


@pytest.mark.parametrize("scale", [-0.3, 0.0, 0.4])
def test_scale_values(scale):
    """Sharper and flatter softmaxes (and a negative scale), with wider inputs."""
    fa = _fa()
    q8, k8, v8, ds = fa_synth.make_fp8_inputs(1, 4, 4, 333, 128, seed=9910, sigma=2.0)
    o, lse = fa.fwd_fp8(*P.to_dev(q8, k8, v8), ds, scale, True)
    torch.cuda.synchronize()
    a = (_np(q8), _np(k8), _np(v8), ds, scale, True)
    ro, rl = oracle.attn_fwd_fp8(*a)
    check(o, lse, ro, rl, oracle.p_rounding_bound(*a), f"scale={scale}", lse_tol(_np(q8), _np(k8), ds, scale))


def test_close_to_bf16_path():
    """On the same dequantised values the FP8 and bf16 forwards agree to the
    E4M3 weight rounding (loose: a mean, not a bound)."""
    fa = _fa()
    q8, k8, v8, ds = fa_synth.make_fp8_inputs(2, 4, 4, 1000, 128, seed=9920)
    o8, l8 = fa.fwd_fp8(*P.to_dev(q8, k8, v8), ds, 0.09, True)
    deq = [(t.view(torch.float8_e4m3fn).float() * s).to(torch.bfloat16).cuda() for t, s in zip((q8, k8, v8), ds)]
    o16, l16 = fa.fwd(*deq, 0.09, True)
    torch.cuda.synchronize()
    diff = (o8.float() - o16.float()).abs()
    assert float(diff.mean()) < 2e-2 * float(o16.float().abs().mean()) + 1e-3, float(diff.mean())
    assert float((l8 - l16).abs().max()) < 2e-2


def test_full_size():
    """The FP8 causal prefill workload (B2 H32 N8192 d128) in the launch
    configuration the bench times: sampled rows of three heads."""
    fa = _fa()
    w = fa_synth.FP8_PREFILL
    q8, k8, v8, ds = fa_synth.make_fp8_inputs(w.B, w.H, w.H, w.N, w.d, seed=w.seed)
    o, lse = fa.fwd_fp8(*P.to_dev(q8, k8, v8), ds, w.scale, w.causal)
    torch.cuda.synchronize()
    qn, kn, vn = _np(q8), _np(k8), _np(v8)
    rows = P.sample_rows(w.N, 24, seed=w.seed)
    for (b, h) in P.heads_to_check(w.B, w.H, 3, seed=w.seed):
        ro, rl, rb = oracle.attn_fwd_fp8_rows(qn, kn, vn, ds, w.scale, w.causal, [(b, h, i) for i in rows])
        check(o[b, h, rows], lse[b, h, rows], ro, rl, rb, f"{w.name} head ({b},{h})",
              lse_tol(qn[b:b + 1, h:h + 1], kn[b:b + 1, h:h + 1], ds, w.scale))


def test_deterministic():
    fa = _fa()
    q8, k8, v8, ds = fa_synth.make_fp8_inputs(1, 8, 2, 1500, 128, seed=9930)
    q8, k8, v8 = P.to_dev(q8, k8, v8)
    a = fa.fwd_fp8(q8, k8, v8, ds, 0.09, True)
    b = fa.fwd_fp8(q8, k8, v8, ds, 0.09, True)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def _codes(x):
    """E4M3 codes (uint8) of a float tensor, round to nearest even."""
    return x.to(torch.float8_e4m3fn).view(torch.uint8)


@pytest.mark.parametrize("pattern", ["rising", "plateau"])
@pytest.mark.parametrize("causal", [False, True])
def test_reference_raises(pattern, causal):
    """Score patterns that drive the lazy reference: 'rising' scores grow
    along the keys, so the reference is raised again and again (O and l
    rescaled, weights redone); 'plateau' keeps every key after the first
    tile 1 nat above the first tile's maximum, so each tile's four-weight
    sums exceed 448 (the byte test runs) while no weight overflows (no
    raise).  Q is all ones, every K row constant, so score j is
    scale * d * t_j exactly."""
    fa = _fa()
    B, H, N, d = 1, 2, 300, 64
    scale = 1.0 / 8
    g = torch.Generator(device="cpu").manual_seed(9940)
    q = torch.ones(B, H, N, d)
    if pattern == "rising":
        t = torch.linspace(0.0, 2.0, N)
    else:
        t = torch.full((N,), 0.125)
        t[:64] = 0.0
    k = t.view(1, 1, N, 1).expand(B, H, N, d).contiguous()
    v = torch.randn(B, H, N, d, generator=g)
    q8, k8, v8 = _codes(q), _codes(k), _codes(v)
    ds = (1.0, 1.0, 1.0)
    o, lse = fa.fwd_fp8(*P.to_dev(q8, k8, v8), ds, scale, causal)
    torch.cuda.synchronize()
    a = (_np(q8), _np(k8), _np(v8), ds, scale, causal)
    ro, rl = oracle.attn_fwd_fp8(*a)
    check(o, lse, ro, rl, oracle.p_rounding_bound(*a), f"{pattern} causal={causal}",
          lse_tol(_np(q8), _np(k8), ds, scale))
