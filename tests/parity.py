"""Helpers that compare the HIP path with the fp64 oracle element by element.

The GPU receives the dtype-rounded inputs; the oracle receives exactly those
values upcast to float64 (fa_synth.to_f64), so the comparison measures the
kernels' arithmetic only.  A failure message names the worst element, the
oracle value there and the output dtype's rounding floor at that magnitude,
so rounding can be told apart from a bug.

Tolerances (max |gpu - oracle|): O, dQ, dK, dV 1e-5 for fp32 inputs and
2e-2 for fp16/bf16; LSE 1e-3 for every dtype.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import fa_synth
import oracle

TOL_OUT = {"f32": 1e-5, "f16": 2e-2, "bf16": 2e-2}
TOL_LSE = 1e-3
MANT_BITS = {"f32": 23, "f16": 10, "bf16": 7}


def half_ulp(x: float, dtype: str) -> float:
    x = abs(x)
    if x == 0.0:
        return 0.0
    return 2.0 ** (math.floor(math.log2(x)) - MANT_BITS[dtype] - 1)


def compare(name: str, got, ref, tol: float, dtype: str, context: str = ""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, f"{name}: shape {got.shape} vs {ref.shape}"
    if not np.all(np.isfinite(got)):
        bad = np.argwhere(~np.isfinite(got))[0]
        raise AssertionError(f"{context} {name}: non-finite value at {tuple(bad)}")
    if got.size == 0:
        return 0.0
    diff = np.abs(got - ref)
    idx = np.unravel_index(int(np.argmax(diff)), diff.shape)
    err = float(diff[idx])
    assert err <= tol, (f"{context} {name}: max abs err {err:.3e} > {tol:.1e} at {idx}; oracle {ref[idx]:.6g}, "
                        f"gpu {got[idx]:.6g}, output rounding floor {half_ulp(ref[idx], dtype):.2e}")
    return err


def to_dev(*ts):
    return [t.cuda() for t in ts]


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def sample_rows(N: int, count: int, seed: int, extra=()):
    """Rows at both ends, at tile boundaries and at random."""
    rng = np.random.default_rng(seed)
    base = {0, 1, N - 1, N // 2}
    for b in (31, 32, 63, 64, 127, 128, 255, 256, 511, 512):
        for r in (b - 1, b, b + 1):
            if 0 <= r < N:
                base.add(r)
    base.update(r for r in extra if 0 <= r < N)
    rest = rng.choice(N, size=min(N, max(0, count - len(base))), replace=False)
    return sorted(base.union(int(r) for r in rest))


def heads_to_check(B: int, H: int, count: int, seed: int):
    rng = np.random.default_rng(seed)
    allh = [(b, h) for b in range(B) for h in range(H)]
    pick = {allh[0], allh[-1]}
    for i in rng.choice(len(allh), size=min(len(allh), count), replace=False):
        pick.add(allh[int(i)])
    return sorted(pick)[:max(count, 2)]


EPS32 = 2.0 ** -23


def out_tol(dtype: str, q=None, k=None, scale: float = 0.0) -> float:
    """Output tolerance.  16-bit: 2e-2.  fp32: 1e-5, widened only when the
    scaled logits are large: an fp32 dot product of length d carries an error
    of order eps32 * sum_c |q_c k_c|, which exp turns into a relative error of
    the weights of |scale| times that.  The widening is 1 (no change) while
    |scale| * max_ij sum_c |q_ic k_jc| <= 16, which holds for the fp32
    single-head workload (scale 1/8, d = 64)."""
    if dtype != "f32" or q is None:
        return TOL_OUT[dtype]
    qa = np.abs(f64(q)).max(axis=(0, 1))  # [N, d] envelope over heads
    ka = np.abs(f64(k)).max(axis=(0, 1))
    bound = abs(scale) * float((qa @ ka.T).max())
    return TOL_OUT["f32"] * max(1.0, bound / 16.0)


def check_fwd_full(q, k, v, o, lse, scale, causal, dtype, context="", lse_tol=TOL_LSE):
    ro, rl = oracle.attn_fwd(f64(q), f64(k), f64(v), scale, causal)
    e1 = compare("O", f64(o), ro, out_tol(dtype, q, k, scale), dtype, context)
    e2 = compare("LSE", f64(lse), rl, lse_tol, dtype, context)
    return e1, e2


def check_fwd_sampled(q, k, v, o, lse, scale, causal, dtype, heads, rows, context="", lse_tol=TOL_LSE):
    """O and LSE at the given (b, h) heads and row indices, one row at a time."""
    worst = (0.0, 0.0)
    for (b, h) in heads:
        qh, kh, vh = (f64(t[b:b + 1, h:h + 1]) for t in (q, k, v))
        ro, rl = oracle.attn_fwd_rows(qh, kh, vh, scale, causal, [(0, 0, i) for i in rows])
        go = f64(o[b, h, rows])
        gl = f64(lse[b, h, rows])
        e1 = compare("O", go, ro, TOL_OUT[dtype], dtype, f"{context} head ({b},{h})")
        e2 = compare("LSE", gl, rl, lse_tol, dtype, f"{context} head ({b},{h})")
        worst = (max(worst[0], e1), max(worst[1], e2))
    return worst


def naive_lse_tol(q, k, scale, dtype, heads=None, rows=None) -> float:
    """The naive path stores S in float16 for 16-bit inputs; LSE is
    1-Lipschitz in the logits (max norm), so its error grows by at most half
    an fp16 ulp of the largest |S| the rows see."""
    if dtype == "f32":
        return TOL_LSE
    qq, kk = f64(q), f64(k)
    if heads is None:
        smax = float(np.abs(scale * np.einsum("bhid,bhjd->bhij", qq, kk)).max())
    else:
        smax = max(float(np.abs(scale * (qq[b, h, rows] @ kk[b, h].T)).max()) for (b, h) in heads)
    return TOL_LSE + half_ulp(smax, "f16")


def workload_tensors(w: fa_synth.Workload, with_dout=None):
    return fa_synth.workload_inputs(w, with_dout)
