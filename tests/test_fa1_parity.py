"""fa_fwd_fa1 (the FlashAttention-1 loop order, through the C ABI) against
the fp64 oracle: the output against the attention definition, and the
running state left in the workspace against the oracle's executable model
of the review's Algorithm 1 with the same block sizes (64 keys, 128
queries).
"""
import math

import numpy as np
import pytest
import torch

import fa_synth
import oracle
from tests import parity as P

pytestmark = pytest.mark.gpu

LOG2E = 1.0 / math.log(2.0)


def _fa():
    import io_aware_exact_03_amd as fa
    return fa


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 17, 64, 65, 128, 129, 300, 513])
def test_small_shapes(N, causal, d, dtype):
    fa = _fa()
    B, H = 2, 2
    scale = 1 / math.sqrt(d)
    q, k, v = fa_synth.make_inputs(B, H, N, d, dtype, seed=9800 + N + d)
    ws = torch.full((fa.fa1_workspace_bytes(B, H, N, d),), 0xFF, dtype=torch.uint8, device="cuda")
    o, lse = fa.fwd_fa1(*P.to_dev(q, k, v), scale, causal, ws=ws)
    torch.cuda.synchronize()
    qq, kk, vv = P.f64(q), P.f64(k), P.f64(v)
    ctx = f"N={N} causal={causal} d={d} {dtype}"
    ro, rl = oracle.attn_fwd(qq, kk, vv, scale, causal)
    P.compare("O", P.f64(o), ro, P.TOL_OUT[dtype], dtype, ctx)
    P.compare("LSE", P.f64(lse), rl, P.TOL_LSE, dtype, ctx)
    # The final running state against Algorithm 1's model (same blocks).
    trace = []
    mo, ml = oracle.online_fa1(qq, kk, vv, scale, causal, br=128, bc=64, trace=trace)
    go, gm, gl = (P.f64(t) for t in fa.fa1_state(ws, B, H, N, d))
    P.compare("O (fp32 state)", go, mo, P.TOL_OUT[dtype], "f32", ctx)
    # m is the row max of scale * S in log2 units; l the sum of exp(s - m)
    row_max = np.stack([np.stack([(scale * (qq[b, h] @ kk[b, h].T) +
                                   (np.where(np.arange(N)[None, :] > np.arange(N)[:, None], -np.inf, 0.0)
                                    if causal else 0.0)).max(axis=1) for h in range(H)]) for b in range(B)])
    P.compare("m", gm, row_max * LOG2E, 1e-3 * max(1.0, float(np.abs(row_max).max())), "f32", ctx)
    P.compare("l", np.log(gl), ml - row_max, 1e-3, "f32", ctx)


def test_matches_fused_forward():
    """Same result as the FA2-order kernel, within rounding."""
    fa = _fa()
    q, k, v = P.to_dev(*fa_synth.make_inputs(2, 4, 1000, 128, "bf16", seed=9810))
    for causal in (False, True):
        a = fa.fwd_fa1(q, k, v, 0.09, causal)
        b = fa.fwd(q, k, v, 0.09, causal)
        torch.cuda.synchronize()
        P.compare("O", P.f64(a[0]), P.f64(b[0]), 2e-2, "bf16", f"causal={causal}")
        P.compare("LSE", P.f64(a[1]), P.f64(b[1]), 1e-3, "bf16", f"causal={causal}")


@pytest.mark.parametrize("scale", [-0.2, 0.0, 0.3])
def test_scale_values(scale):
    fa = _fa()
    q, k, v = fa_synth.make_inputs(1, 2, 333, 128, "bf16", seed=9820)
    o, lse = fa.fwd_fa1(*P.to_dev(q, k, v), scale, True)
    torch.cuda.synchronize()
    ro, rl = oracle.attn_fwd(P.f64(q), P.f64(k), P.f64(v), scale, True)
    P.compare("O", P.f64(o), ro, P.TOL_OUT["bf16"], "bf16", f"scale={scale}")
    P.compare("LSE", P.f64(lse), rl, P.TOL_LSE, "bf16", f"scale={scale}")
