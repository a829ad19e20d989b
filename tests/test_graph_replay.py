"""Entry points captured into a HIP graph and replayed.

A caller that launches short problems back to back can capture the C-ABI
calls on its capturing stream (here torch.cuda.CUDAGraph, whose capture
stream is torch's current stream inside the context) and replay them without
the host cost of each launch; the bench times short workloads that way too.
The kernels are deterministic (no atomics, fixed reduction order), so every
replay must reproduce the eager result bit for bit.  The outputs are poisoned
with NaN by eager work between replays, and each replay is synchronised and
checked on its own.
"""
import math

import pytest
import torch

import fa_synth
from tests import parity as P

pytestmark = pytest.mark.gpu

REPLAYS = 4


def _fa():
    import io_aware_exact_03_amd as fa
    return fa


def _capture(fn):
    """Warm fn up on a side stream, then capture one call of it."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _replay_and_check(g, outs, refs, label):
    for rep in range(REPLAYS):
        for t in outs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (t, r) in enumerate(zip(outs, refs)):
            assert torch.equal(t, r), f"{label}: replay {rep}, output {i} differs from the eager call"


# (B, H, N, d, dtype, causal): the key-split short path, the persistent
# 256-query kernel, a ragged causal bf16 case and the fp32 kernel
FWD_CASES = [(4, 8, 512, 64, "f16", False), (4, 8, 2048, 64, "f16", False), (2, 2, 300, 128, "bf16", True),
             (1, 1, 512, 64, "f32", False)]


@pytest.mark.parametrize("B,H,N,d,dtype,causal", FWD_CASES)
def test_fwd_graph_replays(B, H, N, d, dtype, causal):
    fa = _fa()
    q, k, v = P.to_dev(*fa_synth.make_inputs(B, H, N, d, dtype, seed=7600 + N + d))
    scale = 1.0 / math.sqrt(d)
    o_ref, l_ref = fa.fwd(q, k, v, scale, causal)
    o, lse = torch.empty_like(o_ref), torch.empty_like(l_ref)
    g = _capture(lambda: fa.fwd(q, k, v, scale, causal, out=o, lse=lse))
    _replay_and_check(g, (o, lse), (o_ref, l_ref), f"fwd B{B} H{H} N{N} d{d} {dtype} causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
def test_naive_graph_replays(causal):
    fa = _fa()
    q, k, v = P.to_dev(*fa_synth.make_inputs(2, 4, 512, 64, "f16", seed=7610))
    ref = fa.naive_fwd(q, k, v, 0.125, causal)
    outs = tuple(torch.empty_like(t) for t in ref)
    g = _capture(lambda: fa.naive_fwd(q, k, v, 0.125, causal, out=outs[0], lse=outs[1], s_ws=outs[2],
                                      p_ws=outs[3]))
    # S and P past the causal diagonal are not part of the result
    n = 512
    keep = torch.ones((n, n), dtype=torch.bool, device=q.device)
    if causal:
        keep = torch.tril(keep)
    def view(ts):
        return (ts[0], ts[1], ts[2][..., keep], ts[3][..., keep])
    for rep in range(REPLAYS):
        for t in outs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (t, r) in enumerate(zip(view(outs), view(ref))):
            assert torch.equal(t, r), f"naive causal={causal}: replay {rep}, output {i} differs"


def test_bwd_graph_replays():
    fa = _fa()
    q, k, v, do = P.to_dev(*fa_synth.make_inputs(2, 4, 700, 128, "bf16", seed=7620, with_dout=True))
    o, lse = fa.fwd(q, k, v, 0.09, True)
    ref = fa.bwd(q, k, v, o, do, lse, 0.09, True)  # (dq, dk, dv, delta)
    dq, dk, dv, delta = (torch.empty_like(t) for t in ref)
    g = _capture(lambda: fa.bwd(q, k, v, o, do, lse, 0.09, True, delta=delta, dq=dq, dk=dk, dv=dv))
    _replay_and_check(g, (dq, dk, dv, delta), ref, "bwd B2 H4 N700 d128 bf16 causal")
