"""fa_fwd_chunk (through the C ABI) against the fp64 oracle, element by
element: a chunk of Nq queries, the last Nq of Nk positions, with the
causal mask aligned at the bottom-right corner ("Flash Attention:
IO-awareness principle", section on PagedAttention and chunked prefill).
"""
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


# (Nq, Nk): offsets Nk - Nq of 0, 1, 8, 11, 27, 257 (mod 32: 0, 1, 8, 11, 27, 1), one query, one key.
SIZES = [(1, 1), (1, 300), (17, 300), (64, 64), (100, 357), (256, 1000), (300, 301), (513, 700)]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("sizes", SIZES, ids=lambda s: f"{s[0]}of{s[1]}")
def test_small_shapes(sizes, causal, d, dtype):
    fa = _fa()
    Nq, Nk = sizes
    B, H, Hkv = 2, 4, 2
    q, k, v = fa_synth.make_chunk_inputs(B, H, Hkv, Nq, Nk, d, dtype, 9600 + Nq + Nk + d)
    o, lse = fa.fwd_chunk(*P.to_dev(q, k, v), 1 / math.sqrt(d), causal)
    torch.cuda.synchronize()
    ro, rl = oracle.attn_fwd_chunk(P.f64(q), P.f64(k), P.f64(v), 1 / math.sqrt(d), causal)
    ctx = f"Nq={Nq} Nk={Nk} causal={causal} d={d} {dtype}"
    P.compare("O", P.f64(o), ro, P.TOL_OUT[dtype], dtype, ctx)
    P.compare("LSE", P.f64(lse), rl, P.TOL_LSE, dtype, ctx)


@pytest.mark.parametrize("causal", [False, True])
def test_square_chunk_is_the_square_kernel(causal):
    """Nq = Nk runs the same kernel as fa_fwd_gqa: bitwise equal."""
    fa = _fa()
    q, k, v = P.to_dev(*fa_synth.make_chunk_inputs(1, 8, 2, 777, 777, 128, "bf16", 9700))
    a = fa.fwd_chunk(q, k, v, 0.09, causal)
    b = fa.fwd_gqa(q, k, v, 0.09, causal)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_chunks_reassemble_the_prompt():
    """A prompt run chunk by chunk (each chunk against all keys up to its end)
    matches the square causal kernel on the whole prompt, within rounding."""
    fa = _fa()
    q, k, v = P.to_dev(*fa_synth.make_chunk_inputs(1, 4, 4, 1111, 1111, 128, "bf16", 9710))
    full_o, full_l = fa.fwd(q, k, v, 0.09, True)
    torch.cuda.synchronize()
    for c0, c1 in ((0, 300), (300, 301), (301, 837), (837, 1111)):
        o, lse = fa.fwd_chunk(q[:, :, c0:c1].contiguous(), k[:, :, :c1].contiguous(), v[:, :, :c1].contiguous(),
                              0.09, True)
        torch.cuda.synchronize()
        P.compare("O", P.f64(o), P.f64(full_o[:, :, c0:c1]), 2e-2, "bf16", f"chunk [{c0},{c1})")
        P.compare("LSE", P.f64(lse), P.f64(full_l[:, :, c0:c1]), 1e-3, "bf16", f"chunk [{c0},{c1})")


@pytest.mark.parametrize("scale", [-0.2, 0.0, 0.3])
def test_scale_values(scale):
    fa = _fa()
    q, k, v = fa_synth.make_chunk_inputs(1, 4, 2, 200, 650, 128, "bf16", 9720)
    o, lse = fa.fwd_chunk(*P.to_dev(q, k, v), scale, True)
    torch.cuda.synchronize()
    ro, rl = oracle.attn_fwd_chunk(P.f64(q), P.f64(k), P.f64(v), scale, True)
    P.compare("O", P.f64(o), ro, P.TOL_OUT["bf16"], "bf16", f"scale={scale}")
    P.compare("LSE", P.f64(lse), rl, P.TOL_LSE, "bf16", f"scale={scale}")


def test_full_size():
    """The chunked-prefill workload (2048 queries after 14336 cached keys, 64
    query heads on 8 K/V heads, d = 128, bf16) in the launch configuration
    the bench times: sampled rows of three heads against the oracle."""
    fa = _fa()
    w = fa_synth.CHUNK_PREFILL
    Nk = fa_synth.CHUNK_PREFILL_NK
    q, k, v = fa_synth.make_chunk_inputs(w.B, w.H, w.kv_heads, w.N, Nk, w.d, w.dtype, w.seed)
    o, lse = fa.fwd_chunk(*P.to_dev(q, k, v), w.scale, w.causal)
    torch.cuda.synchronize()
    qq, kk, vv = P.f64(q), P.f64(k), P.f64(v)
    rows = P.sample_rows(w.N, 24, seed=w.seed)
    for (b, h) in P.heads_to_check(w.B, w.H, 3, seed=w.seed):
        ro, rl = oracle.attn_fwd_chunk_rows(qq, kk, vv, w.scale, w.causal, [(b, h, i) for i in rows])
        ctx = f"{w.name} head ({b},{h})"
        P.compare("O", P.f64(o[b, h, rows]), ro, P.TOL_OUT[w.dtype], w.dtype, ctx)
        P.compare("LSE", P.f64(lse[b, h, rows]), rl, P.TOL_LSE, w.dtype, ctx)
