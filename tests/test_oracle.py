"""The fp64 oracle against its pins (CPU only).

Page tags: [triton] "Triton 06: Flash Attention v2" (wonbeomjang.kr);
[review] "Paper review: FlashAttention ... with IO-Awareness"
(osehyeon.github.io); [essay] "Flash Attention: IO-awareness principle"
(hrletsgo.me).
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import attention as A
from tests import oracle_pins as P

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("pin", P.FWD_PINS, ids=lambda f: f.__name__)
def test_forward_pins(pin):
    pin(oracle.attn_fwd)


def test_forward_matches_bruteforce():
    P.pin_bruteforce_fwd(oracle.attn_fwd, oracle.attn_fwd_bruteforce)


def test_row_helper():
    P.pin_rows_helper(oracle.attn_fwd, oracle.attn_fwd_rows)


def test_row_chunking_is_invisible(monkeypatch):
    """Row chunks of the oracle (a memory bound only) do not change results."""
    q, k, v, g = (P.rand((1, 2, 45, 4), s) for s in (1, 2, 3, 4))
    ref = oracle.attn_fwd(q, k, v, 0.5, True)
    refb = oracle.attn_bwd(q, k, v, g, 0.5, True)
    monkeypatch.setattr(A, "ROW_CHUNK", 7)
    got = oracle.attn_fwd(q, k, v, 0.5, True)
    gotb = oracle.attn_bwd(q, k, v, g, 0.5, True)
    for a, b in zip(ref + refb, got + gotb):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def test_finite_differences():
    P.pin_finite_differences(oracle.attn_fwd, oracle.attn_bwd)


def test_delta_identity():
    P.pin_delta_identity(oracle.attn_fwd, oracle.attn_bwd)


def test_gradient_sums():
    P.pin_gradient_sums(oracle.attn_bwd)


def test_torch_autograd():
    P.pin_torch_autograd(oracle.attn_bwd)


def test_backward_matches_bruteforce():
    P.pin_bruteforce_bwd(oracle.attn_bwd, oracle.attn_bwd_bruteforce)


# ---------------------------------------------------------------------------
# tiled models of the algorithm: equal to the definition (decomposition
# identity of [review] 'Tiling'; online update of [essay] 'Tiling')
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n", [1, 2, 3, 16, 33])
def test_online_models_equal_definition(n, causal):
    q, k, v = (P.rand((1, 2, n, 4), 200 + n + s) for s in range(3))
    o, lse = oracle.attn_fwd(q, k, v, 0.45, causal)
    for bm in (1, 2, 5, 8):
        for bn in (1, 2, 5, 8):
            o1, l1 = oracle.online_fa1(q, k, v, 0.45, causal, bm, bn)
            o2, l2 = oracle.online_fa2(q, k, v, 0.45, causal, bm, bn)
            np.testing.assert_allclose(o1, o, rtol=0, atol=1e-12)
            np.testing.assert_allclose(l1, lse, rtol=0, atol=1e-12)
            np.testing.assert_allclose(o2, o, rtol=0, atol=1e-12)
            np.testing.assert_allclose(l2, lse, rtol=0, atol=1e-12)


def test_online_fa2_stage_plan_and_trace():
    """Causal FA2 visits stage-1 blocks, then the diagonal block(s), and never a
    block entirely in the future; l starts at 1 yet ends as the true sum."""
    n, bm, bn = 40, 8, 4
    q, k, v = (P.rand((1, 1, n, 3), 300 + s) for s in range(3))
    tr = []
    oracle.online_fa2(q, k, v, 1.0, True, bm, bn, trace=tr)
    for i in range(-(-n // bm)):
        visited = [(j, st) for (ii, j, st, _, _) in tr if ii == i]
        assert [j for j, _ in visited] == list(range(len(visited)))
        for j, st in visited:
            assert j * bn <= min(n, (i + 1) * bm) - 1  # no future block
            assert st == (1 if (j + 1) * bn <= i * bm else 2)
    # non-causal runs every block as stage 3
    tr = []
    oracle.online_fa2(q, k, v, 1.0, False, bm, bn, trace=tr)
    assert {st for (_, _, st, _, _) in tr} == {3}
    assert len(tr) == (-(-n // bm)) * (-(-n // bn))


def test_online_fa1_trace_running_max():
    """FA1's running max m_i never decreases and ends at the row max."""
    n = 12
    q, k, v = (P.rand((1, 1, n, 3), 400 + s) for s in range(3))
    tr = []
    oracle.online_fa1(q, k, v, 1.0, False, 4, 3, trace=tr)
    for i in range(3):
        ms = [m for (ii, _, m, _) in tr if ii == i]
        for a, b in zip(ms, ms[1:]):
            assert np.all(b >= a)
    s = q[0, 0] @ k[0, 0].T
    final = np.concatenate([m for (ii, j, m, _) in tr if j == 3])
    np.testing.assert_allclose(final, s.max(1), rtol=0, atol=1e-12)


def test_fa1_block_sizes():
    """B_c = ceil(M/4d), B_r = min(B_c, d) ([review] Algorithm 1, step 1)."""
    assert oracle.fa1_block_sizes(1000, 16) == (16, 16)     # ceil(1000/64) = 16
    assert oracle.fa1_block_sizes(81920, 128) == (128, 160)  # 160 KB of bf16 at d=128
    assert oracle.fa1_block_sizes(81920, 64) == (64, 320)
    assert oracle.fa1_block_sizes(100, 64) == (1, 1)


def test_causal_stages_golden():
    """The worked example of [triton] 'Improvement 3'."""
    g = json.load(open(os.path.join(GOLDEN, "triton_fa2_causal_stages.json")))
    c0, c1 = g["cases"]
    (a1, b1), (a2, b2) = oracle.causal_stage_ranges(c0["start_m"], c0["block_m"], c0["block_n"], c0["seq"])
    assert list(range(a1, b1)) == c0["stage1"]
    assert list(range(a2, b2)) == c0["stage2"]
    assert b2 == c0["first_skipped"]
    (a1, b1), (a2, b2) = oracle.causal_stage_ranges(c1["start_m"], c1["block_m"], c1["block_n"], c1["seq"])
    assert b1 - a1 == c1["stage1_count"] and b2 - a2 == c1["stage2_count"]
    assert (b2 - a2) / (b2 - a1) == pytest.approx(1 / 64)


def test_causal_stages_cover_exactly_the_allowed_keys():
    """Stage 1 blocks hold only allowed keys for every row of the block;
    stage 2 blocks straddle; every allowed key is in a visited block."""
    for n in (1, 7, 64, 100, 513):
        for bm in (16, 64, 128, 256):
            for bn in (16, 32, 64, 128):
                for i in range(-(-n // bm)):
                    (a1, b1), (a2, b2) = oracle.causal_stage_ranges(i, bm, bn, n)
                    first, last = i * bm, min(n, (i + 1) * bm) - 1
                    for j in range(a1, b1):
                        assert (j + 1) * bn - 1 <= first
                    for j in range(a2, b2):
                        assert j * bn <= last
                    assert b2 * bn > last  # last row's own key is visited
                    assert (b2 * bn) >= last + 1


def test_nonfinite_guard_in_fa1():
    """Rows with no allowed key in a causal block contribute nothing (the
    exp of -inf minus -inf is taken as 0, never NaN)."""
    q, k, v = (P.rand((1, 1, 9, 2), 500 + s) for s in range(3))
    o, lse = oracle.online_fa1(q, k, v, 1.0, True, 9, 2)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))


# Grouped-query attention ([essay], section on serving: GQA / MQA).

def test_gqa_forward_pins():
    P.pin_gqa_torch_sdpa(oracle.attn_fwd_gqa)
    P.pin_gqa_bruteforce(oracle.attn_fwd_gqa, oracle.attn_fwd_bruteforce)


def test_gqa_backward_pins():
    P.pin_gqa_autograd(oracle.attn_bwd_gqa)
    P.pin_gqa_finite_differences(oracle.attn_fwd_gqa, oracle.attn_bwd_gqa)
    P.pin_gqa_identical_heads(oracle.attn_bwd_gqa)


def test_gqa_rows_helper():
    q, k, v, _ = P._gqa_inputs(2, 6, 2, 17, 4, 390)
    for causal in (False, True):
        o, lse = oracle.attn_fwd_gqa(q, k, v, 0.5, causal)
        rows = [(0, 0, 0), (1, 5, 16), (0, 3, 8), (1, 2, 11)]
        ro, rl = oracle.attn_fwd_rows_gqa(q, k, v, 0.5, causal, rows)
        for n, (b, h, i) in enumerate(rows):
            np.testing.assert_allclose(ro[n], o[b, h, i], rtol=0, atol=1e-13)
            np.testing.assert_allclose(rl[n], lse[b, h, i], rtol=0, atol=1e-13)


def test_gqa_rejects_bad_grouping():
    q, k, v, _ = P._gqa_inputs(1, 6, 4, 5, 3, 395)
    with pytest.raises(ValueError):
        oracle.attn_fwd_gqa(q, k, v, 0.5, False)


# Decode ([lesson] "LLM-serving translation"; split merge: [review]'s softmax
# decomposition).

def test_decode_pins():
    P.pin_decode_is_last_causal_row(oracle.attn_decode, oracle.attn_fwd_gqa)
    P.pin_decode_torch_sdpa(oracle.attn_decode)
    P.pin_decode_closed_forms(oracle.attn_decode)


def test_decode_split_pins():
    P.pin_split_merge(oracle.decode_split_merge, oracle.attn_decode)
    P.pin_partials_torch(oracle.decode_partials)


def test_decode_rejects():
    q, k, v = P._decode_inputs(1, 4, 3, 5, 3, 470)
    with pytest.raises(ValueError):
        oracle.attn_decode(q, k, v, 0.5)
    q, k, v = P._decode_inputs(1, 4, 2, 5, 3, 470)
    with pytest.raises(ValueError):
        oracle.attn_decode(q, k, v, 0.5, [6])
    with pytest.raises(ValueError):
        oracle.decode_partials(q, k, v, 0.5, 2, 2)


# Chunked prefill ([essay], section on PagedAttention and chunked prefill).

def test_chunk_pins():
    P.pin_chunk_is_suffix_of_causal(oracle.attn_fwd_chunk, oracle.attn_fwd_gqa)
    P.pin_chunk_torch_sdpa(oracle.attn_fwd_chunk)
    P.pin_chunked_prefill_reassembles(oracle.attn_fwd_chunk, oracle.attn_fwd_gqa)


def test_chunk_rows_helper():
    q, k, v = P._chunk_inputs(2, 4, 2, 9, 30, 4, 540)
    for causal in (False, True):
        o, lse = oracle.attn_fwd_chunk(q, k, v, 0.5, causal)
        rows = [(0, 0, 0), (1, 3, 8), (0, 2, 4)]
        ro, rl = oracle.attn_fwd_chunk_rows(q, k, v, 0.5, causal, rows)
        for n, (b, h, i) in enumerate(rows):
            np.testing.assert_allclose(ro[n], o[b, h, i], rtol=0, atol=1e-13)
            np.testing.assert_allclose(rl[n], lse[b, h, i], rtol=0, atol=1e-13)


def test_chunk_rejects():
    q, k, v = P._chunk_inputs(1, 4, 2, 9, 5, 4, 545)
    with pytest.raises(ValueError):
        oracle.attn_fwd_chunk(q, k, v, 0.5, True)  # causal chunk longer than its keys


# FP8 ([essay] section "FA2/FA3").

def test_fp8_pins():
    P.pin_e4m3_codebook(oracle.e4m3_decode)
    P.pin_e4m3_round(oracle.e4m3_round, oracle.e4m3_decode)
    P.pin_fp8_attention(oracle.attn_fwd_fp8, oracle.attn_fwd_gqa)
    P.pin_p_rounding_bound(oracle.p_rounding_bound, oracle.attn_fwd_fp8_model, oracle.attn_fwd_fp8)


def test_fp8_rows_helper():
    q8, k8, v8, ds = P._fp8_inputs(2, 4, 2, 19, 8, 630)
    for causal in (False, True):
        o, lse = oracle.attn_fwd_fp8(q8, k8, v8, ds, 0.4, causal)
        bnd = oracle.p_rounding_bound(q8, k8, v8, ds, 0.4, causal)
        rows = [(0, 0, 0), (1, 3, 18), (0, 2, 7)]
        ro, rl, rb = oracle.attn_fwd_fp8_rows(q8, k8, v8, ds, 0.4, causal, rows)
        for n, (b, h, i) in enumerate(rows):
            np.testing.assert_allclose(ro[n], o[b, h, i], rtol=0, atol=1e-12)
            np.testing.assert_allclose(rl[n], lse[b, h, i], rtol=0, atol=1e-12)
            np.testing.assert_allclose(rb[n], bnd[b, h, i], rtol=1e-12, atol=1e-15)
