"""fa_decode (through the C ABI) against the fp64 oracle, element by element:
the final O and LSE against the decode definition, and the pieces of cut
units left in the workspace against the definition over each piece's keys.

Decoding is one query per head against a K/V cache ("Flash Attention -- five
lessons converging into 80 lines", "LLM-serving translation"); the splits
are merged with the softmax decomposition of the FlashAttention review.
"""
import math

import numpy as np
import pytest
import torch

import fa_synth
import oracle
from tests import parity as P

pytestmark = pytest.mark.gpu

TOL_O = 2e-2      # as the forward: P is rounded to the input dtype before PV
TOL_LSE = 1e-3
TOL_PIECE_O = 2e-2
TILE = 128  # keys per tile of the documented partition


def _fa():
    import io_aware_exact_03_amd as fa
    return fa


def _run(B, H, Hkv, Nkv, d, dtype, seed, n_parts, lens=None, ragged=False, scale=None):
    fa = _fa()
    q, k, v, gl = fa_synth.make_decode_inputs(B, H, Hkv, Nkv, d, dtype, seed, ragged)
    if lens is None:
        lens = gl
    scale = 1 / math.sqrt(d) if scale is None else scale
    qd, kd, vd = P.to_dev(q, k, v)
    ld = lens.to(torch.int32).cuda()
    ws = None
    need = fa.decode_workspace_bytes(B, H, Hkv, d, n_parts)
    if need:
        ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")  # NaN-filled
    o, lse = fa.decode(qd, kd, vd, scale, kv_lens=ld, n_parts=n_parts, ws=ws)
    torch.cuda.synchronize()
    return q, k, v, lens, scale, o, lse, ws


def _check(q, k, v, lens, scale, o, lse, dtype, ctx):
    lens_c = [min(max(int(x), 0), k.shape[2]) for x in lens]
    ro, rl = oracle.attn_decode(P.f64(q), P.f64(k), P.f64(v), scale, lens_c)
    P.compare("O", P.f64(o), ro, TOL_O, dtype, ctx)
    gl = P.f64(lse)
    assert np.array_equal(np.isneginf(gl), np.isneginf(rl)), f"{ctx}: -inf LSE rows differ"
    fin = np.isfinite(rl)
    P.compare("LSE", gl[fin], rl[fin], TOL_LSE, dtype, ctx)


GROUPS = [(2, 8, 2), (1, 4, 1), (3, 6, 6), (1, 64, 8), (2, 48, 1)]  # G = 4, MQA, G = 1, G = 8, G = 48 (2 blocks)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Nkv", [1, 100, 700])
@pytest.mark.parametrize("n_parts", [1, 3, 40])
@pytest.mark.parametrize("grp", GROUPS, ids=lambda g: f"B{g[0]}H{g[1]}Hkv{g[2]}")
def test_small_shapes(grp, n_parts, Nkv, d, dtype):
    B, H, Hkv = grp
    ctx = f"B={B} H={H} Hkv={Hkv} Nkv={Nkv} d={d} parts={n_parts} {dtype}"
    res = _run(B, H, Hkv, Nkv, d, dtype, 9900 + Nkv + d + H, n_parts, ragged=True)
    _check(*res[:7], dtype, ctx)


def cut_pieces(lens, H, Hkv, n_parts):
    """The documented partition: units (b, K/V head, block of 32 query heads)
    own ceil(L_b / 128) tiles each, laid end to end and cut into n_parts
    ranges of ceil(T / n_parts) tiles.  Yields (slot, b, hkv, qb, k0, k1) for
    every piece of a unit that was cut."""
    G = H // Hkv
    QB = (G + 31) // 32
    units, P = [], 0
    for b, L in enumerate(lens):
        nb = (L + TILE - 1) // TILE
        for ui in range(Hkv * QB):
            units.append((b * Hkv * QB + ui, b, ui, P, nb, L))
            P += nb
    per = (P + n_parts - 1) // n_parts
    for u, b, ui, P_u, nb, L in units:
        if nb == 0 or P_u // per == (P_u + nb - 1) // per:
            continue
        for w in range(P_u // per, (P_u + nb - 1) // per + 1):
            t0, t1 = max(P_u, w * per), min(P_u + nb, (w + 1) * per)
            yield w + u, b, ui // QB, ui % QB, (t0 - P_u) * TILE, min((t1 - P_u) * TILE, L)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("n_parts", [2, 5, 16, 100])
def test_pieces_match_oracle(n_parts, d):
    """The workspace after the call holds, for every unit cut between parts,
    each piece's O (normalised within the piece) and LSE: checked against
    the decode definition over exactly that piece's keys."""
    fa = _fa()
    B, H, Hkv, Nkv = 3, 8, 2, 900
    lens = torch.tensor([900, 257, 1], dtype=torch.int32)
    q, k, v, lens, scale, o, lse, ws = _run(B, H, Hkv, Nkv, d, "bf16", 9950 + n_parts, n_parts, lens=lens)
    go, gl = (P.f64(t) for t in fa.decode_pieces(ws, B, H, Hkv, d, n_parts))
    qq, kk, vv = P.f64(q), P.f64(k), P.f64(v)
    G = H // Hkv
    n_cut = 0
    for slot, b, hkv, qb, k0, k1 in cut_pieces(lens.tolist(), H, Hkv, n_parts):
        heads = list(range(hkv * G + 32 * qb, min(hkv * G + 32 * qb + 32, (hkv + 1) * G)))
        ro, rl = oracle.attn_decode(qq[b:b + 1, heads], kk[b:b + 1, hkv:hkv + 1, k0:k1],
                                    vv[b:b + 1, hkv:hkv + 1, k0:k1], scale)
        ctx = f"parts={n_parts} d={d} slot={slot} b={b} hkv={hkv} keys [{k0},{k1})"
        P.compare("piece O", go[slot, :len(heads)], ro[0], TOL_PIECE_O, "f32", ctx)
        P.compare("piece LSE", gl[slot, :len(heads)], rl[0], TOL_LSE, "f32", ctx)
        n_cut += 1
    assert n_cut > 0
    _check(q, k, v, lens, scale, o, lse, "bf16", f"parts={n_parts} d={d}")


def test_plan_is_used_by_default():
    fa = _fa()
    B, H, Hkv, Nkv, d = 1, 64, 8, 4096, 128
    n_parts = fa.decode_plan(B, H, Hkv, Nkv, d)
    props = torch.cuda.get_device_properties(0)
    assert n_parts == min(props.multi_processor_count, B * Hkv * (Nkv // TILE))
    q, k, v, lens = fa_synth.make_decode_inputs(B, H, Hkv, Nkv, d, "bf16", 9960)
    o, lse = fa.decode(*P.to_dev(q, k, v), 0.088)
    torch.cuda.synchronize()
    _check(q, k, v, lens, 0.088, o, lse, "bf16", f"plan parts={n_parts}")
    assert fa.decode_plan(1, 8, 8, 100, 128) == 8  # never more parts than tiles


@pytest.mark.parametrize("n_parts", [1, 4, 64])
def test_lengths_edge_cases(n_parts):
    """Length 0 (O = 0, LSE = -inf), 1, a tile boundary, the whole cache, and
    out-of-range values clamped to [0, Nkv]."""
    lens = torch.tensor([0, 1, 128, 129, 640, 1000, -5], dtype=torch.int32)
    res = _run(7, 4, 2, 640, 128, "bf16", 9970, n_parts, lens=lens)
    _check(*res[:7], "bf16", f"lengths parts={n_parts}")
    o = res[5]
    assert bool((o[0] == 0).all()) and bool((o[6] == 0).all())


@pytest.mark.parametrize("n_parts", [1, 5])
def test_no_valid_key_anywhere(n_parts):
    """Every length 0 (or negative): no part has work, the first workgroup
    writes O = 0 and LSE = -inf for every head."""
    lens = torch.tensor([0, -3, 0], dtype=torch.int32)
    res = _run(3, 8, 2, 256, 128, "bf16", 9980, n_parts, lens=lens)
    o, lse = res[5], res[6]
    assert bool((o == 0).all())
    assert bool(torch.isneginf(lse).all())


@pytest.mark.parametrize("n_parts", [1, 7, 200])
def test_many_batches(n_parts):
    """More batches than a wave has lanes: the workgroups locate their
    ranges 64 batches at a time, so empty batches and ranges that start or
    end on either side of a 64-batch boundary must all come out right."""
    g = torch.Generator().manual_seed(9975)
    lens = torch.randint(1, 301, (150,), generator=g, dtype=torch.int32)
    for b in (0, 63, 64, 65, 127, 128, 149):
        lens[b] = 0
    lens[62] = 300
    lens[129] = 1
    res = _run(150, 2, 1, 300, 64, "bf16", 9976, n_parts, lens=lens)
    _check(*res[:7], "bf16", f"B150 parts={n_parts}")


@pytest.mark.parametrize("n_parts", [1, 3])
def test_rows_past_the_length_are_never_read(n_parts):
    """Cache rows at and beyond each length hold NaN; the result is finite and
    equals the oracle's on the valid rows."""
    fa = _fa()
    B, H, Hkv, Nkv, d = 2, 8, 2, 500, 128
    q, k, v, _ = fa_synth.make_decode_inputs(B, H, Hkv, Nkv, d, "bf16", 9980)
    lens = torch.tensor([131, 377], dtype=torch.int32)
    kn, vn = k.clone(), v.clone()
    for b, n in enumerate(lens.tolist()):
        kn[b, :, n:] = float("nan")
        vn[b, :, n:] = float("nan")
    o, lse = fa.decode(*P.to_dev(q, kn, vn), 0.1, kv_lens=lens.cuda(), n_parts=n_parts)
    torch.cuda.synchronize()
    _check(q, k, v, lens, 0.1, o, lse, "bf16", f"NaN tail parts={n_parts}")


@pytest.mark.parametrize("scale", [-0.3, 0.0, 0.4])
def test_scale_values(scale):
    res = _run(2, 8, 2, 333, 128, "bf16", 9990, 3, ragged=True, scale=scale)
    _check(*res[:7], "bf16", f"scale={scale}")


@pytest.mark.parametrize("w", [fa_synth.GQA_DECODE, fa_synth.GQA_DECODE_RAGGED], ids=lambda w: w.name)
def test_full_size(w):
    """The decode workloads at full size in the launch configuration the
    bench times (the library's part plan), every head against the oracle."""
    fa = _fa()
    q, k, v, lens = fa_synth.make_decode_inputs(w.B, w.H, w.kv_heads, w.N, w.d, w.dtype, w.seed,
                                                ragged="ragged" in w.name)
    qd, kd, vd = P.to_dev(q, k, v)
    o, lse = fa.decode(qd, kd, vd, w.scale, kv_lens=lens.cuda())
    torch.cuda.synchronize()
    _check(q, k, v, lens, w.scale, o, lse, w.dtype, w.name)


def test_deterministic():
    fa = _fa()
    q, k, v, lens = fa_synth.make_decode_inputs(4, 16, 4, 3000, 128, "bf16", 9995, ragged=True)
    qd, kd, vd = P.to_dev(q, k, v)
    a = fa.decode(qd, kd, vd, 0.09, kv_lens=lens.cuda(), n_parts=37)
    b = fa.decode(qd, kd, vd, 0.09, kv_lens=lens.cuda(), n_parts=37)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
