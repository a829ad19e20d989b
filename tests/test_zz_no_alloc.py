"""fa_decode_noalloc: the decode step for callers that cannot allocate, with
the pieces of cut units in the library's fixed per-device scratch buffer.

Through the C ABI it must give exactly what fa_decode gives with a caller
workspace (same kernels, same partition, deterministic), on two calls in a
row, the second smaller than the first (the buffer then still holds the
first call's pieces, which must not leak into the second), and the first is
also held to the decode oracle.  Requests beyond the buffer are refused on
the host."""
import ctypes
import math

import numpy as np
import pytest
import torch

import fa_synth
import oracle
from tests import parity as P

FA_OK, FA_ERR_ARG, FA_ERR_SCRATCH = 0, 1, 5
A = 4096  # a 16-byte aligned fake address; never dereferenced on rejected calls


def _lib():
    from io_aware_exact_03_amd import _lib as L
    return L.load()


def test_noalloc_rejects_beyond_scratch():
    lib = _lib()
    from io_aware_exact_03_amd import _lib as L
    # 64 x 64 K/V heads with 1024 parts: 5120 slots of 32 x 128 fp32 = 84 MB
    B, H, Hkv, d, parts = 64, 64, 64, 128, 1024
    assert lib.fa_decode_workspace_bytes(B, H, Hkv, d, parts) > L.DECODE_SCRATCH_BYTES
    assert lib.fa_decode_noalloc(A, A, A, None, A, A, B, H, Hkv, 4096, d, 0.1, parts, 2, None) == FA_ERR_SCRATCH
    # one part needs no scratch at all; argument errors as fa_decode
    assert lib.fa_decode_noalloc(None, A, A, None, A, A, 1, 8, 1, 64, 64, 0.1, 1, 2, None) == FA_ERR_ARG
    assert lib.fa_decode_noalloc(A, A, A, None, A, A, 1, 8, 3, 64, 64, 0.1, 1, 2, None) == FA_ERR_ARG
    assert lib.fa_decode_noalloc(A, A, A, None, A, A, 1, 8, 1, 64, 64, 0.1, 2000, 2, None) == FA_ERR_ARG


def _call_both(B, H, Hkv, Nkv, d, dtype, seed, n_parts):
    import io_aware_exact_03_amd as fa
    lib = _lib()
    q, k, v, lens = fa_synth.make_decode_inputs(B, H, Hkv, Nkv, d, dtype, seed, ragged=True)
    qd, kd, vd = P.to_dev(q, k, v)
    ld = lens.to(torch.int32).cuda()
    scale = 1 / math.sqrt(d)
    need = fa.decode_workspace_bytes(B, H, Hkv, d, n_parts)
    assert need > 0, "the case must cut units"
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    o_ref, lse_ref = fa.decode(qd, kd, vd, scale, kv_lens=ld, n_parts=n_parts, ws=ws)
    o = torch.full_like(qd, float("nan"))
    lse = torch.full((B, H), float("nan"), dtype=torch.float32, device="cuda")
    st = lib.fa_decode_noalloc(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), ld.data_ptr(), o.data_ptr(),
                               lse.data_ptr(), B, H, Hkv, Nkv, d, ctypes.c_float(scale), n_parts,
                               fa.DTYPE_CODES[qd.dtype], ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == FA_OK, st
    torch.cuda.synchronize()
    return q, k, v, lens, scale, o, lse, o_ref, lse_ref


@pytest.mark.gpu
def test_noalloc_matches_workspace_entry_point_twice():
    print("[no_alloc] call 1: B2 H16 Hkv2 Nkv3000 d128 bf16, 64 parts", flush=True)
    q, k, v, lens, scale, o, lse, o_ref, lse_ref = _call_both(2, 16, 2, 3000, 128, "bf16", 9301, 64)
    assert torch.equal(o, o_ref), "O differs from fa_decode's"
    assert torch.equal(lse, lse_ref), "LSE differs from fa_decode's"
    ro, rl = oracle.attn_decode(P.f64(q), P.f64(k), P.f64(v), scale, [int(x) for x in lens])
    P.compare("O", P.f64(o), ro, 2e-2, "bf16", "noalloc call 1")
    P.compare("LSE", P.f64(lse), rl, 1e-3, "bf16", "noalloc call 1")
    # a smaller second call: the buffer still holds call 1's pieces
    print("[no_alloc] call 2: B1 H8 Hkv1 Nkv700 d64 f16, 16 parts", flush=True)
    q, k, v, lens, scale, o, lse, o_ref, lse_ref = _call_both(1, 8, 1, 700, 64, "f16", 9302, 16)
    assert torch.equal(o, o_ref), "O differs from fa_decode's"
    assert torch.equal(lse, lse_ref), "LSE differs from fa_decode's"
    ro, rl = oracle.attn_decode(P.f64(q), P.f64(k), P.f64(v), scale, [int(x) for x in lens])
    P.compare("O", P.f64(o), ro, 2e-2, "f16", "noalloc call 2")
    P.compare("LSE", P.f64(lse), rl, 1e-3, "f16", "noalloc call 2")
    assert np.isfinite(P.f64(o)).all()
