"""Seeded synthetic inputs for exact attention, shared by tests and bench.

This module holds no attention arithmetic: it only draws Gaussian tensors from
a seeded CPU generator, scales them by a standard deviation and rounds them to
the storage dtype (round-to-nearest-even, torch's ``.to``).  Both the fp64
oracle and the HIP path read the very same rounded tensors, so input rounding
never enters a parity error.

The workloads follow the problem statement the pages share: Q, K, V of shape
[B, H, N, d] with a scale on QK^T and an optional causal mask.  The pages
measure on synthetic data with no stated distribution; i.i.d. Gaussians are
the plainest reading.  Draw order is fixed: Q, K, V, then dO.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str
    causal: bool
    scale: float
    seed: int
    sigma_qk: float = 1.0
    sigma_v: float = 1.0
    passes: tuple = field(default=("fwd",))
    naive: bool = False
    Hkv: int = 0  # K/V heads per batch; 0 = H (one K/V head per query head)

    @property
    def kv_heads(self) -> int:
        return self.Hkv or self.H

    def describe(self) -> str:
        kv = f" Hkv={self.Hkv}" if self.Hkv else ""
        return (f"{self.name}: B={self.B} H={self.H}{kv} N={self.N} d={self.d} {self.dtype} "
                f"{'causal' if self.causal else 'non-causal'} scale={self.scale:.6g} seed={self.seed}")


def _c2(n: int) -> Workload:
    return Workload(f"noncausal_fwd_sweep_N{n}_B4_H8_d64_f16", 4, 8, n, 64, "f16", False, 1 / 8,
                    1002 + n, naive=True)


# Single head, non-causal, fp32 (the size the T4 lesson sweeps start from).
SINGLE_HEAD_F32 = Workload("single_head_fwd_N512_d64_f32", 1, 1, 512, 64, "f32", False, 1 / 8, 1001)
# Non-causal fp16 sweep with the naive baseline beside it.
NONCAUSAL_SWEEP = tuple(_c2(n) for n in (512, 1024, 2048, 4096))
# Causal prefill, wide heads.
CAUSAL_PREFILL = Workload("causal_prefill_fwd_B2_H32_N8192_d128_bf16", 2, 32, 8192, 128, "bf16", True,
                          1 / math.sqrt(128), 1003)
# Long causal sequence with wide logits, naive baseline beside it.
LONG_CAUSAL = Workload("long_causal_fwd_B1_H16_N16384_d64_bf16", 1, 16, 16384, 64, "bf16", True, 1 / 8,
                       1004, sigma_qk=2.0, naive=True)
# The causal prefill's shape without the mask, and a longer non-causal
# sequence at d = 128: the forward's rate where no block is cut by the
# diagonal.
NONCAUSAL_PREFILL = Workload("noncausal_prefill_fwd_B2_H32_N8192_d128_bf16", 2, 32, 8192, 128, "bf16", False,
                             1 / math.sqrt(128), 1011)
NONCAUSAL_LONG = Workload("noncausal_fwd_B1_H32_N16384_d128_bf16", 1, 32, 16384, 128, "bf16", False,
                          1 / math.sqrt(128), 1012)
# Causal training step: forward and backward.
TRAIN_STEP = Workload("causal_train_step_B4_H16_N4096_d128_bf16", 4, 16, 4096, 128, "bf16", True,
                      1 / math.sqrt(128), 1005, passes=("fwd", "bwd"))

ALL_WORKLOADS = (SINGLE_HEAD_F32,) + NONCAUSAL_SWEEP + (CAUSAL_PREFILL, LONG_CAUSAL, TRAIN_STEP)

# Grouped-query causal prefill: 64 query heads sharing 8 K/V heads (the
# head counts of the 70B-class model the serving discussion names), forward
# and backward.
# Decode steps of the same model: one new token per sequence against a K/V
# cache.  Batch 1 with a 32K cache (the batch-1 decoding case the serving
# discussion names), and 16 sequences of ragged length up to 8K.
GQA_DECODE = Workload("gqa_decode_B1_H64_Hkv8_N32768_d128_bf16", 1, 64, 32768, 128, "bf16", False,
                      1 / math.sqrt(128), 1007, passes=("decode",), Hkv=8)
GQA_DECODE_RAGGED = Workload("gqa_decode_ragged_B16_H64_Hkv8_N8192_d128_bf16", 16, 64, 8192, 128, "bf16", False,
                             1 / math.sqrt(128), 1008, passes=("decode",), Hkv=8)

# FP8 causal prefill: the causal prefill shape with E4M3 Q, K, V.
FP8_PREFILL = Workload("fp8_causal_prefill_fwd_B2_H32_N8192_d128_e4m3", 2, 32, 8192, 128, "e4m3", True,
                       1 / math.sqrt(128), 1010)

# A chunk of 2048 new prompt tokens after 14336 cached ones (keys 16384),
# same model shape: the causal mask is aligned at the bottom-right corner.
CHUNK_PREFILL = Workload("gqa_chunk_prefill_B1_H64_Hkv8_Nq2048_Nk16384_d128_bf16", 1, 64, 2048, 128, "bf16", True,
                         1 / math.sqrt(128), 1009, passes=("fwd",), Hkv=8)
CHUNK_PREFILL_NK = 16384

GQA_PREFILL = Workload("gqa_causal_prefill_B1_H64_Hkv8_N8192_d128_bf16", 1, 64, 8192, 128, "bf16", True,
                       1 / math.sqrt(128), 1006, passes=("fwd", "bwd"), Hkv=8)


def make_inputs(B: int, H: int, N: int, d: int, dtype: str, seed: int, sigma_qk: float = 1.0,
                sigma_v: float = 1.0, with_dout: bool = False, Hkv: int = 0):
    """Q, K, V (and dO) as CPU tensors of ``dtype``: Q and dO [B,H,N,d], K
    and V [B,Hkv,N,d] (Hkv = 0 means H).

    Q and K are N(0, sigma_qk^2), V and dO are N(0, sigma_v^2) and N(0, 1).
    """
    g = torch.Generator(device="cpu").manual_seed(seed)
    shape = (B, H, N, d)
    kv_shape = (B, Hkv or H, N, d)

    def draw(sigma, shape=shape):
        t = torch.randn(*shape, generator=g, dtype=torch.float32)
        if sigma != 1.0:
            t = t * sigma
        return t.to(DTYPES[dtype])

    q = draw(sigma_qk)
    k = draw(sigma_qk, kv_shape)
    v = draw(sigma_v, kv_shape)
    if not with_dout:
        return q, k, v
    return q, k, v, draw(1.0)


def make_decode_inputs(B: int, H: int, Hkv: int, Nkv: int, d: int, dtype: str, seed: int, ragged: bool = False):
    """One decode step: q [B,H,d], K/V caches [B,Hkv,Nkv,d] (all N(0, 1),
    rounded to ``dtype``) and the valid lengths, an int32 CPU tensor [B]:
    all Nkv, or (ragged) uniform on [1, Nkv].  Draw order: q, K, V, lengths."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    q = torch.randn(B, H, d, generator=g, dtype=torch.float32).to(DTYPES[dtype])
    k = torch.randn(B, Hkv, Nkv, d, generator=g, dtype=torch.float32).to(DTYPES[dtype])
    v = torch.randn(B, Hkv, Nkv, d, generator=g, dtype=torch.float32).to(DTYPES[dtype])
    if ragged:
        lens = torch.randint(1, Nkv + 1, (B,), generator=g, dtype=torch.int32)
    else:
        lens = torch.full((B,), Nkv, dtype=torch.int32)
    return q, k, v, lens


def make_chunk_inputs(B: int, H: int, Hkv: int, Nq: int, Nk: int, d: int, dtype: str, seed: int):
    """A prefill chunk: q [B,H,Nq,d] and K, V [B,Hkv,Nk,d], all N(0, 1)
    rounded to ``dtype``.  Draw order: q, K, V."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    q = torch.randn(B, H, Nq, d, generator=g, dtype=torch.float32).to(DTYPES[dtype])
    k = torch.randn(B, Hkv, Nk, d, generator=g, dtype=torch.float32).to(DTYPES[dtype])
    v = torch.randn(B, Hkv, Nk, d, generator=g, dtype=torch.float32).to(DTYPES[dtype])
    return q, k, v


def make_fp8_inputs(B: int, H: int, Hkv: int, N: int, d: int, seed: int, sigma: float = 1.0):
    """FP8 inputs: Q [B,H,N,d], K and V [B,Hkv,N,d] drawn N(0, sigma^2) in
    fp32, each scaled by its own descale = amax / 448 and rounded to OCP
    E4M3 codes (torch.float8_e4m3fn, round to nearest even).  Returns the
    codes as uint8 tensors and the three descale factors.  Draw order: Q, K, V."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    codes, scales = [], []
    for heads in (H, Hkv, Hkv):
        x = torch.randn(B, heads, N, d, generator=g, dtype=torch.float32) * sigma
        ds = float(x.abs().max()) / 448.0
        codes.append((x / ds).to(torch.float8_e4m3fn).view(torch.uint8))
        scales.append(ds)
    return codes[0], codes[1], codes[2], tuple(scales)


def workload_inputs(w: Workload, with_dout: bool | None = None):
    if with_dout is None:
        with_dout = "bwd" in w.passes
    return make_inputs(w.B, w.H, w.N, w.d, w.dtype, w.seed, w.sigma_qk, w.sigma_v, with_dout, w.Hkv)


def to_f64(t):
    """Exact upcast of a (rounded) CPU tensor to a float64 NumPy array."""
    return t.to(torch.float64).numpy()
