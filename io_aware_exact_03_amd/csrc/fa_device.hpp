// fa_device.hpp -- device building blocks for the gfx950 attention kernels:
// MFMA tile products, wave64 cross-half reductions, element conversions and
// the online-softmax step.
//
// MFMA conventions (v_mfma_f32_32x32x16_{bf16,f16} and v_mfma_f32_32x32x2_f32,
// 64 lanes, lane l, g = l / 32, n = l % 32):
//   A operand (32 x K):  lane l supplies row n, its K-slice for group g;
//   B operand (K x 32):  lane l supplies column n, its K-slice for group g;
//   C/D (32 x 32 fp32): register r of lane l is element
//                        row 8*(r/4) + 4*g + (r%4), column n.
// Both operands of one product take their K-slices with the same (g, t)
// pattern, so the hardware's K order inside an instruction never matters.
//
// Pages cited: "Triton 06: Flash Attention v2" (wonbeomjang.kr),
// Improvement 1 (un-scaled accumulator, alpha correction, one final divide),
// Improvement 2 (exp2 with log2(e) folded into the scale), Improvement 4
// (the running accumulator is the matrix product's C operand); "Flash
// Attention -- five lessons converging into 80 lines" (brianyu43.github.io),
// Lesson 4 (warp reduction for the row max and sum, coalesced loads).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

// Element type tags for the 16-bit paths.
struct BF16 {};
struct F16 {};

// ---------------------------------------------------------------------------
// Matrix products.  c += A(32 x 16) * B(16 x 32) with 8 16-bit elements per
// lane per operand, passed as 16 raw bytes.
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x16 mma16(BF16, const uint4& a, const uint4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mma16(F16, const uint4& a, const uint4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
// fp32: c += A(32 x 2) * B(2 x 32), one element per lane per operand.
__device__ __forceinline__ f32x16 mma32(float a, float b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Conversions, round-to-nearest-even.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t pack2(BF16, float a, float b) {
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint32_t pack2(F16, float a, float b) {
  f16x2 v = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float lo16(BF16, uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi16(BF16, uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float lo16(F16, uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
__device__ __forceinline__ float hi16(F16, uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// ---------------------------------------------------------------------------
// Wave64 reductions across the two 32-lane halves.  v_permlane32_swap
// exchanges the halves; which result holds the partner's value depends on
// the half, so only symmetric combinations are formed from the pair.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float halves_max(float x) {
  const uint32_t u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const uint32_t u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// One online-softmax step for the KB 32x32 score blocks S^T of one 32-query
// column block.  Lane l owns query n = l % 32; register r of block kb is key
// key_base + 32*kb + 8*(r/4) + (r%4), where key_base already includes 4*g.
//
//   m_new = max(m, rowmax(S) * qk_scale)           (cross-half max)
//   p     = exp2(S * qk_scale - m_new)              (in place in s)
//   l     = alpha * l + sum(p),  alpha = exp2(m - m_new)
//
// l is this lane's partial sum over its own keys: alpha is the same on both
// halves, so the halves are added once, at the end.  qk_scale >= 0 (a
// negative scale is folded into the sign of Q), so max(S) * qk_scale is
// the max of the scaled scores.  MASKED keeps only keys < key_lim (the
// causal limit query+1 and the sequence end); masked p are exactly 0 even
// when qk_scale is 0.  A row with no key yet keeps m = -inf and uses 0 in
// place of m_new, so -inf - (-inf) never occurs.
// Returns alpha for the accumulator correction.
// ---------------------------------------------------------------------------
template <int KB, bool MASKED>
__device__ __forceinline__ float softmax_step(f32x16 (&s)[KB], float& m, float& l, float qk_scale,
                                              int key_base, int key_lim) {
  float mx = kNegInf;
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if constexpr (MASKED) {
        const int key = key_base + 32 * kb + 8 * (r / 4) + (r % 4);
        mx = fmaxf(mx, key < key_lim ? s[kb][r] : kNegInf);
      } else {
        mx = fmaxf(mx, s[kb][r]);
      }
    }
  }
  mx = halves_max(mx);
  const float mt = (mx == kNegInf) ? kNegInf : mx * qk_scale;
  const float m_new = fmaxf(m, mt);
  const float m_use = (m_new == kNegInf) ? 0.f : m_new;
  const float alpha = fast_exp2(m - m_use);
  float sum = 0.f;
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float p = fast_exp2(__builtin_fmaf(s[kb][r], qk_scale, -m_use));
      if constexpr (MASKED) {
        const int key = key_base + 32 * kb + 8 * (r / 4) + (r % 4);
        p = key < key_lim ? p : 0.f;
      }
      s[kb][r] = p;
      sum += p;
    }
  }
  l = l * alpha + sum;
  m = m_new;
  return alpha;
}

}  // namespace fa
