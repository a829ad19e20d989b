// fa_ceiling.hip -- what the chip itself sustains, measured by the same
// library the attention kernels live in: a matrix-core-only loop (the
// ceiling a dense bf16 contraction can reach) and streaming copy / read
// loops (the ceiling an HBM-bound kernel can reach).  Attention kernels are
// reported as a fraction of the published peaks and of these measured ones
// ("Flash Attention -- five lessons converging into 80 lines",
// brianyu43.github.io, Lesson 3: effective bandwidth as a fraction of what
// the memory can deliver).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/fa.h"
#include "fa_device.hpp"
#include "fa_kernels.hpp"

namespace fa {

// Matrix cores alone: every wave keeps NACC independent 32x32 fp32
// accumulators and issues v_mfma_f32_32x32x16_bf16 into them round-robin, so
// no product waits for the one before it.  The operands are built from the
// lane index (nothing for the compiler to fold) and every accumulator feeds
// the value written at the end, so no product is dead.  Wave 0 of each
// workgroup also records the shader-clock and constant-clock (100 MHz)
// counters at its start and end.  At most eight waves per workgroup (two
// per SIMD), which leaves 256 registers per lane: no spills.
template <int NACC>
__global__ __launch_bounds__(512) void ceiling_mfma_kernel(float* __restrict__ sink, unsigned long long* __restrict__ clocks, int iters) {
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t w = 0x3F803F80u ^ (lane << 3);  // bf16 pairs near 1.0
  const uint4 a = make_uint4(w, w ^ 0x10001u, w ^ 0x20002u, w ^ 0x30003u);
  const uint4 b = make_uint4(w ^ 0x40004u, w, w ^ 0x50005u, w ^ 0x60006u);
  f32x16 acc[NACC];
#pragma unroll
  for (int i = 0; i < NACC; ++i) acc[i] = f32x16{};
  const bool timer = threadIdx.x == 0;
  unsigned long long t0 = 0, r0 = 0;
  if (timer) {
    t0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < NACC; ++i) acc[i] = mma16(BF16{}, a, b, acc[i]);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NACC; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[i][r];
  sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
  if (timer && clocks != nullptr) {
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    clocks[2 * blockIdx.x] = t1 - t0;
    clocks[2 * blockIdx.x + 1] = r1 - r0;
  }
}

// The streaming kernels give each workgroup one contiguous chunk of the
// buffer (a grid-stride walk, where neighbouring workgroups touch addresses
// a grid apart, sustains about 12% less on this chip) and keep U 16-byte
// accesses per lane in flight.
__device__ __forceinline__ void stream_chunk(size_t n, size_t* lo, size_t* hi) {
  const size_t per = (n + gridDim.x - 1) / gridDim.x;
  *lo = min(n, (size_t)blockIdx.x * per);
  *hi = min(n, *lo + per);
}

// Streaming copy, 8 loads then 8 stores per lane per round.
__global__ __launch_bounds__(256) void ceiling_copy_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                           size_t n) {
  constexpr int U = 8;
  size_t lo, hi;
  stream_chunk(n, &lo, &hi);
  size_t i = lo + threadIdx.x;
  for (; i + (U - 1) * 256 < hi; i += U * 256) {
    uint4 x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) x[u] = src[i + u * 256];
#pragma unroll
    for (int u = 0; u < U; ++u) dst[i + u * 256] = x[u];
  }
  for (; i < hi; i += 256) dst[i] = src[i];
}

// Streaming read, 16 loads per lane per round: every 16-byte chunk is loaded
// once and folded into an XOR per lane, written to sink (one word per lane)
// so no load is dead.
__global__ __launch_bounds__(256) void ceiling_read_kernel(const uint4* __restrict__ src, size_t n,
                                                           uint32_t* __restrict__ sink) {
  constexpr int U = 16;
  size_t lo, hi;
  stream_chunk(n, &lo, &hi);
  size_t i = lo + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (U - 1) * 256 < hi; i += U * 256) {
    uint4 x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) x[u] = src[i + u * 256];
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= x[u].x ^ x[u].y ^ x[u].z ^ x[u].w;
  }
  for (; i < hi; i += 256) acc ^= src[i].x ^ src[i].y ^ src[i].z ^ src[i].w;
  sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

// Vector issue cost, one wave on one SIMD, timed with the shader clock: per
// loop iteration, MODE 0 issues 32 exponentials (v_exp_f32), each after a
// v_mul_f32, on 8 independent chains; MODE 1 issues 96 v_fma_f32 on 24
// independent chains; MODE 2 issues both sets, interleaved by the compiler.
// The softmax of the attention kernels is made of these two kinds of
// instruction; MODE 2 against MODE 0 + MODE 1 shows how far the
// transcendental unit's work overlaps the FMAs of the same wave.
template <int MODE>
__global__ __launch_bounds__(64) void ceiling_valu_kernel(float* __restrict__ sink,
                                                          unsigned long long* __restrict__ cycles, int iters,
                                                          float a, float b) {
  float e[8], f[24];
#pragma unroll
  for (int i = 0; i < 8; ++i) e[i] = 0.001f * (float)(threadIdx.x + i);
#pragma unroll
  for (int i = 0; i < 24; ++i) f[i] = 0.002f * (float)(threadIdx.x + i);
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if constexpr (MODE != 1) {
#pragma unroll
        for (int i = 0; i < 8; ++i) e[i] = __builtin_amdgcn_exp2f(e[i] * 0.5f);
      }
      if constexpr (MODE != 0) {
#pragma unroll
        for (int i = 0; i < 24; ++i) f[i] = __builtin_fmaf(f[i], a, b);
      }
    }
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += e[i];
#pragma unroll
  for (int i = 0; i < 24; ++i) s += f[i];
  sink[threadIdx.x] = s;
  if (threadIdx.x == 0) cycles[0] = t1 - t0;
}

// The 16-bit forward's inner step without HBM traffic: what its mix of
// instructions sustains on the matrix cores.  Eight waves per workgroup (two
// per SIMD), each running 32-key steps of 8 slots; a slot issues one product
// of the score chain S^T = K Q^T (32x32x16, accumulating), the weights of
// two keys (fma, exp2, bf16 pack, row-sum add) and one PV product into one
// of four accumulators, as the forward's slots do.  MODE 0: operands from
// registers.  MODE 1: each slot's A operands come from LDS as in the forward
// (one 16-byte row read for the score product, two 8-byte transposing reads
// for the PV product), read three slots ahead.  MODE 2: MODE 1 plus a
// workgroup barrier every two steps (the forward's one per 64-key tile).
// Operands are built from the lane index, every result feeds the sink.
template <int MODE>
__global__ __launch_bounds__(512) void ceiling_mix_kernel(float* __restrict__ sink,
                                                         unsigned long long* __restrict__ clocks, int iters,
                                                         float a, float b) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[16384];  // 16 KB row-read area, 16 KB transposing-read area
  const int lane = threadIdx.x & 63;
  for (int i = threadIdx.x; i < 16384; i += blockDim.x) lds[i] = (uint16_t)(0x3C00 + (i & 255));
  __syncthreads();
  const uint32_t w0 = 0x3F803F80u ^ ((uint32_t)lane << 3);
  const uint4 ka = make_uint4(w0, w0 ^ 0x10001u, w0 ^ 0x20002u, w0 ^ 0x30003u);
  uint4 qf[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) qf[s] = make_uint4(w0 ^ (s << 1), w0, w0 ^ 0x50005u, w0 ^ (0x60006u + s));
  f32x16 oacc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) oacc[i] = f32x16{};
  f32x16 sA, sB;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    sA[i] = 0.001f * (float)(lane + i);
    sB[i] = 0.f;
  }
  float lsum = 0.f;
  auto row_read = [&](int slot) __attribute__((always_inline)) {
    return *reinterpret_cast<const uint4*>(lds + ((slot & 7) * 1024 + lane * 16) / 2);
  };
  auto tr_read = [&](int slot) __attribute__((always_inline)) {
    const uint16_t* p = lds + (16384 + (slot & 7) * 1024 + lane * 8) / 2;
    const uint2 lo = read_tr_b64(p), hi = read_tr_b64(p + 256);
    return make_uint4(lo.x, lo.y, hi.x, hi.y);
  };
  uint4 ra[4], rb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ra[i] = MODE >= 1 && i < 3 ? row_read(i) : ka;
    rb[i] = MODE >= 1 && i < 3 ? tr_read(i) : ka;
  }
  // PV products take the previous step's packed weights, as in the forward
  uint32_t pkA[8] = {}, pkB[8] = {};
  auto step = [&](const f32x16& cur, f32x16& nxt, uint32_t (&pk)[8], const uint32_t (&pkp)[8])
      __attribute__((always_inline)) {
    const uint4 pp[2] = {make_uint4(pkp[0], pkp[1], pkp[2], pkp[3]), make_uint4(pkp[4], pkp[5], pkp[6], pkp[7])};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if constexpr (MODE >= 1) {
        ra[(k + 3) % 4] = row_read(k + 3);
        rb[(k + 3) % 4] = tr_read(k + 3);
      }
      nxt = mma16(BF16{}, ra[k % 4], qf[k], k == 0 ? f32x16{} : nxt);
      const float p0 = fast_exp2(__builtin_fmaf(cur[2 * k], a, -b));
      const float p1 = fast_exp2(__builtin_fmaf(cur[2 * k + 1], a, -b));
      pk[k] = pack2(BF16{}, p0, p1);
      lsum += p0 + p1;
      oacc[k % 4] = mma16(BF16{}, rb[k % 4], pp[k / 4], oacc[k % 4]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  const bool timer = threadIdx.x == 0;
  unsigned long long t0 = 0, r0 = 0;
  if (timer) {
    t0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  for (int it = 0; it < iters; ++it) {
    step(sA, sB, pkA, pkB);
    step(sB, sA, pkB, pkA);
    if constexpr (MODE == 2) {
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
      __builtin_amdgcn_s_barrier();
    }
  }
  float r = lsum;
#pragma unroll
  for (int i = 0; i < 8; ++i) r += __uint_as_float(pkA[i] & 0x3FFF3FFFu);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int k = 0; k < 16; ++k) r += oacc[i][k];
#pragma unroll
  for (int k = 0; k < 16; ++k) r += sA[k] + sB[k];
  sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = r;
  if (timer && clocks != nullptr) {
    clocks[2 * blockIdx.x] = __builtin_amdgcn_s_memtime() - t0;
    clocks[2 * blockIdx.x + 1] = __builtin_amdgcn_s_memrealtime() - r0;
  }
}

}  // namespace fa

namespace {
constexpr int kStreamGrid = 256 * 8;  // eight workgroups per CU
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
int launch_status(hipError_t e) {
  if (e == hipSuccess) return FA_OK;
  fa::record_hip_error((int)e);
  return FA_ERR_HIP;
}
}  // namespace

extern "C" {

int fa_ceiling_mfma(float* sink, unsigned long long* clocks, int workgroups, int waves, int iters, void* stream) {
  if (sink == nullptr) return FA_ERR_ARG;
  if (workgroups < 1 || iters < 1 || (waves != 4 && waves != 8)) return FA_ERR_ARG;
  if (!aligned16(sink) || (clocks != nullptr && !aligned16(clocks))) return FA_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // Eight accumulators per wave (128 registers) leave room for two waves
  // per SIMD.
  hipLaunchKernelGGL(fa::ceiling_mfma_kernel<8>, dim3((unsigned)workgroups), dim3((unsigned)(64 * waves)), 0, s,
                     sink, clocks, iters);
  return launch_status(hipGetLastError());
}

int fa_ceiling_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (src == nullptr || dst == nullptr || bytes == 0 || bytes % 16 != 0) return FA_ERR_ARG;
  if (!aligned16(src) || !aligned16(dst)) return FA_ERR_ALIGN;
  hipLaunchKernelGGL(fa::ceiling_copy_kernel, dim3(kStreamGrid), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(src), static_cast<uint4*>(dst), bytes / 16);
  return launch_status(hipGetLastError());
}

int fa_ceiling_read(const void* src, size_t bytes, void* sink, void* stream) {
  if (src == nullptr || sink == nullptr || bytes == 0 || bytes % 16 != 0) return FA_ERR_ARG;
  if (!aligned16(src) || !aligned16(sink)) return FA_ERR_ALIGN;
  hipLaunchKernelGGL(fa::ceiling_read_kernel, dim3(kStreamGrid), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(src), bytes / 16, static_cast<uint32_t*>(sink));
  return launch_status(hipGetLastError());
}

size_t fa_ceiling_read_sink_bytes(void) { return (size_t)kStreamGrid * 256 * 4; }

// Scores of the mix loop are sums of products near 1; this scale and shift
// keep its weights exp2(score * scale - shift) well inside range.
constexpr float kMixScale = 1.f / 1024, kMixShift = 4.f;

int fa_ceiling_mix(int mode, float* sink, unsigned long long* clocks, int workgroups, int iters, void* stream) {
  if (!sink || workgroups < 1 || iters < 1 || mode < 0 || mode > 2) return FA_ERR_ARG;
  if (!aligned16(sink) || (clocks != nullptr && !aligned16(clocks))) return FA_ERR_ALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 g((unsigned)workgroups), blk(512);
  if (mode == 0) hipLaunchKernelGGL(fa::ceiling_mix_kernel<0>, g, blk, 0, st, sink, clocks, iters, kMixScale, kMixShift);
  if (mode == 1) hipLaunchKernelGGL(fa::ceiling_mix_kernel<1>, g, blk, 0, st, sink, clocks, iters, kMixScale, kMixShift);
  if (mode == 2) hipLaunchKernelGGL(fa::ceiling_mix_kernel<2>, g, blk, 0, st, sink, clocks, iters, kMixScale, kMixShift);
  return launch_status(hipGetLastError());
}

int fa_ceiling_valu(int mode, float* sink, unsigned long long* cycles, int iters, void* stream) {
  if (!sink || !cycles || iters < 1 || mode < 0 || mode > 2) return FA_ERR_ARG;
  if (!aligned16(sink) || ((uintptr_t)cycles & 7u)) return FA_ERR_ALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (mode == 0) hipLaunchKernelGGL(fa::ceiling_valu_kernel<0>, dim3(1), dim3(64), 0, st, sink, cycles, iters, 0.999f, 0.001f);
  if (mode == 1) hipLaunchKernelGGL(fa::ceiling_valu_kernel<1>, dim3(1), dim3(64), 0, st, sink, cycles, iters, 0.999f, 0.001f);
  if (mode == 2) hipLaunchKernelGGL(fa::ceiling_valu_kernel<2>, dim3(1), dim3(64), 0, st, sink, cycles, iters, 0.999f, 0.001f);
  return launch_status(hipGetLastError());
}

}  // extern "C"
