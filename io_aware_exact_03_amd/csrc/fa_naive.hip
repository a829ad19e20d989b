// fa_naive.hip -- the three-kernel attention that materialises S and P in
// memory: S = scale * Q K^T for every N x N pair, then a row softmax S -> P
// (causal mask applied here), then O = P V.  This is standard attention as in
// Algorithm 0 of "Paper review: FlashAttention ... with IO-Awareness"
// (osehyeon.github.io) and the "naive" implementation of "Flash Attention --
// five lessons converging into 80 lines" (brianyu43.github.io, "Two
// implementations").  It exists to measure the N^2 memory round trips that
// the fused kernel avoids ("Flash Attention: IO-awareness principle",
// hrletsgo.me, the S+P traffic table), so each kernel is a reasonable gfx950
// kernel but none is fused with another.
//
// Storage: S and P are float16 for 16-bit inputs (both f16 and bf16) and
// float32 for fp32 inputs; the softmax computes in fp32.  For bf16 inputs
// the PV product converts V to float16 when staging it (exact for values
// inside float16's normal range).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_device.hpp"
#include "fa_kernels.hpp"

namespace fa {
namespace {

__device__ __forceinline__ uint16_t to_h(float x) { return __builtin_bit_cast(uint16_t, (_Float16)x); }
__device__ __forceinline__ float from_h(uint16_t x) { return (float)__builtin_bit_cast(_Float16, x); }

// ---------------------------------------------------------------------------
// Kernel 1: S = scale * Q K^T.  Workgroup tile 128 queries x 64 keys, one
// wave per 32 query rows; both operands are row-major 16-byte reads.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void naive_qk16(const uint16_t* __restrict__ qg, const uint16_t* __restrict__ kg,
                                                  uint16_t* __restrict__ sg, int N, int n_mt, int n_nt, float scale) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, n = lane & 31, g = lane >> 5;
  long long t = blockIdx.x;
  const int nt = (int)(t % n_nt);
  t /= n_nt;
  const int mt = (int)(t % n_mt);
  const int bh = (int)(t / n_mt);
  const size_t head = (size_t)bh * N * D;
  const int q = mt * 128 + wave * 32 + n;
  uint4 a[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s)
    a[s] = q < N ? *reinterpret_cast<const uint4*>(qg + head + (size_t)q * D + 16 * s + 8 * g) : make_uint4(0, 0, 0, 0);
  f32x16 acc[2] = {f32x16{}, f32x16{}};
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int key = nt * 64 + 32 * cb + n;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      const uint4 b = key < N ? *reinterpret_cast<const uint4*>(kg + head + (size_t)key * D + 16 * s + 8 * g)
                              : make_uint4(0, 0, 0, 0);
      acc[cb] = mma16(T{}, a[s], b, acc[cb]);
    }
  }
  // C layout: register r of column block cb is S[row 8(r/4)+4g+r%4][key n].
  uint16_t* sh = sg + (size_t)bh * N * N;
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int key = nt * 64 + 32 * cb + n;
    if (key >= N) continue;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = mt * 128 + wave * 32 + 8 * (r / 4) + 4 * g + (r % 4);
      if (row < N) sh[(size_t)row * N + key] = to_h(acc[cb][r] * scale);
    }
  }
}

template <int D>
__global__ __launch_bounds__(256) void naive_qk32(const float* __restrict__ qg, const float* __restrict__ kg,
                                                  float* __restrict__ sg, int N, int n_mt, int n_nt, float scale) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, n = lane & 31, g = lane >> 5;
  long long t = blockIdx.x;
  const int nt = (int)(t % n_nt);
  t /= n_nt;
  const int mt = (int)(t % n_mt);
  const int bh = (int)(t / n_mt);
  const size_t head = (size_t)bh * N * D;
  const int q = mt * 128 + wave * 32 + n;
  f32x16 acc[2] = {f32x16{}, f32x16{}};
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int key = nt * 64 + 32 * cb + n;
    for (int s = 0; s < D / 2; ++s) {
      const float av = q < N ? qg[head + (size_t)q * D + 2 * s + g] : 0.f;
      const float bv = key < N ? kg[head + (size_t)key * D + 2 * s + g] : 0.f;
      acc[cb] = mma32(av, bv, acc[cb]);
    }
  }
  float* sh = sg + (size_t)bh * N * N;
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int key = nt * 64 + 32 * cb + n;
    if (key >= N) continue;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = mt * 128 + wave * 32 + 8 * (r / 4) + 4 * g + (r % 4);
      if (row < N) sh[(size_t)row * N + key] = acc[cb][r] * scale;
    }
  }
}

// ---------------------------------------------------------------------------
// Kernel 2: row softmax.  One workgroup of 256 threads per row; the row is
// read once into registers (EPT elements per thread), reduced for max and
// sum through LDS, and written back as P.  Causal: keys after the row get
// P = 0.  Also writes LSE = m + ln l.
// ---------------------------------------------------------------------------
template <typename S, int EPT>
__global__ __launch_bounds__(256) void naive_softmax(const S* __restrict__ sg, S* __restrict__ pg,
                                                     float* __restrict__ lseg, int N, int causal) {
  constexpr int NT = 256;
  __shared__ float red[NT / 64];
  const long long row_id = blockIdx.x;  // bh * N + i
  const int i = (int)(row_id % N);
  const S* srow = sg + (size_t)row_id * N;
  S* prow = pg + (size_t)row_id * N;
  const int lim = causal ? i + 1 : N;  // keys < lim are allowed
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

  float x[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const int col = e * NT + threadIdx.x;
    float v = kNegInf;
    if (col < lim) {
      if constexpr (sizeof(S) == 2) v = from_h(srow[col]); else v = srow[col];
    }
    x[e] = v;
  }
  float m = kNegInf;
#pragma unroll
  for (int e = 0; e < EPT; ++e) m = fmaxf(m, x[e]);
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if (lane == 0) red[wave] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  float l = 0.f;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    x[e] = (x[e] == kNegInf) ? 0.f : __expf(x[e] - m);
    l += x[e];
  }
  for (int off = 32; off > 0; off >>= 1) l += __shfl_xor(l, off);
  if (lane == 0) red[wave] = l;
  __syncthreads();
  l = red[0] + red[1] + red[2] + red[3];
  const float inv = 1.f / l;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const int col = e * NT + threadIdx.x;
    if (col < N) {
      if constexpr (sizeof(S) == 2) prow[col] = to_h(x[e] * inv); else prow[col] = x[e] * inv;
    }
  }
  if (threadIdx.x == 0) lseg[row_id] = m + __logf(l);
}

// Rows longer than the register path: two passes over S (online max/sum,
// then normalise).
template <typename S>
__global__ __launch_bounds__(256) void naive_softmax_long(const S* __restrict__ sg, S* __restrict__ pg,
                                                          float* __restrict__ lseg, int N, int causal) {
  constexpr int NT = 256;
  __shared__ float red_m[NT / 64], red_l[NT / 64];
  const long long row_id = blockIdx.x;
  const int i = (int)(row_id % N);
  const S* srow = sg + (size_t)row_id * N;
  S* prow = pg + (size_t)row_id * N;
  const int lim = causal ? i + 1 : N;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float m = kNegInf, l = 0.f;
  for (int col = threadIdx.x; col < lim; col += NT) {
    float v;
    if constexpr (sizeof(S) == 2) v = from_h(srow[col]); else v = srow[col];
    const float mn = fmaxf(m, v);
    l = l * __expf(m - mn) + __expf(v - mn);
    m = mn;
  }
  for (int off = 32; off > 0; off >>= 1) {
    const float mo = __shfl_xor(m, off), lo = __shfl_xor(l, off);
    const float mn = fmaxf(m, mo);
    const float a = (m == kNegInf) ? 0.f : __expf(m - mn), b = (mo == kNegInf) ? 0.f : __expf(mo - mn);
    l = l * a + lo * b;
    m = mn;
  }
  if (lane == 0) { red_m[wave] = m; red_l[wave] = l; }
  __syncthreads();
  float M = kNegInf;
  for (int w = 0; w < NT / 64; ++w) M = fmaxf(M, red_m[w]);
  float L = 0.f;
  for (int w = 0; w < NT / 64; ++w) L += (red_m[w] == kNegInf) ? 0.f : red_l[w] * __expf(red_m[w] - M);
  const float inv = 1.f / L;
  for (int col = threadIdx.x; col < N; col += NT) {
    float p = 0.f;
    if (col < lim) {
      float v;
      if constexpr (sizeof(S) == 2) v = from_h(srow[col]); else v = srow[col];
      p = __expf(v - M) * inv;
    }
    if constexpr (sizeof(S) == 2) prow[col] = to_h(p); else prow[col] = p;
  }
  if (threadIdx.x == 0) lseg[row_id] = M + __logf(L);
}

// ---------------------------------------------------------------------------
// Kernel 3: O = P V.  Workgroup: 128 query rows (32 per wave) x all d.  P
// (float16) is the A operand, read row-major; V is staged per 64-key block
// into LDS transposed (d-major, keys contiguous) and converted to float16.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void naive_pv16(const uint16_t* __restrict__ pg, const uint16_t* __restrict__ vg,
                                                  uint16_t* __restrict__ og, int N, int n_mt) {
  constexpr int BK = 64, VROW = BK + 8, NT = 256;
  constexpr int KPT = BK * D / 8 / NT;  // 2 (d=64) or 4 (d=128)
  __shared__ __attribute__((aligned(16))) uint16_t vt[D * VROW];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, n = lane & 31, g = lane >> 5;
  const int mt = blockIdx.x % n_mt;
  const int bh = blockIdx.x / n_mt;
  const uint16_t* ph = pg + (size_t)bh * N * N;
  const uint16_t* vh = vg + (size_t)bh * N * D;
  const int q = mt * 128 + wave * 32 + n;
  const int va = tid % (BK / KPT), vdc = tid / (BK / KPT);
  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};
  for (int k0 = 0; k0 < N; k0 += BK) {
    // stage V[k0 .. k0+64) transposed, as float16
    uint4 x[KPT];
#pragma unroll
    for (int e = 0; e < KPT; ++e) {
      const int key = k0 + KPT * va + e;
      x[e] = key < N ? *reinterpret_cast<const uint4*>(vh + (size_t)key * D + 8 * vdc) : make_uint4(0, 0, 0, 0);
    }
    __syncthreads();
    const uint32_t* w = reinterpret_cast<const uint32_t*>(x);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      uint16_t e[4];
#pragma unroll
      for (int kk = 0; kk < KPT; ++kk) {
        const uint32_t word = w[4 * kk + t / 2];
        const float f = (t & 1) ? hi16(T{}, word) : lo16(T{}, word);
        e[kk] = to_h(f);
      }
      uint16_t* dst = &vt[(8 * vdc + t) * VROW + KPT * va];
      if constexpr (KPT == 4)
        *reinterpret_cast<uint2*>(dst) =
            make_uint2((uint32_t)e[0] | ((uint32_t)e[1] << 16), (uint32_t)e[2] | ((uint32_t)e[3] << 16));
      else
        *reinterpret_cast<uint32_t*>(dst) = (uint32_t)e[0] | ((uint32_t)e[1] << 16);
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      const int key = k0 + 16 * s + 8 * g;  // first of this lane's 8 keys
      uint4 a = make_uint4(0, 0, 0, 0);
      if (q < N) {
        if ((N & 7) == 0 && key + 8 <= N) {  // 16-byte aligned full slice
          a = *reinterpret_cast<const uint4*>(ph + (size_t)q * N + key);
        } else {
          uint16_t tmp[8];
#pragma unroll
          for (int e2 = 0; e2 < 8; ++e2) tmp[e2] = (key + e2 < N) ? ph[(size_t)q * N + key + e2] : (uint16_t)0;
          a = make_uint4(tmp[0] | (tmp[1] << 16), tmp[2] | (tmp[3] << 16), tmp[4] | (tmp[5] << 16),
                         tmp[6] | (tmp[7] << 16));
        }
      }
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const uint4 b = *reinterpret_cast<const uint4*>(&vt[(32 * db + n) * VROW + 16 * s + 8 * g]);
        acc[db] = mma16(F16{}, a, b, acc[db]);
      }
    }
  }
  // C layout: register r of d block db is O[row 8(r/4)+4g+r%4][d 32 db + n].
  uint16_t* oh = og + (size_t)bh * N * D;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = mt * 128 + wave * 32 + 8 * (r / 4) + 4 * g + (r % 4);
      if (row < N) {
        const uint32_t w2 = pack2(T{}, acc[db][r], 0.f);
        oh[(size_t)row * D + 32 * db + n] = (uint16_t)(w2 & 0xffffu);
      }
    }
}

template <int D>
__global__ __launch_bounds__(256) void naive_pv32(const float* __restrict__ pg, const float* __restrict__ vg,
                                                  float* __restrict__ og, int N, int n_mt) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, n = lane & 31, g = lane >> 5;
  const int mt = blockIdx.x % n_mt;
  const int bh = blockIdx.x / n_mt;
  const float* ph = pg + (size_t)bh * N * N;
  const float* vh = vg + (size_t)bh * N * D;
  const int q = mt * 128 + wave * 32 + n;
  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};
  for (int k = 0; k < N; k += 2) {
    const int key = k + g;
    const float a = (q < N && key < N) ? ph[(size_t)q * N + key] : 0.f;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const float b = key < N ? vh[(size_t)key * D + 32 * db + n] : 0.f;
      acc[db] = mma32(a, b, acc[db]);
    }
  }
  float* oh = og + (size_t)bh * N * D;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = mt * 128 + wave * 32 + 8 * (r / 4) + 4 * g + (r % 4);
      if (row < N) oh[(size_t)row * D + 32 * db + n] = acc[db][r];
    }
}

template <typename S>
hipError_t launch_softmax(const NaiveArgs& a) {
  const long long rows = (long long)a.BH * a.N;
  if (rows > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const S* s = static_cast<const S*>(a.s);
  S* p = static_cast<S*>(a.p);
  const int causal = a.causal ? 1 : 0;
  const dim3 grid((unsigned)rows), block(256);
  if (a.N <= 256 * 8)
    hipLaunchKernelGGL((naive_softmax<S, 8>), grid, block, 0, a.stream, s, p, a.lse, a.N, causal);
  else if (a.N <= 256 * 16)
    hipLaunchKernelGGL((naive_softmax<S, 16>), grid, block, 0, a.stream, s, p, a.lse, a.N, causal);
  else if (a.N <= 256 * 32)
    hipLaunchKernelGGL((naive_softmax<S, 32>), grid, block, 0, a.stream, s, p, a.lse, a.N, causal);
  else if (a.N <= 256 * 64)
    hipLaunchKernelGGL((naive_softmax<S, 64>), grid, block, 0, a.stream, s, p, a.lse, a.N, causal);
  else
    hipLaunchKernelGGL((naive_softmax_long<S>), grid, block, 0, a.stream, s, p, a.lse, a.N, causal);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t run16(const NaiveArgs& a) {
  const int n_mt = (a.N + 127) / 128, n_nt = (a.N + 63) / 64;
  const long long g1 = (long long)a.BH * n_mt * n_nt;
  const long long g3 = (long long)a.BH * n_mt;
  if (g1 > 0x7fffffffLL || g3 > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((naive_qk16<T, D>), dim3((unsigned)g1), dim3(256), 0, a.stream,
                     static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                     static_cast<uint16_t*>(a.s), a.N, n_mt, n_nt, a.scale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_softmax<uint16_t>(a);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((naive_pv16<T, D>), dim3((unsigned)g3), dim3(256), 0, a.stream,
                     static_cast<const uint16_t*>(a.p), static_cast<const uint16_t*>(a.v),
                     static_cast<uint16_t*>(a.o), a.N, n_mt);
  return hipGetLastError();
}

template <int D>
hipError_t run32(const NaiveArgs& a) {
  const int n_mt = (a.N + 127) / 128, n_nt = (a.N + 63) / 64;
  const long long g1 = (long long)a.BH * n_mt * n_nt;
  const long long g3 = (long long)a.BH * n_mt;
  if (g1 > 0x7fffffffLL || g3 > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((naive_qk32<D>), dim3((unsigned)g1), dim3(256), 0, a.stream, static_cast<const float*>(a.q),
                     static_cast<const float*>(a.k), static_cast<float*>(a.s), a.N, n_mt, n_nt, a.scale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_softmax<float>(a);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((naive_pv32<D>), dim3((unsigned)g3), dim3(256), 0, a.stream, static_cast<const float*>(a.p),
                     static_cast<const float*>(a.v), static_cast<float*>(a.o), a.N, n_mt);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_naive(const NaiveArgs& a) {
  if (a.dtype == 0) return a.d == 64 ? run32<64>(a) : run32<128>(a);
  if (a.dtype == 1) return a.d == 64 ? run16<F16, 64>(a) : run16<F16, 128>(a);
  return a.d == 64 ? run16<BF16, 64>(a) : run16<BF16, 128>(a);
}

}  // namespace fa
