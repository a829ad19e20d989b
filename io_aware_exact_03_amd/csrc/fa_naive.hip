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
// wave per 32 query rows; both operands are row-major 16-byte reads.  This
// element-wise writer serves row lengths that are not a multiple of eight.
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

// The same product for rows of 16-byte multiples (N % 8 == 0), written the
// way a memory-bound kernel should write: each wave computes S^T (keys x its
// 32 queries), so a lane holds one query's keys in runs of four; the tile of
// 128 queries x 128 keys is staged in LDS as float16 rows and stored with
// 16-byte accesses, sixteen lanes per 256-byte row segment.  K is staged in
// LDS once per workgroup (rows padded by 16 bytes) and read by all four waves.
template <typename T, int D>
__global__ __launch_bounds__(256) void naive_qk16_v(const uint16_t* __restrict__ qg, const uint16_t* __restrict__ kg,
                                                    uint16_t* __restrict__ sg, int N, int n_mt, int n_nt,
                                                    float scale) {
  constexpr int BQ = 128, BK = 128, KROW = D + 8, SROW = BK + 8, CPR = D / 8;
  constexpr int LDS_ELEMS = (BK * KROW > BQ * SROW) ? BK * KROW : BQ * SROW;
  __shared__ __attribute__((aligned(16))) uint16_t lds[LDS_ELEMS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, n = lane & 31, g = lane >> 5;
  long long t = blockIdx.x;
  const int nt = (int)(t % n_nt);
  t /= n_nt;
  const int mt = (int)(t % n_mt);
  const int bh = (int)(t / n_mt);
  const size_t head = (size_t)bh * N * D;
  const int q0 = mt * BQ, k0 = nt * BK;
  // K tile -> LDS (zeros past N)
#pragma unroll
  for (int c = 0; c < BK * CPR / 256; ++c) {
    const int idx = c * 256 + tid, key = idx / CPR, ch = idx % CPR;
    const uint4 x = k0 + key < N ? *reinterpret_cast<const uint4*>(kg + head + (size_t)(k0 + key) * D + 8 * ch)
                                 : make_uint4(0, 0, 0, 0);
    *reinterpret_cast<uint4*>(&lds[key * KROW + 8 * ch]) = x;
  }
  // Q fragments (B operand of S^T = K Q^T): query q0 + 32 wave + n
  const int q = q0 + 32 * wave + n;
  uint4 qf[D / 16];
#pragma unroll
  for (int s2 = 0; s2 < D / 16; ++s2)
    qf[s2] = q < N ? *reinterpret_cast<const uint4*>(qg + head + (size_t)q * D + 16 * s2 + 8 * g) : make_uint4(0, 0, 0, 0);
  __syncthreads();
  f32x16 acc[BK / 32];
#pragma unroll
  for (int cb = 0; cb < BK / 32; ++cb) {
    acc[cb] = f32x16{};
#pragma unroll
    for (int s2 = 0; s2 < D / 16; ++s2) {
      const uint4 a = *reinterpret_cast<const uint4*>(&lds[(32 * cb + n) * KROW + 16 * s2 + 8 * g]);
      acc[cb] = mma16(T{}, a, qf[s2], acc[cb]);
    }
  }
  __syncthreads();  // every wave is done with K: the buffer now stages S
  // register r of block cb: key 32 cb + 8 (r / 4) + 4 g + r % 4, query n
#pragma unroll
  for (int cb = 0; cb < BK / 32; ++cb)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint2 w = make_uint2((uint32_t)to_h(acc[cb][4 * j] * scale) | ((uint32_t)to_h(acc[cb][4 * j + 1] * scale) << 16),
                                 (uint32_t)to_h(acc[cb][4 * j + 2] * scale) | ((uint32_t)to_h(acc[cb][4 * j + 3] * scale) << 16));
      *reinterpret_cast<uint2*>(&lds[(32 * wave + n) * SROW + 32 * cb + 8 * j + 4 * g]) = w;
    }
  __syncthreads();
  uint16_t* sh = sg + (size_t)bh * N * N;
  constexpr int CH = BK / 8;  // 16-byte chunks per staged row
#pragma unroll
  for (int pass = 0; pass < BQ * CH / 256; ++pass) {
    const int row = pass * (256 / CH) + tid / CH, ch = tid % CH;
    const int qq = q0 + row, key = k0 + 8 * ch;
    if (qq < N && key < N)  // N % 8 == 0: the chunk is whole
      *reinterpret_cast<uint4*>(sh + (size_t)qq * N + key) = *reinterpret_cast<const uint4*>(&lds[row * SROW + 8 * ch]);
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
// P = 0.  Also writes LSE = m + ln l.  This element-wise form serves rows
// whose length is not a multiple of eight (and fp32 rows).
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

// The same softmax for float16 rows of 16-byte multiples (N % 8 == 0): a row
// belongs to TPR threads (one wave, or the whole workgroup for long rows),
// each of which moves CPT 16-byte chunks, eight elements per load and per
// store.  Causal rows read only their visible chunks and write zeros past
// the diagonal.
template <int TPR, int CPT>
__global__ __launch_bounds__(256) void naive_softmax_v16(const uint16_t* __restrict__ sg, uint16_t* __restrict__ pg,
                                                         float* __restrict__ lseg, int N, int causal,
                                                         long long rows) {
  static_assert(TPR == 64 || TPR == 256, "a wave or the workgroup per row");
  constexpr int RPW = 256 / TPR;  // rows per workgroup
  __shared__ float red[4];
  const int t = threadIdx.x % TPR, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const long long row_id = (long long)blockIdx.x * RPW + threadIdx.x / TPR;
  const bool row_ok = row_id < rows;
  const int i = row_ok ? (int)(row_id % N) : 0;
  const int lim = causal ? i + 1 : N;  // keys < lim are allowed
  const int nch = N / 8;
  const uint4* srow = reinterpret_cast<const uint4*>(sg + (size_t)(row_ok ? row_id : 0) * N);
  uint4* prow = reinterpret_cast<uint4*>(pg + (size_t)(row_ok ? row_id : 0) * N);
  float x[CPT][8];
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int ch = c * TPR + t;
    const bool any = row_ok && ch < nch && 8 * ch < lim;
    const uint4 w = any ? srow[ch] : make_uint4(0, 0, 0, 0);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float v = from_h((uint16_t)((e & 1) ? (ws[e / 2] >> 16) : (ws[e / 2] & 0xffffu)));
      x[c][e] = (any && 8 * ch + e < lim) ? v : kNegInf;
    }
  }
  float m = kNegInf;
#pragma unroll
  for (int c = 0; c < CPT; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) m = fmaxf(m, x[c][e]);
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if constexpr (TPR == 256) {
    if (lane == 0) red[wave] = m;
    __syncthreads();
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
  }
  float l = 0.f;
#pragma unroll
  for (int c = 0; c < CPT; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      x[c][e] = (x[c][e] == kNegInf) ? 0.f : __expf(x[c][e] - m);
      l += x[c][e];
    }
  for (int off = 32; off > 0; off >>= 1) l += __shfl_xor(l, off);
  if constexpr (TPR == 256) {
    if (lane == 0) red[wave] = l;
    __syncthreads();
    l = red[0] + red[1] + red[2] + red[3];
  }
  const float inv = 1.f / l;
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int ch = c * TPR + t;
    if (row_ok && ch < nch) {
      uint32_t o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        o[e] = (uint32_t)to_h(x[c][2 * e] * inv) | ((uint32_t)to_h(x[c][2 * e + 1] * inv) << 16);
      prow[ch] = make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
  if (row_ok && t == 0) lseg[row_id] = m + __logf(l);
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
    // this block's P (the A operand: 8 keys of the lane's query row per
    // product), loaded first so it arrives while V is staged
    uint4 pa[BK / 16];
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
      pa[s] = a;
    }
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
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const uint4 b = *reinterpret_cast<const uint4*>(&vt[(32 * db + n) * VROW + 16 * s + 8 * g]);
        acc[db] = mma16(F16{}, pa[s], b, acc[db]);
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

// float16 rows of 16-byte multiples: the vector softmax, a wave per row up
// to 2048 keys, the workgroup per row up to 32768.  Returns false if the row
// length has no vector variant.
bool launch_softmax_v16(const NaiveArgs& a, hipError_t* err) {
  const int N = a.N;
  if ((N & 7) != 0 || N > 256 * 8 * 16) return false;
  const long long rows = (long long)a.BH * N;
  const uint16_t* s = static_cast<const uint16_t*>(a.s);
  uint16_t* p = static_cast<uint16_t*>(a.p);
  const int causal = a.causal ? 1 : 0;
  auto go = [&](auto kern, int rpw) {
    const long long grid = (rows + rpw - 1) / rpw;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), 0, a.stream, s, p, a.lse, N, causal, rows);
  };
  if (N <= 64 * 8) go(naive_softmax_v16<64, 1>, 4);
  else if (N <= 64 * 16) go(naive_softmax_v16<64, 2>, 4);
  else if (N <= 64 * 32) go(naive_softmax_v16<64, 4>, 4);
  else if (N <= 256 * 16) go(naive_softmax_v16<256, 2>, 1);
  else if (N <= 256 * 32) go(naive_softmax_v16<256, 4>, 1);
  else if (N <= 256 * 64) go(naive_softmax_v16<256, 8>, 1);
  else go(naive_softmax_v16<256, 16>, 1);
  *err = hipGetLastError();
  return true;
}

template <typename S>
hipError_t launch_softmax(const NaiveArgs& a) {
  const long long rows = (long long)a.BH * a.N;
  if (rows > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if constexpr (sizeof(S) == 2) {
    hipError_t e;
    if (launch_softmax_v16(a, &e)) return e;
  }
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
  const int n_mt = (a.N + 127) / 128, n_nt = (a.N + 63) / 64, n_nt128 = (a.N + 127) / 128;
  const long long g1 = (long long)a.BH * n_mt * n_nt;
  const long long g3 = (long long)a.BH * n_mt;
  if (g1 > 0x7fffffffLL || g3 > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if ((a.N & 7) == 0) {  // 16-byte rows: the staged, row-contiguous S writer
    hipLaunchKernelGGL((naive_qk16_v<T, D>), dim3((unsigned)((long long)a.BH * n_mt * n_nt128)), dim3(256), 0,
                       a.stream, static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                       static_cast<uint16_t*>(a.s), a.N, n_mt, n_nt128, a.scale);
  } else {
    hipLaunchKernelGGL((naive_qk16<T, D>), dim3((unsigned)g1), dim3(256), 0, a.stream,
                       static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                       static_cast<uint16_t*>(a.s), a.N, n_mt, n_nt, a.scale);
  }
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
