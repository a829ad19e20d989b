// fa_fwd.hip -- fused exact-attention forward for gfx950 (MI355X).
//
// One workgroup owns one block of BM query rows of one (batch, head) and
// finishes its output rows alone: query blocks outside, K/V blocks inside
// ("Flash Attention: IO-awareness principle", hrletsgo.me, section "FA2/FA3";
// "Triton 06: Flash Attention v2", wonbeomjang.kr, the forward flow summary).
// Per K/V block, on chip: S^T = K Q^T on MFMA, the online-softmax step with
// exp2 and the scale pre-multiplied by log2(e), and O^T += V^T P^T on MFMA
// with the running accumulator as the C operand (Improvements 1, 2, 4).  The
// causal case runs unmasked blocks, then the masked diagonal block, and never
// reads blocks in the future (Improvement 3).  One divide per row at the end;
// LSE = (m + log2 l) * ln 2 is stored for the backward pass.
//
// gfx950 layout choices (not from the pages, which target NVIDIA parts):
// * Each wave owns QB column blocks of 32 queries.  Computing S^T (keys x
//   queries) puts every lane on ONE query, so the row max and row sum are
//   in-lane plus one exchange of the two 32-lane halves, and the softmax
//   correction alpha is lane-local for the O^T accumulator as well.
// * The fp32 S^T accumulator registers, converted to 16-bit, are directly
//   the B operand of the O^T product: no LDS round trip for P.  That product
//   needs V with keys contiguous per lane, so V is stored transposed in LDS,
//   with the keys of each 16-key group permuted (bits 2 and 3 of the key
//   index swapped) to match the accumulator's key order.
// * K (row-major, 16-byte row padding) and V^T (padded rows) are
//   double-buffered in LDS; the next block's global loads are in flight
//   while the current block computes; one barrier per block.
// * Workgroups are renumbered so each XCD (own L2) works on whole heads,
//   heaviest causal query blocks first.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fa_device.hpp"
#include "fa_plan.hpp"
#include "fa_kernels.hpp"

namespace fa {

// ===========================================================================
// 16-bit (bf16 / fp16) forward
// ===========================================================================
template <typename T, int D, int BN, int NW, int QB, bool CAUSAL>
struct Fwd16 {
  static constexpr int NT = NW * 64;
  static constexpr int QW = 32 * QB;        // queries per wave
  static constexpr int BM = NW * QW;        // queries per workgroup
  static constexpr int KROW = D + 8;        // K row stride in LDS (elements)
  static constexpr int VROW = BN + 8;       // V^T row stride in LDS (elements)
  static constexpr int DS = D / 16;         // k-steps of the S product
  static constexpr int KB = BN / 32;        // 32-key blocks per K/V block
  static constexpr int DB = D / 32;         // 32-wide d blocks of O
  static constexpr int KCH = BN * D / 8;    // 16-byte chunks of a K block
  static constexpr int KLD = KCH / NT;      // K chunks per thread
  static constexpr int KPT = BN * D / 8 / NT;  // keys per thread in the V transpose
  static_assert(KCH % NT == 0, "K block must split evenly over threads");
  static_assert(KPT == 2 || KPT == 4, "V transpose packs 2 or 4 keys per thread");
  static_assert(BN % 32 == 0 && D % 32 == 0, "tile shape");
  static constexpr int LDS_K = BN * KROW;   // elements per K buffer
  static constexpr int LDS_V = D * VROW;    // elements per V^T buffer
};

template <typename T, int D, int BN, int NW, int QB, bool CAUSAL>
__global__ __launch_bounds__(NW * 64) void fwd16_kernel(
    const uint16_t* __restrict__ qg, const uint16_t* __restrict__ kg, const uint16_t* __restrict__ vg,
    uint16_t* __restrict__ og, float* __restrict__ lseg, int N, int n_qblk, float qk_scale,
    uint32_t qsign) {
  using C = Fwd16<T, D, BN, NW, QB, CAUSAL>;
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[2][C::LDS_K];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[2][C::LDS_V];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 31;
  const int g = lane >> 5;

  int bh, qblk;
  tile_of(xcd_remap(blockIdx.x, gridDim.x), n_qblk, CAUSAL, &bh, &qblk);
  const size_t head = (size_t)bh * (size_t)N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2;
  const rsrc_t qrs = make_rsrc(qg + head, head_bytes);
  const rsrc_t krs = make_rsrc(kg + head, head_bytes);
  const rsrc_t vrs = make_rsrc(vg + head, head_bytes);

  const int q0 = qblk * C::BM;
  const int qw0 = q0 + wave * C::QW;  // first query of this wave

  // ---- Q fragments, held in registers for the whole kernel --------------
  // B operand of S^T = K Q^T: lane supplies Q[query n][16 s + 8 g + 0..7].
  // Rows past N read as zeros.
  uint4 qf[QB][C::DS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const uint32_t row = qw0 + 32 * qb + n;
#pragma unroll
    for (int s = 0; s < C::DS; ++s) {
      uint4 x = load16(qrs, (row * D + 16 * s + 8 * g) * 2);
      x.x ^= qsign; x.y ^= qsign; x.z ^= qsign; x.w ^= qsign;
      qf[qb][s] = x;
    }
  }

  // ---- key-block plan ---------------------------------------------------
  // Blocks [0, j_unm) hold only keys visible to every query of the
  // workgroup and lie before the sequence tail: no mask at all (the pages'
  // unmasked stage).  Blocks [j_unm, j_end) straddle the diagonal or hold
  // the tail: masked per key; each wave also skips blocks wholly in its
  // future.  Blocks from j_end on are never read.
  const int n_kv = (N + BN - 1) / BN;
  const int full_blocks = N / BN;
  int j_end = n_kv, j_unm = full_blocks;
  if (CAUSAL) {
    j_end = min(n_kv, (min(q0 + C::BM, N) - 1) / BN + 1);
    int s1, s2;
    causal_stages(q0, min(q0 + C::BM, N), BN, &s1, &s2);
    j_unm = min(s1, full_blocks);
  }
  int w_s2 = n_kv;
  const bool wave_live = qw0 < N;
  if (CAUSAL && wave_live) {
    int w_s1;
    causal_stages(qw0, min(qw0 + C::QW, N), BN, &w_s1, &w_s2);
  }

  // ---- global -> register staging of one K/V block -----------------------
  uint4 kst[C::KLD];
  uint4 vst[C::KPT];
  const int va = tid % (BN / C::KPT);   // key group of this thread
  const int vdc = tid / (BN / C::KPT);  // d chunk (8 elements) of this thread

  auto load_block = [&](int j) {
    const uint32_t key0 = j * BN;
#pragma unroll
    for (int i = 0; i < C::KLD; ++i) {
      const int c = tid + i * C::NT;
      const uint32_t row = key0 + c / (D / 8), col = (c % (D / 8)) * 8;
      kst[i] = load16(krs, (row * D + col) * 2);
    }
#pragma unroll
    for (int e = 0; e < C::KPT; ++e) {
      const uint32_t row = key0 + C::KPT * va + e;
      vst[e] = load16(vrs, (row * D + 8 * vdc) * 2);
    }
  };
  auto store_block = [&](int buf) {
#pragma unroll
    for (int i = 0; i < C::KLD; ++i) {
      const int c = tid + i * C::NT;
      const int row = c / (D / 8), col = (c % (D / 8)) * 8;
      *reinterpret_cast<uint4*>(&k_lds[buf][row * C::KROW + col]) = kst[i];
    }
    // V^T: KPT keys x 8 d of V become 8 rows of V^T (keys in tpos order).
    store_transposed<C::KPT>(&v_lds[buf][8 * vdc * C::VROW], C::VROW, tpos(C::KPT * va), vst);
  };

  // ---- running state --------------------------------------------------
  f32x16 oacc[QB][C::DB];
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = kNegInf;
    l_run[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < C::DB; ++db) oacc[qb][db] = f32x16{};
  }

  // One K/V block on this wave's queries.  MASKED is a compile-time choice
  // so the unmasked stage carries no per-key compare at all.
  auto tile = [&](int j, int buf, auto masked) {
    constexpr bool MASKED = decltype(masked)::value;
    // S^T = K_j Q^T  (keys x queries), fp32 accumulate.
    f32x16 s[QB][C::KB];
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb) {
#pragma unroll
      for (int st = 0; st < C::DS; ++st) {
        const uint4 a =
            *reinterpret_cast<const uint4*>(&k_lds[buf][(32 * kb + n) * C::KROW + 16 * st + 8 * g]);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[qb][kb] = mma16(T{}, a, qf[qb][st], st == 0 ? f32x16{} : s[qb][kb]);
      }
    }
    // Online softmax, then P^T packed to 16-bit as the B operand.
    uint4 pp[QB][C::KB * 2];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int query = qw0 + 32 * qb + n;
      const int key_base = j * BN + 4 * g;
      const int key_lim = CAUSAL ? min(query + 1, N) : N;
      const float mt = tile_max<C::KB, MASKED>(s[qb], qk_scale, key_base, key_lim);
      float alpha;
      if (raise_max(mt, m_run[qb], l_run[qb], &alpha)) {
#pragma unroll
        for (int db = 0; db < C::DB; ++db) oacc[qb][db] *= alpha;
      }
      const float m_use = (m_run[qb] == kNegInf) ? 0.f : m_run[qb];
      l_run[qb] += tile_exp<C::KB, MASKED>(s[qb], qk_scale, m_use, key_base, key_lim);
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const f32x16& v = s[qb][kb];
          pp[qb][2 * kb + h] = make_uint4(pack2(T{}, v[8 * h + 0], v[8 * h + 1]), pack2(T{}, v[8 * h + 2], v[8 * h + 3]),
                                          pack2(T{}, v[8 * h + 4], v[8 * h + 5]), pack2(T{}, v[8 * h + 6], v[8 * h + 7]));
        }
      }
    }
    // O^T += V_j^T P^T  (d x queries), accumulator as C operand.
#pragma unroll
    for (int kk = 0; kk < C::KB * 2; ++kk) {
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        const uint4 a =
            *reinterpret_cast<const uint4*>(&v_lds[buf][(32 * db + n) * C::VROW + 16 * kk + 8 * g]);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) oacc[qb][db] = mma16(T{}, a, pp[qb][kk], oacc[qb][db]);
      }
    }
  };

  if (j_end > 0) {
    load_block(0);
    store_block(0);
  }
  __syncthreads();

  int j = 0;
  for (; j < j_unm; ++j) {  // unmasked stage: every wave, every key visible
    const int buf = j & 1;
    const bool more = j + 1 < j_end;
    if (more) load_block(j + 1);
    tile(j, buf, std::false_type{});
    if (more) store_block(buf ^ 1);
    __syncthreads();
  }
  for (; j < j_end; ++j) {  // masked stage: diagonal blocks and the sequence tail
    const int buf = j & 1;
    const bool more = j + 1 < j_end;
    if (more) load_block(j + 1);
    if (wave_live && (!CAUSAL || j < w_s2)) tile(j, buf, std::true_type{});
    if (more) store_block(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: one divide per row, store O and the natural-log LSE ------
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int query = qw0 + 32 * qb + n;
    const float l_tot = halves_sum(l_run[qb]);
    const float inv = 1.f / l_tot;
    if (query < N) {
      uint16_t* orow = og + head + (size_t)query * D;
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const f32x16& v = oacc[qb][db];
          const uint2 w = make_uint2(pack2(T{}, v[4 * rq + 0] * inv, v[4 * rq + 1] * inv),
                                     pack2(T{}, v[4 * rq + 2] * inv, v[4 * rq + 3] * inv));
          *reinterpret_cast<uint2*>(orow + 32 * db + 8 * rq + 4 * g) = w;
        }
      }
      if (g == 0) lseg[(size_t)bh * N + query] = (m_run[qb] + __log2f(l_tot)) * kLn2;
    }
  }
}

// ===========================================================================
// fp32 forward: same structure on v_mfma_f32_32x32x2_f32, P kept in fp32.
// ===========================================================================
template <int D, int BN, int NW, bool CAUSAL>
struct Fwd32 {
  static constexpr int NT = NW * 64;
  static constexpr int BM = NW * 32;
  static constexpr int KROW = D + 2;   // floats; column reads hit 64 distinct banks
  static constexpr int VROW = D + 8;   // floats; the two halves read disjoint banks
  static constexpr int KB = BN / 32;
  static constexpr int DB = D / 32;
  static constexpr int KCH = BN * D / 4;  // float4 chunks per block
  static constexpr int LD = KCH / NT;
  static_assert(KCH % NT == 0, "block must split evenly over threads");
};

template <int D, int BN, int NW, bool CAUSAL>
__global__ __launch_bounds__(NW * 64) void fwd32_kernel(const float* __restrict__ qg, const float* __restrict__ kg,
                                                        const float* __restrict__ vg, float* __restrict__ og,
                                                        float* __restrict__ lseg, int N, int n_qblk,
                                                        float qk_scale, float qsign) {
  using C = Fwd32<D, BN, NW, CAUSAL>;
  __shared__ __attribute__((aligned(16))) float k_lds[2][BN * C::KROW];
  __shared__ __attribute__((aligned(16))) float v_lds[2][BN * C::VROW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 31;
  const int g = lane >> 5;

  int bh, qblk;
  tile_of(xcd_remap(blockIdx.x, gridDim.x), n_qblk, CAUSAL, &bh, &qblk);
  const size_t head = (size_t)bh * (size_t)N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 4;
  const rsrc_t qrs = make_rsrc(qg + head, head_bytes);
  const rsrc_t krs = make_rsrc(kg + head, head_bytes);
  const rsrc_t vrs = make_rsrc(vg + head, head_bytes);
  const int q0 = qblk * C::BM;
  const int qw0 = q0 + wave * 32;
  const int query = qw0 + n;

  // B operand of S^T: lane supplies Q[query][2 s + g] (zeros past N).
  float qf[D / 2];
#pragma unroll
  for (int s = 0; s < D / 2; ++s) qf[s] = load4f(qrs, ((uint32_t)query * D + 2 * s + g) * 4) * qsign;

  const int n_kv = (N + BN - 1) / BN;
  const int full_blocks = N / BN;
  int j_end = n_kv, j_unm = full_blocks;
  if (CAUSAL) {
    j_end = min(n_kv, (min(q0 + C::BM, N) - 1) / BN + 1);
    int s1, s2;
    causal_stages(q0, min(q0 + C::BM, N), BN, &s1, &s2);
    j_unm = min(s1, full_blocks);
  }
  int w_s2 = n_kv;
  const bool wave_live = qw0 < N;
  if (CAUSAL && wave_live) {
    int w_s1;
    causal_stages(qw0, min(qw0 + 32, N), BN, &w_s1, &w_s2);
  }

  float4 kst[C::LD], vst[C::LD];
  auto load_block = [&](int j) {
#pragma unroll
    for (int i = 0; i < C::LD; ++i) {
      const int c = tid + i * C::NT;
      const uint32_t row = j * BN + c / (D / 4), col = (c % (D / 4)) * 4;
      kst[i] = load16f(krs, (row * D + col) * 4);
      vst[i] = load16f(vrs, (row * D + col) * 4);
    }
  };
  auto store_block = [&](int buf) {
#pragma unroll
    for (int i = 0; i < C::LD; ++i) {
      const int c = tid + i * C::NT;
      const int row = c / (D / 4), col = (c % (D / 4)) * 4;
      float2* kd = reinterpret_cast<float2*>(&k_lds[buf][row * C::KROW + col]);
      kd[0] = make_float2(kst[i].x, kst[i].y);
      kd[1] = make_float2(kst[i].z, kst[i].w);
      *reinterpret_cast<float4*>(&v_lds[buf][row * C::VROW + col]) = vst[i];
    }
  };

  f32x16 oacc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) oacc[db] = f32x16{};
  float m_run = kNegInf, l_run = 0.f;

  auto tile = [&](int j, int buf, auto masked) {
    constexpr bool MASKED = decltype(masked)::value;
    f32x16 s[C::KB];
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb) {
      s[kb] = f32x16{};
#pragma unroll
      for (int st = 0; st < D / 2; ++st)
        s[kb] = mma32(k_lds[buf][(32 * kb + n) * C::KROW + 2 * st + g], qf[st], s[kb]);
    }
    const int key_base = j * BN + 4 * g;
    const int key_lim = CAUSAL ? min(query + 1, N) : N;
    const float mt = tile_max<C::KB, MASKED>(s, qk_scale, key_base, key_lim);
    float alpha;
    if (raise_max(mt, m_run, l_run, &alpha)) {
#pragma unroll
      for (int db = 0; db < C::DB; ++db) oacc[db] *= alpha;
    }
    const float m_use = (m_run == kNegInf) ? 0.f : m_run;
    l_run += tile_exp<C::KB, MASKED>(s, qk_scale, m_use, key_base, key_lim);
    // O^T += V^T P^T: k-step r of key block kb uses key 32 kb + 8(r/4) + 4g + r%4
    // on both operands (the accumulator register r and the V row read).
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 32 * kb + 8 * (r / 4) + 4 * g + (r % 4);
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
          oacc[db] = mma32(v_lds[buf][key * C::VROW + 32 * db + n], s[kb][r], oacc[db]);
      }
    }
  };

  if (j_end > 0) {
    load_block(0);
    store_block(0);
  }
  __syncthreads();
  int j = 0;
  for (; j < j_unm; ++j) {
    const int buf = j & 1;
    const bool more = j + 1 < j_end;
    if (more) load_block(j + 1);
    tile(j, buf, std::false_type{});
    if (more) store_block(buf ^ 1);
    __syncthreads();
  }
  for (; j < j_end; ++j) {
    const int buf = j & 1;
    const bool more = j + 1 < j_end;
    if (more) load_block(j + 1);
    if (wave_live && (!CAUSAL || j < w_s2)) tile(j, buf, std::true_type{});
    if (more) store_block(buf ^ 1);
    __syncthreads();
  }

  const float l_tot = halves_sum(l_run);
  const float inv = 1.f / l_tot;
  if (query < N) {
    float* orow = og + head + (size_t)query * D;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const f32x16& v = oacc[db];
        *reinterpret_cast<float4*>(orow + 32 * db + 8 * rq + 4 * g) =
            make_float4(v[4 * rq] * inv, v[4 * rq + 1] * inv, v[4 * rq + 2] * inv, v[4 * rq + 3] * inv);
      }
    if (g == 0) lseg[(size_t)bh * N + query] = (m_run + __log2f(l_tot)) * kLn2;
  }
}

// ===========================================================================
// launchers
// ===========================================================================
namespace {

// Tile per head dim: 8 waves x 32 queries (two waves per SIMD, so one wave's
// softmax overlaps the other's matrix products), 64 keys per block for
// d = 128 and 128 for d = 64.  Must agree with fwd_tile() in fa_plan.hpp.
template <int D>
struct Tile16 {
  static constexpr int BN = D == 128 ? 64 : 128, NW = 8, QB = 1;
};

template <typename T, int D, bool CAUSAL>
hipError_t launch16(const FwdArgs& a) {
  constexpr int BN = Tile16<D>::BN, NW = Tile16<D>::NW, QB = Tile16<D>::QB;
  using C = Fwd16<T, D, BN, NW, QB, CAUSAL>;
  const int n_qblk = (a.N + C::BM - 1) / C::BM;
  const long long grid = (long long)n_qblk * a.BH;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fwd16_kernel<T, D, BN, NW, QB, CAUSAL>), dim3((unsigned)grid), dim3(C::NT), 0, a.stream,
                     static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                     static_cast<const uint16_t*>(a.v), static_cast<uint16_t*>(a.o), a.lse, a.N, n_qblk,
                     a.qk_scale, a.neg ? 0x80008000u : 0u);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch32(const FwdArgs& a) {
  constexpr int BN = 64, NW = 4;
  using C = Fwd32<D, BN, NW, CAUSAL>;
  const int n_qblk = (a.N + C::BM - 1) / C::BM;
  const long long grid = (long long)n_qblk * a.BH;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fwd32_kernel<D, BN, NW, CAUSAL>), dim3((unsigned)grid), dim3(C::NT), 0, a.stream,
                     static_cast<const float*>(a.q), static_cast<const float*>(a.k), static_cast<const float*>(a.v),
                     static_cast<float*>(a.o), a.lse, a.N, n_qblk, a.qk_scale, a.neg ? -1.f : 1.f);
  return hipGetLastError();
}

template <typename T>
hipError_t dispatch16(const FwdArgs& a) {
  if (a.d == 64) return a.causal ? launch16<T, 64, true>(a) : launch16<T, 64, false>(a);
  return a.causal ? launch16<T, 128, true>(a) : launch16<T, 128, false>(a);
}

}  // namespace

hipError_t launch_fwd(const FwdArgs& a) {
  switch (a.dtype) {
    case 0:
      if (a.d == 64) return a.causal ? launch32<64, true>(a) : launch32<64, false>(a);
      return a.causal ? launch32<128, true>(a) : launch32<128, false>(a);
    case 1: return dispatch16<F16>(a);
    default: return dispatch16<BF16>(a);
  }
}

}  // namespace fa
