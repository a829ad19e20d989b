// fa_bwd.hip -- exact-attention backward with recomputation, for gfx950.
//
// Three launches on one stream ("Triton 06: Flash Attention v2",
// wonbeomjang.kr, "Backward" and the forward/backward flow summary; "Flash
// Attention: IO-awareness principle", hrletsgo.me, "Recomputation"):
//   1. Delta_i = rowsum(dO_i * O_i)
//   2. dK/dV: one workgroup per block of keys, looping over query blocks;
//      P recomputed from the saved LSE, dV += P^T dO,
//      dS = P * (dO V^T - Delta), dK += scale * dS^T Q
//   3. dQ:    one workgroup per block of queries, looping over key blocks;
//      dQ += scale * dS K
// No N x N matrix is stored and no atomics are used: every output element
// is written by exactly one workgroup, so results are deterministic.
//
// Layout choices on gfx950 (the pages show no code for these kernels):
// * dK/dV computes S = Q K^T (queries x keys) so each lane owns one key:
//   the fp32 accumulators of P and dS, packed to 16-bit, are directly the A
//   operand of the dV and dK products, whose B operands (dO and Q with the
//   queries as contraction index) come from transposed LDS copies whose
//   query order matches the accumulator registers.
// * dQ computes S^T (keys x queries) like the forward, so each lane owns one
//   query; dS^T is the B operand of dQ^T = K^T dS^T with K^T in LDS.
// * Per-query LSE and Delta are lane-local in dQ and read from LDS (four
//   16-byte broadcast reads per 32 queries) in dK/dV.
// * The next query/key block is loaded into registers while the current one
//   computes; LDS is double-buffered with one barrier per block.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fa_device.hpp"
#include "fa_kernels.hpp"
#include "fa_plan.hpp"

namespace fa {
namespace {

constexpr float kPosInf = __builtin_huge_valf();

template <typename T>
__device__ __forceinline__ uint4 pack8(T, const f32x16& v, int h) {
  return make_uint4(pack2(T{}, v[8 * h + 0], v[8 * h + 1]), pack2(T{}, v[8 * h + 2], v[8 * h + 3]),
                    pack2(T{}, v[8 * h + 4], v[8 * h + 5]), pack2(T{}, v[8 * h + 6], v[8 * h + 7]));
}

// ---------------------------------------------------------------------------
// 1. Delta_i = sum_c dO_ic O_ic (fp32), D/8 lanes per row.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(const uint16_t* __restrict__ og,
                                                        const uint16_t* __restrict__ dog,
                                                        float* __restrict__ delta, long long rows) {
  constexpr int LPR = D / 8, RPB = 256 / LPR;
  const long long row = (long long)blockIdx.x * RPB + threadIdx.x / LPR;
  const int c = threadIdx.x % LPR;
  float acc = 0.f;
  if (row < rows) {
    const uint4 a = *reinterpret_cast<const uint4*>(og + row * D + 8 * c);
    const uint4 b = *reinterpret_cast<const uint4*>(dog + row * D + 8 * c);
    const uint32_t wa[4] = {a.x, a.y, a.z, a.w}, wb[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc = __builtin_fmaf(lo16(T{}, wa[i]), lo16(T{}, wb[i]), acc);
      acc = __builtin_fmaf(hi16(T{}, wa[i]), hi16(T{}, wb[i]), acc);
    }
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < rows && c == 0) delta[row] = acc;
}

// ---------------------------------------------------------------------------
// 2. dK, dV.  A workgroup owns NP groups of 32 keys and loops over 32-query
// blocks.  Each key group is served by a pair of waves on one SIMD with
// split roles, two of the four products each:
//   wave A (waves 0..NP-1):  S = Q K^T, P = exp2(S*c - LSE2), dV += P^T dO
//   wave B (waves NP..2NP-1): dP = dO V^T, dS = P * (dP - Delta), dK += dS^T Q
// B runs one query block behind A: in iteration i, A works on block i while
// B works on block i-1, whose P (fp32, lane-private LDS slots) A wrote in
// iteration i-1.  So the two waves of a SIMD never wait for each other
// inside an iteration, and A's exponentials overlap B's products.
// Q, dO, LSE and Delta go from global memory straight into LDS (no
// registers), two blocks ahead, through four slots: A's block, B's block and
// the two blocks in flight.  P cycles through two buffers.  One barrier per
// iteration, which waits only for the older block in flight.  A negative
// scale is applied by negating K, so Q lands in LDS unchanged.
// ---------------------------------------------------------------------------
template <int D>
struct KV {
  static constexpr int NP = 4, NW = 2 * NP, NT = 64 * NW, KW = 32, BNK = NP * KW, BMQ = 32;
  static constexpr int DS = D / 16, DB = D / 32, CPR = D / 8;
  static constexpr int RPL = 64 / CPR;            // tile rows per 1 KB wave load
  static constexpr int PPA = BMQ / RPL;           // 1 KB pieces per Q (or dO) block
  static constexpr int LPB = 2 * PPA / NW;        // pieces per wave per block
  static_assert(LPB >= 1 && 2 * PPA == LPB * NW, "staging split");
};

// Uniform state of one dK/dV wave.
struct KVWave {
  int wave, lane, n, g, pw, kw0, N;
  bool role_a;
  float qk_scale;
  rsrc_t qrs, dors, lrs, drs;
};

// Issue the loads of query block i into LDS: piece t = wave LPB + e covers
// tile rows (t % PPA) RPL .. + RPL of Q (t < PPA) or of dO; lane l fills LDS
// bytes 16 l of the piece, i.e. tile row l / CPR and stored chunk l % CPR,
// which holds the row's logical chunk (l % CPR) ^ swz_chunk(row).  Waves 0
// and 1 also load LSE and Delta.  Returns nothing; the caller counts loads.
template <int D>
__device__ __forceinline__ void kv_issue(const KVWave& w, int i, uint16_t* __restrict__ q_dst,
                                         uint16_t* __restrict__ do_dst, float* __restrict__ l_dst,
                                         float* __restrict__ d_dst) {
  using C = KV<D>;
  const int lrow = w.lane / C::CPR;
#pragma unroll
  for (int e = 0; e < C::LPB; ++e) {
    const int t = w.wave * C::LPB + e;
    const bool is_q = t < C::PPA;  // wave-uniform
    const int row = (t % C::PPA) * C::RPL + lrow;
    const int chunk = (w.lane % C::CPR) ^ swz_chunk<D>(row);
    const uint32_t off = ((uint32_t)(i * C::BMQ + row) * D + 8 * chunk) * 2;
    const int piece = (t % C::PPA) * C::RPL * D;
    if (is_q) load_lds16(w.qrs, q_dst + piece, off);
    else load_lds16(w.dors, do_dst + piece, off);
  }
  if (w.wave == 0) load_lds4(w.lrs, l_dst, (uint32_t)(i * C::BMQ + w.lane) * 4);
  if (w.wave == 1) load_lds4(w.drs, d_dst, (uint32_t)(i * C::BMQ + w.lane) * 4);
}

// One iteration of a wave's work.  Every LDS tile it touches arrives as a
// distinct __restrict__ pointer, which tells the compiler that the loads it
// issues into the next slots do not alias what it reads this iteration, so
// it does not wait for those loads before each read.
template <typename T, int D, bool CAUSAL>
__device__ __forceinline__ void kv_iter(
    const KVWave& w, int i, bool work, bool ahead, const uint4 (&kv)[KV<D>::DS], f32x16 (&acc)[KV<D>::DB],
    const uint16_t* __restrict__ lhs, const uint16_t* __restrict__ rhs, const float* __restrict__ rowv,
    float4* __restrict__ x_out, const float4* __restrict__ x_in, uint16_t* __restrict__ nq,
    uint16_t* __restrict__ ndo, float* __restrict__ nl, float* __restrict__ nd) {
  using C = KV<D>;
  if (ahead) kv_issue<D>(w, i + 2, nq, ndo, nl, nd);
  if (!work) return;
  const int n = w.n, g = w.g, lane = w.lane;
  // Register r of the 32x32 accumulator is query 8 (r/4) + 4 g + r%4 of the
  // block; the lane's key is kw0 + n.  A chain's LDS operands are all
  // requested before its first product, and the second chain's transposed
  // operands before the vector work; the fences keep them there.
  uint4 ra[C::DS];
#pragma unroll
  for (int st = 0; st < C::DS; ++st) ra[st] = read_row<D>(lhs, n, 16 * st + 8 * g);
  float4 v4[4], p4[4];
#pragma unroll
  for (int rq = 0; rq < 4; ++rq) {
    v4[rq] = *reinterpret_cast<const float4*>(&rowv[8 * rq + 4 * g]);  // A: LSE, B: Delta
    if (!w.role_a) p4[rq] = x_in[64 * rq + lane];
  }
  __builtin_amdgcn_sched_barrier(0);
  f32x16 sd = f32x16{};  // A: S, B: dP
#pragma unroll
  for (int st = 0; st < C::DS; ++st) sd = mma16(T{}, ra[st], kv[st], sd);
  uint4 rb[2 * C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) {
    rb[2 * db] = read_tr<D>(rhs, 0, 32 * db, lane);
    rb[2 * db + 1] = read_tr<D>(rhs, 16, 32 * db, lane);
  }
  __builtin_amdgcn_sched_barrier(0);
  if (w.role_a) {
    const int q_first = i * C::BMQ;
    const bool need_mask = CAUSAL && q_first < w.kw0 + C::KW - 1;
    const int key = w.kw0 + n;
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const float lv[4] = {v4[rq].x, v4[rq].y, v4[rq].z, v4[rq].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // P = exp2(s |scale| log2 e - LSE log2 e).  A query past the end has
        // Q, dO and Delta all zero (LSE reads as 0), so its P adds nothing.
        float p = fast_exp2(__builtin_fmaf(sd[4 * rq + e], w.qk_scale, -lv[e] * kLog2e));
        if (need_mask) p = (key <= q_first + 8 * rq + 4 * g + e) ? p : 0.f;
        sd[4 * rq + e] = p;
      }
      x_out[64 * rq + lane] = make_float4(sd[4 * rq], sd[4 * rq + 1], sd[4 * rq + 2], sd[4 * rq + 3]);
    }
  } else {
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const float dv4[4] = {v4[rq].x, v4[rq].y, v4[rq].z, v4[rq].w};
      const float pv[4] = {p4[rq].x, p4[rq].y, p4[rq].z, p4[rq].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) sd[4 * rq + e] = pv[e] * (sd[4 * rq + e] - dv4[e]);
    }
  }
  const uint4 pk0 = pack8(T{}, sd, 0), pk1 = pack8(T{}, sd, 1);
#pragma unroll
  for (int db = 0; db < C::DB; ++db) {
    acc[db] = mma16(T{}, pk0, rb[2 * db], acc[db]);
    acc[db] = mma16(T{}, pk1, rb[2 * db + 1], acc[db]);
  }
}

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(512) void bwd_dkdv_kernel(
    const uint16_t* __restrict__ qg, const uint16_t* __restrict__ kg, const uint16_t* __restrict__ vg,
    const uint16_t* __restrict__ dog, const float* __restrict__ lseg, const float* __restrict__ deltag,
    float* __restrict__ dkg, float* __restrict__ dvg, int N, int n_kblk, int BH, float qk_scale,
    float dk_scale, uint32_t ksign) {
  using C = KV<D>;
  __shared__ __attribute__((aligned(16))) uint16_t q_lds[4][C::BMQ * D];   // swizzled row-major
  __shared__ __attribute__((aligned(16))) uint16_t do_lds[4][C::BMQ * D];
  __shared__ __attribute__((aligned(16))) float4 x_lds[2][C::NP][4 * 64];  // P, A -> B
  __shared__ __attribute__((aligned(16))) float lse_lds[4][64];            // raw LSE (first BMQ used)
  __shared__ __attribute__((aligned(16))) float dl_lds[4][64];

  KVWave w;
  w.lane = threadIdx.x & 63;
  w.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform, in a scalar register
  w.n = w.lane & 31;
  w.g = w.lane >> 5;
  w.role_a = w.wave < C::NP;
  w.pw = w.wave % C::NP;  // key group; waves pw and pw + NP share a SIMD
  w.N = N;
  w.qk_scale = qk_scale;
  // One block of BNK keys of one (batch, head), start to finish.
  auto block = [&](int bh, int kblk) __attribute__((always_inline)) {
  const size_t head = (size_t)bh * (size_t)N * D;
  const uint32_t head_bytes = (uint32_t)((size_t)N * D * 2);
  w.qrs = make_rsrc(qg + head, head_bytes);
  w.dors = make_rsrc(dog + head, head_bytes);
  w.lrs = make_rsrc(lseg + (size_t)bh * N, (uint32_t)N * 4);
  w.drs = make_rsrc(deltag + (size_t)bh * N, (uint32_t)N * 4);
  w.kw0 = kblk * C::BNK + w.pw * C::KW;  // first key of this pair
  const bool pair_live = w.kw0 < N;

  // A holds K (sign-flipped for a negative scale), B holds V, as the B
  // operand of Q K^T / dO V^T: kv[s] = row kw0 + n, columns 16 s + 8 g .. + 8.
  uint4 kv[C::DS];
  {
    const rsrc_t rs = make_rsrc((w.role_a ? kg : vg) + head, head_bytes);
    const uint32_t sgn = w.role_a ? ksign : 0u;
#pragma unroll
    for (int s = 0; s < C::DS; ++s) {
      const uint4 a = load16(rs, ((uint32_t)(w.kw0 + w.n) * D + 16 * s + 8 * w.g) * 2);
      kv[s] = make_uint4(a.x ^ sgn, a.y ^ sgn, a.z ^ sgn, a.w ^ sgn);
    }
  }
  f32x16 acc[C::DB];  // A: dV, B: dK (unscaled); rows = keys, columns = d
#pragma unroll
  for (int db = 0; db < C::DB; ++db) acc[db] = f32x16{};

  const int n_qblk = (N + C::BMQ - 1) / C::BMQ;
  const int i_lo = CAUSAL ? (kblk * C::BNK) / C::BMQ : 0;
  auto block_active = [&](int i) {
    return pair_live && (!CAUSAL || min((i + 1) * C::BMQ, N) - 1 >= w.kw0);
  };
  // Loads this wave issues per block (the barrier count below depends on it).
  const bool extra = w.wave < 2;

  wait_vmem();  // K or V fragments above
  kv_issue<D>(w, i_lo, q_lds[i_lo & 3], do_lds[i_lo & 3], lse_lds[i_lo & 3], dl_lds[i_lo & 3]);
  if (i_lo + 1 < n_qblk) {
    const int s1 = (i_lo + 1) & 3;
    kv_issue<D>(w, i_lo + 1, q_lds[s1], do_lds[s1], lse_lds[s1], dl_lds[s1]);
    if (extra) lds_barrier<C::LPB + 1>();
    else lds_barrier<C::LPB>();
  } else {
    lds_barrier<0>();
  }

  // Iteration i: A works on block i (slot i & 3), B on block i - 1 (slot
  // (i - 1) & 3); block i + 2 is loaded into slot (i + 2) & 3, whose last
  // reader (B, block i - 2) finished before the previous barrier.
  for (int i = i_lo; i <= n_qblk; ++i) {
    const bool ahead = i + 2 < n_qblk;
    const int sa = i & 3, sb = (i - 1) & 3, sn = (i + 2) & 3;
    const bool work = w.role_a ? (i < n_qblk && block_active(i)) : (i > i_lo && block_active(i - 1));
    const int s_own = w.role_a ? sa : sb;
    kv_iter<T, D, CAUSAL>(w, i, work, ahead, kv, acc,
                          w.role_a ? q_lds[s_own] : do_lds[s_own],   // row-read operand
                          w.role_a ? do_lds[s_own] : q_lds[s_own],   // transposed-read operand
                          w.role_a ? lse_lds[s_own] : dl_lds[s_own],
                          x_lds[i & 1][w.pw], x_lds[(i - 1) & 1][w.pw],
                          q_lds[sn], do_lds[sn], lse_lds[sn], dl_lds[sn]);
    // Block i + 1 (loaded one iteration ago) must be in LDS after this barrier;
    // block i + 2's loads may stay in flight.
    if (!ahead) lds_barrier<0>();
    else if (extra) lds_barrier<C::LPB + 1>();
    else lds_barrier<C::LPB>();
  }

  // Register r of d block db is key kw0 + 8(r/4) + 4g + r%4, column 32 db + n.
  float* out = (w.role_a ? dvg : dkg) + head;
  const float sc = w.role_a ? 1.f : dk_scale;
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kr = w.kw0 + 8 * (r / 4) + 4 * w.g + (r % 4);
      if (kr < N) out[(size_t)kr * D + 32 * db + w.n] = acc[db][r] * sc;
    }
  };

  // Persistent loop over equal-cost items (items_per_head / item_blocks);
  // in each round every XCD works on a contiguous range of items.  The
  // heavier key block of a causal pair (the lower one) goes first.
  const int per_head = items_per_head(n_kblk, CAUSAL);
  const int n_items = BH * per_head;
  for (int L = xcd_remap(blockIdx.x, gridDim.x); L < n_items; L += gridDim.x) {
    const int bh = L / per_head;
    int lo, hi;
    const int nb = item_blocks(L % per_head, n_kblk, CAUSAL, &lo, &hi);
    for (int t = 0; t < nb; ++t) {
      block(bh, t == 0 ? lo : hi);
      __syncthreads();  // the next block reuses the LDS buffers
    }
  }
}

// ---------------------------------------------------------------------------
// 3. dQ.  Workgroup = 8 waves x 32 queries (two waves per SIMD); inner loop
// over 64-key blocks, each taken as two 32-key sub-blocks.  K and V sit
// row-major (swizzled) in LDS: rows feed S^T = K Q^T and dP^T = V dO^T,
// transposing reads give K^T for dQ^T += K^T dS^T.
// ---------------------------------------------------------------------------
template <int D>
struct QG {
  static constexpr int NW = 8, NT = 64 * NW, BM = NW * 32, BN = 64;
  static constexpr int DS = D / 16, DB = D / 32, KB = BN / 32, CPR = D / 8;
  static constexpr int LDC = BN * CPR / NT;  // 16-byte chunks of K (and of V) per thread per block
  static_assert(LDC >= 1 && BN * CPR % NT == 0, "staging split");
};

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(512) void bwd_dq_kernel(
    const uint16_t* __restrict__ qg, const uint16_t* __restrict__ kg, const uint16_t* __restrict__ vg,
    const uint16_t* __restrict__ dog, const float* __restrict__ lseg, const float* __restrict__ deltag,
    float* __restrict__ dqg, int N, int n_qblk, int BH, float qk_scale, float dq_scale, uint32_t qsign) {
  using C = QG<D>;
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[2][C::BN * D];  // swizzled row-major
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[2][C::BN * D];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, n = lane & 31, g = lane >> 5;
  // One block of BM queries of one (batch, head), start to finish.
  auto qblock = [&](int bh, int qblk) __attribute__((always_inline)) {
  const size_t head = (size_t)bh * (size_t)N * D;
  const uint32_t head_bytes = (uint32_t)((size_t)N * D * 2);
  const rsrc_t krs = make_rsrc(kg + head, head_bytes), vrs = make_rsrc(vg + head, head_bytes);
  const int q0 = qblk * C::BM;
  const int qw0 = q0 + wave * 32;
  const int query = qw0 + n;

  // Q and dO of this lane's query as the B operands (zero past the end).
  uint4 qf[C::DS], dof[C::DS];
  {
    const rsrc_t qrs = make_rsrc(qg + head, head_bytes), dors = make_rsrc(dog + head, head_bytes);
#pragma unroll
    for (int s = 0; s < C::DS; ++s) {
      const uint32_t off = ((uint32_t)query * D + 16 * s + 8 * g) * 2;
      uint4 a = load16(qrs, off);
      a.x ^= qsign; a.y ^= qsign; a.z ^= qsign; a.w ^= qsign;
      qf[s] = a;
      dof[s] = load16(dors, off);
    }
  }
  const float lse2 = query < N ? lseg[(size_t)bh * N + query] * kLog2e : kPosInf;
  const float dl = query < N ? deltag[(size_t)bh * N + query] : 0.f;

  f32x16 dq[C::DB];  // dQ^T: rows = d, columns = queries
#pragma unroll
  for (int db = 0; db < C::DB; ++db) dq[db] = f32x16{};

  const int n_kv = (N + C::BN - 1) / C::BN;
  int j_end = n_kv;
  if (CAUSAL) j_end = min(n_kv, (min(q0 + C::BM, N) - 1) / C::BN + 1);
  int w_s1 = n_kv, w_s2 = n_kv;
  const bool wave_live = qw0 < N;
  if (CAUSAL && wave_live) causal_stages(qw0, min(qw0 + 32, N), C::BN, &w_s1, &w_s2);
  const int full_blocks = N / C::BN;
  const int key_lim = CAUSAL ? min(query + 1, N) : N;

  uint4 ks[C::LDC], vs[C::LDC];
  auto load_block = [&](int j) {
#pragma unroll
    for (int e = 0; e < C::LDC; ++e) {
      const int c = tid + e * C::NT;
      const uint32_t off = ((uint32_t)(j * C::BN + c / C::CPR) * D + 8 * (c % C::CPR)) * 2;
      ks[e] = load16(krs, off);
      vs[e] = load16(vrs, off);
    }
  };
  auto store_block = [&](int buf) {
#pragma unroll
    for (int e = 0; e < C::LDC; ++e) {
      const int c = tid + e * C::NT;
      const int off = swz<D>(c / C::CPR, 8 * (c % C::CPR));
      *reinterpret_cast<uint4*>(&k_lds[buf][off]) = ks[e];
      *reinterpret_cast<uint4*>(&v_lds[buf][off]) = vs[e];
    }
  };

  if (j_end > 0) {
    load_block(0);
    store_block(0);
  }
  wait_vmem();  // Q, dO fragments above
  __syncthreads();

  // Blocks [0, j_unm) need no mask for this wave (every key visible to all
  // its queries, none past the end); the rest are masked per key.  The two
  // stages are separate loops with the mask fixed at compile time; every
  // iteration of either ends in the same barrier, so all waves of the
  // workgroup still meet at each block.
  const int j_unm = min(CAUSAL ? w_s1 : n_kv, full_blocks);
  auto block = [&](int j, auto masked) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked)::value;
    const int buf = j & 1;
    const bool more = j + 1 < j_end;
    if (more) load_block(j + 1);
    const bool active = wave_live && (!CAUSAL || j < w_s2);
    if (active) {
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb) {
        f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int st = 0; st < C::DS; ++st) {
          s = mma16(T{}, read_row<D>(k_lds[buf], 32 * kb + n, 16 * st + 8 * g), qf[st], s);
          dp = mma16(T{}, read_row<D>(v_lds[buf], 32 * kb + n, 16 * st + 8 * g), dof[st], dp);
        }
        // Register r is key j BN + 32 kb + 8(r/4) + 4g + r%4.
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = fast_exp2(__builtin_fmaf(s[r], qk_scale, -lse2));
          if constexpr (MASKED) {
            const int kr = j * C::BN + 32 * kb + 8 * (r / 4) + 4 * g + (r % 4);
            p = kr < key_lim ? p : 0.f;
          }
          dp[r] = p * (dp[r] - dl);
        }
        const uint4 ds0 = pack8(T{}, dp, 0), ds1 = pack8(T{}, dp, 1);
        // dQ^T += K^T dS^T over this sub-block's 32 keys (two 16-key chunks).
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          dq[db] = mma16(T{}, read_tr<D>(k_lds[buf], 32 * kb, 32 * db, lane), ds0, dq[db]);
          dq[db] = mma16(T{}, read_tr<D>(k_lds[buf], 32 * kb + 16, 32 * db, lane), ds1, dq[db]);
        }
      }
    }
    if (more) store_block(buf ^ 1);
    __syncthreads();
  };
  int j = 0;
  for (; j < min(j_unm, j_end); ++j) block(j, std::false_type{});
  for (; j < j_end; ++j) block(j, std::true_type{});

  if (query < N) {
    float* row = dqg + head + (size_t)query * D;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const f32x16& v = dq[db];
        *reinterpret_cast<float4*>(row + 32 * db + 8 * rq + 4 * g) =
            make_float4(v[4 * rq] * dq_scale, v[4 * rq + 1] * dq_scale, v[4 * rq + 2] * dq_scale,
                        v[4 * rq + 3] * dq_scale);
      }
  }
  };

  // Persistent loop over equal-cost items, as in the dK/dV pass; the
  // heavier query block of a causal pair (the higher one) goes first.
  const int per_head = items_per_head(n_qblk, CAUSAL);
  const int n_items = BH * per_head;
  for (int L = xcd_remap(blockIdx.x, gridDim.x); L < n_items; L += gridDim.x) {
    const int bh = L / per_head;
    int lo, hi;
    const int nb = item_blocks(L % per_head, n_qblk, CAUSAL, &lo, &hi);
    for (int t = 0; t < nb; ++t) {
      qblock(bh, t + 1 < nb ? hi : lo);
      __syncthreads();  // the next block reuses the LDS buffers
    }
  }
}

// ---------------------------------------------------------------------------
template <typename T, int D, bool CAUSAL>
hipError_t run(const BwdArgs& a, int stage) {
  const long long rows = (long long)a.BH * a.N;
  constexpr int RPB = 256 / (D / 8);
  const long long g1 = (rows + RPB - 1) / RPB;
  const int n_kblk = (a.N + KV<D>::BNK - 1) / KV<D>::BNK;
  const int n_qblk = (a.N + QG<D>::BM - 1) / QG<D>::BM;
  long long g2 = (long long)items_per_head(n_kblk, CAUSAL) * a.BH;
  long long g3 = (long long)items_per_head(n_qblk, CAUSAL) * a.BH;
  if (g1 > 0x7fffffffLL || g2 > 0x7fffffffLL || g3 > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  // dK/dV and dQ run persistent grids of one workgroup per CU (registers
  // allow one 512-thread workgroup per CU), never more than their items.
  int dev = 0, cus = 0;
  hipError_t de = hipGetDevice(&dev);
  if (de == hipSuccess) de = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (de != hipSuccess) return de;
  if (g2 > cus) g2 = cus;
  if (g3 > cus) g3 = cus;
  const float qk_scale = fabsf(a.scale) * kLog2eHost;
  const uint32_t qsign = a.scale < 0.f ? 0x80008000u : 0u;
  const auto* q = static_cast<const uint16_t*>(a.q);
  const auto* k = static_cast<const uint16_t*>(a.k);
  const auto* v = static_cast<const uint16_t*>(a.v);
  const auto* o = static_cast<const uint16_t*>(a.o);
  const auto* dout = static_cast<const uint16_t*>(a.dout);
  if (stage == 0 || stage == 1) {
    hipLaunchKernelGGL((bwd_delta_kernel<T, D>), dim3((unsigned)g1), dim3(256), 0, a.stream, o, dout, a.delta, rows);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (stage == 0 || stage == 2) {
    hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, CAUSAL>), dim3((unsigned)g2), dim3(KV<D>::NT), 0, a.stream, q, k, v, dout,
                       a.lse, a.delta, a.dk, a.dv, a.N, n_kblk, a.BH, qk_scale, a.scale, qsign);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (stage == 0 || stage == 3) {
    hipLaunchKernelGGL((bwd_dq_kernel<T, D, CAUSAL>), dim3((unsigned)g3), dim3(QG<D>::NT), 0, a.stream, q, k, v, dout,
                       a.lse, a.delta, a.dq, a.N, n_qblk, a.BH, qk_scale, a.scale, qsign);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <typename T>
hipError_t dispatch(const BwdArgs& a, int stage) {
  if (a.d == 64) return a.causal ? run<T, 64, true>(a, stage) : run<T, 64, false>(a, stage);
  return a.causal ? run<T, 128, true>(a, stage) : run<T, 128, false>(a, stage);
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& a, int stage) {
  if (a.dtype == 1) return dispatch<F16>(a, stage);
  if (a.dtype == 2) return dispatch<BF16>(a, stage);
  return hipErrorNotSupported;  // fp32 is rejected by the ABI before this point
}

}  // namespace fa
