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
//   queries as contraction index) come from transposing reads of the
//   row-major Q and dO tiles in LDS.
// * dQ computes S^T (keys x queries) like the forward, so each lane owns one
//   query; dS^T is the B operand of dQ^T = K^T dS^T, K^T from transposing
//   reads of the row-major K tile.
// * Per-query LSE and Delta are lane-local in dQ and read from LDS (four
//   16-byte broadcast reads per 32 queries) in dK/dV.
// * Every tile goes from global memory straight into LDS (buffer_load ...
//   lds) through a ring of slots loaded ahead of use: Q/dO blocks in dK/dV
//   (three slots, one block ahead, continuing across blocks), K/V tiles in
//   dQ (four slots, three tiles ahead); both grids are persistent.
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
// 2. dK, dV.  A workgroup owns NP groups of 32 keys and loops over 64-query
// blocks.  Each key group is served by a pair of waves on one SIMD with
// split roles, two of the four products each:
//   wave A (waves 0..NP-1):  S = Q K^T, P = exp2(S*c - LSE2), dV += P^T dO
//   wave B (waves NP..2NP-1): dP = dO V^T, dS = P * (dP - Delta), dK += dS^T Q
// B runs one query block behind A: in iteration i, A works on block i while
// B works on block i-1, whose P A wrote to LDS (fp16) in iteration i-1.  So
// the two waves of a SIMD never wait for each other inside an iteration.
// Each wave takes its block as two 32-query halves in four phases, so the
// vector work of one half runs under the matrix products of the other:
//   A: S0 | S1 + weights P0 | dV(P0) + weights P1 | dV(P1)
//   B: dP0 | dP1 + dS0 | dK(dS0) + dS1 | dK(dS1)
// Q and dO go from global memory straight into LDS (no registers) one
// block ahead through three slots (A's block, B's block, the block in
// flight); waves 0 and 1 stage -LSE log2(e) and -Delta of the block in
// flight.  One barrier
// per iteration.  A negative scale is applied by negating K, so Q lands in
// LDS unchanged.
// ---------------------------------------------------------------------------
template <int D>
struct KV {
  static constexpr int NP = 4, NW = 2 * NP, NT = 64 * NW, KW = 32, BNK = NP * KW, BMQ = 64, NSLOT = 3;
  static constexpr int DS = D / 16, DB = D / 32, CPR = D / 8;
  static constexpr int RPL = 64 / CPR;            // tile rows per 1 KB wave load
  static constexpr int PPA = BMQ / RPL;           // 1 KB pieces per Q (or dO) block
  static constexpr int LPB = 2 * PPA / NW;        // pieces per wave per block
  static_assert(LPB >= 1 && 2 * PPA == LPB * NW, "staging split");
  static_assert(2 * DB == DS, "one product per slot in every phase");
};

// Lane index from the lane masks (no input register), so that the compiler
// can recompute lane-derived values where they are used instead of keeping
// them live across the whole kernel.
__device__ __forceinline__ int lane_id() { return (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

// State of one dK/dV wave: uniform values, and the lane's position.
struct KVWave {
  int wave, pw, kw0, N;
  bool role_a;
  float qk_scale;
  __device__ __forceinline__ int lane() const { return lane_id(); }
  __device__ __forceinline__ int n() const { return lane_id() & 31; }
  __device__ __forceinline__ int g() const { return lane_id() >> 5; }
};
// Buffer resources of the query head a segment reads: Q, dO, LSE, Delta.
struct KVSrc {
  rsrc_t qrs, dors, lrs, drs;
};

// Issue the loads of query block i: piece t = wave LPB + e covers tile rows
// (t % PPA) RPL .. + RPL of Q (t < PPA) or of dO, straight into LDS; lane l
// fills LDS bytes 16 l of the piece, i.e. tile row l / CPR and stored chunk
// l % CPR, which holds the row's logical chunk (l % CPR) ^ swz_chunk(row).
// Wave 0 loads the block's LSE and wave 1 its Delta into a register
// (returned); once it has arrived they store -LSE log2(e) and -Delta into
// LDS (kv_stage_rows).
template <int D>
__device__ __forceinline__ float kv_issue(const KVWave& w, const KVSrc& src, int i, uint16_t* __restrict__ q_dst,
                                          uint16_t* __restrict__ do_dst) {
  using C = KV<D>;
  float val = 0.f;
  if (w.wave == 0) val = load4f(src.lrs, (uint32_t)(i * C::BMQ + w.lane()) * 4);
  if (w.wave == 1) val = load4f(src.drs, (uint32_t)(i * C::BMQ + w.lane()) * 4);
  const int lrow = w.lane() / C::CPR;
#pragma unroll
  for (int e = 0; e < C::LPB; ++e) {
    const int t = w.wave * C::LPB + e;
    const bool is_q = t < C::PPA;  // wave-uniform
    const int row = (t % C::PPA) * C::RPL + lrow;
    const int chunk = (w.lane() % C::CPR) ^ swz_chunk<D>(row);
    const uint32_t off = ((uint32_t)(i * C::BMQ + row) * D + 8 * chunk) * 2;
    const int piece = (t % C::PPA) * C::RPL * D;
    if (is_q) load_lds16(src.qrs, q_dst + piece, off);
    else load_lds16(src.dors, do_dst + piece, off);
  }
  return val;
}
// The per-row values of a block as the waves consume them: -LSE log2(e)
// (added by A's weights) and -Delta (the initial accumulator of B's dP, so
// the dP product yields dP - Delta directly).
__device__ __forceinline__ void kv_stage_rows(const KVWave& w, float val, float* __restrict__ l_dst,
                                              float* __restrict__ d_dst) {
  if (w.wave == 0) l_dst[w.lane()] = -val * kLog2e;
  if (w.wave == 1) d_dst[w.lane()] = -val;
}

// One iteration of a wave's work on its block: four phases over the two
// halves (see above), each of NS slots with one matrix product and a share
// of the other half's vector work; LDS reads run two slots ahead.  Register
// r of a 32x32 accumulator is query 32 h + 8 (r/4) + 4 g + r%4 of the block
// (half h), the lane's key is kw0 + n.  A query past N has Q = 0, LSE = 0
// and dO = Delta = 0, so whatever weight it gets adds nothing.  Every LDS
// tile arrives as a distinct __restrict__ pointer, which tells the compiler
// that the loads issued into the next slot do not alias what is read here,
// so it does not wait for those loads before each read.
template <typename T, int D, bool ROLE_A, bool MASK>
__device__ __forceinline__ void kv_iter(const KVWave& w, int i, const uint4 (&kv)[KV<D>::DS],
                                        f32x16 (&acc)[KV<D>::DB], const uint16_t* __restrict__ lhs,
                                        const uint16_t* __restrict__ rhs, const float* __restrict__ rowv,
                                        uint4* __restrict__ x_out, const uint4* __restrict__ x_in) {
  using C = KV<D>;
  constexpr int NS = C::DS;        // products per phase
  constexpr int EP = 16 / NS;      // accumulator elements of vector work per slot (2 or 4)
  const int n = w.n(), g = w.g(), lane = w.lane();
  const int q_first = i * C::BMQ;
  const int key = w.kw0 + n;

  // Row operand (A: Q, B: dO) fragment k of half h; transposed operand (A:
  // dO, B: Q) fragment k of half h (16-query chunk k / DB, d block k % DB).
  // In the swizzled layout every fragment sits at a per-lane base XOR a
  // constant plus a row offset, because the chunk permutation only touches
  // the low (within-row) address bits: row reads at (R ^ 16 k) + 32 h D,
  // transposing reads at (T ^ 32 (k % DB) [^ 16 for the second 8 rows]) +
  // (32 h + 16 (k / DB) [+ 8]) D, in elements.  The two bases pass through an
  // empty asm so the compiler computes each address next to its read instead
  // of keeping dozens of precomputed addresses live across the loop.
  // (Byte offsets: one XOR per fragment, the row part is the read's
  // immediate offset.)
  uint32_t R = 2u * (uint32_t)swz<D>(n, 8 * g);
  uint32_t Tb = 2u * (uint32_t)swz<D>(4 * g + ((lane & 15) >> 2), 16 * ((lane >> 4) & 1) + 4 * (lane & 3));
  asm volatile("" : "+v"(R), "+v"(Tb));
  const char* lb = reinterpret_cast<const char*>(lhs);
  const char* rb = reinterpret_cast<const char*>(rhs);
  auto rowf = [&](int h, int k) __attribute__((always_inline)) {
    return *reinterpret_cast<const uint4*>(lb + (R ^ (32 * k)) + 64 * h * D);
  };
  auto trf = [&](int h, int k) __attribute__((always_inline)) {
    const uint32_t r0 = 2 * (32 * h + 16 * (k / C::DB)) * D;
    const uint32_t t = Tb ^ (64 * (k % C::DB));
    const uint2 x = read_tr_b64(reinterpret_cast<const uint16_t*>(rb + t + r0));
    const uint2 y = read_tr_b64(reinterpret_cast<const uint16_t*>(rb + (t ^ 32) + r0 + 16 * D));
    return make_uint4(x.x, x.y, y.x, y.y);
  };
  // Per-row values (A: -LSE log2 e, B: Delta) of the elements a slot's
  // vector work touches: elements EP k .. of half h, i.e. rows 32 h +
  // 8 (r/4) + 4 g + r%4; one float4 covers four consecutive elements.
  auto rowv4 = [&](int h, int q) __attribute__((always_inline)) {
    return *reinterpret_cast<const float4*>(&rowv[32 * h + 8 * q + 4 * g]);
  };
  // B: the 16 row values of half h as an accumulator (register r <-> row).
  auto rowacc = [&](int h) __attribute__((always_inline)) {
    f32x16 c;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 x = rowv4(h, q);
      c[4 * q] = x.x; c[4 * q + 1] = x.y; c[4 * q + 2] = x.z; c[4 * q + 3] = x.w;
    }
    return c;
  };
  // fp16 P of half h: 8 words per lane, stored / read in two 16-byte pieces.
  auto put_p = [&](int h, int piece, const uint32_t (&ph)[8]) __attribute__((always_inline)) {
    x_out[(2 * h + piece) * 64 + lane] = make_uint4(ph[4 * piece], ph[4 * piece + 1], ph[4 * piece + 2],
                                                    ph[4 * piece + 3]);
  };
  auto get_p = [&](int h, uint32_t (&ph)[8]) __attribute__((always_inline)) {
    const uint4 x0 = x_in[(2 * h) * 64 + lane], x1 = x_in[(2 * h + 1) * 64 + lane];
    ph[0] = x0.x; ph[1] = x0.y; ph[2] = x0.z; ph[3] = x0.w;
    ph[4] = x1.x; ph[5] = x1.y; ph[6] = x1.z; ph[7] = x1.w;
  };
  // Vector work of slot k on half h (elements r0 = EP k .. r0 + EP - 1).
  //  A: p = exp2(s qk - LSE log2 e) (masked on the diagonal), packed to
  //     16-bit for dV += P^T dO and to fp16 for wave B (stored as soon as a
  //     16-byte piece is complete).
  //  B: dS = P (dP - Delta) with P from the fp16 copy, packed to 16-bit for
  //     dK += dS^T Q.
  auto vec = [&](int h, int k, const f32x16& sd, const float4& v4, uint32_t (&pk)[8], uint32_t (&ph)[8])
      __attribute__((always_inline)) {
    const int r0 = EP * k;
    const float vq[4] = {v4.x, v4.y, v4.z, v4.w};
    const float* v = vq + (r0 % 4);
#pragma unroll
    for (int e = 0; e < EP; e += 2) {
      const int r = r0 + e;
      if constexpr (ROLE_A) {
        float p0 = fast_exp2(__builtin_fmaf(sd[r], w.qk_scale, v[e]));
        float p1 = fast_exp2(__builtin_fmaf(sd[r + 1], w.qk_scale, v[e + 1]));
        if constexpr (MASK) {
          const int q = q_first + 32 * h + 8 * (r / 4) + 4 * g + (r % 4);
          p0 = key <= q ? p0 : 0.f;
          p1 = key <= q + 1 ? p1 : 0.f;
        }
        pk[r / 2] = pack2(T{}, p0, p1);
        ph[r / 2] = pack2(F16{}, p0, p1);
      } else {
        // fp16 P times dP - Delta (the accumulator), one mixed-precision
        // multiply-add each
        const _Float16 h0 = __builtin_bit_cast(_Float16, (uint16_t)(ph[r / 2] & 0xffffu));
        const _Float16 h1 = __builtin_bit_cast(_Float16, (uint16_t)(ph[r / 2] >> 16));
        pk[r / 2] = pack2(T{}, __builtin_fmaf((float)h0, sd[r], 0.f), __builtin_fmaf((float)h1, sd[r + 1], 0.f));
        (void)v;
      }
    }
    if constexpr (ROLE_A) {
      if ((r0 + EP) % 8 == 0) put_p(h, (r0 + EP) / 8 - 1, ph);
    }
  };

  f32x16 s0, s1;
  uint4 a[3], b[3];
  float4 vv[2];  // row values: the float4 in use and the next one
  uint32_t pk0[8], pk1[8], ph0[8], ph1[8];
  constexpr int SPQ = 4 / EP;  // slots per float4 of row values

  // ---- phase 1: the first half's product chain ----------------------------
  a[0] = rowf(0, 0);
  a[1] = rowf(0, 1);
  f32x16 c0 = f32x16{}, c1 = f32x16{};  // initial accumulators (B: -Delta rows)
  if constexpr (!ROLE_A) {
    get_p(0, ph0);
    c0 = rowacc(0);
  }
#pragma unroll
  for (int k = 0; k < NS; ++k) {
    a[(k + 2) % 3] = k + 2 < NS ? rowf(0, k + 2) : rowf(1, k + 2 - NS);
    if constexpr (ROLE_A) {
      if (k == NS - 1) vv[0] = rowv4(0, 0);
    } else {
      if (k == NS - 1) c1 = rowacc(1);
    }
    s0 = mma16(T{}, a[k % 3], kv[k], k == 0 ? c0 : s0);
    __builtin_amdgcn_sched_barrier(0);
  }
  // ---- phase 2: the second half's chain, the first half's vector work ----
  // (The three fragment registers rotate continuously across phases: the
  // first two fragments of a phase were read into slots NS % 3, (NS+1) % 3.)
#pragma unroll
  for (int k = 0; k < NS; ++k) {
    if (k + 2 < NS) a[(NS + k + 2) % 3] = rowf(1, k + 2);
    else b[k + 2 - NS] = trf(0, k + 2 - NS);
    if constexpr (ROLE_A) {
      if (k % SPQ == 0) vv[(k / SPQ + 1) % 2] = k + SPQ < NS ? rowv4(0, (k + SPQ) / SPQ) : rowv4(1, 0);
    } else {
      if (k == NS - 2) get_p(1, ph1);
    }
    s1 = mma16(T{}, a[(NS + k) % 3], kv[k], k == 0 ? c1 : s1);
    vec(0, k, s0, vv[(k / SPQ) % 2], pk0, ph0);
    __builtin_amdgcn_sched_barrier(0);
  }
  // ---- phase 3: the first half's second product, the second half's vector work
  {
    const uint4 pp[2] = {make_uint4(pk0[0], pk0[1], pk0[2], pk0[3]), make_uint4(pk0[4], pk0[5], pk0[6], pk0[7])};
#pragma unroll
    for (int k = 0; k < NS; ++k) {
      b[(k + 2) % 3] = k + 2 < NS ? trf(0, k + 2) : trf(1, k + 2 - NS);
      if constexpr (ROLE_A) {
        if (k % SPQ == 0 && k + SPQ < NS) vv[(k / SPQ + 1) % 2] = rowv4(1, (k + SPQ) / SPQ);
      }
      acc[k % C::DB] = mma16(T{}, pp[k / C::DB], b[k % 3], acc[k % C::DB]);
      vec(1, k, s1, vv[(k / SPQ) % 2], pk1, ph1);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // ---- phase 4: the second half's second product --------------------------
  {
    const uint4 pp[2] = {make_uint4(pk1[0], pk1[1], pk1[2], pk1[3]), make_uint4(pk1[4], pk1[5], pk1[6], pk1[7])};
#pragma unroll
    for (int k = 0; k < NS; ++k) {
      if (k + 2 < NS) b[(NS + k + 2) % 3] = trf(1, k + 2);
      acc[k % C::DB] = mma16(T{}, pp[k / C::DB], b[(NS + k) % 3], acc[k % C::DB]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// GROUPED = false compiles the one-query-head-per-K/V-head case (G = 1)
// without the query-head index, which costs registers.
//
// The workgroup walks a sequence of segments: one block of BNK keys of one
// K/V head together with one query head that reads it (G segments per block
// under GQA), i.e. the query blocks i_lo .. n_qblk - 1 of that head.  With
// wave B one query block behind wave A, a segment takes n_qblk - i_lo + 1
// iterations: in the first only A has products to compute, in the last only
// B.  Segments run back to back without draining: the last iteration loads
// the next segment's first query block, and each wave does its block-change
// work in its idle iteration -- A in the last (store dV, load the next
// block's K), B in the first (store the previous block's dK, load this
// block's V).  The barrier that ends every iteration waits for all loads and
// stores, so that work runs under the other wave's products.
template <typename T, int D, bool CAUSAL, bool GROUPED>
__global__ __launch_bounds__(512) void bwd_dkdv_kernel(
    const uint16_t* __restrict__ qg, const uint16_t* __restrict__ kg, const uint16_t* __restrict__ vg,
    const uint16_t* __restrict__ dog, const float* __restrict__ lseg, const float* __restrict__ deltag,
    float* __restrict__ dkg, float* __restrict__ dvg, int N, int n_kblk, int BHkv, int G,
    float qk_scale, float dk_scale, uint32_t ksign) {
  using C = KV<D>;
  // All of LDS is one variable.  The compiler matches loads into LDS
  // against later LDS reads per variable: with the ring slots of Q in an
  // array of their own, every read of one slot would wait for the loads
  // just issued into the next.  The barriers' explicit waits order the
  // loads and the reads.
  struct Lds {
    uint16_t q[C::NSLOT][C::BMQ * D];   // swizzled row-major
    uint16_t dO[C::NSLOT][C::BMQ * D];
    uint4 x[2][C::NP][4 * 64];          // fp16 P, A -> B
    float lse[C::NSLOT][C::BMQ];        // -LSE log2(e)
    float dl[C::NSLOT][C::BMQ];         // -Delta
  };
  __shared__ __attribute__((aligned(16))) Lds lds;
  auto& q_lds = lds.q;
  auto& do_lds = lds.dO;
  auto& x_lds = lds.x;
  auto& lse_lds = lds.lse;
  auto& dl_lds = lds.dl;

  KVWave w;
  w.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform, in a scalar register
  w.role_a = w.wave < C::NP;
  w.pw = w.wave % C::NP;  // key group; waves pw and pw + NP share a SIMD
  w.N = N;
  w.qk_scale = qk_scale;

  const int n_qblk = (N + C::BMQ - 1) / C::BMQ;
  const uint32_t head_bytes = (uint32_t)((size_t)N * D * 2);
  const int n_group = GROUPED ? G : 1;

  // ---- segment cursor ------------------------------------------------------
  // Persistent walk over equal-cost items (items_per_head / item_blocks) of
  // the K/V heads; in each round every XCD works on a contiguous range of
  // items.  Cursor (L, t, j): item L, its block t (the heavier, lower key
  // block of a causal pair first), query head j of the group.
  struct Seg {
    int bkv, kblk, j;
  };
  const int per_head = items_per_head(n_kblk, CAUSAL);
  const int n_items = BHkv * per_head;
  auto seg_at = [&](int L, int t, int j, Seg& sg) {
    if (L >= n_items) return false;
    int lo, hi;
    item_blocks(L % per_head, n_kblk, CAUSAL, &lo, &hi);
    sg.bkv = L / per_head;
    sg.kblk = t == 0 ? lo : hi;
    sg.j = j;
    return true;
  };
  auto advance = [&](int& L, int& t, int& j) {
    if (++j < n_group) return;
    j = 0;
    int lo, hi;
    if (++t < item_blocks(L % per_head, n_kblk, CAUSAL, &lo, &hi)) return;
    t = 0;
    L += gridDim.x;
  };
  auto qhead_of = [&](const Seg& sg) { return GROUPED ? q_head_of(sg.bkv, G, sg.j) : sg.bkv; };
  // Loads of query block i of query head qh into a ring slot (the buffer
  // resources are rebuilt per call: scalar work, and no live registers).
  auto issue = [&](int qh, int i, uint16_t* __restrict__ q_dst, uint16_t* __restrict__ do_dst)
      __attribute__((always_inline)) {
    KVSrc r;
    r.qrs = make_rsrc(qg + (size_t)qh * N * D, head_bytes);
    r.dors = make_rsrc(dog + (size_t)qh * N * D, head_bytes);
    r.lrs = make_rsrc(lseg + (size_t)qh * N, (uint32_t)N * 4);
    r.drs = make_rsrc(deltag + (size_t)qh * N, (uint32_t)N * 4);
    return kv_issue<D>(w, r, i, q_dst, do_dst);
  };
  auto first_qblk = [&](const Seg& sg) { return CAUSAL ? (sg.kblk * C::BNK) / C::BMQ : 0; };
  auto same_block = [&](const Seg& x, const Seg& y) { return x.bkv == y.bkv && x.kblk == y.kblk; };

  // A holds K (sign-flipped for a negative scale), B holds V, as the B
  // operand of Q K^T / dO V^T: kv[s] = row kw0 + n, columns 16 s + 8 g .. + 8.
  // Rows past N read as zeros.
  uint4 kv[C::DS];
  auto load_kv = [&](const Seg& sg) __attribute__((always_inline)) {
    const int kw0 = sg.kblk * C::BNK + w.pw * C::KW;
    const rsrc_t rs = make_rsrc((w.role_a ? kg : vg) + (size_t)sg.bkv * N * D, head_bytes);
    const uint32_t sgn = w.role_a ? ksign : 0u;
#pragma unroll
    for (int s = 0; s < C::DS; ++s) {
      const uint4 a = load16(rs, ((uint32_t)(kw0 + w.n()) * D + 16 * s + 8 * w.g()) * 2);
      kv[s] = make_uint4(a.x ^ sgn, a.y ^ sgn, a.z ^ sgn, a.w ^ sgn);
    }
  };
  f32x16 acc[C::DB];  // A: dV, B: dK (unscaled); rows = keys, columns = d
  // Register r of d block db is key kw0 + 8(r/4) + 4g + r%4, column 32 db + n.
  // Buffer stores: rows past N fall outside the head's range and are dropped.
  auto store_acc = [&](int bkv, int kblk) __attribute__((always_inline)) {
    const int kw0 = kblk * C::BNK + w.pw * C::KW;
    const rsrc_t rs = make_rsrc((w.role_a ? dvg : dkg) + (size_t)bkv * N * D, (uint32_t)((size_t)N * D * 4));
    const float sc = w.role_a ? 1.f : dk_scale;
    const uint32_t base = ((uint32_t)(kw0 + 4 * w.g()) * D + w.n()) * 4;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[db][r] * sc), rs,
                                              base + (uint32_t)((8 * (r / 4) + (r % 4)) * D + 32 * db) * 4, 0, 0);
#pragma unroll
    for (int db = 0; db < C::DB; ++db) acc[db] = f32x16{};
  };

  // ---- first segment: A's K, the first query block ------------------------
  int cL = xcd_remap(blockIdx.x, gridDim.x), ct = 0, cj = 0;
  Seg cur;
  if (!seg_at(cL, ct, cj, cur)) return;  // uniform: the grid never exceeds the items
#pragma unroll
  for (int db = 0; db < C::DB; ++db) acc[db] = f32x16{};
  if (w.role_a) load_kv(cur);
  int qh = qhead_of(cur);
  float row_in = issue(qh, first_qblk(cur), q_lds[0], do_lds[0]);
  kv_stage_rows(w, row_in, lse_lds[0], dl_lds[0]);
  lds_barrier<0>();

  // Element (query block) i of the current segment sits in ring slot
  // (sb + i - i_lo) % 3.
  int sb = 0;
  // A block change leaves the finished block's dV in A's accumulators and its
  // dK in B's; each wave stores them just before its first product of the
  // new segment (A: iteration i_lo, B: iteration i_lo + 1), so the stores
  // drain under full-rate products.
  int prev_bkv = -1, prev_kblk = 0;  // the block whose dV / dK is still in the accumulators (-1: none)
  bool b_change = true;  // B: new block at this segment; a previous block's dK to store
  while (true) {
    int nL = cL, nt = ct, nj = cj;
    advance(nL, nt, nj);
    Seg nxt;
    const bool has_next = seg_at(nL, nt, nj, nxt);
    const bool a_change = !has_next || !same_block(cur, nxt);
    w.kw0 = cur.kblk * C::BNK + w.pw * C::KW;  // first key of this pair
    const bool pair_live = w.kw0 < N;
    const int i_lo = first_qblk(cur);
    auto block_active = [&](int i) {
      return pair_live && (!CAUSAL || min((i + 1) * C::BMQ, N) - 1 >= w.kw0);
    };
    // A block needs the causal mask when its first query is left of the
    // pair's last key (only the diagonal block of the pair).
    auto block_masked = [&](int i) { return CAUSAL && i * C::BMQ < w.kw0 + C::KW - 1; };
    auto a_work = [&](int i, const uint16_t* __restrict__ qa, const uint16_t* __restrict__ da,
                      const float* __restrict__ la, auto may_mask, auto first) __attribute__((always_inline)) {
      constexpr bool MAY_MASK = decltype(may_mask)::value;
      if (decltype(first)::value && prev_bkv >= 0) store_acc(prev_bkv, prev_kblk);  // first product of a new block
      if (!block_active(i)) return;
      if (MAY_MASK && block_masked(i))
        kv_iter<T, D, true, true>(w, i, kv, acc, qa, da, la, x_lds[i & 1][w.pw], x_lds[(i + 1) & 1][w.pw]);
      else
        kv_iter<T, D, true, false>(w, i, kv, acc, qa, da, la, x_lds[i & 1][w.pw], x_lds[(i + 1) & 1][w.pw]);
    };
    // B's work on element i - 1 in iteration i.
    auto b_work = [&](int i, const uint16_t* __restrict__ qb, const uint16_t* __restrict__ db_,
                      const float* __restrict__ dlb, auto first) __attribute__((always_inline)) {
      if (decltype(first)::value && prev_bkv >= 0) store_acc(prev_bkv, prev_kblk);  // first product of a new block
      if (block_active(i - 1))
        kv_iter<T, D, false, false>(w, i - 1, kv, acc, db_, qb, dlb, x_lds[i & 1][w.pw], x_lds[(i + 1) & 1][w.pw]);
    };

    // ---- iteration i_lo: A's first block; B changes block if needed -------
    {
      const int sa = sb, sn = (sb + 1) % 3;
      const bool ahead = i_lo + 1 < n_qblk;
      if (ahead) row_in = issue(qh, i_lo + 1, q_lds[sn], do_lds[sn]);
      if (w.role_a) {
        a_work(i_lo, q_lds[sa], do_lds[sa], lse_lds[sa], std::true_type{}, std::true_type{});
      } else if (b_change) {
        load_kv(cur);
      }
      if (ahead) kv_stage_rows(w, row_in, lse_lds[sn], dl_lds[sn]);
      lds_barrier<0>();
    }
    // ---- iterations i_lo + 1 .. n_qblk - 1: both waves --------------------
    // Iteration i: A on block i (slot sa), B on block i - 1 (slot sa - 1),
    // block i + 1 loaded into slot sa + 1, whose last reader (B, block i - 2)
    // finished before the previous barrier.
    // role: 0 = this wave's role decided at run time, 1 = A, 2 = B (the
    // unrolled loop below runs one copy per role, so that A's and B's
    // accumulators never meet in a join, which would cost a register copy
    // of the whole accumulator per iteration).
    auto mid = [&](int i, uint16_t* __restrict__ qa, uint16_t* __restrict__ da, float* __restrict__ la,
                   uint16_t* __restrict__ qb, uint16_t* __restrict__ db_, float* __restrict__ dlb,
                   uint16_t* __restrict__ qn, uint16_t* __restrict__ dn, float* __restrict__ ln,
                   float* __restrict__ dln, auto may_mask, auto role) __attribute__((always_inline)) {
      constexpr int ROLE = decltype(role)::value;
      const bool ahead = i + 1 < n_qblk;
      if (ahead) row_in = issue(qh, i + 1, qn, dn);
      // may_mask marks iteration i_lo + 1: A's block may be masked there, and
      // it is B's first product of the segment.
      if (ROLE == 1 || (ROLE == 0 && w.role_a)) a_work(i, qa, da, la, may_mask, std::false_type{});
      else b_work(i, qb, db_, dlb, may_mask);
      // Block i + 1 must be in LDS after this barrier (waves 0 and 1 first
      // store its row values, whose loads have arrived by now).
      if (ahead) kv_stage_rows(w, row_in, ln, dln);
      lds_barrier<0>();
    };
    // A pair's keys start at kw0 = 128 kblk + 32 pw, so its only masked block
    // (the one holding query kw0) is block 2 kblk + pw / 2: i_lo or i_lo + 1.
    static_assert(C::BNK == 2 * C::BMQ && C::KW == 32 && C::NP == 4, "masked block at i_lo or i_lo + 1");
    if (i_lo + 1 < n_qblk) {
      const int sa = (sb + 1) % 3, sp = sb, sn = (sb + 2) % 3;
      mid(i_lo + 1, q_lds[sa], do_lds[sa], lse_lds[sa], q_lds[sp], do_lds[sp], dl_lds[sp], q_lds[sn], do_lds[sn],
          lse_lds[sn], dl_lds[sn], std::true_type{}, std::integral_constant<int, 0>{});
    }
    // The rest, unrolled over the three slots so every LDS base is an
    // immediate: stream position c = sb + i - i_lo, slot c % 3.
    auto rest = [&](auto role) __attribute__((always_inline)) {
      const int c_beg = sb + 2, c_end = sb + n_qblk - 1 - i_lo;  // i from i_lo + 2 to n_qblk - 1
      for (int c0 = c_beg - c_beg % 3; c0 <= c_end; c0 += 3) {
#pragma unroll
        for (int jj = 0; jj < 3; ++jj) {
          const int c = c0 + jj;
          if (c >= c_beg && c <= c_end) {
            mid(c - sb + i_lo, q_lds[jj], do_lds[jj], lse_lds[jj], q_lds[(jj + 2) % 3], do_lds[(jj + 2) % 3],
                dl_lds[(jj + 2) % 3], q_lds[(jj + 1) % 3], do_lds[(jj + 1) % 3], lse_lds[(jj + 1) % 3],
                dl_lds[(jj + 1) % 3], std::false_type{}, role);
          }
        }
      }
    };
    if (w.role_a) rest(std::integral_constant<int, 1>{});
    else rest(std::integral_constant<int, 2>{});
    // ---- iteration n_qblk: B's last block; A changes block if needed ------
    // The next segment's first block goes into the slot after B's.
    const int s_b = (sb + n_qblk - 1 - i_lo) % 3, s_n = (s_b + 1) % 3;
    {
      if (has_next) row_in = issue(qhead_of(nxt), first_qblk(nxt), q_lds[s_n], do_lds[s_n]);
      if (w.role_a) {
        if (a_change && has_next) load_kv(nxt);  // A's K is dead; its dV waits in acc
      } else if (i_lo + 1 == n_qblk) {
        b_work(n_qblk, q_lds[s_b], do_lds[s_b], dl_lds[s_b], std::true_type{});
      } else {
        b_work(n_qblk, q_lds[s_b], do_lds[s_b], dl_lds[s_b], std::false_type{});
      }
      if (has_next) kv_stage_rows(w, row_in, lse_lds[s_n], dl_lds[s_n]);
      lds_barrier<0>();
    }
    if (!has_next) break;
    b_change = a_change;
    prev_bkv = a_change ? cur.bkv : -1;
    prev_kblk = cur.kblk;
    cur = nxt;
    cL = nL;
    ct = nt;
    cj = nj;
    qh = qhead_of(cur);
    sb = s_n;
  }
  // The last block's dV (A) and dK (B).
  store_acc(cur.bkv, cur.kblk);
}

// ---------------------------------------------------------------------------
// 3. dQ.  Workgroup = 8 waves x 32 queries (two waves per SIMD), the same
// organisation as the forward: K and V tiles of BN keys go from global
// memory straight into LDS (swizzled row-major) through four buffers, three
// tiles ahead; rows feed S^T = K Q^T and dP^T = V dO^T, transposing reads
// give K^T for dQ^T += K^T dS^T.  Each lane owns one query, so its LSE and
// Delta are two registers.  Per 32-key sub-block u a wave issues the score
// and dP products of sub-block u+1 in slots, each followed by its share of
// u's vector work (P and dS), then the dQ product of u.  Only a wave's last
// sub-block (the diagonal, or the sequence tail) is masked.
// ---------------------------------------------------------------------------
template <int D, int NW_ = FA_DQ_WAVES>
struct QG {
  static constexpr int NW = NW_, NT = 64 * NW, BM = NW * 32;
  static constexpr int BN = D == 128 ? 64 : 128;  // 16 KB of K and of V per tile
  static constexpr int DS = D / 16, DB = D / 32, SUB = BN / 32, CPR = D / 8;
  static constexpr int RPP = 64 / CPR;            // tile rows per 1 KB wave load
  static constexpr int PPT = BN / RPP;            // 1 KB pieces per K (or V) tile
  static constexpr int LPW = 2 * PPT / NW;        // loads per wave per tile
  static constexpr int NBUF = 4;
  static_assert(SUB % 2 == 0 && LPW >= 1 && LPW * NW == 2 * PPT && 2 * DB == DS, "tile shape");
};

template <typename T, int D, bool CAUSAL, int NW>
__global__ __launch_bounds__(512) void bwd_dq_kernel(
    const uint16_t* __restrict__ qg, const uint16_t* __restrict__ kg, const uint16_t* __restrict__ vg,
    const uint16_t* __restrict__ dog, const float* __restrict__ lseg, const float* __restrict__ deltag,
    float* __restrict__ dqg, int N, int n_qblk, int BH, int G, float qk_scale, float dq_scale,
    uint32_t qsign) {
  using C = QG<D, NW>;
  constexpr int BN = C::BN, DS = C::DS, DB = C::DB, SUB = C::SUB, NS = C::DS;
  // Swizzled row-major tiles, one LDS variable (loads into one ring slot
  // then do not make the compiler wait before reads of another).
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[C::NBUF][BN * D];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[C::NBUF][BN * D];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 31, g = lane >> 5;
  const uint32_t head_bytes = (uint32_t)((size_t)N * D * 2);

  // Q and dO of this lane's query as the B operands, and its LSE and Delta
  // (zeros past the end; the LSE and Delta loads are range-checked too, and
  // a query past N is made harmless by LSE = +inf below).  The next
  // block's values are loaded at the end of the current block, after the
  // last use of these registers, and arrive under its epilogue; a negative
  // scale flips Q's sign bits at the block's first use, so nothing waits
  // for the data at the load.
  uint4 qf[DS], dof[DS];
  float lse_in, dl;
  auto load_rows = [&](int bh, int qblk) __attribute__((always_inline)) {
    const size_t head = (size_t)bh * (size_t)N * D;
    const rsrc_t qrs = make_rsrc(qg + head, head_bytes), dors = make_rsrc(dog + head, head_bytes);
    int nn = n, gg = g;  // through an empty asm: offsets formed here, not hoisted and spilled
    asm volatile("" : "+v"(nn), "+v"(gg));
    const int query = qblk * C::BM + wave * 32 + nn;
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      const uint32_t off = ((uint32_t)query * D + 16 * s + 8 * gg) * 2;
      qf[s] = load16(qrs, off);
      dof[s] = load16(dors, off);
    }
    lse_in = load4f(make_rsrc(lseg + (size_t)bh * N, (uint32_t)N * 4), (uint32_t)query * 4);
    dl = load4f(make_rsrc(deltag + (size_t)bh * N, (uint32_t)N * 4), (uint32_t)query * 4);
  };

  // One block of BM queries of one (batch, head), start to finish; the
  // block (nbh, nqblk) comes next (nbh < 0: none).
  auto qblock = [&](int bh, int qblk, int nbh, int nqblk) __attribute__((always_inline)) {
  const size_t head = (size_t)bh * (size_t)N * D;
  const size_t kvhead = (size_t)kv_head_of(bh, G) * (size_t)N * D;  // shared by G query heads
  const rsrc_t krs = make_rsrc(kg + kvhead, head_bytes), vrs = make_rsrc(vg + kvhead, head_bytes);
  const int q0 = qblk * C::BM;
  const int qw0 = q0 + wave * 32;
  const int query = qw0 + n;
  float lse2;  // LSE log2(e), set once the rows have arrived (prologue)

  // Key plan, as in the forward: the wave's queries see sub-blocks
  // [0, u_last]; only u_last is masked.
  const int n_sub = (N + 31) / 32;
  const bool wave_live = qw0 < N;
  const int u_last = !wave_live ? -1 : (CAUSAL ? qw0 / 32 : n_sub - 1);
  const int last_live = min(C::NW - 1, (N - 1 - q0) / 32);
  const int u_end = CAUSAL ? (q0 / 32 + last_live) : (n_sub - 1);
  const int j_end = u_end / SUB + 1;
  const int key_lim = CAUSAL ? min(query + 1, N) : N;

  // Tile loads (as in the forward): piece t = wave LPW + e holds RPP rows of
  // K (t < PPT) or V; lane l fills LDS bytes 16 l of the piece.
  auto issue = [&](int j, uint16_t* __restrict__ kd, uint16_t* __restrict__ vd) __attribute__((always_inline)) {
    const int lrow = lane / C::CPR;
#pragma unroll
    for (int e = 0; e < C::LPW; ++e) {
      const int t = wave * C::LPW + e;
      const int p = t % C::PPT;
      const int row = p * C::RPP + lrow;
      const int chunk = (lane % C::CPR) ^ swz_chunk<D>(row);
      const uint32_t off = ((uint32_t)(j * BN + row) * D + 8 * chunk) * 2;
      if (t < C::PPT) load_lds16(krs, kd + p * C::RPP * D, off);
      else load_lds16(vrs, vd + p * C::RPP * D, off);
    }
  };

  // Fragment addresses in the swizzled tiles: row reads at (R ^ 16 k) +
  // 32 sb D, transposing reads at (T ^ 32 (k % DB) [^ 16]) + rows D (see the
  // dK/dV pass); the bases go through an empty asm so the addresses are
  // formed next to their reads.
  uint32_t R = (uint32_t)swz<D>(n, 8 * g);
  uint32_t Tb = (uint32_t)swz<D>(4 * g + ((lane & 15) >> 2), 16 * ((lane >> 4) & 1) + 4 * (lane & 3));
  asm volatile("" : "+v"(R), "+v"(Tb));
  auto rowfrag = [&](const uint16_t* t, int sb, int k) __attribute__((always_inline)) {
    return *reinterpret_cast<const uint4*>(t + ((R ^ (16 * k)) + 32 * sb * D));
  };
  auto trfrag = [&](const uint16_t* t, int sb, int k) __attribute__((always_inline)) {
    const uint32_t r0 = (32 * sb + 16 * (k / DB)) * D;
    const uint32_t x = Tb ^ (32 * (k % DB));
    const uint2 lo = read_tr_b64(t + (x + r0));
    const uint2 hi = read_tr_b64(t + ((x ^ 16) + r0 + 8 * D));
    return make_uint4(lo.x, lo.y, hi.x, hi.y);
  };

  f32x16 dq[DB];  // dQ^T: rows = d, columns = queries
#pragma unroll
  for (int db = 0; db < DB; ++db) dq[db] = f32x16{};
  f32x16 sA, dA, sB, dB;  // S^T and dP^T of even / odd sub-blocks

  // P and dS of one sub-block's elements [r0, r0 + EP): register r is key
  // key0 + 8 (r/4) + 4 g + r%4.  A query past N has dO = 0 and Delta = 0
  // (its LSE is +inf, so P = 0).
  auto vec = [&](const f32x16& s, const f32x16& dp, int key0, int r0, int ep, uint32_t (&pk)[8], auto masked)
      __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked)::value;
#pragma unroll
    for (int r = r0; r < r0 + ep; r += 2) {
      float p0 = fast_exp2(__builtin_fmaf(s[r], qk_scale, -lse2));
      float p1 = fast_exp2(__builtin_fmaf(s[r + 1], qk_scale, -lse2));
      if constexpr (MASKED) {
        const int kr = key0 + 8 * (r / 4) + 4 * g + (r % 4);
        p0 = kr < key_lim ? p0 : 0.f;
        p1 = kr + 1 < key_lim ? p1 : 0.f;
      }
      pk[r / 2] = pack2(T{}, p0 * (dp[r] - dl), p1 * (dp[r + 1] - dl));
    }
  };
  // dQ^T += K^T dS^T over sub-block sb of a K tile (two 16-key chunks).
  auto dq_gemm = [&](const uint16_t* kt, int sb, const uint32_t (&pk)[8]) __attribute__((always_inline)) {
    const uint4 pp[2] = {make_uint4(pk[0], pk[1], pk[2], pk[3]), make_uint4(pk[4], pk[5], pk[6], pk[7])};
    uint4 b[3];
    b[0] = trfrag(kt, sb, 0);
    b[1] = trfrag(kt, sb, 1);
#pragma unroll
    for (int k = 0; k < NS; ++k) {
      if (k + 2 < NS) b[(k + 2) % 3] = trfrag(kt, sb, k + 2);
      dq[k % DB] = mma16(T{}, b[k % 3], pp[k / DB], dq[k % DB]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // S^T and dP^T of sub-block sb of a K/V tile, not overlapped (prologue).
  auto sdp = [&](const uint16_t* kt, const uint16_t* vt, int sb, f32x16& s, f32x16& dp)
      __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < NS; ++k) {
      s = mma16(T{}, rowfrag(kt, sb, k), qf[k], k == 0 ? f32x16{} : s);
      dp = mma16(T{}, rowfrag(vt, sb, k), dof[k], k == 0 ? f32x16{} : dp);
    }
  };
  // One step for an unmasked sub-block u (S^T, dP^T in cur): the products
  // of sub-block u+1 (rows 32 nsb.. of tiles kn / vn) in NS slots, each with
  // its share of u's vector work, then u's dQ product (K tile kt, rows 32 sb..).
  auto step = [&](const f32x16& cs, const f32x16& cd, f32x16& ns, f32x16& nd, const uint16_t* kn,
                  const uint16_t* vn, int nsb, const uint16_t* kt, int sb) __attribute__((always_inline)) {
    constexpr int EPS = 16 / NS;
    uint4 a[3], c[3];
    a[0] = rowfrag(kn, nsb, 0); c[0] = rowfrag(vn, nsb, 0);
    a[1] = rowfrag(kn, nsb, 1); c[1] = rowfrag(vn, nsb, 1);
    uint32_t pk[8];
#pragma unroll
    for (int k = 0; k < NS; ++k) {
      if (k + 2 < NS) {
        a[(k + 2) % 3] = rowfrag(kn, nsb, k + 2);
        c[(k + 2) % 3] = rowfrag(vn, nsb, k + 2);
      }
      ns = mma16(T{}, a[k % 3], qf[k], k == 0 ? f32x16{} : ns);
      nd = mma16(T{}, c[k % 3], dof[k], k == 0 ? f32x16{} : nd);
      vec(cs, cd, 0, EPS * k, EPS, pk, std::false_type{});
      __builtin_amdgcn_sched_barrier(0);
    }
    dq_gemm(kt, sb, pk);
  };

  // One tile j (buffers kc / vc, next kn / vn): this wave's steps u < u_last
  // in it, and the loads of tile j + 3 (restrict: see the forward).
  auto tile = [&](int j, const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
                  const uint16_t* __restrict__ kn, const uint16_t* __restrict__ vn, uint16_t* __restrict__ kl,
                  uint16_t* __restrict__ vl, bool load) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < SUB; ++i) {
      // tile j + 3's loads go out halfway through the tile rather than
      // right after the barrier, where every wave's first reads are
      if (i == SUB / 2 && load) issue(j + 3, kl, vl);
      const int u = j * SUB + i;
      if (u < u_last) {
        const uint16_t* kt = i + 1 < SUB ? kc : kn;
        const uint16_t* vt = i + 1 < SUB ? vc : vn;
        if (i % 2 == 0) step(sA, dA, sB, dB, kt, vt, (i + 1) % SUB, kc, i);
        else step(sB, dB, sA, dA, kt, vt, (i + 1) % SUB, kc, i);
      }
    }
  };

  // ---- prologue: tiles 0..2 in flight, wait for 0 and 1 ------------------
  issue(0, k_lds[0], v_lds[0]);
  if (j_end > 1) issue(1, k_lds[1], v_lds[1]);
  if (j_end > 2) {
    issue(2, k_lds[2], v_lds[2]);
    lds_barrier<C::LPW>();
  } else {
    lds_barrier<0>();
  }
  if (qsign != 0) {
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      qf[s].x ^= qsign; qf[s].y ^= qsign; qf[s].z ^= qsign; qf[s].w ^= qsign;
    }
  }
  lse2 = query < N ? lse_in * kLog2e : kPosInf;
  if (wave_live) sdp(k_lds[0], v_lds[0], 0, sA, dA);

  // ---- main loop, unrolled over the buffers (immediate LDS offsets) ------
  for (int j0 = 0; j0 < j_end; j0 += C::NBUF) {
#pragma unroll
    for (int jj = 0; jj < C::NBUF; ++jj) {
      const int j = j0 + jj;
      if (j < j_end) {
        const bool load = j + 3 < j_end;
        tile(j, k_lds[jj], v_lds[jj], k_lds[(jj + 1) % C::NBUF], v_lds[(jj + 1) % C::NBUF],
             k_lds[(jj + 3) % C::NBUF], v_lds[(jj + 3) % C::NBUF], load);
        if (load) lds_barrier<C::LPW>();
        else lds_barrier<0>();
      }
    }
  }
  // No load is in flight here (the loop's last barrier waited for all of
  // them); saying so spares the tail and the dQ staging below a wait for
  // loads the compiler would otherwise take as pending.
  vm_wait<0>();
  // The wave's last (masked) sub-block; its tile is among the last four of
  // the workgroup, still in LDS.
  if (wave_live) {
    const uint16_t* kt = k_lds[(u_last / SUB) % C::NBUF];
    const f32x16 cs = (u_last % 2 == 0) ? sA : sB, cd = (u_last % 2 == 0) ? dA : dB;
    uint32_t pk[8];
    vec(cs, cd, 32 * u_last, 0, 16, pk, std::true_type{});
    dq_gemm(kt, u_last % SUB, pk);
  }

  // dQ through LDS, as the forward's O: each wave stages its 32 x D fp32
  // tile in its own part of the idle ring (16-byte chunk c of row r at chunk
  // c ^ (r mod chunks per row)), then every store instruction writes whole
  // rows (64 lanes x 16 bytes); range-checked buffer stores drop rows past N.
  lds_only_barrier();  // every wave's tail has finished reading the ring
  if (wave_live) {
    constexpr int CH = D / 4;  // 16-byte chunks per fp32 row
    float* stage = reinterpret_cast<float*>(wave < C::NW / 2 ? &k_lds[0][0] : &v_lds[0][0]) +
                   (wave % (C::NW / 2)) * 32 * D;
    static_assert((C::NW / 2) * 32 * D * 4 <= C::NBUF * BN * D * 2, "dQ staging fits in half the ring");
    // Lane values through an empty asm: the addresses are formed here
    // rather than hoisted out of the persistent loop and kept live.
    int nn = n, gg = g;
    asm volatile("" : "+v"(nn), "+v"(gg));
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const f32x16& v = dq[db];
        const int c = 8 * db + 2 * rq + gg;
        *reinterpret_cast<float4*>(stage + nn * D + 4 * (c ^ (nn % CH))) =
            make_float4(v[4 * rq] * dq_scale, v[4 * rq + 1] * dq_scale, v[4 * rq + 2] * dq_scale,
                        v[4 * rq + 3] * dq_scale);
      }
    // The next block's rows (the tail above was the last use of the rows,
    // and the accumulator is in LDS now).
    if (nbh >= 0) load_rows(nbh, nqblk);
    const rsrc_t drs = make_rsrc(dqg + head, (uint32_t)((size_t)N * D * 4));
    int li = lane;  // through an empty asm: addresses formed here, not hoisted
    asm volatile("" : "+v"(li));
    constexpr int ROWS = 64 / CH;
#pragma unroll
    for (int i = 0; i < 32 / ROWS; ++i) {
      const int r = ROWS * i + li / CH, c = li % CH;
      const float4 x = *reinterpret_cast<const float4*>(stage + r * D + 4 * (c ^ (r % CH)));
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u32, x), drs,
                                             ((uint32_t)(qw0 + r) * D + 4 * c) * 4, 0, 0);
    }
  } else if (nbh >= 0) {
    load_rows(nbh, nqblk);
  }
  };

  // Persistent loop over equal-cost items, as in the dK/dV pass; the
  // heavier query block of a causal pair (the higher one) goes first.
  const int per_head = items_per_head(n_qblk, CAUSAL);
  const int n_items = BH * per_head;
  // Block t of item L (heavy first); false past the item's blocks.
  auto block_at = [&](int L, int t, int* bh, int* qb) {
    if (L >= n_items) return false;
    int lo, hi;
    const int nb = item_blocks(L % per_head, n_qblk, CAUSAL, &lo, &hi);
    if (t >= nb) return false;
    *bh = L / per_head;
    *qb = t + 1 < nb ? hi : lo;
    return true;
  };
  int L = xcd_remap(blockIdx.x, gridDim.x), t = 0, bh = -1, qb = -1;
  if (block_at(L, 0, &bh, &qb)) load_rows(bh, qb);
  while (bh >= 0) {  // one call site: the block body is large
    int nbh = -1, nqb = -1;
    if (block_at(L, t + 1, &nbh, &nqb)) {
      ++t;
    } else {
      L += gridDim.x;
      t = 0;
      if (!block_at(L, 0, &nbh, &nqb)) nbh = -1;
    }
    qblock(bh, qb, nbh, nqb);
    // The next block's loads reuse the LDS buffers; this block's dQ stores
    // may still be in flight.
    lds_only_barrier();
    bh = nbh;
    qb = nqb;
  }
}

// ---------------------------------------------------------------------------
template <typename T, int D, bool CAUSAL>
hipError_t run(const BwdArgs& a, int stage) {
  const long long rows = (long long)a.BH * a.N;
  constexpr int RPB = 256 / (D / 8);
  const long long g1 = (rows + RPB - 1) / RPB;
  const int n_kblk = (a.N + KV<D>::BNK - 1) / KV<D>::BNK;
  int n_qblk = (a.N + QG<D>::BM - 1) / QG<D>::BM;
  long long g2 = (long long)items_per_head(n_kblk, CAUSAL) * (a.BH / a.G);
  long long g3 = (long long)items_per_head(n_qblk, CAUSAL) * a.BH;
  if (g1 > 0x7fffffffLL || g2 > 0x7fffffffLL || g3 > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  // dK/dV and dQ run persistent grids of one workgroup per CU (registers
  // allow one 512-thread workgroup per CU), never more than their items.
  int dev = 0, cus = 0;
  hipError_t de = hipGetDevice(&dev);
  if (de == hipSuccess) de = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (de != hipSuccess) return de;
  // dQ items that would fill at most half the CUs: 128-query items on four
  // waves, one per SIMD, so that twice the CUs work
  const bool dq4 = QG<D>::NW == 8 && 2 * g3 <= cus;
  if (dq4) {
    n_qblk = (a.N + QG<D, 4>::BM - 1) / QG<D, 4>::BM;
    g3 = (long long)items_per_head(n_qblk, CAUSAL) * a.BH;
  }
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
    if (a.G > 1)
      hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, CAUSAL, true>), dim3((unsigned)g2), dim3(KV<D>::NT), 0, a.stream, q, k,
                         v, dout, a.lse, a.delta, a.dk, a.dv, a.N, n_kblk, a.BH / a.G, a.G, qk_scale, a.scale, qsign);
    else
      hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, CAUSAL, false>), dim3((unsigned)g2), dim3(KV<D>::NT), 0, a.stream, q,
                         k, v, dout, a.lse, a.delta, a.dk, a.dv, a.N, n_kblk, a.BH, 1, qk_scale, a.scale, qsign);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (stage == 0 || stage == 3) {
    if (dq4)
      hipLaunchKernelGGL((bwd_dq_kernel<T, D, CAUSAL, 4>), dim3((unsigned)g3), dim3(QG<D, 4>::NT), 0, a.stream, q, k,
                         v, dout, a.lse, a.delta, a.dq, a.N, n_qblk, a.BH, a.G, qk_scale, a.scale, qsign);
    else
      hipLaunchKernelGGL((bwd_dq_kernel<T, D, CAUSAL, QG<D>::NW>), dim3((unsigned)g3), dim3(QG<D>::NT), 0, a.stream, q,
                         k, v, dout, a.lse, a.delta, a.dq, a.N, n_qblk, a.BH, a.G, qk_scale, a.scale, qsign);
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
