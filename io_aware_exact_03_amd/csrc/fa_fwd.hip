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
// * Each wave owns 32 queries.  Computing S^T (keys x queries) puts every
//   lane on ONE query, so the softmax statistics are in-lane plus one
//   exchange of the two 32-lane halves, and the correction alpha is
//   lane-local for the O^T accumulator as well.
// * The fp32 S^T accumulator registers, rounded to 16 bits, are directly the
//   B operand of O^T += V^T P^T: no LDS round trip for P.  V stays row-major
//   in LDS and reaches that product through transposing reads
//   (ds_read_b64_tr_b16).
// * K and V tiles go from global memory straight into LDS (no registers),
//   swizzled row-major, through a ring of five tile buffers, three tiles
//   ahead; one barrier per tile.  The ring is laid out so that nearly every
//   LDS read takes its address from a per-lane base plus an immediate.
// * Software pipeline inside each wave, per 32-key sub-block u: the S^T
//   product of u+1 and the PV product of u-1 are issued slot by slot with
//   the exponentials of u spread between them, so the matrix cores and the
//   vector/transcendental units overlap within one wave; eight waves (two
//   per SIMD) cover the rest.
// * The reference max is raised lazily (only when a weight would exceed
//   2^8), so the common path computes no row max and the O rescale is rare;
//   exact, since O, l and the LSE all use the same reference.
// * A persistent grid walks equal-cost work items (a causal item pairs a
//   heavy query block with a light one of the same head); each XCD (own L2)
//   works on a contiguous range of items, i.e. on shared heads.
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
// Workgroup: 8 waves x 32 queries (BM = 256, two waves per SIMD; a build may
// define FA_FWD16_WAVES = 4 to time the one-wave-per-SIMD shape), or 4 waves
// (BM = 128) for problems whose 256-query items would leave CUs idle.  K/V tiles
// of BN keys go from global memory straight into LDS (no registers), row-major
// with the XOR chunk swizzle, into five buffers: the previous tile (whose V
// the first step still reads), the tile being consumed, the next one (whose
// first score product starts in the current tile's last step) and two in
// flight.  K feeds S^T = K Q^T with 16-byte row reads; V
// feeds O^T += V^T P^T through transposing reads (ds_read_b64_tr_b16).
template <typename T, int D, int BN, bool CAUSAL, int NW_ = FA_FWD16_WAVES>
struct Fwd16 {
  static constexpr int NW = NW_, NT = NW * 64, BM = NW * 32;
  static constexpr int DS = D / 16;          // k-steps of the S product
  static constexpr int DB = D / 32;          // 32-wide d blocks of O
  static constexpr int SUB = BN / 32;        // 32-key sub-blocks per tile
  static constexpr int CPR = D / 8;          // 16-byte chunks per K/V row
  static constexpr int RPP = 64 / CPR;       // tile rows per 1 KB wave load
  static constexpr int PPT = BN / RPP;       // 1 KB pieces per K (or V) tile
  static constexpr int LPW = 2 * PPT / NW;   // loads per wave per tile
  static constexpr int NBUF = 5;
  static_assert(SUB % 2 == 0, "score registers alternate per sub-block");
  static_assert(LPW >= 1 && LPW * NW == 2 * PPT, "tile loads split evenly over waves");
  static_assert(LPW < 16, "vmcnt range");
};

// A sub-block's weights p = exp2(S q - m) are accepted when this lane's sum
// of its 16 weights stays at or below 2^8 (so every weight does); otherwise
// the reference max is raised to the true row max (plus the lift below) and
// the weights are redone.
constexpr float kSumLimit = 256.f;
// A raised reference sits this far (log2 units) above the row max it was
// raised to, so later, larger scores stay under the limit longer.  bf16
// weights keep their relative precision at any scale, so for bf16 the lift
// costs nothing; fp16 weights far below the maximum would fall into fp16's
// subnormal range sooner, so for fp16 the reference is the row max itself.
constexpr float ref_lift(BF16) { return 8.f; }
constexpr float ref_lift(F16) { return 0.f; }

template <typename T, int D, int BN, bool CAUSAL, int NW>
__global__ __launch_bounds__(512) void fwd16_kernel(
    const uint16_t* __restrict__ qg, const uint16_t* __restrict__ kg, const uint16_t* __restrict__ vg,
    uint16_t* __restrict__ og, float* __restrict__ lseg, int Nq, int Nk, int qshift, int koff, int n_qblk,
    int BH, int G, float qk_scale, uint32_t qsign) {
  using C = Fwd16<T, D, BN, CAUSAL, NW>;
  constexpr int DS = C::DS, DB = C::DB, SUB = C::SUB;
  // Swizzled row-major tiles, V below K: the transposing V reads of ring
  // slots 0-3 then reach their address with a per-lane base register and
  // the 16-bit immediate offset alone (no address add per read).
  __shared__ __attribute__((aligned(16))) uint16_t kv_lds[2][C::NBUF][BN * D];
  auto& v_lds = kv_lds[0];
  auto& k_lds = kv_lds[1];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 31;
  const int g = lane >> 5;

  // ---- Q fragments of the current query block, held in registers --------
  // B operand of S^T = K Q^T: lane supplies Q[query][16 s + 8 g + 0..7];
  // rows outside [0, Nq) read as zeros (a negative row wraps to an offset
  // past the buffer).  A negative scale flips Q's sign bits, at the block's
  // first use rather than at the load, so that nothing waits for the data
  // early: the next block's fragments are loaded at the end of the current
  // block and arrive under its epilogue.
  //
  // Query rows are indexed virtually: virtual row i' is query i' - qshift,
  // and with the causal mask it sees keys j <= i' + koff, koff a multiple of
  // 32.  A query offset off = Nk - Nq (the queries are the last Nq of Nk
  // positions) becomes koff = off - off % 32 and qshift = off % 32, so the
  // diagonal always falls on whole 32-key sub-blocks.  Square attention has
  // qshift = koff = 0.
  uint4 qf[DS];
  auto load_q = [&](int bh, int qblk) __attribute__((always_inline)) {
    const rsrc_t rs = make_rsrc(qg + (size_t)bh * (size_t)Nq * D, (uint32_t)Nq * D * 2);
    const int q = qblk * C::BM + 32 * wave + n - qshift;
#pragma unroll
    for (int s = 0; s < DS; ++s) qf[s] = load16(rs, ((uint32_t)q * D + 16 * s + 8 * g) * 2);
  };

  // ---- tile loads: global -> LDS ------------------------------------------
  // Piece t (0 .. 2 PPT - 1) = wave LPW + e holds RPP tile rows of K
  // (t < PPT) or V.  Lane l fills LDS bytes 16 l of the piece: row l / CPR,
  // stored chunk l % CPR, which holds the row's logical chunk
  // (l % CPR) ^ swz_chunk(row).  Rows past Nk read as zeros.
  auto issue_tile = [&](const rsrc_t& krs, const rsrc_t& vrs, int j, uint16_t* __restrict__ kd,
                        uint16_t* __restrict__ vd) __attribute__((always_inline)) {
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
  auto kv_rsrc = [&](int bh, rsrc_t* krs, rsrc_t* vrs) __attribute__((always_inline)) {
    const size_t kvhead = (size_t)kv_head_of(bh, G) * (size_t)Nk * D;  // shared by G query heads
    const uint32_t head_bytes = (uint32_t)Nk * D * 2;
    *krs = make_rsrc(kg + kvhead, head_bytes);
    *vrs = make_rsrc(vg + kvhead, head_bytes);
  };
  // Tiles query block qblk reads: up to the diagonal sub-block of its last
  // wave with live queries (causal), else to the key tail.
  auto tiles_of = [&](int qblk) __attribute__((always_inline)) {
    const int q0 = qblk * C::BM;
    const int last_live = min(C::NW - 1, (Nq + qshift - 1 - q0) / 32);  // q0 < Nq + qshift always
    const int u_end = CAUSAL ? ((q0 + koff) / 32 + last_live) : ((Nk + 31) / 32 - 1);
    return u_end / SUB + 1;
  };
  // A block's first three tiles go to ring slots 0-2.  They are issued
  // before the block starts: by the block before it, as soon as its last
  // tile reads are done, so they arrive under its epilogue.
  auto issue_first = [&](int bh, int qblk) __attribute__((always_inline)) {
    rsrc_t krs, vrs;
    kv_rsrc(bh, &krs, &vrs);
    const int je = tiles_of(qblk);
    issue_tile(krs, vrs, 0, k_lds[0], v_lds[0]);
    if (je > 1) issue_tile(krs, vrs, 1, k_lds[1], v_lds[1]);
    if (je > 2) issue_tile(krs, vrs, 2, k_lds[2], v_lds[2]);
  };

  // One query block of one (batch, head), start to finish; (nbh, nqblk) is
  // the block this workgroup runs next (nbh < 0: none).  Its first three
  // tiles and its Q fragments are in flight when it starts.
  auto block = [&](int bh, int qblk, int nbh, int nqblk) __attribute__((always_inline)) {
  const size_t head = (size_t)bh * (size_t)Nq * D;
  rsrc_t krs, vrs;
  kv_rsrc(bh, &krs, &vrs);

  const int q0 = qblk * C::BM;
  const int qw0 = q0 + 32 * wave;  // first query of this wave
  const int query = qw0 + n;       // this lane's query

  // ---- key plan ------------------------------------------------------------
  // The wave's queries see the 32-key sub-blocks [0, u_last].  Every
  // sub-block before u_last is visible to all of them and lies before the
  // sequence end, so only u_last is masked: for the causal case it is the
  // diagonal sub-block (keys qw0 .. qw0 + 31, the pages' masked stage),
  // otherwise the sub-block holding the sequence tail.  Sub-blocks after
  // u_last (the future) are never computed.  A wave whose queries all lie
  // past the last query (u_last = -1) only helps load tiles.  In virtual
  // rows the diagonal sub-block of the wave is (qw0 + koff) / 32.
  const int NqV = Nq + qshift;  // virtual rows
  const int n_sub = (Nk + 31) / 32;
  const bool wave_live = qw0 < NqV;
  const int u_last = !wave_live ? -1 : (CAUSAL ? (qw0 + koff) / 32 : n_sub - 1);
  const int j_end = tiles_of(qblk);  // tiles this workgroup reads
  const int key_lim = CAUSAL ? min(query + koff + 1, Nk) : Nk;

  auto issue = [&](int j, uint16_t* kd, uint16_t* vd) __attribute__((always_inline)) {
    issue_tile(krs, vrs, j, kd, vd);
  };

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
  float m_run = 0.f, l_run = 0.f;  // m_run: reference max, log2 units
  f32x16 sA, sB;                    // scores of even / odd sub-blocks

  // S^T of one sub-block (32 keys x 32 queries) from rows 32 sb .. of a K tile.
  // In the swizzled layout every fragment sits at a per-lane base XOR a
  // constant plus a row offset (the chunk permutation only touches the
  // within-row address bits): row reads at (R ^ 32 k) + 64 sb D bytes,
  // transposing reads at (T ^ 64 (k % DB) [^ 32]) + 2 rows D.  The bases go
  // through an empty asm so each address is formed next to its read.
  // The K ring lies kKOff bytes above the V ring; that distance is carried in
  // the K base register (the XOR touches bits 5-7 only, so (Rb + kKOff) ^ x =
  // (Rb ^ x) + kKOff), which leaves each K read's immediate offset within the
  // 16-bit range for ring slots 0-3.
  constexpr uint32_t kKOff = sizeof(v_lds);
  uint32_t Rb = 2u * (uint32_t)swz<D>(n, 8 * g) + kKOff;
  uint32_t Tb = 2u * (uint32_t)swz<D>(4 * g + ((lane & 15) >> 2), 16 * ((lane >> 4) & 1) + 4 * (lane & 3));
  asm volatile("" : "+v"(Rb), "+v"(Tb));
  auto kfrag = [&](const uint16_t* kt, int sb, int k) __attribute__((always_inline)) {
    return *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(kt) - kKOff + (Rb ^ (32 * k)) + 64 * sb * D);
  };
  auto vfrag = [&](const uint16_t* vt, int sb, int k) __attribute__((always_inline)) {
    const char* base = reinterpret_cast<const char*>(vt);
    const uint32_t r0 = 2 * (32 * sb + 16 * (k / DB)) * D;
    const uint32_t t = Tb ^ (64 * (k % DB));
    const uint2 lo = read_tr_b64(reinterpret_cast<const uint16_t*>(base + t + r0));
    const uint2 hi = read_tr_b64(reinterpret_cast<const uint16_t*>(base + (t ^ 32) + r0 + 16 * D));
    return make_uint4(lo.x, lo.y, hi.x, hi.y);
  };
  auto s_gemm = [&](const uint16_t* kt, int sb, f32x16& s) __attribute__((always_inline)) {
#pragma unroll
    for (int st = 0; st < DS; ++st)
      s = mma16(T{}, kfrag(kt, sb, st), qf[st], st == 0 ? f32x16{} : s);
  };
  // Weights of sub-block `cur` (first key key0) with the current reference,
  // packed to 16-bit as the B operand of the PV product; returns the lane sum.
  auto exp_pack = [&](const f32x16& cur, int key0, uint32_t (&pk)[8], auto masked) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked)::value;
    float part[2] = {0.f, 0.f};
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      float p0 = fast_exp2(__builtin_fmaf(cur[r], qk_scale, -m_run));
      float p1 = fast_exp2(__builtin_fmaf(cur[r + 1], qk_scale, -m_run));
      if constexpr (MASKED) {
        const int kb = key0 + 4 * g + 8 * (r / 4) + (r % 4);
        p0 = kb < key_lim ? p0 : 0.f;
        p1 = kb + 1 < key_lim ? p1 : 0.f;
      }
      pk[r / 2] = pack2(T{}, p0, p1);
      part[(r / 2) % 2] = r < 4 ? first_pair(T{}, pk[r / 2], p0, p1)
                                : add_pair(T{}, pk[r / 2], p0, p1, part[(r / 2) % 2]);
    }
    return part[0] + part[1];
  };
  // Rare path: some lane's weights exceeded the limit.  Raise the reference
  // to the true row max of this sub-block (plus the lift) where it is
  // higher, rescale O and l, and redo the weights.  Exact: O, l and the LSE
  // share the reference.
  auto raise_redo = [&](const f32x16& cur, int key0, uint32_t (&pk)[8], auto masked) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked)::value;
    f32x16 c1[1] = {cur};
    const float mt = tile_max<1, MASKED>(c1, qk_scale, key0 + 4 * g, key_lim);
    const float m_new = fmaxf(m_run, mt + ref_lift(T{}));
    const float alpha = fast_exp2(m_run - m_new);
    l_run *= alpha;
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
    return exp_pack(cur, key0, pk, masked);
  };
  // Accept the weights of a sub-block, or raise the reference and redo them.
  auto settle = [&](const f32x16& cur, int key0, uint32_t (&pk)[8], float lsum, auto masked)
      __attribute__((always_inline)) {
    if (__builtin_amdgcn_ballot_w64(!(lsum <= kSumLimit)) != 0) lsum = raise_redo(cur, key0, pk, masked);
    l_run += lsum;
  };

  // Operand fragments.  Product k (0 .. NS-1) of a sub-block's score product
  // takes K rows 32 sb + n, columns 16 k + 8 g; product k of its PV product
  // takes the 16 keys 16 (k / DB) .. of the sub-block, d block k % DB.
  constexpr int NS = DS;  // = 2 DB: both products of a sub-block have NS steps
  static_assert(NS == 2 * DB, "slot pairing");
  // O^T += V^T P^T over one sub-block, not overlapped (the wave's last ones).
  auto pv_gemm = [&](const uint16_t* vt, int sb, const uint32_t (&pk)[8]) __attribute__((always_inline)) {
    const uint4 pp[2] = {make_uint4(pk[0], pk[1], pk[2], pk[3]), make_uint4(pk[4], pk[5], pk[6], pk[7])};
    uint4 b[3];
    b[0] = vfrag(vt, sb, 0);
    b[1] = vfrag(vt, sb, 1);
#pragma unroll
    for (int k = 0; k < NS; ++k) {
      if (k + 2 < NS) b[(k + 2) % 3] = vfrag(vt, sb, k + 2);
      oacc[k % DB] = mma16(T{}, b[k % 3], pp[k / DB], oacc[k % DB]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Software pipeline over the wave's sub-blocks.  Step u issues, in NS
  // slots, the score product of sub-block u+1 and the PV product of u-1,
  // one matrix product of each per slot, and spreads the weights of u (whose
  // scores the previous step produced) evenly over the slots, so the vector
  // and transcendental work hides under the matrix products.  LDS reads run
  // two slots ahead and cross into the next step: ka / vb carry the first
  // two K and V fragments the next step consumes.
  constexpr int PD = 3;  // fragments read ahead of the product that uses them
  static_assert(PD <= NS, "prefetch distance");
  uint4 ka[PD], vb[PD];
  // Packed weights of the even and the odd sub-blocks: step u writes the
  // array of u's parity and its PV product reads the other one (u - 1), so
  // no copy is needed between steps.  A tile holds an even number of
  // sub-blocks, so the parity is a compile-time fact inside the tile loop.
  uint32_t pkA[8], pkB[8];
  auto step = [&](f32x16& cur, int key0, f32x16& nxt, const uint16_t* kt, int ksb, const uint16_t* vt, int vsb,
                  const uint16_t* kt2, int ksb2, const uint16_t* vt2, int vsb2, uint32_t (&pk)[8],
                  const uint32_t (&pkp)[8], auto with_pv) __attribute__((always_inline)) {
    constexpr bool PV = decltype(with_pv)::value;
    constexpr int EPS = 16 / NS;  // weights per slot
    const uint4 pp[2] = {make_uint4(pkp[0], pkp[1], pkp[2], pkp[3]), make_uint4(pkp[4], pkp[5], pkp[6], pkp[7])};
    uint4 a[PD + 1], b[PD + 1];
#pragma unroll
    for (int i = 0; i < PD; ++i) {
      a[i] = ka[i];
      b[i] = vb[i];
    }
    float lsum = 0.f;  // one chain: its links are a slot apart
#pragma unroll
    for (int k = 0; k < NS; ++k) {
      if (k + PD < NS) {
        a[(k + PD) % (PD + 1)] = kfrag(kt, ksb, k + PD);
        if constexpr (PV) b[(k + PD) % (PD + 1)] = vfrag(vt, vsb, k + PD);
      } else {
        ka[k + PD - NS] = kfrag(kt2, ksb2, k + PD - NS);
        vb[k + PD - NS] = vfrag(vt2, vsb2, k + PD - NS);
      }
      nxt = mma16(T{}, a[k % (PD + 1)], qf[k], k == 0 ? f32x16{} : nxt);
#pragma unroll
      for (int e = 0; e < EPS; e += 2) {
        const int r = k * EPS + e;
        const float p0 = fast_exp2(__builtin_fmaf(cur[r], qk_scale, -m_run));
        const float p1 = fast_exp2(__builtin_fmaf(cur[r + 1], qk_scale, -m_run));
        pk[r / 2] = pack2(T{}, p0, p1);
        lsum = r == 0 ? first_pair(T{}, pk[0], p0, p1) : add_pair(T{}, pk[r / 2], p0, p1, lsum);
      }
      if constexpr (PV) oacc[k % DB] = mma16(T{}, b[k % (PD + 1)], pp[k / DB], oacc[k % DB]);
      __builtin_amdgcn_sched_barrier(0);
    }
    // The rare redo rebuilds pk; this use keeps the compiler from moving the
    // packs into the common branch, out of the interleave.
#pragma unroll
    for (int i = 0; i < 8; ++i) asm volatile("" ::"v"(pk[i]));
    settle(cur, key0, pk, lsum, std::false_type{});
  };

  // One tile j (buffers: kc / vc this tile, kn the next, vp the previous):
  // this wave's steps u = j SUB + i with 1 <= u < u_last, and the loads of
  // tile j + 3.  The tiles arrive as separate __restrict__ pointers, which
  // tells the compiler that the loads into kl / vl do not alias the tiles
  // read here, so it does not wait for them before each LDS read.
  auto tile = [&](int j, const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
                  const uint16_t* __restrict__ kn, const uint16_t* __restrict__ vp, uint16_t* __restrict__ kl,
                  uint16_t* __restrict__ vl, bool load) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < SUB; ++i) {
      // tile j + 3's loads go out halfway through the tile rather than
      // right after the barrier, where every wave's first reads are
      if (i == SUB / 2 && load) issue(j + 3, kl, vl);
      const int u = j * SUB + i;
      f32x16& cur = (i % 2 == 0) ? sA : sB;
      f32x16& nxt = (i % 2 == 0) ? sB : sA;
      uint32_t(&pk)[8] = (i % 2 == 0) ? pkA : pkB;
      uint32_t(&pkp)[8] = (i % 2 == 0) ? pkB : pkA;
      if (u >= 1 && u < u_last) {
        const uint16_t* kt = i + 1 < SUB ? kc : kn;        // sub-block u + 1
        const uint16_t* vt = i >= 1 ? vc : vp;             // sub-block u - 1
        const uint16_t* kt2 = i + 2 < SUB ? kc : kn;       // sub-block u + 2
        step(cur, 32 * u, nxt, kt, (i + 1) % SUB, vt, (i + SUB - 1) % SUB, kt2, (i + 2) % SUB, vc, i, pk, pkp,
             std::true_type{});
      }
    }
  };

  // ---- prologue: tiles 0..2 and Q were issued before the block; wait for
  // all of them (and for the previous block's O stores, issued after them).
  lds_barrier<0>();
  if (qsign != 0) {
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      qf[s].x ^= qsign; qf[s].y ^= qsign; qf[s].z ^= qsign; qf[s].w ^= qsign;
    }
  }
  if (wave_live) {
    s_gemm(k_lds[0], 0, sA);
    f32x16 s1[1] = {sA};
    // key 0 is visible to every query
    m_run = tile_max<1, true>(s1, qk_scale, 4 * g, key_lim) + ref_lift(T{});
    if (u_last >= 1) {
      // step 0: scores of sub-block 1, weights of 0, no PV product yet
      const uint16_t* k2 = k_lds[2 / SUB];
#pragma unroll
      for (int i = 0; i < PD; ++i) ka[i] = kfrag(k_lds[0], 1, i);
      step(sA, 0, sB, k_lds[0], 1, v_lds[0], 0, k2, 2 % SUB, v_lds[0], 0, pkA, pkB, std::false_type{});
    }
  }

  // ---- main loop, unrolled over the buffers so that every LDS offset is a
  // compile-time immediate ---------------------------------------------------
  constexpr int NB5 = C::NBUF;
  for (int j0 = 0; j0 < j_end; j0 += NB5) {
#pragma unroll
    for (int jj = 0; jj < NB5; ++jj) {
      const int j = j0 + jj;
      if (j < j_end) {
        const bool load = j + 3 < j_end;
        tile(j, k_lds[jj], v_lds[jj], k_lds[(jj + 1) % NB5], v_lds[(jj + NB5 - 1) % NB5], k_lds[(jj + 3) % NB5],
             v_lds[(jj + 3) % NB5], load);
        // Tiles j + 1 and j + 2 must be in LDS after this barrier; tile
        // j + 3's loads may stay in flight.
        if (load) lds_barrier<C::LPW>();
        else lds_barrier<0>();
      }
    }
  }
  // The loop's last barrier waited for every load (no tile load follows the
  // final three tiles), so this wait costs nothing; it tells the compiler
  // that no tile load is pending, which spares the LDS accesses below a
  // wait for the global loads issued after them.
  vm_wait<0>();
  // The wave's last two sub-blocks: the PV product of u_last - 1 and the
  // masked weights and PV product of u_last.  Their tiles are among the
  // last five of the workgroup (a wave's last sub-block is at most seven
  // sub-blocks before the workgroup's), so they are still in LDS: no load
  // was issued after the final one.
  if (wave_live) {
    if (u_last >= 1) {
      uint32_t pkl[8];  // weights of sub-block u_last - 1, from the array of its parity
#pragma unroll
      for (int i = 0; i < 8; ++i) pkl[i] = (u_last & 1) ? pkA[i] : pkB[i];
      pv_gemm(v_lds[((u_last - 1) / SUB) % NB5], (u_last - 1) % SUB, pkl);
    }
    const uint16_t* vt = v_lds[(u_last / SUB) % NB5];
    const f32x16 cur = (u_last % 2 == 0) ? sA : sB;
    uint32_t pk[8];
    const float lsum = exp_pack(cur, 32 * u_last, pk, std::true_type{});
    settle(cur, 32 * u_last, pk, lsum, std::true_type{});
    pv_gemm(vt, u_last % SUB, pk);
  }

  // The next block's Q (the tail above was the last use of this block's),
  // in flight during the epilogue.
  if (nbh >= 0) load_q(nbh, nqblk);

  // ---- epilogue: one divide per row, store O and the natural-log LSE ------
  // A lane holds 4-element pieces of its own query's row, so storing from
  // registers would make every store instruction touch 32 rows.  Instead
  // each wave stages its 32 x D tile of O in its own part of ring slots 3
  // and 4 (idle now: the next block's first tiles go to slots 0-2 as soon
  // as every wave's tail has read the ring), swizzled row-major, and reads
  // it back so that every store instruction writes whole rows (64 lanes x
  // 16 bytes).
  const float l_tot = halves_sum(l_run);
  const float inv = 1.f / l_tot;
  const int qrow = query - qshift;  // the real query of this lane's virtual row
  if (wave_live && g == 0 && qrow >= 0 && qrow < Nq) lseg[(size_t)bh * Nq + qrow] = (m_run + __log2f(l_tot)) * kLn2;
  lds_only_barrier();  // every wave's tail has finished reading the ring
  static_assert(4 * 32 * D <= 2 * BN * D, "four waves' O tiles fit in two ring slots");
  uint16_t* stage = (wave < 4 ? v_lds[3] : k_lds[3]) + (wave % 4) * 32 * D;
  // Read-back instruction i covers rows 64 i / CPR .. of the tile: lane l
  // takes row (64 i + l) / CPR, 16-byte chunk l % CPR.  A wave reads back
  // only its own tile, so no barrier sits between its writes and reads.
  // Both come before the next block's tile loads, which the compiler would
  // otherwise make them wait for (it cannot tell the LDS ranges apart).
  constexpr int CPR = D / 8, ROWS = 64 / CPR;
  uint4 ox[32 / ROWS];
  int li = lane;
  if (wave_live) {
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const f32x16& v = oacc[db];
        const uint2 w = make_uint2(pack2(T{}, v[4 * rq + 0] * inv, v[4 * rq + 1] * inv),
                                   pack2(T{}, v[4 * rq + 2] * inv, v[4 * rq + 3] * inv));
        *reinterpret_cast<uint2*>(stage + swz<D>(n, 32 * db + 8 * rq + 4 * g)) = w;
      }
    }
    // The lane index goes through an empty asm so the addresses are formed
    // here, not hoisted and kept live.
    asm volatile("" : "+v"(li));
#pragma unroll
    for (int i = 0; i < 32 / ROWS; ++i) {
      const int r = ROWS * i + li / CPR, c = li % CPR;
      ox[i] = *reinterpret_cast<const uint4*>(stage + swz<D>(r, 8 * c));
    }
  }
  if (nbh >= 0) issue_first(nbh, nqblk);
  if (wave_live) {
    // Buffer stores, whole rows per instruction: rows past Nq, or before 0
    // (virtual rows, whose offset wraps), fall outside the head's range and
    // are dropped.
    const int q_first = qw0 - qshift;  // the real query of the wave's row 0
    const rsrc_t ors = make_rsrc(og + head, (uint32_t)Nq * D * 2);
#pragma unroll
    for (int i = 0; i < 32 / ROWS; ++i) {
      const int r = ROWS * i + li / CPR, c = li % CPR;
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u32, ox[i]), ors,
                                             ((uint32_t)(q_first + r) * D + 8 * c) * 2, 0, 0);
    }
  }
  };

  // Persistent loop: the grid holds one workgroup per CU and each walks
  // its share of equal-cost work items (items_per_head / item_blocks).
  // Logical item L = r G + xcd_remap(blockIdx), so in every round r each
  // XCD works on a contiguous range of items, i.e. on shared heads.  The
  // heavier query block of a causal pair goes first.
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
  if (block_at(L, 0, &bh, &qb)) {
    load_q(bh, qb);
    issue_first(bh, qb);
  }
  while (bh >= 0) {  // one call site: the block body is large
    int nbh = -1, nqb = -1;
    if (block_at(L, t + 1, &nbh, &nqb)) {
      ++t;
    } else {
      L += gridDim.x;
      t = 0;
      if (!block_at(L, 0, &nbh, &nqb)) nbh = -1;
    }
    block(bh, qb, nbh, nqb);
    // Every wave has read its staged O before the next block's tile loads
    // reach slots 3 and 4; the O stores may still be in flight.
    lds_only_barrier();
    bh = nbh;
    qb = nqb;
  }
}
// ===========================================================================
// 16-bit forward for short sequences on few heads: the keys of a block are
// split among the waves of its workgroup
// ===========================================================================
// When B H ceil(N / 256) work items leave CUs idle and every key a block can
// see fits in LDS (at most KMAX keys), the query blocks shrink to 64 rows and
// each workgroup's eight waves split the work as two 32-query groups x four
// key ranges of at most SMAX 32-key sub-blocks.  A wave fetches what it
// reads straight into LDS (swizzled row-major, as the persistent kernel's
// tiles): its group's Q rows, then K, then V of its sub-blocks.  It waits
// only for its own loads, so no barrier stands between the loads and the
// products, and its score products start while V is still arriving; the two
// query groups of a key range both fetch it and write identical bytes to
// identical LDS addresses.  With at most SMAX sub-blocks per wave the
// softmax needs no running correction: the wave forms S^T = K Q^T for all of
// them, takes the exact row max once, then adds the weights and
// O^T += V^T P^T sub-block by sub-block.  Only the sub-block that holds the
// causal diagonal or the sequence end is masked.  The four partial results
// of a query group are merged through LDS with the log-sum-exp form of the
// softmax decomposition ("Paper review: FlashAttention ...",
// osehyeon.github.io, "Tiling"): M = max_r m_r, L = sum_r l_r 2^(m_r - M),
// O = sum_r O_r 2^(m_r - M) / L.  Square attention only (queries and keys
// share positions).
template <int D>
struct FwdSplit {
  static constexpr int NW = 8, NT = 64 * NW, QG = 2, KQ = 4, BM = 32 * QG;
  static constexpr int DS = D / 16, DB = D / 32, CPR = D / 8;
  static constexpr int KMAX = D == 64 ? 512 : 256;  // keys of K and V in 128 KB
  static constexpr int RPP = 64 / CPR;              // rows per 1 KB wave load
  static constexpr int PPS = 32 / RPP;              // wave loads per 32-row sub-block of K (or V)
  static constexpr int SMAX = KMAX / 32 / KQ;       // sub-blocks per key range, at most
  static constexpr int PROW = D + 4;                // floats per row of a partial O (padded)
  static constexpr int KV_BYTES = 2 * KMAX * D * 2 + BM * D * 2;  // K, V, then the block's Q rows
  static constexpr int PART_BYTES = NW * 32 * PROW * 4;
  static constexpr int LDS_BYTES = KV_BYTES > PART_BYTES ? KV_BYTES : PART_BYTES;
  static_assert(PPS + 2 * PPS * SMAX < 64, "vmcnt range");
};

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(512) void fwd16_split_kernel(
    const uint16_t* __restrict__ qg, const uint16_t* __restrict__ kg, const uint16_t* __restrict__ vg,
    uint16_t* __restrict__ og, float* __restrict__ lseg, int N, int n_qblk, int G, float qk_scale,
    uint32_t qsign) {
  using C = FwdSplit<D>;
  constexpr int DS = C::DS, DB = C::DB, CPR = C::CPR, PPS = C::PPS, SMAX = C::SMAX;
  __shared__ __attribute__((aligned(16))) unsigned char lds_raw[C::LDS_BYTES];
  __shared__ float mrg_m[C::QG][C::KQ][32], mrg_l[C::QG][C::KQ][32];
  uint16_t* k_lds = reinterpret_cast<uint16_t*>(lds_raw);
  uint16_t* v_lds = k_lds + C::KMAX * D;
  uint16_t* q_lds = v_lds + C::KMAX * D;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 31, g = lane >> 5;
  const int qgrp = wave & 1, kq = wave >> 1;
  // The blocks of one head go to one XCD (contiguous logical numbers per
  // XCD), where they share the head's K/V in that XCD's L2.
  const int lb = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = lb / n_qblk, qblk = lb % n_qblk;
  const int q0 = qblk * C::BM;
  const int qw0 = q0 + 32 * qgrp;  // first query of this wave
  const int query = qw0 + n;
  const uint32_t head_bytes = (uint32_t)N * D * 2;
  const size_t kvhead = (size_t)kv_head_of(bh, G) * (size_t)N * D;
  const rsrc_t krs = make_rsrc(kg + kvhead, head_bytes);
  const rsrc_t vrs = make_rsrc(vg + kvhead, head_bytes);

  // ---- this wave's sub-blocks ---------------------------------------------
  // The block's visible keys form ns sub-blocks, dealt to the four key
  // ranges; a causal wave stops at its diagonal sub-block (qw0 / 32), and a
  // wave whose queries all lie past N has nothing to do.
  const int kend = CAUSAL ? min(q0 + C::BM, N) : N;  // <= KMAX (host-checked)
  const int ns = (kend + 31) / 32;
  const int u0 = kq * ns / C::KQ;
  int ul = (kq + 1) * ns / C::KQ - 1;
  if (CAUSAL) ul = min(ul, qw0 / 32);
  if (qw0 >= N) ul = u0 - 1;
  const int nsb = max(ul - u0 + 1, 0);  // 0 .. SMAX
  // The one sub-block that needs the mask: the diagonal, or the one that
  // holds the sequence end when N is not a multiple of 32.  Keys before it
  // are visible to every query of the wave.
  const int mu = CAUSAL ? qw0 / 32 : (N % 32 != 0 ? ns - 1 : -1);
  const int key_lim = CAUSAL ? min(query + 1, N) : N;

  const rsrc_t qrs = make_rsrc(qg + (size_t)bh * N * D, head_bytes);
  uint4 qf[DS];
  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
  float m_raw = kNegInf;               // row max of the raw scores
  float m_run = kNegInf, l_run = 0.f;  // row max (scaled, log2 units) and this lane's sum

  // Slot i of the wave holds sub-block u0 + i; slots past the wave's last
  // sub-block hold the block's last one again (loaded, not used).
  uint16_t* const qs = q_lds + qgrp * 32 * D;
  auto slot_u = [&](int i) { return min(u0 + i, ns - 1); };
  auto kslot = [&](int i) { return k_lds + 32 * slot_u(i) * D; };
  auto vslot = [&](int i) { return v_lds + 32 * slot_u(i) * D; };
  {
    // Wave load p of 32 rows fills RPP of them: lane l writes bytes 16 l,
    // i.e. row RPP p + l / CPR, stored chunk l % CPR holding the row's
    // logical chunk (l % CPR) ^ swz_chunk(row) (the swizzle repeats every 16
    // rows, so slot rows and block rows agree).  Rows past N read as zeros.
    // Every wave issues the same loads in the same order, so the count still
    // in flight behind any of them is a compile-time constant.
    auto issue32 = [&](const rsrc_t& rs, uint16_t* dst, int row0) __attribute__((always_inline)) {
#pragma unroll
      for (int p = 0; p < PPS; ++p) {
        const int row = p * C::RPP + lane / CPR;
        const int chunk = (lane % CPR) ^ swz_chunk<D>(row);
        load_lds16_untracked(rs, lds_addr(dst + p * C::RPP * D), ((uint32_t)(row0 + row) * D + 8 * chunk) * 2);
      }
    };
    issue32(qrs, qs, qw0);
#pragma unroll
    for (int i = 0; i < SMAX; ++i) issue32(krs, kslot(i), 32 * slot_u(i));
#pragma unroll
    for (int i = 0; i < SMAX; ++i) issue32(vrs, vslot(i), 32 * slot_u(i));

    // ---- scores of every slot, then the exact row max over them -----------
    f32x16 sc[SMAX];
    auto scores = [&](auto ic) __attribute__((always_inline)) {
      constexpr int i = decltype(ic)::value;
      if (i >= nsb) return;
      // Q and this slot's K are in LDS once only later K slots and the V
      // slots may remain in flight
      vm_wait<(SMAX - 1 - i) * PPS + SMAX * PPS>();
      lds_fence();
      if (i == 0) {
        // Q fragments (B operand of S^T = K Q^T): lane supplies
        // Q[query][16 s + 8 g + 0..7]; a negative scale flips their sign bits
#pragma unroll
        for (int s = 0; s < DS; ++s) {
          qf[s] = read_row<D>(qs, n, 16 * s + 8 * g);
          qf[s].x ^= qsign; qf[s].y ^= qsign; qf[s].z ^= qsign; qf[s].w ^= qsign;
        }
      }
      const uint16_t* kt = kslot(i);
      f32x16 s = f32x16{};
#pragma unroll
      for (int st = 0; st < DS; ++st) s = mma16(T{}, read_row<D>(kt, n, 16 * st + 8 * g), qf[st], s);
      sc[i] = s;
      const int u = u0 + i;
      // raw max; only the diagonal / sequence-end sub-block has invisible keys
      if (u == mu) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kb = 32 * u + 4 * g + 8 * (r / 4) + (r % 4);
          m_raw = fmaxf(m_raw, kb < key_lim ? s[r] : kNegInf);
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) m_raw = fmaxf(m_raw, s[r]);
      }
    };
    // ---- weights and O^T += V^T P^T, slot by slot --------------------------
    auto accumulate = [&](auto ic) __attribute__((always_inline)) {
      constexpr int i = decltype(ic)::value;
      if (i >= nsb) return;
      const int u = u0 + i;
      const f32x16& s = sc[i];
      uint32_t pk[8];
      // weights packed to 16 bits (the B operand of the PV product); returns
      // this lane's sum of them
      auto weights = [&](auto masked) __attribute__((always_inline)) {
        constexpr bool MASKED = decltype(masked)::value;
        float part[2] = {0.f, 0.f};
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          float p0 = fast_exp2(__builtin_fmaf(s[r], qk_scale, -m_run));
          float p1 = fast_exp2(__builtin_fmaf(s[r + 1], qk_scale, -m_run));
          if constexpr (MASKED) {
            const int kb = 32 * u + 4 * g + 8 * (r / 4) + (r % 4);
            p0 = kb < key_lim ? p0 : 0.f;
            p1 = kb + 1 < key_lim ? p1 : 0.f;
          }
          pk[r / 2] = pack2(T{}, p0, p1);
          part[(r / 2) % 2] = r < 4 ? first_pair(T{}, pk[r / 2], p0, p1)
                                    : add_pair(T{}, pk[r / 2], p0, p1, part[(r / 2) % 2]);
        }
        return part[0] + part[1];
      };
      l_run += (u == mu) ? weights(std::true_type{}) : weights(std::false_type{});
      const uint4 pp[2] = {make_uint4(pk[0], pk[1], pk[2], pk[3]), make_uint4(pk[4], pk[5], pk[6], pk[7])};
      // this slot's V is in LDS once only the later V slots remain in flight
      vm_wait<(SMAX - 1 - i) * PPS>();
      lds_fence();
      const uint16_t* vt = vslot(i);
#pragma unroll
      for (int k2 = 0; k2 < DS; ++k2) {
        const uint4 b = read_tr<D>(vt, 16 * (k2 / DB), 32 * (k2 % DB), lane);
        oacc[k2 % DB] = mma16(T{}, b, pp[k2 / DB], oacc[k2 % DB]);
      }
    };
    scores(std::integral_constant<int, 0>{});
    scores(std::integral_constant<int, 1>{});
    if constexpr (SMAX == 4) {
      scores(std::integral_constant<int, 2>{});
      scores(std::integral_constant<int, 3>{});
    }
    // the two lane halves hold different keys of the same queries; the
    // scale is >= 0, so scaling the raw max gives the max of the scaled scores
    m_run = halves_max(m_raw) * qk_scale;
    accumulate(std::integral_constant<int, 0>{});
    accumulate(std::integral_constant<int, 1>{});
    if constexpr (SMAX == 4) {
      accumulate(std::integral_constant<int, 2>{});
      accumulate(std::integral_constant<int, 3>{});
    }
  }
  const float m = nsb > 0 ? m_run : kNegInf;

  // ---- merge the four key ranges of each query group ----------------------
  const float l_tot = halves_sum(l_run);
  if (g == 0) {
    mrg_m[qgrp][kq][n] = m;
    mrg_l[qgrp][kq][n] = l_tot;
  }
  // Every load into LDS has landed (a wave with idle slots, or none live,
  // still has loads in flight here, which the compiler does not know of)
  // before the partial results below overwrite K and V.
  vm_wait<0>();
  lds_fence();
  __syncthreads();  // every wave is done with K and V, and m, l are shared
  float M = kNegInf;
#pragma unroll
  for (int r = 0; r < C::KQ; ++r) M = fmaxf(M, mrg_m[qgrp][r][n]);
  float L = 0.f;
#pragma unroll
  for (int r = 0; r < C::KQ; ++r) {
    const float mr = mrg_m[qgrp][r][n];
    L += (mr == kNegInf) ? 0.f : mrg_l[qgrp][r][n] * fast_exp2(mr - M);
  }
  const float wself = (m == kNegInf) ? 0.f : fast_exp2(m - M) / L;
  // this wave's weighted partial O, row-major [32][PROW] fp32: register r of
  // d block db is column 32 db + 8 (r / 4) + 4 g + r % 4 of row n
  float* part = reinterpret_cast<float*>(lds_raw) + wave * 32 * C::PROW;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<float4*>(part + n * C::PROW + 32 * db + 8 * j + 4 * g) =
          make_float4(oacc[db][4 * j] * wself, oacc[db][4 * j + 1] * wself, oacc[db][4 * j + 2] * wself,
                      oacc[db][4 * j + 3] * wself);
  if (kq == 0 && g == 0 && query < N) lseg[(size_t)bh * N + query] = (M + __log2f(L)) * kLn2;
  __syncthreads();
  // O = the sum of the four partials, 8 elements (16 bytes) per store
  const rsrc_t ors = make_rsrc(og + (size_t)bh * N * D, head_bytes);
  for (int c = threadIdx.x; c < C::BM * CPR; c += C::NT) {
    const int row = c / CPR, ch = c % CPR, grp = row / 32, rn = row % 32;
    float acc8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < C::KQ; ++r) {
      const float* src = reinterpret_cast<const float*>(lds_raw) + (2 * r + grp) * 32 * C::PROW + rn * C::PROW + 8 * ch;
      const float4 x = *reinterpret_cast<const float4*>(src);
      const float4 y = *reinterpret_cast<const float4*>(src + 4);
      acc8[0] += x.x; acc8[1] += x.y; acc8[2] += x.z; acc8[3] += x.w;
      acc8[4] += y.x; acc8[5] += y.y; acc8[6] += y.z; acc8[7] += y.w;
    }
    const uint4 o = make_uint4(pack2(T{}, acc8[0], acc8[1]), pack2(T{}, acc8[2], acc8[3]),
                               pack2(T{}, acc8[4], acc8[5]), pack2(T{}, acc8[6], acc8[7]));
    // rows past N fall outside the head's range and are dropped
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u32, o), ors,
                                           ((uint32_t)(q0 + row) * D + 8 * ch) * 2, 0, 0);
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
                                                        float* __restrict__ lseg, int N, int n_qblk, int G,
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
  const size_t kvhead = (size_t)kv_head_of(bh, G) * (size_t)N * D;
  const rsrc_t krs = make_rsrc(kg + kvhead, head_bytes);
  const rsrc_t vrs = make_rsrc(vg + kvhead, head_bytes);
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

// ===========================================================================
// fp32 forward for short sequences on few heads: one 32-query block per
// workgroup, its keys split over the eight waves
// ===========================================================================
// When the 128-query blocks of the fp32 kernel leave CUs idle, each
// workgroup takes one block of 32 queries and its eight waves split the
// block's visible keys into eight ranges of 32-key sub-blocks.  Each wave
// runs the online softmax of the fp32 kernel over its range, and the eight
// partial results are merged through LDS with the log-sum-exp form of the
// softmax decomposition ("Paper review: FlashAttention ...",
// osehyeon.github.io, "Tiling").  The operands come straight from global
// memory (through L1/L2; no K/V tile is shared within the workgroup): in
// S^T = K Q^T the contraction may run over the head dimension in any order,
// so lane half g supplies elements g D/2 .. g D/2 + D/2 - 1 of its K and Q
// rows, contiguous floats; O^T += V^T P^T takes, as in the fp32 kernel, the
// key of accumulator register r on both operands.
template <int D>
struct Fwd32Split {
  static constexpr int NW = 8, NT = 64 * NW, BM = 32;
  static constexpr int DB = D / 32, HD = D / 2;  // d blocks of O; dimensions per lane half
  static constexpr int PROW = D + 4;             // floats per row of a partial O (padded)
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(512) void fwd32_split_kernel(const float* __restrict__ qg, const float* __restrict__ kg,
                                                          const float* __restrict__ vg, float* __restrict__ og,
                                                          float* __restrict__ lseg, int N, int n_qblk, int G,
                                                          float qk_scale, float qsign) {
  using C = Fwd32Split<D>;
  constexpr int DB = C::DB, HD = C::HD;
  __shared__ __attribute__((aligned(16))) float part[C::NW][32 * C::PROW];
  __shared__ float mrg_m[C::NW][32], mrg_l[C::NW][32];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 31, g = lane >> 5;
  // the blocks of one head go to one XCD, where they share its K/V in L2
  const int lb = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = lb / n_qblk, qblk = lb % n_qblk;
  const int q0 = qblk * C::BM, query = q0 + n;
  const uint32_t head_bytes = (uint32_t)N * D * 4;
  const rsrc_t qrs = make_rsrc(qg + (size_t)bh * N * D, head_bytes);
  const size_t kvhead = (size_t)kv_head_of(bh, G) * (size_t)N * D;
  const rsrc_t krs = make_rsrc(kg + kvhead, head_bytes);
  const rsrc_t vrs = make_rsrc(vg + kvhead, head_bytes);

  // The block's visible keys form ns sub-blocks, dealt to the eight waves.
  // Only the last one can hold invisible keys (the causal diagonal, or the
  // sequence end); keys before it are visible to every query of the block.
  const int kend = CAUSAL ? min(q0 + C::BM, N) : N;
  const int ns = (kend + 31) / 32;
  const int u0 = wave * ns / C::NW, u1 = (wave + 1) * ns / C::NW;
  const int key_lim = CAUSAL ? min(query + 1, N) : N;

  // Q (B operand of S^T = K Q^T): lane half g holds elements g HD .. of its
  // query's row, zeros past N; a negative scale flips its sign.
  float qf[HD];
#pragma unroll
  for (int t = 0; t < HD / 4; ++t) {
    const float4 x = load16f(qrs, ((uint32_t)query * D + g * HD + 4 * t) * 4);
    qf[4 * t] = x.x * qsign; qf[4 * t + 1] = x.y * qsign; qf[4 * t + 2] = x.z * qsign; qf[4 * t + 3] = x.w * qsign;
  }

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
  float m_run = kNegInf, l_run = 0.f;
  for (int u = u0; u < u1; ++u) {
    const int key0 = 32 * u;
    f32x16 s1[1] = {f32x16{}};
#pragma unroll
    for (int t = 0; t < HD / 4; ++t) {
      const float4 kx = load16f(krs, ((uint32_t)(key0 + n) * D + g * HD + 4 * t) * 4);
      s1[0] = mma32(kx.x, qf[4 * t], s1[0]);
      s1[0] = mma32(kx.y, qf[4 * t + 1], s1[0]);
      s1[0] = mma32(kx.z, qf[4 * t + 2], s1[0]);
      s1[0] = mma32(kx.w, qf[4 * t + 3], s1[0]);
    }
    const bool masked = u == ns - 1;
    const float mt = masked ? tile_max<1, true>(s1, qk_scale, key0 + 4 * g, key_lim)
                            : tile_max<1, false>(s1, qk_scale, 0, 0);
    float alpha;
    if (raise_max(mt, m_run, l_run, &alpha)) {
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
    }
    const float m_use = (m_run == kNegInf) ? 0.f : m_run;
    l_run += masked ? tile_exp<1, true>(s1, qk_scale, m_use, key0 + 4 * g, key_lim)
                    : tile_exp<1, false>(s1, qk_scale, m_use, 0, 0);
    // O^T += V^T P^T: k-step r takes key key0 + 8 (r / 4) + 4 g + r % 4 on
    // both operands (rows past N read as zeros and carry weight 0)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = key0 + 8 * (r / 4) + 4 * g + (r % 4);
#pragma unroll
      for (int db = 0; db < DB; ++db)
        oacc[db] = mma32(load4f(vrs, ((uint32_t)key * D + 32 * db + n) * 4), s1[0][r], oacc[db]);
    }
  }

  // ---- merge the eight key ranges ------------------------------------------
  // this wave's (m, l) and its un-normalised O, row-major [32][PROW]:
  // register r of d block db is column 32 db + 8 (r / 4) + 4 g + r % 4 of row n
  const float l_tot = halves_sum(l_run);
  if (g == 0) {
    mrg_m[wave][n] = m_run;
    mrg_l[wave][n] = l_tot;
  }
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<float4*>(&part[wave][n * C::PROW + 32 * db + 8 * j + 4 * g]) =
          make_float4(oacc[db][4 * j], oacc[db][4 * j + 1], oacc[db][4 * j + 2], oacc[db][4 * j + 3]);
  __syncthreads();
  // M = max_w m_w, L = sum_w l_w 2^(m_w - M), O = sum_w O_w 2^(m_w - M) / L;
  // thread c forms row c / (D / 4), columns 4 (c % (D / 4)) .. + 3
  const size_t head = (size_t)bh * N * D;
  for (int c = threadIdx.x; c < 32 * D / 4; c += C::NT) {
    const int row = c / (D / 4), col = 4 * (c % (D / 4));
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < C::NW; ++w) M = fmaxf(M, mrg_m[w][row]);
    float L = 0.f;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int w = 0; w < C::NW; ++w) {
      const float mw = mrg_m[w][row];
      const float wt = (mw == kNegInf) ? 0.f : fast_exp2(mw - M);
      L += wt * mrg_l[w][row];
      const float4 x = *reinterpret_cast<const float4*>(&part[w][row * C::PROW + col]);
      o.x += wt * x.x; o.y += wt * x.y; o.z += wt * x.z; o.w += wt * x.w;
    }
    if (q0 + row < N) {
      const float inv = 1.f / L;
      *reinterpret_cast<float4*>(og + head + (size_t)(q0 + row) * D + col) =
          make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
      if (col == 0) lseg[(size_t)bh * N + q0 + row] = (M + __log2f(L)) * kLn2;
    }
  }
}

// Tile per head dim: 8 waves x 32 queries (two waves per SIMD), 64 keys per
// tile for d = 128 and 128 for d = 64 (16 KB of K and of V per tile either
// way; five such buffers fill the LDS, so d = 128 has no larger tile).
// Must agree with fwd_tile() in fa_plan.hpp.
template <int D>
struct Tile16 {
  static constexpr int BN = D == 128 ? 64 : FA_FWD16_BN_D64;
};

// The key-split kernel serves square problems whose work items leave CUs
// idle and whose keys fit its LDS.
template <int D>
bool split_keys(const FwdArgs& a, int items, int cus) {
  return a.Nk == a.N && items < cus && a.N <= FwdSplit<D>::KMAX;
}

// The persistent kernel with NW waves per workgroup: one workgroup per CU
// (the LDS ring takes the whole 160 KB), never more workgroups than items.
template <typename T, int D, bool CAUSAL, int NW>
hipError_t launch16_nw(const FwdArgs& a, int cus, int qshift, int koff) {
  constexpr int BN = Tile16<D>::BN;
  using C = Fwd16<T, D, BN, CAUSAL, NW>;
  const int n_qblk = (a.N + qshift + C::BM - 1) / C::BM;
  const long long items = (long long)items_per_head(n_qblk, CAUSAL) * a.BH;
  if (items > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const int grid = (int)(items < cus ? items : cus);
  hipLaunchKernelGGL((fwd16_kernel<T, D, BN, CAUSAL, NW>), dim3((unsigned)grid), dim3(C::NT), 0, a.stream,
                     static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                     static_cast<const uint16_t*>(a.v), static_cast<uint16_t*>(a.o), a.lse, a.N, a.Nk, qshift, koff,
                     n_qblk, a.BH, a.G, a.qk_scale, a.neg ? 0x80008000u : 0u);
  return hipGetLastError();
}

template <typename T, int D, bool CAUSAL>
hipError_t launch16(const FwdArgs& a) {
  constexpr int BN = Tile16<D>::BN;
  using C = Fwd16<T, D, BN, CAUSAL>;
  // Causal queries are the last N of Nk positions: offset Nk - N, split into
  // a multiple of 32 (koff) and a shift of the virtual query rows (qshift).
  const int off = CAUSAL ? a.Nk - a.N : 0;
  const int qshift = off % 32, koff = off - qshift;
  const int n_qblk = (a.N + qshift + C::BM - 1) / C::BM;
  const long long items = (long long)items_per_head(n_qblk, CAUSAL) * a.BH;
  if (items > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  if (split_keys<D>(a, (int)items, cus)) {
    // fewer items than CUs: 64-query blocks, keys split inside the workgroup
    using S = FwdSplit<D>;
    const int nb = (a.N + S::BM - 1) / S::BM;
    hipLaunchKernelGGL((fwd16_split_kernel<T, D, CAUSAL>), dim3((unsigned)(nb * a.BH)), dim3(S::NT), 0, a.stream,
                       static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                       static_cast<const uint16_t*>(a.v), static_cast<uint16_t*>(a.o), a.lse, a.N, nb, a.G,
                       a.qk_scale, a.neg ? 0x80008000u : 0u);
    return hipGetLastError();
  }
  // At most half as many 256-query items as CUs: 128-query items on four
  // waves fill twice the CUs; a CU then runs one wave per SIMD, slower per
  // query than two, but twice the CUs work.
  if (C::NW == 8 && 2 * items <= cus) return launch16_nw<T, D, CAUSAL, 4>(a, cus, qshift, koff);
  return launch16_nw<T, D, CAUSAL, C::NW>(a, cus, qshift, koff);
}

template <int D, bool CAUSAL>
hipError_t launch32(const FwdArgs& a) {
  constexpr int BN = 64, NW = 4;
  using C = Fwd32<D, BN, NW, CAUSAL>;
  const int n_qblk = (a.N + C::BM - 1) / C::BM;
  const long long grid = (long long)n_qblk * a.BH;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  if (a.Nk == a.N && grid < cus) {
    // fewer 128-query blocks than CUs: 32-query blocks, keys split inside
    using S = Fwd32Split<D>;
    const long long nb = (a.N + S::BM - 1) / S::BM;
    if (nb * a.BH > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((fwd32_split_kernel<D, CAUSAL>), dim3((unsigned)(nb * a.BH)), dim3(S::NT), 0, a.stream,
                       static_cast<const float*>(a.q), static_cast<const float*>(a.k),
                       static_cast<const float*>(a.v), static_cast<float*>(a.o), a.lse, a.N, (int)nb, a.G,
                       a.qk_scale, a.neg ? -1.f : 1.f);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((fwd32_kernel<D, BN, NW, CAUSAL>), dim3((unsigned)grid), dim3(C::NT), 0, a.stream,
                     static_cast<const float*>(a.q), static_cast<const float*>(a.k), static_cast<const float*>(a.v),
                     static_cast<float*>(a.o), a.lse, a.N, n_qblk, a.G, a.qk_scale, a.neg ? -1.f : 1.f);
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
