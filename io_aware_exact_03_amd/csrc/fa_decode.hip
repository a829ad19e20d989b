// fa_decode.hip -- decoding: the newest query of every head against its
// K/V cache, the keys shared out evenly among workgroups, the pieces of
// heads cut between workgroups merged.
//
// Pages cited: "Flash Attention -- five lessons converging into 80 lines"
// (brianyu43.github.io), "LLM-serving translation" (in decoding Q has one
// row per head); "Flash Attention: IO-awareness principle" (hrletsgo.me),
// section on serving (with few K/V heads and batch 1 a decode step has too
// few tiles to fill the GPU, hence kernels that split the keys); "Paper
// review: FlashAttention ... with IO-Awareness" (osehyeon.github.io), the
// softmax decomposition under "Tiling" (max and normaliser of a
// concatenation from those of its parts), which merges the pieces.
//
// Decoding reads every cached key and value once and does 4 d flops per key
// per query head, so it is bound by HBM bandwidth, not by the matrix cores.
// The design keeps the K/V stream as wide and deep as LDS allows and spends
// matrix-core work freely: the G query heads that share a K/V head are the
// 32 columns of one MFMA product (padded with zeros), so each K/V element
// is read from HBM once for the whole group.
//
// Work split (fa_plan.hpp): the key tiles of every unit (batch, K/V head,
// block of 32 query heads) are laid end to end and cut into as many equal
// ranges as there are workgroups, so ragged batches stay balanced.
// Split kernel, one workgroup per range, walking its range unit by unit:
//   * a unit's piece is cut into 32-key sub-tiles and wave w takes sub-tiles
//     w, w + NW, w + 2 NW, ...: every wave streams its own keys, with no
//     workgroup barrier, K and V rows straight into the wave's own LDS rings
//     (buffer_load ... lds, rows swizzled as in the forward), several
//     sub-tiles ahead, so each CU has many loads outstanding, which a
//     bandwidth-bound stream needs;
//   * per step a wave runs the score products of its next sub-tile on the
//     matrix cores while its vector units form the current sub-tile's
//     weights, then the current PV product;
//   * the buffer range of the head ends at its valid length, so keys past it
//     read as zeros (never a stale or non-finite cache entry) and are masked;
//   * S^T = K Q^T on v_mfma_f32_32x32x16 (lane = query head, registers =
//     keys), an online softmax in base 2 per wave, O^T += V^T P^T with V^T
//     from transposing LDS reads;
//   * at the end of a unit's piece the waves' (m, l, O) are combined through
//     LDS; a whole unit is written to the outputs, a piece to its workspace
//     slot.
// Merge kernel (more than one range), one workgroup per (unit, query
// column) that was cut: with M = max_s LSE_s and w_s = exp(LSE_s - M),
// LSE = M + ln sum w_s and O = sum w_s O_s / sum w_s.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_device.hpp"
#include "fa_kernels.hpp"
#include "fa_plan.hpp"

namespace fa {
namespace {

template <int D, int NW_, int NSLOT_>
struct Dec {
  static constexpr int NW = NW_, NT = 64 * NW, NSLOT = NSLOT_;
  static constexpr int DS = D / 16, DB = D / 32, CPR = D / 8;
  static constexpr int RPP = 64 / CPR;          // sub-tile rows per 1 KB wave load
  static constexpr int VL = 32 / RPP;           // 1 KB loads per 32-key K or V sub-tile
  static constexpr int KSLOT = NSLOT - 1;       // K ring slots (K runs one fewer sub-tile ahead)
  static constexpr int EPT = D / (2 * NW);      // output elements per thread in the combine
  static constexpr int OROW = D + 4;            // padded fp32 row of a wave's O in LDS (16-byte rows)
  static_assert((NSLOT + KSLOT) * NW * 32 * D * 2 <= 160 * 1024, "rings fit in LDS");
  static_assert(EPT % 8 == 0, "combine vector width");
  static_assert(NW * 32 * (OROW + 2) * 4 <= NW * NSLOT * 32 * D * 2, "combine fits in the ring");
};

// Valid length of batch b, clamped to [0, Nkv].
__device__ __forceinline__ int decode_len(const int* kv_lens, int b, int Nkv) {
  const int l = kv_lens ? kv_lens[b] : Nkv;
  return l < 0 ? 0 : (l > Nkv ? Nkv : l);
}

// Wave-wide sum and inclusive prefix sum of an int over the 64 lanes.
__device__ __forceinline__ int wave_total(int v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(v, off, 64);
    if (lane >= off) v += y;
  }
  return v;
}

// Sums of tiles over all batches (T) and over batches < blim (P), and the
// tiles of batch blim itself (nb), computed by each wave on its own from one
// pass over the lengths: no LDS and no barrier, and no second, dependent
// read of a length.  Wave-uniform.
__device__ __forceinline__ void decode_wave_sums(const int* kv_lens, int B, int Nkv, int UB, int blim, int* T_out,
                                                 int* P_out, int* nb_out) {
  const int lane = threadIdx.x & 63;
  int sT = 0, sP = 0, nb = 0;
  for (int c0 = 0; c0 < B; c0 += 64) {
    const int b = c0 + lane;
    const int t = b < B ? decode_tiles(decode_len(kv_lens, b, Nkv)) : 0;
    sT += t * UB;
    sP += b < blim ? t * UB : 0;
    if (blim >= c0 && blim < c0 + 64) nb = __builtin_amdgcn_readlane(t, blim - c0);
  }
  *T_out = __builtin_amdgcn_readfirstlane(wave_total(sT));
  *P_out = __builtin_amdgcn_readfirstlane(wave_total(sP));
  *nb_out = nb;
}

// The partition, computed by each wave on its own: the total tile count T,
// the tiles per part, and the batch b holding tile part * per with the
// first tile P_b of that batch and its own tile count (b = B, P_b = T when
// the part is empty).
// Batches go 64 at a time through a wave-wide prefix sum.  Wave-uniform.
__device__ __forceinline__ void decode_wave_plan(const int* kv_lens, int B, int Nkv, int UB, int parts_total,
                                                 int part, int* T_out, int* per_out, int* b_out, int* Pb_out,
                                                 int* nb_out) {
  const int lane = threadIdx.x & 63;
  int sum = 0;
  for (int b = lane; b < B; b += 64) sum += decode_tiles(decode_len(kv_lens, b, Nkv)) * UB;
  const int T = __builtin_amdgcn_readfirstlane(wave_total(sum));
  const int per = (T + parts_total - 1) / parts_total;
  const int target = part * per;
  *T_out = T;
  *per_out = per;
  *b_out = B;
  *Pb_out = T;
  *nb_out = 0;
  if (target >= T) return;
  int base = 0;
  for (int c0 = 0; c0 < B; c0 += 64) {
    const int b = c0 + lane;
    const int v = b < B ? decode_tiles(decode_len(kv_lens, b, Nkv)) * UB : 0;
    const int incl = base + wave_incl_scan(v);
    const uint64_t hit = __builtin_amdgcn_ballot_w64(v > 0 && incl - v <= target && target < incl);
    if (hit != 0) {
      const int src = __builtin_ctzll(hit);
      *b_out = c0 + src;
      *Pb_out = __builtin_amdgcn_readlane(incl - v, src);
      *nb_out = __builtin_amdgcn_readlane(v, src) / UB;
      return;
    }
    base = __builtin_amdgcn_readlane(incl, 63);
  }
}

template <typename T, int D, int NW, int NSLOT>
__global__ __launch_bounds__(64 * NW) void decode_split_kernel(
    const uint16_t* __restrict__ qg, const uint16_t* __restrict__ kg, const uint16_t* __restrict__ vg,
    const int* __restrict__ kv_lens, uint16_t* __restrict__ og, float* __restrict__ lseg,
    float* __restrict__ opart, float* __restrict__ lpart, int B, int H, int G, int Nkv, float qk_scale) {
  using C = Dec<D, NW, NSLOT>;
  constexpr int DS = C::DS, DB = C::DB;
  // Each wave's rings: NSLOT V and NSLOT - 1 K sub-tiles of 32 swizzled rows.
  __shared__ __attribute__((aligned(16))) uint16_t ring[NW][NSLOT][32 * D];
  __shared__ __attribute__((aligned(16))) uint16_t kring[NW][C::KSLOT][32 * D];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 31, g = lane >> 5;
  const int Hkv = H / G, QB = decode_query_blocks(G), UB = Hkv * QB;

  // Batches with no valid key: O = 0, LSE = -inf (no part owns them).  The
  // lengths are read 64 at a time, one per lane; every wave finds the same
  // batches and the workgroup writes each.
  if (blockIdx.x == 0) {
    for (int c0 = 0; c0 < B; c0 += 64) {
      uint64_t zero = __builtin_amdgcn_ballot_w64(c0 + lane < B && decode_len(kv_lens, c0 + lane, Nkv) == 0);
      while (zero != 0) {
        const int bz = c0 + __builtin_ctzll(zero);
        zero &= zero - 1;
        for (int i = threadIdx.x; i < H * D; i += C::NT) og[((size_t)bz * H) * D + i] = 0;
        for (int i = threadIdx.x; i < H; i += C::NT) lseg[(size_t)bz * H + i] = kNegInf;
      }
    }
  }

  // This part's tile range; consecutive parts share an XCD (and its L2),
  // which the query blocks of one K/V head read in turn.
  const int w = xcd_remap(blockIdx.x, gridDim.x);
  int Ttot, per, b, P_b, nb;
  decode_wave_plan(kv_lens, B, Nkv, UB, (int)gridDim.x, w, &Ttot, &per, &b, &P_b, &nb);
  int t = w * per;
  const int t_end = min(t + per, Ttot);
  if (t >= t_end) return;

  // The unit holding tile t: batch b (first tile P_b, nb tiles per unit),
  // unit ui of the batch.
  int ui = (t - P_b) / nb;
  int P_u = P_b + ui * nb;

  f32x16 oacc[DB];
  float m_run, l_run;  // base-2 running max; this half's share of l

  // Keys [k0, k1) of unit (b, ui), the whole unit or not.
  auto segment = [&](int k0, int k1, int len, bool whole, int slot) __attribute__((always_inline)) {
    const int hkv = ui / QB, qb = ui % QB;
    const int bkv = b * Hkv + hkv;
    const int nq = min(32, G - 32 * qb);  // live query columns
    const int bh0 = bkv * G + 32 * qb;    // flat query head of column 0

    // Q^T fragments (MFMA B operand): lane (n, g) holds query head n,
    // elements 16 k + 8 g .. + 8; dead columns are zero.
    uint4 qf[DS];
#pragma unroll
    for (int k = 0; k < DS; ++k)
      qf[k] = n < nq ? *reinterpret_cast<const uint4*>(qg + (size_t)(bh0 + n) * D + 16 * k + 8 * g)
                     : make_uint4(0u, 0u, 0u, 0u);

    // The buffer range ends at the valid length: later rows read as zeros.
    const uint32_t valid_bytes = (uint32_t)len * D * 2;
    const rsrc_t krs = make_rsrc(kg + (size_t)bkv * Nkv * D, valid_bytes);
    const rsrc_t vrs = make_rsrc(vg + (size_t)bkv * Nkv * D, valid_bytes);

    // This wave's sub-tiles: s = wave + NW i for i < n_mine, keys
    // k0 + 32 s .. + 31.
    const int n_sub = (k1 - k0 + 31) / 32;
    const int n_mine = n_sub > wave ? (n_sub - 1 - wave) / NW + 1 : 0;

    // Loads of the wave's i-th sub-tile: its K rows and its V rows each into
    // a ring slot (row r, stored chunk c holds global chunk c ^
    // swz_chunk(r)), straight from global memory.  The loads are issued so
    // that the compiler does not track them (it would otherwise wait for
    // all of them wherever its view of the stream's branches is unsure);
    // the stream below waits for them explicitly.
    auto issue_rows = [&](const rsrc_t& rs, int i, uint16_t* dst) __attribute__((always_inline)) {
      const int key0 = k0 + 32 * (wave + NW * i);
      const int lrow = lane / C::CPR;
#pragma unroll
      for (int e = 0; e < C::VL; ++e) {
        const int row = e * C::RPP + lrow;
        const int ch = (lane % C::CPR) ^ swz_chunk<D>(row);
        load_lds16_untracked(rs, lds_addr(dst + e * C::RPP * D), ((uint32_t)(key0 + row) * D + 8 * ch) * 2);
      }
    };

#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
    m_run = kNegInf;
    l_run = 0.f;

    // Operand fragments, read from a slot into registers: K fragment k of
    // lane (n, g) is key n, elements 16 k + 8 g .. + 8 (A operand of S^T =
    // K Q^T); V^T fragment h DB + db covers keys 16 h .. and d block db (A
    // operand of O^T += V^T P^T).
    // In the swizzled layout every fragment sits at a per-lane base XOR a
    // constant plus a row offset (the chunk permutation only touches the
    // address bits within a row): K fragment k at Rb ^ 32 k bytes, the two
    // transposing reads of V^T fragment (h, db) at (Tb ^ 64 db) + 32 h D and
    // (Tb ^ 64 db ^ 32) + (32 h + 16) D.  The bases pass through an empty
    // asm at each use, so the addresses are formed next to their reads
    // rather than kept live for every slot of the unrolled loop.
    const uint32_t Rb = 2u * (uint32_t)swz<D>(n, 8 * g);
    const uint32_t Tb = 2u * (uint32_t)swz<D>(4 * g + ((lane & 15) >> 2), 16 * ((lane >> 4) & 1) + 4 * (lane & 3));
    auto read_k = [&](const uint16_t* __restrict__ kt, uint4 (&kfr)[DS]) __attribute__((always_inline)) {
      uint32_t rb = Rb;
      asm volatile("" : "+v"(rb));
      const char* base = reinterpret_cast<const char*>(kt);
#pragma unroll
      for (int k = 0; k < DS; ++k) kfr[k] = *reinterpret_cast<const uint4*>(base + (rb ^ (32 * k)));
    };
    auto read_v = [&](const uint16_t* __restrict__ vt, uint4 (&vfr)[2 * DB]) __attribute__((always_inline)) {
      uint32_t tb = Tb;
      asm volatile("" : "+v"(tb));
      const char* base = reinterpret_cast<const char*>(vt);
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const uint32_t t = tb ^ (64 * db);
          const uint2 lo = read_tr_b64(reinterpret_cast<const uint16_t*>(base + t + 32 * h * D));
          const uint2 hi = read_tr_b64(reinterpret_cast<const uint16_t*>(base + (t ^ 32) + (32 * h + 16) * D));
          vfr[h * DB + db] = make_uint4(lo.x, lo.y, hi.x, hi.y);
        }
    };
    // Once this wave's LDS reads have returned, their slots may be refilled.
    auto reads_done = [&]() __attribute__((always_inline)) {
      lds_fence();
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt, expcnt free
    };

    // Scores of a sub-tile: two independent product chains (even and odd
    // k), summed.  Register r of S^T is key key0 + 8 (r / 4) + 4 g + r % 4.
    f32x16 scur;  // scores of the sub-tile whose weights the next step computes
    // Lazy reference max, as in the forward: the wave's first sub-tile sets
    // the reference to its row max (it holds a valid key); later weights are
    // accepted while each lane's sum of its 16 weights stays at or below
    // 2^8, otherwise (rare) the reference is raised to the row max and O, l
    // rescaled.  Exact: O, l and the LSE share the reference.  Keys past
    // k1 (only in a segment's last sub-tile) get weight zero.
    auto row_max = [&](int key0) __attribute__((always_inline)) {
      float mx = kNegInf;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = key0 + 8 * (r / 4) + 4 * g + (r % 4);
        mx = fmaxf(mx, key < k1 ? scur[r] * qk_scale : kNegInf);
      }
      return halves_max(mx);
    };
    auto weight = [&](int key0, int r) __attribute__((always_inline)) {
      const int key = key0 + 8 * (r / 4) + 4 * g + (r % 4);
      return key < k1 ? fast_exp2(__builtin_fmaf(scur[r], qk_scale, -m_run)) : 0.f;
    };
    // The rare raise, then the row sum joins l and the weights of scur
    // (x) go into the PV product with V^T fragments vfr.
    auto finish = [&](int key0, float (&x)[16], float psum, const uint4 (&vfr)[2 * DB]) __attribute__((always_inline)) {
      if (__builtin_amdgcn_ballot_w64(!(psum <= 256.f)) != 0) {
        const float m_new = fmaxf(m_run, row_max(key0));
        const float alpha = fast_exp2(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
        m_run = m_new;
        psum = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          x[r] = weight(key0, r);
          psum += x[r];
        }
      }
      l_run += psum;
      // P^T as the B operand of O^T += V^T P^T: registers 8 h .. 8 h + 7
      // are the keys of 16-key step h in the order read_tr delivers V^T's rows.
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint4 pk = make_uint4(pack2(T{}, x[8 * h + 0], x[8 * h + 1]), pack2(T{}, x[8 * h + 2], x[8 * h + 3]),
                                    pack2(T{}, x[8 * h + 4], x[8 * h + 5]), pack2(T{}, x[8 * h + 6], x[8 * h + 7]));
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[db] = mma16(T{}, vfr[h * DB + db], pk, oacc[db]);
      }
    };

    // The wave's stream.  K rows of sub-tile j go into K slot j % KA, V rows
    // into V slot j % VA, straight from global memory with loads the
    // compiler does not track.  Software pipeline: step i computes the
    // weights of sub-tile i (scores from step i - 1) while the matrix cores
    // run the score products of sub-tile i + 1, then the PV product of i.
    // So step i reads K(i + 1) and refills its slot with K(i + 1 + KA) once
    // the read has returned, and reads V(i) just before the PV product (to
    // keep its registers free meanwhile) and refills that slot with
    // V(i + VA) after it.  Issue order:
    // K(0) V(0) K(1) V(1) V(2), then K(2) when K(0) has been read, then
    // K(i + 3) V(i + 3) in step i.  So in step i >= 2 the last of K(i + 1)
    // and V(i) is followed by V(i + 1), K(i + 2) and V(i + 2) (those that
    // exist), in step 1 by K(3) and V(3), and in step 0 only K(2) can be in
    // flight (the prologue waited for the rest); waiting until only those
    // are outstanding (in-order counter) means K(i + 1) and V(i) are in LDS.
    // Only this wave reads its slots, so no barrier.  The loop is unrolled
    // over KA VA steps so every LDS offset is fixed.
    constexpr int KA = C::KSLOT, VA = NSLOT, UNR = KA * VA;
    static_assert(KA == 2 && VA == 3, "issue order and waits");
    uint16_t* const myring = ring[wave][0];
    uint16_t* const mykring = kring[wave][0];
    auto kslot = [&](int j) __attribute__((always_inline)) { return mykring + (j % KA) * 32 * D; };
    auto vslot = [&](int j) __attribute__((always_inline)) { return myring + (j % VA) * 32 * D; };
#pragma unroll
    for (int s0 = 0; s0 < VA; ++s0) {
      if (s0 < KA && s0 < n_mine) issue_rows(krs, s0, kslot(s0));
      if (s0 < n_mine) issue_rows(vrs, s0, vslot(s0));
    }
    // Prologue: wait for everything in flight (the first sub-tiles and the
    // query fragments: the compiler tracks the query loads but not the tile
    // loads behind them, so a wait it placed for the fragments would hold a
    // later step until every tile load issued so far had arrived; after this
    // wait it has none to place), the scores of sub-tile 0, the reference.
    if (n_mine > 0) {
      vm_wait<0>();
      uint4 kfr[DS];
      read_k(kslot(0), kfr);
      reads_done();
      if (KA < n_mine) issue_rows(krs, KA, kslot(0));
      f32x16 s0 = f32x16{}, s1 = f32x16{};
#pragma unroll
      for (int k = 0; k < DS; k += 2) {
        s0 = mma16(T{}, kfr[k], qf[k], s0);
        s1 = mma16(T{}, kfr[k + 1], qf[k + 1], s1);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) scur[r] = s0[r] + s1[r];
      m_run = row_max(k0 + 32 * wave);
    }
    // Step i < n_mine - 1 (a next sub-tile exists; sub-tile i has no key
    // past k1).  kt: K slot of i + 1, vt: V slot of i.
    auto step = [&](int i, uint16_t* __restrict__ kt, uint16_t* __restrict__ vt) __attribute__((always_inline)) {
      const int key0 = k0 + 32 * (wave + NW * i);
      uint4 kfr[DS];
      read_k(kt, kfr);
      reads_done();
      if (i + 1 + KA < n_mine) issue_rows(krs, i + 1 + KA, kt);
      // scores of i + 1 on the matrix cores, weights of i beside them: one
      // product, then two weights
      f32x16 s0 = f32x16{}, s1 = f32x16{};
      float x[16], psum = 0.f;
#pragma unroll
      for (int k = 0; k < DS; ++k) {
        if (k % 2 == 0) s0 = mma16(T{}, kfr[k], qf[k], s0);
        else s1 = mma16(T{}, kfr[k], qf[k], s1);
#pragma unroll
        for (int e = 0; e < 16 / DS; ++e) {
          const int r = k * (16 / DS) + e;
          x[r] = fast_exp2(__builtin_fmaf(scur[r], qk_scale, -m_run));
          psum += x[r];
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      uint4 vfr[2 * DB];
      read_v(vt, vfr);
      finish(key0, x, psum, vfr);
      reads_done();
      if (i + VA < n_mine) issue_rows(vrs, i + VA, vt);
#pragma unroll
      for (int r = 0; r < 16; ++r) scur[r] = s0[r] + s1[r];
    };
    // The last step: weights (possibly masked) of the last sub-tile and its
    // PV product, no next scores.
    auto last_step = [&](int i) __attribute__((always_inline)) {
      const int key0 = k0 + 32 * (wave + NW * i);
      uint4 vfr[2 * DB];
      read_v(vslot(i), vfr);
      float x[16], psum = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        x[r] = weight(key0, r);
        psum += x[r];
      }
      finish(key0, x, psum, vfr);
    };
    for (int i0 = 0; i0 < n_mine - 1; i0 += UNR) {
#pragma unroll
      for (int jj = 0; jj < UNR; ++jj) {
        const int i = i0 + jj;
        if (i < n_mine - 1) {
          // loads issued after the last of K(i + 1) and V(i), see above
          const int later = i == 0 ? 1 : (i == 1 ? (3 < n_mine ? 2 : 0) : 1 + (i + 2 < n_mine ? 2 : 0));
          if (later == 3) vm_wait<3 * C::VL>();
          else if (later == 2) vm_wait<2 * C::VL>();
          else if (later == 1) vm_wait<C::VL>();
          else vm_wait<0>();
          lds_fence();
          step(i, kslot(jj + 1), vslot(jj));
        }
      }
    }
    if (n_mine > 0) {
      vm_wait<0>();
      lds_fence();
      last_step(n_mine - 1);
    }

    // Combine the waves through LDS (the rings are free after this barrier:
    // every wave's last wait left no load in flight).
    __syncthreads();
    float* orow = reinterpret_cast<float*>(&ring[0][0][0]);  // [NW][32][OROW]
    float* mrow = orow + NW * 32 * C::OROW;                   // [NW][32]
    float* lrow = mrow + NW * 32;                             // [NW][32]
    const float l_tot = halves_sum(l_run);
    if (g == 0) {
      mrow[wave * 32 + n] = m_run;
      lrow[wave * 32 + n] = l_tot;
    }
    // registers 4 j .. 4 j + 3 of a d block are four consecutive elements
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<float4*>(orow + (wave * 32 + n) * C::OROW + 32 * db + 8 * j + 4 * g) =
            make_float4(oacc[db][4 * j], oacc[db][4 * j + 1], oacc[db][4 * j + 2], oacc[db][4 * j + 3]);
    __syncthreads();

    const int col = threadIdx.x % 32, e0 = (threadIdx.x / 32) * C::EPT;
    if (col < nq) {
      // Wave 0's first sub-tile holds the segment's first key, so some
      // wave's max is finite; a wave without keys has m = -inf, weight 0.
      float M = kNegInf;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, mrow[ww * 32 + col]);
      float ew[NW], Lsum = 0.f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) {
        ew[ww] = fast_exp2(mrow[ww * 32 + col] - M);
        Lsum += ew[ww] * lrow[ww * 32 + col];
      }
      const float inv = 1.f / Lsum;
      float o[C::EPT];
#pragma unroll
      for (int e = 0; e < C::EPT; ++e) o[e] = 0.f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) {
        const float* src = orow + (ww * 32 + col) * C::OROW + e0;
#pragma unroll
        for (int e = 0; e < C::EPT; e += 4) {
          const float4 x = *reinterpret_cast<const float4*>(src + e);
          o[e] += ew[ww] * x.x;
          o[e + 1] += ew[ww] * x.y;
          o[e + 2] += ew[ww] * x.z;
          o[e + 3] += ew[ww] * x.w;
        }
      }
      const float lse = (M + __log2f(Lsum)) * kLn2;
      if (whole) {  // the final result of these query heads
        uint16_t* dst = og + (size_t)(bh0 + col) * D + e0;
#pragma unroll
        for (int e = 0; e < C::EPT; e += 8) {
          uint4 v;
          v.x = pack2(T{}, o[e + 0] * inv, o[e + 1] * inv);
          v.y = pack2(T{}, o[e + 2] * inv, o[e + 3] * inv);
          v.z = pack2(T{}, o[e + 4] * inv, o[e + 5] * inv);
          v.w = pack2(T{}, o[e + 6] * inv, o[e + 7] * inv);
          *reinterpret_cast<uint4*>(dst + e) = v;
        }
        if (e0 == 0) lseg[bh0 + col] = lse;
      } else {  // this segment's (O normalised within it, LSE) for the merge
        float* dst = opart + ((size_t)slot * 32 + col) * D + e0;
#pragma unroll
        for (int e = 0; e < C::EPT; e += 4)
          *reinterpret_cast<float4*>(dst + e) = make_float4(o[e] * inv, o[e + 1] * inv, o[e + 2] * inv, o[e + 3] * inv);
        if (e0 == 0) lpart[(size_t)slot * 32 + col] = lse;
      }
    }
    __syncthreads();  // the next segment refills the rings
  };

  // Walk the range unit by unit.
  for (;;) {
    const int seg_end = min(t_end, P_u + nb);
    const int len = decode_len(kv_lens, b, Nkv);
    segment((t - P_u) * kDecodeTileKeys, min((seg_end - P_u) * kDecodeTileKeys, len), len,
            t == P_u && seg_end == P_u + nb, w + b * UB + ui);
    t = seg_end;
    if (t >= t_end) break;
    P_u += nb;
    if (++ui == UB) {  // next batch with keys
      ui = 0;
      do nb = decode_tiles(decode_len(kv_lens, ++b, Nkv));
      while (nb == 0);
    }
  }
}

// Merge of the pieces of one (unit, live query column) that was cut between
// parts: the 256 threads are 8 piece groups x 32 element chunks.  Each group
// folds every 8th piece with the same decomposition (a running max and
// rescaled sums), loading four pieces' LSEs and output chunks at once so
// that one memory latency covers them; the 8 groups are then combined
// through LDS.  With uniform lengths (kv_lens null) the unit's first tile
// has a closed form; otherwise block sums over the batch lengths locate it.
template <typename T, int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(const float* __restrict__ opart,
                                                           const float* __restrict__ lpart,
                                                           const int* __restrict__ kv_lens,
                                                           uint16_t* __restrict__ og, float* __restrict__ lseg,
                                                           int B, int H, int G, int Nkv, int n_parts) {
  constexpr int CH = D / 32;  // floats per element chunk
  constexpr int U = 4;        // pieces per group in flight
  __shared__ float red[8][D];
  __shared__ float rs[2][8];
  const int Hkv = H / G, QB = decode_query_blocks(G), UB = Hkv * QB, CPU = min(32, G);
  const int u = blockIdx.x / CPU, col = blockIdx.x % CPU;
  const int b = u / UB, ui = u % UB, qb = ui % QB;
  if (col >= min(32, G - 32 * qb)) return;  // (block-uniform returns throughout)
  int Ttot, P_b, nb;
  if (kv_lens == nullptr) {
    nb = decode_tiles(Nkv);
    Ttot = B * UB * nb;
    P_b = b * UB * nb;
  } else {
    decode_wave_sums(kv_lens, B, Nkv, UB, b, &Ttot, &P_b, &nb);
  }
  if (nb == 0) return;
  const int per = (Ttot + n_parts - 1) / n_parts;
  const int P_u = P_b + ui * nb;
  const int w_first = P_u / per, w_last = (P_u + nb - 1) / per;
  if (w_first == w_last) return;  // one part held the whole unit and wrote it
  const int np = w_last - w_first + 1;
  const size_t slot0 = (size_t)w_first + u;

  const int tid = threadIdx.x, c = tid % 32, grp = tid / 32;
  // this group's running max (natural log units), weight sum and sums
  float m = kNegInf, wsum = 0.f;
  float acc[CH] = {};
  for (int i0 = grp; i0 < np; i0 += 8 * U) {
    float li[U];
    float oi[U][CH];
#pragma unroll
    for (int q = 0; q < U; ++q) {
      const int i = i0 + 8 * q;
      li[q] = kNegInf;
#pragma unroll
      for (int e = 0; e < CH; ++e) oi[q][e] = 0.f;
      if (i < np) {
        li[q] = lpart[(slot0 + i) * 32 + col];
        // CH consecutive floats, 4 CH bytes aligned (the workspace is)
        const float* src = opart + ((slot0 + i) * 32 + col) * D + CH * c;
        if constexpr (CH == 4) {
          const float4 x = *reinterpret_cast<const float4*>(src);
          oi[q][0] = x.x; oi[q][1] = x.y; oi[q][2] = x.z; oi[q][3] = x.w;
        } else {
          static_assert(CH == 2, "d = 64 or 128");
          const float2 x = *reinterpret_cast<const float2*>(src);
          oi[q][0] = x.x; oi[q][1] = x.y;
        }
      }
    }
    float mb = m;
#pragma unroll
    for (int q = 0; q < U; ++q) mb = fmaxf(mb, li[q]);
    if (mb == kNegInf) continue;  // nothing live yet (every LSE of a cut piece is finite)
    const float r = fast_exp2((m - mb) * kLog2e);  // m = -inf gives 0
    wsum *= r;
#pragma unroll
    for (int e = 0; e < CH; ++e) acc[e] *= r;
#pragma unroll
    for (int q = 0; q < U; ++q) {
      const float wi = fast_exp2((li[q] - mb) * kLog2e);  // absent pieces: exp(-inf) = 0
      wsum += wi;
#pragma unroll
      for (int e = 0; e < CH; ++e) acc[e] += wi * oi[q][e];
    }
    m = mb;
  }
  // combine the groups: M = max m_g, each group's sums scaled by exp(m_g - M)
  if (c == 0) rs[0][grp] = m;
  __syncthreads();
  float M = kNegInf;
#pragma unroll
  for (int q = 0; q < 8; ++q) M = fmaxf(M, rs[0][q]);
  const float sg = m == kNegInf ? 0.f : fast_exp2((m - M) * kLog2e);
#pragma unroll
  for (int e = 0; e < CH; ++e) red[grp][CH * c + e] = acc[e] * sg;
  if (c == 0) rs[1][grp] = wsum * sg;
  __syncthreads();
  if (grp == 0) {
    float W = 0.f;
#pragma unroll
    for (int q = 0; q < 8; ++q) W += rs[1][q];
    const float inv = 1.f / W;
    float o[CH];
#pragma unroll
    for (int e = 0; e < CH; ++e) {
      float v = 0.f;
#pragma unroll
      for (int q = 0; q < 8; ++q) v += red[q][CH * c + e];
      o[e] = v * inv;
    }
    const int bh = (b * Hkv + ui / QB) * G + 32 * qb + col;
    uint16_t* dst = og + (size_t)bh * D + CH * c;
#pragma unroll
    for (int e = 0; e < CH; e += 2) *reinterpret_cast<uint32_t*>(dst + e) = pack2(T{}, o[e], o[e + 1]);
    if (c == 0) lseg[bh] = M + __log2f(W) * kLn2;
  }
}

template <typename T, int D>
hipError_t run(const DecodeArgs& a) {
  constexpr int NW = 4, NSLOT = 3;
  using C = Dec<D, NW, NSLOT>;
  const float qk_scale = a.scale * kLog2eHost;
  hipLaunchKernelGGL((decode_split_kernel<T, D, NW, NSLOT>), dim3((unsigned)a.parts), dim3(C::NT), 0, a.stream,
                     static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                     static_cast<const uint16_t*>(a.v), a.kv_lens, static_cast<uint16_t*>(a.o), a.lse, a.opart,
                     a.lpart, a.B, a.H, a.G, a.Nkv, qk_scale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.parts == 1) return e;
  // one workgroup per (unit, query column that a unit can have live)
  const long long units = (long long)a.B * (a.H / a.G) * decode_query_blocks(a.G);
  const long long grid = units * (a.G < 32 ? a.G : 32);
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((decode_merge_kernel<T, D>), dim3((unsigned)grid), dim3(256), 0, a.stream, a.opart,
                     a.lpart, a.kv_lens, static_cast<uint16_t*>(a.o), a.lse, a.B, a.H, a.G, a.Nkv, a.parts);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a) {
  if (a.dtype == 2) return a.d == 128 ? run<BF16, 128>(a) : run<BF16, 64>(a);
  return a.d == 128 ? run<F16, 128>(a) : run<F16, 64>(a);
}

}  // namespace fa
