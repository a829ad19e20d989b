// fa_fp8.hip -- forward with FP8 (OCP E4M3) Q, K, V on the gfx950 8-bit
// matrix product v_mfma_f32_32x32x64_f8f6f4, whose dense rate is twice the
// 16-bit one.
//
// Pages cited: "Flash Attention: IO-awareness principle" (hrletsgo.me),
// section "FA2/FA3" (FA3's FP8 mode); "Triton 06: Flash Attention v2"
// (wonbeomjang.kr), Improvements 1-3 (un-scaled accumulator, exp2 with
// log2(e) folded into the scale, causal blocks split into unmasked and
// masked ones).
//
// Inputs are FP8 codes with one dequantisation factor per tensor (value =
// code * descale).  The algorithm is the fused forward's: per query block
// (8 waves x 32 queries) K and V tiles of 64 keys stream through an LDS
// ring; per tile each wave computes S^T = K Q^T (lane = query, registers =
// keys), P 2^8 = exp2(x - m + 8) in fp32 against a lazily raised reference
// m, the row sum in fp32, and P 2^8 rounded to E4M3 as the B operand of
// O^T += V^T P^T.  The 2^8 keeps small weights in E4M3's range; it cancels
// between O's accumulator and the row sum.
//
// Operand layouts of the 8-bit product (measured on the chip): lane (r, g)
// of an operand holds row (or column) r = lane % 32 and 32 bytes whose
// contraction index is the same for both operands at the same (g, byte).
// So the score product reads 32 consecutive bytes of a K row (d = 64 s +
// 32 g + byte) against the same bytes of Q; the PV product pairs byte
// 16 b + r of lane (n, g) with key 32 b + 8 (r / 4) + 4 g + r % 4 -- the
// keys of register r of score block b -- so the packed P needs no shuffle,
// and V^T's matching bytes come from ds_read_b64_tr_b8: element e of lane
// i in a 16-lane group is byte i % 8 of the 8 bytes addressed by lane
// 2 e + i / 8 of the group.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_device.hpp"
#include "fa_kernels.hpp"
#include "fa_plan.hpp"

namespace fa {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v2i_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x16 mma_fp8(const v8i& a, const v8i& b, const f32x16& c) {
  // formats 0/0 = E4M3 for both operands, no block scales
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Headroom of the lazy reference, log2 units: after a raise the largest
// weight is 2^(8 - kFp8Lift), and scores may grow by kFp8Lift + log2(448 /
// 256) before the next raise.  Weights below 2^-9 / 2^8 of the reference
// (2^(-17 + kFp8Lift) of the row max) round to zero.
constexpr float kFp8Lift = 2.f;

template <int D>
struct Fp8 {
  static constexpr int NW = 8, NT = 64 * NW, BM = 32 * NW, BN = 64, NBUF = 4;
  static constexpr int DS = D / 64;        // 64-byte contraction steps of the score product
  static constexpr int DB = D / 32;        // 32-wide d blocks of O
  static constexpr int CPR = D / 16;       // 16-byte chunks per row
  static constexpr int RPP = 1024 / D;     // rows per 1 KB wave load
  static constexpr int PPT = BN / RPP;     // 1 KB pieces per K (or V) tile
  static constexpr int LPW = 2 * PPT / NW; // loads per wave per tile
  static_assert(LPW >= 1 && LPW * NW == 2 * PPT && PPT % LPW == 0 && 3 * LPW < 64, "tile loads");
};

// Stored 16-byte chunk of logical chunk c in row r.  D = 128: the two low
// bits of (r >> 1) & 7 swapped; D = 64: (r >> 2) & 3.  Both keep the 32-byte
// row reads of K and the transposing 8-byte reads of V free of bank
// conflicts.
template <int D>
__device__ __forceinline__ int fp8_swz(int r) {
  if (D == 128) {
    const int x = (r >> 1) & 7;
    return ((x & 1) << 1) | ((x >> 1) & 1) | (x & 4);
  }
  return (r >> 2) & 3;
}
template <int D>
__device__ __forceinline__ int fp8_off(int row, int chunk) {  // byte offset of (row, logical chunk)
  return row * D + 16 * (chunk ^ fp8_swz<D>(row));
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(512) void fwd_fp8_kernel(const uint8_t* __restrict__ qg, const uint8_t* __restrict__ kg,
                                                      const uint8_t* __restrict__ vg, uint16_t* __restrict__ og,
                                                      float* __restrict__ lseg, int N, int n_qblk, int BH, int G,
                                                      float qk_scale, float o_scale, uint32_t qsign) {
  using C = Fp8<D>;
  constexpr int BN = C::BN, DS = C::DS, DB = C::DB;
  // One LDS variable for both rings: the compiler matches loads into LDS
  // against later LDS reads per variable, and would make the reads of one
  // slot wait for the loads just issued into another.  The barriers' explicit
  // waits order loads and reads.
  __shared__ __attribute__((aligned(16))) uint8_t kv_lds[2][C::NBUF][BN * D];
  auto& k_lds = kv_lds[0];
  auto& v_lds = kv_lds[1];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 31, g = lane >> 5;

  auto block = [&](int bh, int qblk) __attribute__((always_inline)) {
    const size_t head = (size_t)bh * N * D;
    const size_t kvhead = (size_t)kv_head_of(bh, G) * N * D;
    const uint32_t head_bytes = (uint32_t)N * D;
    const rsrc_t qrs = make_rsrc(qg + head, head_bytes);
    const rsrc_t krs = make_rsrc(kg + kvhead, head_bytes);
    const rsrc_t vrs = make_rsrc(vg + kvhead, head_bytes);
    const int q0 = qblk * C::BM;
    const int qw0 = q0 + 32 * wave;
    const int query = qw0 + n;
    const bool wave_live = qw0 < N;

    // Q fragments: lane (n, g), step s: bytes 64 s + 32 g .. + 32 of row `query`.
    v8i qf[DS];
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      const uint4 a = load16(qrs, (uint32_t)query * D + 64 * s + 32 * g);
      const uint4 b = load16(qrs, (uint32_t)query * D + 64 * s + 32 * g + 16);
      // a negative score factor flips Q's sign bits, so qk_scale >= 0
      qf[s] = v8i{(int)(a.x ^ qsign), (int)(a.y ^ qsign), (int)(a.z ^ qsign), (int)(a.w ^ qsign),
                  (int)(b.x ^ qsign), (int)(b.y ^ qsign), (int)(b.z ^ qsign), (int)(b.w ^ qsign)};
    }

    // Tiles this workgroup reads, and the last one each wave needs.
    const int n_tiles = (N + BN - 1) / BN;
    const int last_row = min(q0 + C::BM, N) - 1;
    const int j_end = CAUSAL ? min(n_tiles, last_row / BN + 1) : n_tiles;
    const int key_lim = CAUSAL ? min(query + 1, N) : N;

    // Waves 0 .. NW/2 - 1 load K tiles, the others V tiles: K tile jk into
    // slot kd, V tile jv into slot vd, each only if that tile exists.  LDS row
    // r, stored chunk c holds global chunk c ^ fp8_swz(r) of key j BN + r;
    // rows past N read as zeros.
    auto issue = [&](int jk, uint8_t* __restrict__ kd, int jv, uint8_t* __restrict__ vd) __attribute__((always_inline)) {
      const int lrow = lane / C::CPR;
      const bool k_wave = wave * C::LPW < C::PPT;
      if (!(k_wave ? jk < j_end : jv >= 0 && jv < j_end)) return;
#pragma unroll
      for (int e = 0; e < C::LPW; ++e) {
        const int t = wave * C::LPW + e;
        const int p = t % C::PPT;
        const int row = p * C::RPP + lrow;
        const int ch = (lane % C::CPR) ^ fp8_swz<D>(row);
        if (k_wave) load_lds16(krs, kd + p * C::RPP * D, (uint32_t)(jk * BN + row) * D + 16 * ch);
        else load_lds16(vrs, vd + p * C::RPP * D, (uint32_t)(jv * BN + row) * D + 16 * ch);
      }
    };

    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
    float m_run = kNegInf, l_run = 0.f;  // base-2 running max; this half's share of l

    // V^T fragment of d block db (A operand of O^T += V^T P^T): four
    // transposing reads, read t giving bytes 8 t .. 8 t + 7, i.e. keys
    // 32 (t / 2) + 16 (t % 2) + 8 (e / 4) + 4 g + e % 4, e = 0..7.
    const int tg = lane >> 4, tj = lane & 15;  // 16-lane group, lane in group
    auto vfrag = [&](const uint8_t* vt, int db) __attribute__((always_inline)) {
      v8i r;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int e = tj >> 1;
        const int row = 32 * (t >> 1) + 16 * (t & 1) + 8 * (e >> 2) + 4 * g + (e & 3);
        const int chunk = 2 * db + (tg & 1);
        const uint8_t* p = vt + fp8_off<D>(row, chunk) + 8 * (tj & 1);
        const v2i_t x = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) v2i_t*)(p));
        r[2 * t] = x[0];
        r[2 * t + 1] = x[1];
      }
      return r;
    };

    // Raw scores S^T (before the scale) of the two 32-key blocks of the K
    // tile kt; register r of block b is key 32 b + 8 (r / 4) + 4 g + r % 4
    // of the tile.
    auto s_gemm = [&](const uint8_t* __restrict__ kt, f32x16 (&sc)[2]) __attribute__((always_inline)) {
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        sc[b] = f32x16{};
#pragma unroll
        for (int s = 0; s < DS; ++s) {
          const int row = 32 * b + n;
          const uint4 x0 = *reinterpret_cast<const uint4*>(kt + fp8_off<D>(row, 4 * s + 2 * g));
          const uint4 x1 = *reinterpret_cast<const uint4*>(kt + fp8_off<D>(row, 4 * s + 2 * g + 1));
          const v8i a = v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
          sc[b] = mma_fp8(a, qf[s], sc[b]);
        }
      }
    };

    // Softmax of tile j with a lazy reference.  The weights are
    // P 2^8 = exp2(x qk_scale - (m - 8)) against a reference m that is only
    // raised when some weight would leave E4M3's range (> 448): the common
    // path computes no row max and never rescales.  The fp32 sum of a word's
    // four weights is at least each of them (rounded sums of non-negative
    // terms never fall below a term), so while every such sum is at most 448
    // no weight overflows and nothing more is tested.  Otherwise the packed
    // bytes are tested: an overflow shows as a NaN code (E4M3 has no
    // infinity; the conversion does not saturate).  Then (rare; always on a
    // row's first tile, where m is -inf and the sums are infinite) m is
    // raised to the tile's row max plus kFp8Lift, O and l are rescaled and
    // the weights redone.  The lift keeps later, slightly larger scores in
    // range.  qk_scale >= 0, so the max of the raw scores gives the max.
    // MASK: keys past a lane's limit get weight zero (set directly; an
    // infinite score times a zero qk_scale would be NaN).
    // Word w of the packed weights: keys 32 (w / 4) + 8 (w % 4) + 4 g + i.
    auto weight_word = [&](const f32x16 (&sc)[2], int j, auto mask_tag, v8i& pk, float& psum, float& qmax, float base,
                           int w)
        __attribute__((always_inline)) {
      constexpr bool MASK = decltype(mask_tag)::value;
      const int b = w / 4, r = 4 * (w % 4);
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = fast_exp2(__builtin_fmaf(sc[b][r + i], qk_scale, -base));
        if (MASK && j * BN + 32 * b + 8 * (r / 4) + 4 * g + i >= key_lim) p[i] = 0.f;
      }
      const float s4 = (p[0] + p[1]) + (p[2] + p[3]);
      psum = w == 0 ? s4 : psum + s4;
      qmax = w == 0 ? s4 : fmaxf(qmax, s4);
      // the two conversions fill the low and the high half of the word,
      // overwriting the codes it held before in place
      int word = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], pk[w], false);
      word = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], word, true);
      pk[w] = word;
    };
    auto weights = [&](const f32x16 (&sc)[2], int j, auto mask_tag, v8i& pk, float& psum, float& qmax)
        __attribute__((always_inline)) {
      const float base = m_run - 8.f;  // -inf before the first raise: every weight overflows
#pragma unroll
      for (int w = 0; w < 8; ++w) weight_word(sc, j, mask_tag, pk, psum, qmax, base, w);
    };
    // The overflow test and the rare raise; then the tile's sum joins l.
    auto settle = [&](const f32x16 (&sc)[2], int j, auto mask_tag, v8i& pk, float& psum, float& qmax)
        __attribute__((always_inline)) {
      constexpr bool MASK = decltype(mask_tag)::value;
      // !(<=) also takes an infinite or NaN group sum to the byte test
      if (__builtin_amdgcn_ballot_w64(!(qmax <= 448.f)) != 0) {
        uint32_t ovf = 0;
#pragma unroll
        for (int w = 0; w < 8; ++w)  // a byte whose low seven bits are all set is a NaN code
          ovf |= (((uint32_t)pk[w] & 0x7F7F7F7Fu) + 0x01010101u) & 0x80808080u;
        if (__builtin_amdgcn_ballot_w64(ovf != 0) != 0) {
          float mx = kNegInf;
#pragma unroll
          for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const bool vis = !MASK || j * BN + 32 * b + 8 * (r / 4) + 4 * g + (r % 4) < key_lim;
              mx = fmaxf(mx, vis ? sc[b][r] : kNegInf);
            }
          mx = halves_max(mx);
          mx = mx == kNegInf ? kNegInf : mx * qk_scale;
          const float m_new = fmaxf(m_run, mx == kNegInf ? kNegInf : mx + kFp8Lift);
          const float alpha = m_run == kNegInf ? 0.f : fast_exp2(m_run - m_new);
          l_run *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
          m_run = m_new;
          weights(sc, j, mask_tag, pk, psum, qmax);
        }
      }
      l_run += psum;
    };

    // Ring and pipeline.  Iteration j computes the scores of tile j + 1, the
    // weights of tile j (already scored) and the PV product of tile j - 1
    // (weighted in iteration j - 1).  Neither product depends on the vector
    // work beside it, so the eight matrix instructions are spread through the
    // weights and one wave keeps both units busy.  Loads run ahead: K tile
    // j + 3 and V tile j + 2 go out in iteration j, into the slots that K
    // tile j - 1 (scored in iteration j - 2) and V tile j - 2 (read in
    // iteration j - 1) have left.  The barrier at the top of iteration j
    // makes K tile j + 1 and V tile j - 1 visible; the loads still allowed in
    // flight are each wave's latest.
    static_assert(C::NBUF == 4, "ring of four K and four V slots");
    issue(0, k_lds[0], -1, v_lds[3]);
    issue(1, k_lds[1], 0, v_lds[0]);
    issue(2, k_lds[2], 1, v_lds[1]);
    // prologue: K tile 0 in LDS (K waves issued up to three tiles), its scores
    if (j_end > 2) lds_barrier<2 * C::LPW>();
    else if (j_end > 1) lds_barrier<C::LPW>();
    else lds_barrier<0>();
    f32x16 sA[2], sB[2];
    s_gemm(k_lds[0], sA);
    v8i pkA = v8i{}, pkB = v8i{};  // E4M3 weights of alternate tiles
    // One iteration; the loop runs two per trip so the score and weight
    // registers alternate without copies.  The ring slots arrive as distinct
    // __restrict__ pointers: with that, the compiler does not make the reads
    // of one slot wait for the loads just issued into another.
    auto step_in = [&](int j, f32x16 (&cur)[2], f32x16 (&nxt)[2], const v8i& prv, v8i& pk,
                       const uint8_t* __restrict__ kn, const uint8_t* __restrict__ vt,
                       uint8_t* __restrict__ kl, uint8_t* __restrict__ vl, auto mask_tag, auto pv_tag)
        __attribute__((always_inline)) {
      constexpr bool PV = decltype(pv_tag)::value;
      if (j + 1 < j_end) {
        if (j + 2 < j_end) lds_barrier<C::LPW>();
        else lds_barrier<0>();
      }
      issue(j + 3, kl, j + 2, vl);
      // The step's matrix instructions: the PV products of tile j - 1 (d
      // blocks 0 .. DB - 1), then the score products of tile j + 1, ordered so
      // the two k-steps of a key block are not adjacent.  Past the last tile
      // the scores are of stale slot contents and unused.  Each takes its A
      // operand from LDS, read LA instructions ahead.
      constexpr int NPV = PV ? DB : 0, NMM = NPV + 2 * DS, LA = 2;
      auto read_a = [&](int i) __attribute__((always_inline)) {
        if (i < NPV) return vfrag(vt, i);
        const int b = (i - NPV) % 2, st = (i - NPV) / 2;
        const int row = 32 * b + n;
        const uint4 x0 = *reinterpret_cast<const uint4*>(kn + fp8_off<D>(row, 4 * st + 2 * g));
        const uint4 x1 = *reinterpret_cast<const uint4*>(kn + fp8_off<D>(row, 4 * st + 2 * g + 1));
        return v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
      };
      auto mma = [&](int i, const v8i& a) __attribute__((always_inline)) {
        if (i < NPV) {
          oacc[i] = mma_fp8(a, prv, oacc[i]);
        } else {
          const int b = (i - NPV) % 2, st = (i - NPV) / 2;
          nxt[b] = mma_fp8(a, qf[st], st == 0 ? f32x16{} : nxt[b]);
        }
      };
      // Weight word w runs before matrix instructions i with i * 8 / NMM == w;
      // scheduling barriers keep that order, so one wave issues vector work
      // while its own matrix instructions execute.
      v8i ops[NMM];
#pragma unroll
      for (int i = 0; i < LA && i < NMM; ++i) ops[i] = read_a(i);
      float psum, qmax;
      const float base = m_run - 8.f;  // -inf before the first raise: every weight overflows
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int w = 0; w < 8; ++w) {
#pragma unroll
        for (int i = 0; i < NMM; ++i)
          if (i * 8 / NMM == w && i + LA < NMM) ops[i + LA] = read_a(i + LA);
        weight_word(cur, j, mask_tag, pk, psum, qmax, base, w);
        int mm = 0;
#pragma unroll
        for (int i = 0; i < NMM; ++i)
          if (i * 8 / NMM == w) {
            mma(i, ops[i]);
            ++mm;
          }
        // within the chunk: its LDS reads, then the vector work, then the
        // matrix instruction
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
        __builtin_amdgcn_sched_group_barrier(0x402, 32, 0);
        if (mm) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // at most one per chunk (NMM <= 8)
        __builtin_amdgcn_sched_barrier(0);
      }
      settle(cur, j, mask_tag, pk, psum, qmax);
    };
    // The first iteration has no PV product before it.
    auto step = [&](int j, f32x16 (&cur)[2], f32x16 (&nxt)[2], const v8i& prv, v8i& pk, auto mask_tag, auto pv_tag)
        __attribute__((always_inline)) {
      step_in(j, cur, nxt, prv, pk, k_lds[(j + 1) % C::NBUF], v_lds[(j + 3) % C::NBUF], k_lds[(j + 3) % C::NBUF],
              v_lds[(j + 2) % C::NBUF], mask_tag, pv_tag);
    };
    // Tiles every key of which every query of the block sees run without
    // the mask; the rest (the diagonal tiles, the sequence tail) with it.
    // Each range has one code path, so the accumulators need no merging.
    // Between iterations the scores of the next tile are in sA and the
    // weights of the previous one in pkB.
    auto run = [&](int j0, int j1, auto mask_tag) __attribute__((always_inline)) {
      int j = j0;
      if (j == 0 && j < j1) {
        step(0, sA, sB, pkB, pkA, mask_tag, std::false_type{});
        sA[0] = sB[0];
        sA[1] = sB[1];
        pkB = pkA;
        j = 1;
      }
      for (; j + 1 < j1; j += 2) {
        step(j, sA, sB, pkB, pkA, mask_tag, std::true_type{});
        step(j + 1, sB, sA, pkA, pkB, mask_tag, std::true_type{});
      }
      if (j < j1) {
        step(j, sA, sB, pkB, pkA, mask_tag, std::true_type{});
        sA[0] = sB[0];
        sA[1] = sB[1];
        pkB = pkA;
      }
    };
    const int j_full = min(j_end, CAUSAL ? q0 / BN : N / BN);
    run(0, j_full, std::false_type{});
    run(j_full, j_end, std::true_type{});
    // The last tile's PV product.  Its V tile is in LDS and visible: the
    // barrier of the second-to-last iteration waited for every load (the
    // prologue's, with a single tile).
    {
      const uint8_t* vt = v_lds[(j_end - 1) % C::NBUF];
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] = mma_fp8(vfrag(vt, db), pkB, oacc[db]);
    }
    // No tile load is in flight (none is issued for the last three tiles, and
    // the last barrier waited for all); saying so spares the O staging below
    // a wait for loads the compiler would otherwise take as pending.
    vm_wait<0>();

    // O = acc * (V descale / 2^8) / l, LSE = (m + log2 l) ln 2.  O goes
    // through LDS as in the 16-bit forward: each wave stages its 32 x D bf16
    // tile in the idle ring and writes whole rows per store instruction.
    const float l_tot = halves_sum(l_run);  // sum of P 2^8
    const float inv = o_scale / l_tot;
    if (wave_live && g == 0 && query < N) lseg[(size_t)bh * N + query] = (m_run + __log2f(l_tot) - 8.f) * kLn2;
    lds_only_barrier();  // every wave has finished reading the ring
    if (wave_live) {
      static_assert(C::NW * 32 * D * 2 <= 2 * C::NBUF * BN * D, "O staging fits in the ring");
      uint16_t* stage = reinterpret_cast<uint16_t*>(wave < C::NW / 2 ? &k_lds[0][0] : &v_lds[0][0]) +
                        (wave % (C::NW / 2)) * 32 * D;
      int nn = n, gg = g;  // through an empty asm: addresses formed here, not hoisted
      asm volatile("" : "+v"(nn), "+v"(gg));
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const f32x16& v = oacc[db];
          const uint2 w = make_uint2(pack2(BF16{}, v[4 * rq + 0] * inv, v[4 * rq + 1] * inv),
                                     pack2(BF16{}, v[4 * rq + 2] * inv, v[4 * rq + 3] * inv));
          *reinterpret_cast<uint2*>(stage + swz<D>(nn, 32 * db + 8 * rq + 4 * gg)) = w;
        }
      // Store instruction i: lane l writes row (64 i + l) / CPR, chunk l % CPR;
      // rows past N fall outside the range of the buffer stores.
      constexpr int CPR = D / 8, ROWS = 64 / CPR;
      const rsrc_t ors = make_rsrc(og + head, (uint32_t)N * D * 2);
      int li = lane;
      asm volatile("" : "+v"(li));
#pragma unroll
      for (int i = 0; i < 32 / ROWS; ++i) {
        const int r = ROWS * i + li / CPR, c = li % CPR;
        const uint4 x = *reinterpret_cast<const uint4*>(stage + swz<D>(r, 8 * c));
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u32, x), ors,
                                               ((uint32_t)(qw0 + r) * D + 8 * c) * 2, 0, 0);
      }
    }
  };

  // Persistent loop over equal-cost items, as the 16-bit forward.
  const int per_head = items_per_head(n_qblk, CAUSAL);
  const int n_items = BH * per_head;
  for (int L = xcd_remap(blockIdx.x, gridDim.x); L < n_items; L += gridDim.x) {
    int lo, hi;
    const int nb = item_blocks(L % per_head, n_qblk, CAUSAL, &lo, &hi);
    for (int t = 0; t < nb; ++t) {
      block(L / per_head, t + 1 < nb ? hi : lo);  // the heavier block of a causal pair first
      __syncthreads();                            // the next block's loads reuse the ring
    }
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const Fp8Args& a) {
  using C = Fp8<D>;
  const int n_qblk = (a.N + C::BM - 1) / C::BM;
  const long long items = (long long)items_per_head(n_qblk, CAUSAL) * a.BH;
  if (items > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int grid = (int)(items < cus ? items : cus);
  const float f = a.scale * a.q_descale * a.k_descale;
  const float qk_scale = fabsf(f) * kLog2eHost;
  const uint32_t qsign = f < 0.f ? 0x80808080u : 0u;
  const float o_scale = a.v_descale;  // l and the PV products both carry the 2^8
  hipLaunchKernelGGL((fwd_fp8_kernel<D, CAUSAL>), dim3((unsigned)grid), dim3(C::NT), 0, a.stream,
                     static_cast<const uint8_t*>(a.q), static_cast<const uint8_t*>(a.k),
                     static_cast<const uint8_t*>(a.v), static_cast<uint16_t*>(a.o), a.lse, a.N, n_qblk, a.BH, a.G,
                     qk_scale, o_scale, qsign);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_fp8(const Fp8Args& a) {
  if (a.d == 128) return a.causal ? launch<128, true>(a) : launch<128, false>(a);
  return a.causal ? launch<64, true>(a) : launch<64, false>(a);
}

}  // namespace fa
