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
// * K (row-major, 16-byte row padding) and V^T (padded rows) sit in three
//   LDS buffers: the block being consumed, the next one (whose first
//   S product starts inside the current block's last step), and the one
//   after, whose global loads are in flight meanwhile; one barrier per block.
// * Software pipeline inside each wave, per 32-key sub-block u: the S^T
//   product of sub-block u+1 is issued in chunks interleaved with the
//   exponentials of sub-block u, and the PV product of u is interleaved with
//   the row max of u+1, so the matrix cores and the vector/transcendental
//   units overlap within one wave; eight waves (two per SIMD) cover the rest.
// * The reference max is raised lazily (only when a sub-block's max exceeds
//   it by more than a fixed slack), so the O rescale is rare; exact, since
//   O, l and the LSE all use the same reference.
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
  static_assert(QB == 1, "one 32-query block per wave");
  constexpr int KB = C::KB, DB = C::DB, DS = C::DS;
  // Three K/V buffers: iteration j reads K_{j+1} and V_j while block j+2 is
  // staged into the third.
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[3][C::LDS_K];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[3][C::LDS_V];

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
  const int query = qw0 + n;          // this lane's query

  // ---- Q fragments, held in registers for the whole kernel --------------
  // B operand of S^T = K Q^T: lane supplies Q[query][16 s + 8 g + 0..7];
  // rows past N read as zeros.
  uint4 qf[DS];
#pragma unroll
  for (int s = 0; s < DS; ++s) {
    uint4 x = load16(qrs, ((uint32_t)query * D + 16 * s + 8 * g) * 2);
    x.x ^= qsign; x.y ^= qsign; x.z ^= qsign; x.w ^= qsign;
    qf[s] = x;
  }

  // ---- key-block plan ---------------------------------------------------
  // Blocks [0, j_unm) hold only keys visible to every query of the
  // workgroup and lie before the sequence tail: no mask (the pages'
  // unmasked stage).  Blocks [j_unm, j_end) straddle the diagonal or hold
  // the tail and are masked per key.  Blocks from j_end on are never read.
  const int n_kv = (N + BN - 1) / BN;
  const int full_blocks = N / BN;
  int j_end = n_kv, j_unm = full_blocks;
  if (CAUSAL) {
    j_end = min(n_kv, (min(q0 + C::BM, N) - 1) / BN + 1);
    int s1, s2;
    causal_stages(q0, min(q0 + C::BM, N), BN, &s1, &s2);
    j_unm = min(s1, full_blocks);
  }
  const int key_lim = CAUSAL ? min(query + 1, N) : N;

  // ---- global -> register -> LDS staging of one K/V block -----------------
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

  // ---- pieces of one 32-key sub-block --------------------------------------
  // A K/V tile of BN keys holds SUB = BN/32 sub-blocks; sub-block u is
  // sub-block u % SUB of tile u / SUB.  The softmax pipeline runs per
  // sub-block (two 16-register score sets in flight); barriers and staging
  // run per tile.
  constexpr int SUB = BN / 32;
  // S^T = K Q^T for sub-block `sb` of tile buffer `buf` (32 keys x 32 queries).
  auto s_gemm = [&](int buf, int sb, f32x16 (&s)[1]) {
#pragma unroll
    for (int st = 0; st < DS; ++st) {
      const uint4 a = *reinterpret_cast<const uint4*>(&k_lds[buf][(32 * sb + n) * C::KROW + 16 * st + 8 * g]);
      s[0] = mma16(T{}, a, qf[st], st == 0 ? f32x16{} : s[0]);
    }
  };
  // p = exp2(S * qk_scale - m) packed to 16-bit (the B operand of the PV
  // product); returns this lane's sum of p.  key0 = first key of the sub-block.
  auto exp_pack = [&](int key0, f32x16 (&s)[1], float m_use, uint4 (&pp)[2], auto masked) {
    constexpr bool MASKED = decltype(masked)::value;
    const float sum = tile_exp<1, MASKED>(s, qk_scale, m_use, key0 + 4 * g, key_lim);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const f32x16& v = s[0];
      pp[h] = make_uint4(pack2(T{}, v[8 * h + 0], v[8 * h + 1]), pack2(T{}, v[8 * h + 2], v[8 * h + 3]),
                         pack2(T{}, v[8 * h + 4], v[8 * h + 5]), pack2(T{}, v[8 * h + 6], v[8 * h + 7]));
    }
    return sum;
  };
  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
  // O^T += V^T P^T for sub-block `sb` of tile buffer `buf`.
  auto pv_gemm = [&](int buf, int sb, const uint4 (&pp)[2]) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const uint4 a =
            *reinterpret_cast<const uint4*>(&v_lds[buf][(32 * db + n) * C::VROW + 32 * sb + 16 * h + 8 * g]);
        oacc[db] = mma16(T{}, a, pp[h], oacc[db]);
      }
  };

  float m_run = kNegInf, l_run = 0.f;
  // Scaled row max (log2 units) of the sub-block whose exponentials run in
  // the next step, found in the current step and checked in the next one.
  float m_pend = kNegInf;
  auto m_ref = [&] { return m_run == kNegInf ? 0.f : m_run; };
  // Raise the reference max if a sub-block's scores need it; rescale the
  // accumulator (only when some lane of the wave raised).
  auto update_max = [&](float mt) {
    float alpha;
    if (raise_max(mt, m_run, l_run, &alpha)) {
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
    }
  };

  // One pipeline step: sub-block u's softmax and PV product, overlapped with
  // sub-block u+1's score product and row max.
  //   phase A: S_{u+1} = K Q^T   ||  p_u = exp2(S_u - m), packed
  //   phase B: O += V P_u        ||  rowmax(S_{u+1})
  // Each phase is written as chunks of one matrix product plus its share of
  // the VALU work, fenced so the compiler keeps the interleave; LDS reads
  // run two fragments ahead of their products.
  //
  // The reference max for S_u is checked lazily: phase A starts the
  // exponentials with the current reference while the compare and the
  // wave vote on S_u's max (found in the previous step) complete under its
  // products.  Only if some lane's max exceeds the reference by more than
  // the slack (rare) are the reference raised, O and l rescaled and the
  // exponentials redone from S_u, still in registers.  So the max no longer
  // sits between two steps.
  auto step = [&](int key_u, int vbuf, int vsb, f32x16 (&cur)[1], int kbuf_n, int ksb_n, f32x16 (&nxt)[1],
                  auto masked) {
    constexpr bool MASKED = decltype(masked)::value;
    constexpr int EPC = 16 / DS;  // exponentials per product in phase A
    const bool grow = m_pend > m_run + kMaxSlack;  // false while m_pend is -inf
    const bool redo = __builtin_amdgcn_ballot_w64(grow) != 0;  // wave-uniform
    const float m_use = m_ref();
    const int kbase = key_u + 4 * g;
    const uint16_t* krow = &k_lds[kbuf_n][(32 * ksb_n + n) * C::KROW + 8 * g];
    uint4 a[3];
    a[0] = *reinterpret_cast<const uint4*>(krow);
    a[1] = *reinterpret_cast<const uint4*>(krow + 16);
    float part[4] = {0.f, 0.f, 0.f, 0.f};
    uint32_t pk[8];
#pragma unroll
    for (int st = 0; st < DS; ++st) {
      if (st + 2 < DS) a[(st + 2) % 3] = *reinterpret_cast<const uint4*>(krow + 16 * (st + 2));
      nxt[0] = mma16(T{}, a[st % 3], qf[st], st == 0 ? f32x16{} : nxt[0]);
#pragma unroll
      for (int e = 0; e < EPC; e += 2) {
        const int r = st * EPC + e;  // registers r, r+1 of cur
        float p0 = fast_exp2(__builtin_fmaf(cur[0][r], qk_scale, -m_use));
        float p1 = fast_exp2(__builtin_fmaf(cur[0][r + 1], qk_scale, -m_use));
        if constexpr (MASKED) {
          p0 = kbase + 8 * (r / 4) + (r % 4) < key_lim ? p0 : 0.f;
          p1 = kbase + 8 * ((r + 1) / 4) + ((r + 1) % 4) < key_lim ? p1 : 0.f;
        }
        part[r % 4] += p0;
        part[(r + 1) % 4] += p1;
        pk[r / 2] = pack2(T{}, p0, p1);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    uint4 pp[2] = {make_uint4(pk[0], pk[1], pk[2], pk[3]), make_uint4(pk[4], pk[5], pk[6], pk[7])};
    if (redo) {
      const float m_new = grow ? m_pend : m_run;
      const float alpha = grow ? fast_exp2(m_run - m_new) : 1.f;  // m_run = -inf gives 0
      l_run *= alpha;
      m_run = m_new;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
      const float sum = exp_pack(key_u, cur, m_ref(), pp, masked);
      part[0] = sum;
      part[1] = part[2] = part[3] = 0.f;
    }
    l_run += (part[0] + part[1]) + (part[2] + part[3]);
    // phase B: 2 x DB products; the row max of S_{u+1} is spread over them.
    const uint16_t* vrow = &v_lds[vbuf][n * C::VROW + 32 * vsb + 8 * g];
    uint4 b[3];
    b[0] = *reinterpret_cast<const uint4*>(vrow);
    b[1] = *reinterpret_cast<const uint4*>(vrow + 32 * C::VROW);
    constexpr int NB = 2 * DB;  // products in phase B, index i -> (h = i / DB, db = i % DB)
    constexpr int MPC = (16 + NB - 1) / NB;  // S_{u+1} registers folded into the max per product
    float mx = kNegInf;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      if (i + 2 < NB) {
        const int h = (i + 2) / DB, db = (i + 2) % DB;
        b[(i + 2) % 3] = *reinterpret_cast<const uint4*>(vrow + 32 * db * C::VROW + 16 * h);
      }
      oacc[i % DB] = mma16(T{}, b[i % 3], pp[i / DB], oacc[i % DB]);
      if (i >= 1) {  // S_{u+1} is complete once phase A's products drained
#pragma unroll
        for (int r = (i - 1) * MPC; r < i * MPC && r < 16; ++r) {
          if constexpr (MASKED) {
            const int key = kbase + 32 + 8 * (r / 4) + (r % 4);
            mx = fmaxf(mx, key < key_lim ? nxt[0][r] : kNegInf);
          } else {
            mx = fmaxf(mx, nxt[0][r]);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int r = (NB - 1) * MPC; r < 16; ++r) {
      if constexpr (MASKED) {
        const int key = kbase + 32 + 8 * (r / 4) + (r % 4);
        mx = fmaxf(mx, key < key_lim ? nxt[0][r] : kNegInf);
      } else {
        mx = fmaxf(mx, nxt[0][r]);
      }
    }
    mx = halves_max(mx);
    m_pend = mx == kNegInf ? kNegInf : mx * qk_scale;
  };
  // The last sub-block: softmax and PV only.
  auto last_step = [&](int key_u, int vbuf, int vsb, f32x16 (&cur)[1]) {
    update_max(m_pend);
    uint4 pp[2];
    l_run += exp_pack(key_u, cur, m_ref(), pp, std::true_type{});
    pv_gemm(vbuf, vsb, pp);
  };

  // One tile j (tiles j and j+1 are in LDS at buffers b0, b1): its SUB
  // pipeline steps, the last of which starts on tile j+1; tile j+2 is staged
  // into the third buffer meanwhile.
  f32x16 sA[1], sB[1];  // sub-blocks with even / odd index
  // With an odd number of sub-blocks per tile the register roles swap from
  // one tile to the next, so the tile body exists in both orders.
  auto tile_iter_p = [&](int j, auto masked, f32x16 (&e)[1], f32x16 (&o)[1]) {
    const bool stage = j + 2 < j_end;
    if (stage) load_block(j + 2);
    const int b0 = j % 3, b1 = b0 == 2 ? 0 : b0 + 1, b2 = b1 == 2 ? 0 : b1 + 1;
#pragma unroll
    for (int i = 0; i < SUB; ++i) {
      const int key_u = j * BN + 32 * i;
      const int kb_n = i + 1 < SUB ? b0 : b1, ks_n = i + 1 < SUB ? i + 1 : 0;
      if (i % 2 == 0) step(key_u, b0, i, e, kb_n, ks_n, o, masked);
      else step(key_u, b0, i, o, kb_n, ks_n, e, masked);
    }
    if (stage) store_block(b2);
    __syncthreads();
  };
  auto tile_iter = [&](int j, auto masked) {
    if ((SUB % 2 == 1) && (j & 1)) tile_iter_p(j, masked, sB, sA);
    else tile_iter_p(j, masked, sA, sB);
  };

  // ---- prologue: tiles 0 and 1 into LDS, S of sub-block 0 and its max ------
  load_block(0);
  store_block(0);
  if (j_end > 1) {
    load_block(1);
    store_block(1);
  }
  __syncthreads();
  s_gemm(0, 0, sA);
  if (0 < j_unm) update_max(tile_max<1, false>(sA, qk_scale, 4 * g, key_lim));
  else update_max(tile_max<1, true>(sA, qk_scale, 4 * g, key_lim));

  // ---- main loop over tiles that have a next tile ---------------------------
  int j = 0;
  for (; j + 1 < j_unm; ++j) tile_iter(j, std::false_type{});  // tiles j, j+1 unmasked
  for (; j + 1 < j_end; ++j) tile_iter(j, std::true_type{});
  // ---- last tile: its sub-blocks, the final one without a successor -------
  auto last_tile = [&](f32x16 (&e)[1], f32x16 (&o)[1]) {
    const int b0 = j % 3;
#pragma unroll
    for (int i = 0; i < SUB; ++i) {
      const int key_u = j * BN + 32 * i;
      if (i + 1 < SUB) {
        if (i % 2 == 0) step(key_u, b0, i, e, b0, i + 1, o, std::true_type{});
        else step(key_u, b0, i, o, b0, i + 1, e, std::true_type{});
      } else {
        if (i % 2 == 0) last_step(key_u, b0, i, e);
        else last_step(key_u, b0, i, o);
      }
    }
  };
  if ((SUB % 2 == 1) && (j & 1)) last_tile(sB, sA);
  else last_tile(sA, sB);

  // ---- epilogue: one divide per row, store O and the natural-log LSE ------
  const float l_tot = halves_sum(l_run);
  const float inv = 1.f / l_tot;
  if (query < N) {
    uint16_t* orow = og + head + (size_t)query * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const f32x16& v = oacc[db];
        const uint2 w = make_uint2(pack2(T{}, v[4 * rq + 0] * inv, v[4 * rq + 1] * inv),
                                   pack2(T{}, v[4 * rq + 2] * inv, v[4 * rq + 3] * inv));
        *reinterpret_cast<uint2*>(orow + 32 * db + 8 * rq + 4 * g) = w;
      }
    }
    if (g == 0) lseg[(size_t)bh * N + query] = (m_run + __log2f(l_tot)) * kLn2;
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
  static constexpr int NW = 8, QB = 1;
  static constexpr int BN = D == 128 ? 64 : 128;
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
