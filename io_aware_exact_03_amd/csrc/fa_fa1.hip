// fa_fa1.hip -- the FlashAttention-1 loop order, kept as an ablation of the
// forward: K/V blocks in the outer loop, query blocks inside, and the
// running O, l, m of every query block read from HBM and written back at
// every step.
//
// Pages cited: "Paper review: FlashAttention: Fast and Memory-Efficient
// Exact Attention with IO-Awareness" (osehyeon.github.io), Algorithm 1 and
// the softmax decomposition under "Tiling"; "Flash Attention: IO-awareness
// principle" (hrletsgo.me), section "FA2/FA3" (FA1 spreads the work on one
// query block's output over the K/V loop, FA2 swaps the loops so each
// workgroup finishes its own output block).
//
// As in FA1, one workgroup runs one (batch, head): for every K/V block j
// (64 keys, staged in LDS) it walks every query block i (128 queries, 32
// per wave): loads Q_i, O_i, l_i, m_i from global memory, computes
// S = scale Q_i K_j^T on MFMA, m~ = rowmax, P~ = exp(S - m~), l~ = rowsum,
// m_new = max(m_i, m~), l_new = e^{m_i - m_new} l_i + e^{m~ - m_new} l~ and
// O_i <- (l_i e^{m_i - m_new} O_i + e^{m~ - m_new} P~ V_j) / l_new, and
// writes O_i, l_i, m_i back.  O_i lives in an fp32 workspace; a last pass
// writes O in the input type and LSE = m + ln l.  Under the causal mask the
// query blocks wholly before block j are skipped and the straddling ones
// are masked.  Exponentials are base 2 with log2(e) folded into the scale,
// as in the fused forward, so m in the workspace is in log2 units.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_device.hpp"
#include "fa_kernels.hpp"
#include "fa_plan.hpp"

namespace fa {
namespace {

template <int D>
struct Fa1 {
  static constexpr int NW = 4, NT = 64 * NW;
  static constexpr int BC = 64;                 // keys per K/V block
  static constexpr int BR = 32 * NW;            // queries per query block
  static constexpr int DS = D / 16, DB = D / 32, CPR = D / 8;
  static constexpr int RPP = 64 / CPR;          // rows per 1 KB wave load
  static constexpr int PPT = BC / RPP;          // 1 KB pieces per K (or V) block
  static constexpr int LPW = 2 * PPT / NW;      // loads per wave per block
  static_assert(LPW * NW == 2 * PPT && LPW < 64, "load split");
};

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(256) void fa1_kernel(const uint16_t* __restrict__ qg, const uint16_t* __restrict__ kg,
                                                  const uint16_t* __restrict__ vg, uint16_t* __restrict__ og,
                                                  float* __restrict__ lseg, float* __restrict__ ows,
                                                  float* __restrict__ mws, float* __restrict__ lws, int N,
                                                  float qk_scale) {
  using C = Fa1<D>;
  constexpr int BC = C::BC, BR = C::BR, DS = C::DS, DB = C::DB;
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[BC * D];  // swizzled rows
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[BC * D];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 31, g = lane >> 5;
  const int bh = blockIdx.x;
  const size_t head = (size_t)bh * N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2;
  const rsrc_t qrs = make_rsrc(qg + head, head_bytes);
  const rsrc_t krs = make_rsrc(kg + head, head_bytes);
  const rsrc_t vrs = make_rsrc(vg + head, head_bytes);
  float* ow = ows + head;
  float* mw = mws + (size_t)bh * N;
  float* lw = lws + (size_t)bh * N;
  const int Tc = (N + BC - 1) / BC, Tr = (N + BR - 1) / BR;

  for (int j = 0; j < Tc; ++j) {
    // K_j, V_j into LDS (rows past N read as zeros).
    {
      const int lrow = lane / C::CPR;
#pragma unroll
      for (int e = 0; e < C::LPW; ++e) {
        const int t = wave * C::LPW + e;
        const int p = t % C::PPT;
        const int row = p * C::RPP + lrow;
        const int ch = (lane % C::CPR) ^ swz_chunk<D>(row);
        const uint32_t off = ((uint32_t)(j * BC + row) * D + 8 * ch) * 2;
        if (t < C::PPT) load_lds16(krs, &k_lds[p * C::RPP * D], off);
        else load_lds16(vrs, &v_lds[p * C::RPP * D], off);
      }
      lds_barrier<0>();
    }
    // Causal: query block i sees block j iff its last row reaches key j BC.
    const int i0 = CAUSAL ? (j * BC) / BR : 0;
    for (int i = i0; i < Tr; ++i) {
      const int query = i * BR + 32 * wave + n;  // this lane's query
      if (i * BR + 32 * wave >= N) continue;      // the wave has no live row here
      // Q_i fragments (B operand of S^T = K_j Q_i^T)
      uint4 qf[DS];
#pragma unroll
      for (int s = 0; s < DS; ++s) qf[s] = load16(qrs, ((uint32_t)query * D + 16 * s + 8 * g) * 2);
      // S^T for the two 32-key halves of block j; register r of half h is
      // key j BC + 32 h + 8 (r / 4) + 4 g + r % 4.
      f32x16 sc[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        sc[h] = f32x16{};
#pragma unroll
        for (int s = 0; s < DS; ++s) sc[h] = mma16(T{}, read_row<D>(k_lds, 32 * h + n, 16 * s + 8 * g), qf[s], sc[h]);
      }
      const int key_lim = CAUSAL ? min(query + 1, N) : N;
      float mt = kNegInf;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = j * BC + 32 * h + 8 * (r / 4) + 4 * g + (r % 4);
          sc[h][r] = key < key_lim ? sc[h][r] * qk_scale : kNegInf;
          mt = fmaxf(mt, sc[h][r]);
        }
      mt = halves_max(mt);  // m~ (log2 units); -inf when the row sees no key here
      float lt = 0.f;
      uint4 pk[4];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float p0 = mt == kNegInf ? 0.f : fast_exp2(sc[h][r] - mt);
          const float p1 = mt == kNegInf ? 0.f : fast_exp2(sc[h][r + 1] - mt);
          lt += p0 + p1;
          const uint32_t w = pack2(T{}, p0, p1);
          const int word = (16 * h + r) / 2;  // 0..15 -> pk[word / 4]
          if (word % 4 == 0) pk[word / 4].x = w;
          else if (word % 4 == 1) pk[word / 4].y = w;
          else if (word % 4 == 2) pk[word / 4].z = w;
          else pk[word / 4].w = w;
        }
      lt = halves_sum(lt);
      // P~ V_j as O^T += V_j^T P~^T: 16-key step s2 uses registers 8 s2 ..
      f32x16 pv[DB];
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        pv[db] = f32x16{};
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) pv[db] = mma16(T{}, read_tr<D>(v_lds, 16 * s2, 32 * db, lane), pk[s2], pv[db]);
      }
      // The running state of this row from HBM (nothing yet at j = 0).
      float mi = kNegInf, li = 0.f;
      if (j > 0) {
        mi = mw[query < N ? query : 0];
        li = lw[query < N ? query : 0];
      }
      const float mn = fmaxf(mi, mt);
      const float a_old = mi == kNegInf ? 0.f : fast_exp2(mi - mn);
      const float a_new = mt == kNegInf ? 0.f : fast_exp2(mt - mn);
      const float ln = a_old * li + a_new * lt;
      const float inv = ln > 0.f ? 1.f / ln : 0.f;
      const float c_old = li * a_old * inv, c_new = a_new * inv;
      // O_i <- (l_i e^{m_i - m_new} O_i + e^{m~ - m_new} P~ V_j) / l_new;
      // register r of d block db is column 32 db + 8 (r / 4) + 4 g + r % 4.
      if (query < N) {
        float* orow = ow + (size_t)query * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int rq = 0; rq < 4; ++rq) {
            float4* p4 = reinterpret_cast<float4*>(orow + 32 * db + 8 * rq + 4 * g);
            const float4 old = j > 0 ? *p4 : make_float4(0.f, 0.f, 0.f, 0.f);
            *p4 = make_float4(c_old * old.x + c_new * pv[db][4 * rq + 0], c_old * old.y + c_new * pv[db][4 * rq + 1],
                              c_old * old.z + c_new * pv[db][4 * rq + 2], c_old * old.w + c_new * pv[db][4 * rq + 3]);
          }
        if (g == 0) {
          mw[query] = mn;
          lw[query] = ln;
        }
      }
    }
    __syncthreads();  // every wave is done with K_j, V_j before the next block replaces them
  }

  // O in the input type and LSE = (m + log2 l) ln 2.  Each lane reads back
  // what it wrote itself.
  for (int i = 0; i < Tr; ++i) {
    const int query = i * BR + 32 * wave + n;
    if (query >= N) continue;
    const float* orow = ow + (size_t)query * D;
    uint16_t* dst = og + head + (size_t)query * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const float4 x = *reinterpret_cast<const float4*>(orow + 32 * db + 8 * rq + 4 * g);
        *reinterpret_cast<uint2*>(dst + 32 * db + 8 * rq + 4 * g) = make_uint2(pack2(T{}, x.x, x.y), pack2(T{}, x.z, x.w));
      }
    if (g == 0) lseg[(size_t)bh * N + query] = (mw[query] + __log2f(lw[query])) * kLn2;
  }
}

template <typename T, int D>
hipError_t run(const Fa1Args& a) {
  const float qk_scale = a.scale * kLog2eHost;
  if (a.causal)
    hipLaunchKernelGGL((fa1_kernel<T, D, true>), dim3((unsigned)a.BH), dim3(Fa1<D>::NT), 0, a.stream,
                       static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                       static_cast<const uint16_t*>(a.v), static_cast<uint16_t*>(a.o), a.lse, a.ows, a.mws, a.lws, a.N,
                       qk_scale);
  else
    hipLaunchKernelGGL((fa1_kernel<T, D, false>), dim3((unsigned)a.BH), dim3(Fa1<D>::NT), 0, a.stream,
                       static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                       static_cast<const uint16_t*>(a.v), static_cast<uint16_t*>(a.o), a.lse, a.ows, a.mws, a.lws, a.N,
                       qk_scale);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fa1(const Fa1Args& a) {
  if (a.dtype == 2) return a.d == 128 ? run<BF16, 128>(a) : run<BF16, 64>(a);
  return a.d == 128 ? run<F16, 128>(a) : run<F16, 64>(a);
}

}  // namespace fa
