// fa_device.hpp -- device building blocks for the gfx950 attention kernels:
// MFMA tile products, wave64 cross-half reductions, element conversions and
// the online-softmax step.
//
// MFMA conventions (v_mfma_f32_32x32x16_{bf16,f16} and v_mfma_f32_32x32x2_f32,
// 64 lanes, lane l, g = l / 32, n = l % 32):
//   A operand (32 x K):  lane l supplies row n, its K-slice for group g;
//   B operand (K x 32):  lane l supplies column n, its K-slice for group g;
//   C/D (32 x 32 fp32): register r of lane l is element
//                        row 8*(r/4) + 4*g + (r%4), column n.
// Both operands of one product take their K-slices with the same (g, t)
// pattern, so the hardware's K order inside an instruction never matters.
//
// Pages cited: "Triton 06: Flash Attention v2" (wonbeomjang.kr),
// Improvement 1 (un-scaled accumulator, alpha correction, one final divide),
// Improvement 2 (exp2 with log2(e) folded into the scale), Improvement 4
// (the running accumulator is the matrix product's C operand); "Flash
// Attention -- five lessons converging into 80 lines" (brianyu43.github.io),
// Lesson 4 (warp reduction for the row max and sum, coalesced loads).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

// Element type tags for the 16-bit paths.
struct BF16 {};
struct F16 {};

// ---------------------------------------------------------------------------
// Matrix products.  c += A(32 x 16) * B(16 x 32) with 8 16-bit elements per
// lane per operand, passed as 16 raw bytes.
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x16 mma16(BF16, const uint4& a, const uint4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mma16(F16, const uint4& a, const uint4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
// fp32: c += A(32 x 2) * B(2 x 32), one element per lane per operand.
__device__ __forceinline__ f32x16 mma32(float a, float b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Conversions, round-to-nearest-even.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t pack2(BF16, float a, float b) {
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint32_t pack2(F16, float a, float b) {
  f16x2 v = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, v);
}
// acc + a + b for a softmax row sum, where w = pack2(a, b).  fp16: one dot
// product of the packed pair with (1, 1), i.e. the sum of the rounded
// values (relative error at most 2^-11 each, inside the LSE bound of 1e-3
// even when one weight carries the whole row).  bf16 rounding (2^-9) would
// not be, so there the fp32 values are added.
__device__ __forceinline__ float add_pair(BF16, uint32_t, float a, float b, float acc) { return acc + a + b; }
__device__ __forceinline__ float add_pair(F16, uint32_t w, float, float, float acc) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w), __builtin_bit_cast(f16x2, 0x3C003C00u), acc, false);
}
// The first pair of a row sum: a + b, without a zero to add to first (the
// compiler cannot drop 0 + x, which differs from x when x is -0).
__device__ __forceinline__ float first_pair(BF16, uint32_t, float a, float b) { return a + b; }
__device__ __forceinline__ float first_pair(F16, uint32_t w, float a, float b) { return add_pair(F16{}, w, a, b, 0.f); }
__device__ __forceinline__ float lo16(BF16, uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi16(BF16, uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float lo16(F16, uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
__device__ __forceinline__ float hi16(F16, uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// ---------------------------------------------------------------------------
// Wave64 reductions across the two 32-lane halves.  v_permlane32_swap
// exchanges the halves; which result holds the partner's value depends on
// the half, so only symmetric combinations are formed from the pair.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float halves_max(float x) {
  const uint32_t u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const uint32_t u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// Buffer loads.  A buffer resource covers one (batch, head) slice of
// `bytes` bytes; the hardware range check returns zeros for any read at or
// past the end, which is how ragged tails are zero-filled without branches.
// Offsets are 32-bit: the host rejects heads of 2 GiB or more.
// ---------------------------------------------------------------------------
// Wait until every vector-memory load this wave issued has returned
// (s_waitcnt vmcnt(0), the other counters left free).  Placed after the
// loads that precede a prefetching loop: the compiler's wait insertion cannot
// tell those loads from the loop's own prefetches once the loop has been
// entered, and otherwise puts a wait for the whole prefetch in front of the
// first matrix products of every iteration.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// Wait until at most N of this wave's vector-memory operations are
// outstanding (s_waitcnt vmcnt(N); the other counters left free).
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef unsigned int v4u32 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_void_t;
constexpr int kRsrcWord3 = 0x00020000;  // raw (untyped) buffer, 32-bit data format

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}
__device__ __forceinline__ uint4 load16(rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}
__device__ __forceinline__ float4 load16f(rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}
__device__ __forceinline__ float load4f(rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 0));
}

// Loads straight into LDS (no registers): the wave's 64 lanes each fetch
// 16 (or 4) bytes from byte offset `byte_off` of the buffer and the hardware
// writes lane l's bytes to dst + 16 l (or 4 l); dst must be the same for the
// whole wave (it travels in M0).  Reads past the buffer's end write zeros.
// The data is in LDS once this wave's vmcnt says the load has returned; other
// waves see it after a barrier that follows that wait.  dst must be an
// element pointer into a __shared__ array, not the bare array name.
__device__ __forceinline__ void load_lds16(rsrc_t r, void* dst, uint32_t byte_off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t)dst, 16, byte_off, 0, 0, 0);
}
__device__ __forceinline__ void load_lds4(rsrc_t r, void* dst, uint32_t byte_off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t)dst, 4, byte_off, 0, 0, 0);
}
// The same 16-byte load straight into LDS, issued from inline assembly so
// that the compiler does not track it.  The compiler's wait insertion cannot
// tell one LDS range from another for these loads and would make the first
// LDS read after them wait for all; with this form it adds no wait at all,
// and the caller waits explicitly (vm_wait, then lds_fence) before it reads
// the destination.  lds_dst is the wave-uniform LDS byte address (through
// M0); the load has no result registers.  Counted in vmcnt like any load.
// The asm sets M0 itself and declares it clobbered; the compiler does not
// preserve M0 around it (it warns so), which is safe only while the kernel
// keeps no value of its own in M0 across these loads: the kernels that use
// this form issue no compiler-tracked load into LDS and no indexed register
// access (their assembly shows no other M0 use).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(lds_void_t)(const_cast<void*>(p));
}
__device__ __forceinline__ void load_lds16_untracked(rsrc_t r, uint32_t lds_dst, uint32_t byte_off) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds"
      :
      : "s"(lds_dst), "v"(byte_off), "s"(r)
      : "memory", "m0");
}
// Keeps the compiler from moving memory accesses across this point (after an
// explicit wait for loads it does not track).
__device__ __forceinline__ void lds_fence() { asm volatile("" ::: "memory"); }

// Workgroup barrier for loops that keep loads into LDS in flight across
// it.  __syncthreads() fences all LDS writes, including those loads, so it
// would wait for every one of them; here the caller names how many of its
// most recent vector-memory loads may stay outstanding (NCNT, in issue
// order), all LDS instructions of the wave are waited for, and the empty
// asm statements keep the compiler from moving memory accesses across the
// barrier.  A wave that reads data loaded by another wave must do so only
// after a barrier at which the loading wave waited for that load.
template <int NCNT>
__device__ __forceinline__ void lds_barrier() {
  // s_waitcnt immediate: vmcnt bits 3:0 and 15:14, expcnt 6:4 (left at its
  // maximum), lgkmcnt 11:8 (zero).
  static_assert(NCNT >= 0 && NCNT < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((NCNT & 15) | 0x0070 | ((NCNT >> 4) << 14));  // vmcnt(NCNT) lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Workgroup barrier that waits only for this wave's LDS operations, not for
// its outstanding global loads and stores (lgkmcnt(0), vmcnt left free):
// enough before another wave may overwrite LDS this wave has read.
__device__ __forceinline__ void lds_only_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt at their maxima
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------------------
// Online softmax, split so the kernel can decide on the correction once per
// wave.  Scores are the KB 32x32 blocks S^T of one 32-query column block:
// lane l owns query n = l % 32; register r of block kb is key
// key_base + 32*kb + 8*(r/4) + (r%4), where key_base already includes 4*g.
// qk_scale >= 0 (a negative scale is folded into the sign of Q), so the max
// of the raw scores times qk_scale is the max of the scaled scores.  MASKED
// keeps only keys < key_lim (the causal limit query+1 and the sequence end).
// ---------------------------------------------------------------------------

// Row max of the scaled scores of this block (same on both lane halves);
// -inf when the row has no visible key here.
template <int KB, bool MASKED>
__device__ __forceinline__ float tile_max(const f32x16 (&s)[KB], float qk_scale, int key_base, int key_lim) {
  float mx = kNegInf;
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if constexpr (MASKED) {
        const int key = key_base + 32 * kb + 8 * (r / 4) + (r % 4);
        mx = fmaxf(mx, key < key_lim ? s[kb][r] : kNegInf);
      } else {
        mx = fmaxf(mx, s[kb][r]);
      }
    }
  }
  mx = halves_max(mx);
  return (mx == kNegInf) ? kNegInf : mx * qk_scale;
}

// p = exp2(S * qk_scale - m) in place; masked p are exactly 0 (also when
// qk_scale is 0).  Returns this lane's sum of p.
template <int KB, bool MASKED>
__device__ __forceinline__ float tile_exp(f32x16 (&s)[KB], float qk_scale, float m, int key_base, int key_lim) {
  float sum[4] = {0.f, 0.f, 0.f, 0.f};  // four chains instead of one long dependent one
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float p = fast_exp2(__builtin_fmaf(s[kb][r], qk_scale, -m));
      if constexpr (MASKED) {
        const int key = key_base + 32 * kb + 8 * (r / 4) + (r % 4);
        p = key < key_lim ? p : 0.f;
      }
      s[kb][r] = p;
      sum[r % 4] += p;
    }
  }
  return (sum[0] + sum[1]) + (sum[2] + sum[3]);
}

// Running-max bookkeeping with a tolerance.  The reference for the exponent
// (m) is raised only when a block's max exceeds it by more than kMaxSlack
// (log2 units); until then the weights exp2(t - m) may reach 2^kMaxSlack,
// which fp32 accumulators and 16-bit P represent with the same relative
// precision.  Because the accumulator, the row sum and the final LSE all
// use the same m, the result is the same exact softmax: only the points at
// which the accumulator is rescaled change, and a wave skips the rescale
// (a multiply over the whole accumulator) whenever no lane needs it.
constexpr float kMaxSlack = 8.f;

// Returns true (wave-uniform) when some lane of the wave must rescale; then
// *alpha holds this lane's factor (1 for lanes that keep their m) and m, l
// are updated.  m = -inf means "no visible key yet".
__device__ __forceinline__ bool raise_max(float mt, float& m, float& l, float* alpha) {
  const bool grow = mt > m + kMaxSlack;  // false while mt is -inf
  if (__builtin_amdgcn_ballot_w64(grow) == 0) return false;
  const float m_new = grow ? mt : m;
  *alpha = grow ? fast_exp2(m - m_new) : 1.f;  // m = -inf gives 0
  l *= *alpha;
  m = m_new;
  return true;
}


// ---------------------------------------------------------------------------
// Transposed LDS tiles.  A 16-bit tile that feeds an MFMA operand with the
// row index as contraction index is stored transposed (row index
// contiguous).  Inside every 16-row group, row kappa sits at position
// tpos(kappa) = kappa with bits 2 and 3 swapped: a 32x32 accumulator gives
// lane half g the rows {4g..4g+3, 8+4g..8+4g+3} of each 16-row group in
// registers 0..7, and tpos puts exactly those rows at positions 8g..8g+7,
// so one 16-byte LDS read returns a lane's eight elements in register order.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int tpos(int kappa) {
  return (kappa & ~0xC) | ((kappa & 4) << 1) | ((kappa & 8) >> 1);
}

// Write KPT consecutive rows x 8 columns (16-bit, one uint4 per row, rows
// starting at a multiple of KPT) transposed: column t goes to row t of
// `dst` (row stride `stride` elements) at position `pos` = tpos(first row).
// One v_perm_b32 builds each output dword from two input dwords.
template <int KPT>
__device__ __forceinline__ void store_transposed(uint16_t* dst, int stride, int pos, const uint4 (&x)[KPT]) {
  static_assert(KPT == 2 || KPT == 4, "2 or 4 rows per thread");
  const uint32_t* w = reinterpret_cast<const uint32_t*>(x);  // w[4*row + i]: columns 2i, 2i+1
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t sel = h ? 0x07060302u : 0x05040100u;  // high or low halves of the two words
      uint16_t* p = dst + (2 * i + h) * stride + pos;
      const uint32_t a = __builtin_amdgcn_perm(w[4 + i], w[i], sel);
      if constexpr (KPT == 4) {
        const uint32_t b = __builtin_amdgcn_perm(w[12 + i], w[8 + i], sel);
        *reinterpret_cast<uint2*>(p) = make_uint2(a, b);
      } else {
        *reinterpret_cast<uint32_t*>(p) = a;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Swizzled row-major LDS tiles.  A 16-bit tile with rows of D elements
// (D = 64 or 128, no padding) keeps its 16-byte chunks XOR-permuted per row,
// chunk c of row r at chunk c ^ swz_chunk(r).  The permutation makes two
// access patterns bank-conflict free at once:
//  * 16-byte row reads: 16 consecutive rows, one chunk each (an MFMA operand
//    whose contraction index runs along the row);
//  * transposing 8-byte reads (ds_read_b64_tr_b16): per half wave 4
//    consecutive rows x 64 bytes (an MFMA operand whose contraction index
//    runs down the columns).
// Row padding serves only one of the two.
// ---------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ int swz_chunk(int row) {
  static_assert(D == 64 || D == 128, "row width");
  return D == 128 ? 4 * (row & 3) + ((row >> 2) & 3) : 4 * ((row >> 1) & 1) + ((row >> 2) & 3);
}
template <int D>
__device__ __forceinline__ int swz(int row, int col) {  // element offset of (row, col)
  return row * D + (((col >> 3) ^ swz_chunk<D>(row)) << 3) + (col & 7);
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 read_tr_b64(const uint16_t* p) {
  const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(p));
  return __builtin_bit_cast(uint2, v);
}

// An MFMA 16-bit operand fragment read across rows of a swizzled tile: lane
// (c = lane % 32, g = lane / 32) receives column col0 + c of rows
// r0 + 4g + {0..3} and then r0 + 8 + 4g + {0..3} (r0 a multiple of 16, col0
// a multiple of 32), i.e. the row order of a 32x32 accumulator packed to
// 16 bits.  ds_read_b64_tr_b16 hands lane i of each 16-lane group element e
// of the 4-element vector addressed by lane 4e + i/4, so lane p addresses
// row p/4 and columns 4(p%4)..4(p%4)+3 of its group's 4 x 16 block.
template <int D>
__device__ __forceinline__ uint4 read_tr(const uint16_t* tile, int r0, int col0, int lane) {
  const int p = lane & 15, row = r0 + 4 * (lane >> 5) + (p >> 2);
  const int col = col0 + 16 * ((lane >> 4) & 1) + 4 * (p & 3);
  const uint2 a = read_tr_b64(tile + swz<D>(row, col));
  const uint2 b = read_tr_b64(tile + swz<D>(row + 8, col));
  return make_uint4(a.x, a.y, b.x, b.y);
}
template <int D>
__device__ __forceinline__ uint4 read_row(const uint16_t* tile, int row, int col) {
  return *reinterpret_cast<const uint4*>(tile + swz<D>(row, col));
}

}  // namespace fa
