// fa_plan.hpp -- integer planning shared by the host ABI and the kernels:
// causal key-block stages, workgroup-to-tile order, tile shapes.
//
// Pages cited: "Triton 06: Flash Attention v2" (wonbeomjang.kr),
// Improvement 3 (causal mask split into an unmasked stage and a masked
// diagonal stage); "Flash Attention: IO-awareness principle" (hrletsgo.me),
// section "FA2/FA3" (query blocks in the outer loop, each workgroup finishes
// its own output block with no cross-block synchronisation).
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define FA_HD __host__ __device__ __forceinline__
#else
#define FA_HD inline
#endif

namespace fa {

constexpr float kLog2eHost = 1.4426950408889634f;

// Key-block plan of the causal split for the query rows [row0, row_end):
// blocks j < s1_end hold only keys <= row0 (their last key, (j+1)*bn - 1, is
// at or left of the first row) and need no mask; blocks s1_end <= j < s2_end
// straddle the diagonal and are masked; blocks from s2_end on lie wholly in
// the future and are skipped.
//
// The page classifies block j as unmasked when its first key is left of
// the block's first row, which is exact only when the query block size is a
// multiple of bn; the comparison below is exact for any sizes.
FA_HD void causal_stages(int row0, int row_end, int bn, int* s1_end, int* s2_end) {
  // (j+1)*bn - 1 <= row0  <=>  j <= (row0 + 1)/bn - 1
  *s1_end = (row0 + 1) / bn;
  *s2_end = (row_end - 1) / bn + 1;
}

// Workgroups are dealt round-robin to the 8 XCDs (hardware id b runs on XCD
// b % 8), and each XCD has its own L2.  Renumber so that every XCD gets one
// contiguous range of logical tiles: tiles of one (batch, head) then share
// an L2 and its K/V stream.  Bijective on [0, total) for any total.
FA_HD int xcd_remap(int b, int total) {
  constexpr int NX = 8;
  const int xcd = b % NX, slot = b / NX;
  const int q = total / NX, r = total % NX;
  return (xcd < r) ? xcd * (q + 1) + slot : r * (q + 1) + (xcd - r) * q + slot;
}

// Logical tile -> (batch*head, query block).  Within one (batch, head) the
// causal order runs from the last query block (most key blocks) to the
// first, so long workgroups start early and the tail is short.
FA_HD void tile_of(int logical, int n_qblk, bool causal, int* bh, int* qblk) {
  *bh = logical / n_qblk;
  const int j = logical % n_qblk;
  *qblk = causal ? (n_qblk - 1 - j) : j;
}

// Work items of the persistent kernels.  Their grids hold one workgroup
// per CU and each workgroup walks a list of items.  Under the causal mask
// the blocks of a head cost a linear ramp: query block i of the forward and
// of dQ costs about i + 1 key tiles, key block j of dK/dV about n - j query
// tiles.  Item p therefore pairs block p with block n_blk - 1 - p, so every
// item costs about the same and a round-robin deal of items keeps the CUs
// balanced (an odd middle block is an item of its own).  Without the mask
// all blocks cost the same: one block per item.
FA_HD int items_per_head(int n_blk, bool causal) { return causal ? (n_blk + 1) / 2 : n_blk; }

// Blocks of item p of a head: *lo = p and, for a causal pair, *hi =
// n_blk - 1 - p (else -1).  Returns how many (1 or 2).
FA_HD int item_blocks(int p, int n_blk, bool causal, int* lo, int* hi) {
  *lo = p;
  *hi = causal ? n_blk - 1 - p : -1;
  if (*hi == p) *hi = -1;
  return *hi < 0 ? 1 : 2;
}

// Grouped heads (GQA; MQA when one K/V head serves all): the H query heads
// of a batch share H / G K/V heads, G consecutive query heads per K/V head.
// With flat indices bh = b H + h (query) and b (H / G) + h / G (K/V), and
// G dividing H, the K/V head of bh is simply bh / G, and the query heads of
// flat K/V head bkv are bkv G .. bkv G + G - 1.
FA_HD int kv_head_of(int bh, int G) { return bh / G; }
FA_HD int q_head_of(int bkv, int G, int j) { return bkv * G + j; }

// Decoding (one query per head over a K/V cache).  A unit is one (batch,
// K/V head, block of 32 query heads of its group), u = (b Hkv + hkv) QB +
// qb; it owns the ceil(len_b / kDecodeTileKeys) key tiles of its batch's
// valid length.  The units' tiles are laid end to end (T in all) and cut
// into n_parts ranges of per = ceil(T / n_parts) tiles, one workgroup each:
// part w takes tiles [w per, min((w + 1) per, T)).  The piece of unit u a
// part holds is a segment; a segment that is not the whole unit leaves its
// result in workspace slot w + u, to be merged.
constexpr int kDecodeTileKeys = 128;
constexpr int kDecodeMaxParts = 1024;
FA_HD int decode_tiles(int len) { return (len + kDecodeTileKeys - 1) / kDecodeTileKeys; }
FA_HD int decode_query_blocks(int G) { return (G + 31) / 32; }

// Tile constants of the 16-bit forward and of the dQ kernel.  The defaults
// are the shapes the library ships; a build may define others (each wave
// owns 32 queries; BN is the K/V tile of the d = 64 forward) to time the
// alternatives.
#ifndef FA_FWD16_WAVES
#define FA_FWD16_WAVES 8
#endif
#ifndef FA_FWD16_BN_D64
#define FA_FWD16_BN_D64 128
#endif
#ifndef FA_DQ_WAVES
#define FA_DQ_WAVES 8
#endif
static_assert(FA_FWD16_WAVES == 4 || FA_FWD16_WAVES == 8, "forward waves per workgroup");
static_assert(FA_FWD16_BN_D64 == 64 || FA_FWD16_BN_D64 == 128, "forward K/V tile at d = 64");
static_assert(FA_DQ_WAVES == 4 || FA_DQ_WAVES == 8, "dQ waves per workgroup");

// Forward tile shapes (query rows per workgroup, keys per K/V block, waves).
struct FwdTile {
  int bm, bn, waves;
};

FA_HD FwdTile fwd_tile(int d, bool is_f32) {
  if (is_f32) return FwdTile{128, 64, 4};
  return FwdTile{32 * FA_FWD16_WAVES, d == 128 ? 64 : FA_FWD16_BN_D64, FA_FWD16_WAVES};
}

}  // namespace fa
