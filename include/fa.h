/*
 * fa.h -- C ABI of the MI355X (gfx950) exact-attention library, libfa.so.
 *
 * What the library computes.  For every batch b and head h, with Q, K, V the
 * N x d slices of that (b, h):
 *
 *     S = scale * Q K^T            (N x N, never stored by fa_fwd / fa_bwd)
 *     P = softmax(S) row-wise      (causal: S_ij = -inf for j > i)
 *     O = P V                      (N x d)
 *     LSE_i = ln sum_j exp(S_ij)   (natural log, over the allowed j)
 *
 * This is standard attention as defined by Algorithm 0 of "Paper review:
 * FlashAttention: Fast and Memory-Efficient Exact Attention with IO-Awareness"
 * (osehyeon.github.io), with the 1/sqrt(d)-style scale of "Flash Attention:
 * IO-awareness principle" (hrletsgo.me, section on standard attention's
 * bottleneck) taken as an argument.  fa_fwd computes it the FlashAttention-2
 * way ("Triton 06: Flash Attention v2", wonbeomjang.kr, Improvements 1-4):
 * Q row-blocks outside, K/V blocks inside, S and P kept on chip.  fa_bwd
 * recomputes P from LSE ("Backward" and the forward/backward flow summary on
 * the same page).  fa_naive_fwd is the three-kernel path that writes S and P
 * to memory ("Flash Attention -- five lessons converging into 80 lines",
 * brianyu43.github.io, "Two implementations").
 *
 * Layout.  Q, K, V, O, dO are [B, H, N, d] contiguous row-major (d fastest)
 * in the element type `dtype`.  LSE and Delta are float32 [B, H, N].  dQ, dK,
 * dV are float32 [B, H, N, d].  Naive S and P workspaces are [B, H, N, N],
 * float16 when dtype is 16-bit (f16 or bf16) and float32 when dtype is f32.
 *
 * Supported values.  d in {64, 128} (else FA_ERR_UNSUPPORTED); N >= 1 (any
 * value; ragged tails are masked); B, H >= 1; causal in {0, 1}; scale finite
 * (zero and negative allowed).  One (batch, head) slice of Q must stay below
 * 2 GiB, N * d * element size < 2^31 (the kernels address a head with
 * 32-bit buffer offsets), else FA_ERR_UNSUPPORTED.  causal = 1 keeps key j for query i iff
 * j <= i (square, top-left aligned, diagonal kept).
 *
 * Ownership.  The caller allocates and frees every buffer, workspaces
 * included.  The library never allocates, frees or synchronises, and keeps
 * no state between calls except a thread-local copy of the last HIP error.
 * All device pointers are on the current HIP device.  `stream` is a
 * hipStream_t (NULL = the default stream).  Calls enqueue work and return:
 * results are ready when the stream is; a fault in a kernel shows at the
 * caller's next synchronisation.
 *
 * Errors.  Every entry point returns an fa_status synchronously.  All
 * argument checks run on the host before any HIP call, so a rejected call
 * touches no device state: null pointer -> FA_ERR_ARG; shape or size
 * overflowing int64 -> FA_ERR_ARG; a device pointer not 16-byte aligned ->
 * FA_ERR_ALIGN; unsupported d or dtype (and f32 in fa_bwd) ->
 * FA_ERR_UNSUPPORTED.  A launch failure reported by
 * hipGetLastError() -> FA_ERR_HIP; fa_last_hip_error() then returns that
 * hipError_t value for the calling thread.  No C++ exception crosses the ABI.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { FA_F32 = 0, FA_F16 = 1, FA_BF16 = 2 } fa_dtype;

typedef enum {
  FA_OK = 0,
  FA_ERR_ARG = 1,
  FA_ERR_UNSUPPORTED = 2,
  FA_ERR_ALIGN = 3,
  FA_ERR_HIP = 4,
  FA_ERR_SCRATCH = 5
} fa_status;

/*
 * Fused forward.  Reads q, k, v; writes o (dtype, [B,H,N,d]) and lse
 * (float32 [B,H,N], natural log).  One pass over K/V per query block with
 * the online softmax: running max and sum per row, an un-scaled accumulator
 * rescaled when the max grows, one divide at the end, exp2 with
 * log2(e) folded into the scale, and a per-row LSE saved for fa_bwd
 * ("Triton 06: Flash Attention v2", Improvements 1-3).  Causal runs the
 * fully visible key blocks without a mask and masks only the diagonal
 * blocks; key blocks wholly in the future are never read.  Short 16-bit
 * problems with fewer 256-query work items than compute units, whose keys
 * fit in LDS (N <= 512 at d = 64, N <= 256 at d = 128), run 64-query
 * blocks instead, each block's keys split over four waves and the partial
 * results merged with the log-sum-exp form of the softmax decomposition
 * ("Paper review: FlashAttention ...", "Tiling"); the result is the same
 * softmax up to rounding.
 * q, k, v, o, lse: device pointers, 16-byte aligned, not aliased with each
 * other.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int N, int d, float scale, int causal, int dtype, void* stream);

/*
 * Fused backward with recomputation ("Triton 06: Flash Attention v2",
 * "Backward" and the flow summary; "Flash Attention: IO-awareness
 * principle", "Recomputation").  Inputs q, k, v, o (the fa_fwd output),
 * dout (dO), all dtype [B,H,N,d], and lse (float32 [B,H,N], natural log,
 * as fa_fwd wrote it).  Three launches on `stream`, in order:
 *   1. Delta_i = sum_c dO_ic * O_ic  -> delta_ws (float32 [B,H,N])
 *   2. per K/V block: P recomputed from LSE; dV += P^T dO;
 *      dS = P * (dO V^T - Delta); dK += scale * dS^T Q      -> dk, dv
 *   3. per Q block:  dQ += scale * dS K                      -> dq
 * dq, dk, dv are float32 [B,H,N,d] and are fully overwritten (no zeroing
 * needed).  delta_ws is caller-owned scratch that holds Delta afterwards.
 * dtype f16 and bf16 are supported; f32 returns FA_ERR_UNSUPPORTED.  The
 * fp32 gradients of one head must stay below 2 GiB including the last
 * block's padding, (N + 255) * d * 4 < 2^31 (N <= 4,194,048 at d = 128),
 * else FA_ERR_UNSUPPORTED.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
           const float* lse, float* delta_ws, float* dq, float* dk, float* dv,
           int B, int H, int N, int d, float scale, int causal, int dtype, void* stream);

/*
 * One launch of fa_bwd, for timing each kernel on its own: stage 1 writes
 * Delta, stage 2 writes dK and dV (needs Delta), stage 3 writes dQ (needs
 * Delta).  Calling stages 1, 2, 3 in order on one stream does exactly what
 * fa_bwd does.  Same arguments and checks as fa_bwd; a stage outside 1..3
 * -> FA_ERR_ARG.
 */
int fa_bwd_stage(int stage, const void* q, const void* k, const void* v, const void* o,
                 const void* dout, const float* lse, float* delta_ws, float* dq, float* dk,
                 float* dv, int B, int H, int N, int d, float scale, int causal, int dtype,
                 void* stream);

/*
 * Grouped-query attention (GQA; MQA when Hkv = 1), the head sharing that
 * "Flash Attention: IO-awareness principle" names in its section on serving
 * (fewer K/V heads, hence fewer tiles of K/V work).  The H query heads of a
 * batch share Hkv K/V heads: query head h reads K/V head h / (H / Hkv), so
 * G = H / Hkv consecutive query heads form a group.  The result for query
 * head h is exactly fa_fwd's with K, V replaced by that K/V head's slices.
 * q, o: dtype [B,H,N,d]; k, v: dtype [B,Hkv,N,d]; lse: float32 [B,H,N].
 * Requires 1 <= Hkv <= H and H % Hkv == 0, else FA_ERR_ARG; every other
 * argument, check and error as fa_fwd.  fa_fwd(...) is
 * fa_fwd_gqa(..., H, Hkv = H, ...).
 */
int fa_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int Hkv, int N, int d, float scale, int causal, int dtype,
               void* stream);

/*
 * Chunked prefill ("Flash Attention: IO-awareness principle", section on
 * PagedAttention and chunked prefill: serving feeds the kernel a chunk of
 * the prompt at a time over contiguous K/V).  Nq new queries are the last
 * Nq of Nk positions: with causal = 1, query i (0-based in the chunk) keeps
 * key j iff j <= i + (Nk - Nq), the square causal mask aligned at the
 * bottom-right corner; with causal = 0 every query sees all Nk keys.  K/V
 * heads are shared as in fa_fwd_gqa.
 * q, o: dtype [B,H,Nq,d]; k, v: dtype [B,Hkv,Nk,d]; lse: float32 [B,H,Nq].
 * Requires Nq <= Nk when causal (else FA_ERR_ARG); dtype f16 or bf16 when
 * Nq != Nk (f32 -> FA_ERR_UNSUPPORTED); other checks and errors as
 * fa_fwd_gqa.  fa_fwd_gqa(..., N, ...) is fa_fwd_chunk(..., Nq = N, Nk = N, ...).
 */
int fa_fwd_chunk(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int H, int Hkv, int Nq, int Nk, int d, float scale, int causal, int dtype,
                 void* stream);

/*
 * Backward of fa_fwd_gqa.  q, o, dout: dtype [B,H,N,d]; k, v: dtype
 * [B,Hkv,N,d]; lse, delta_ws: float32 [B,H,N]; dq: float32 [B,H,N,d];
 * dk, dv: float32 [B,Hkv,N,d], each the sum over the K/V head's G query
 * heads of what fa_bwd would give that query head (the chain rule through
 * the shared K and V).  The dK/dV kernel walks a K/V block's G query heads
 * in turn and accumulates on chip, so dk and dv are written once, fully
 * overwritten, with no atomics.  Same three launches, checks and errors as
 * fa_bwd, plus 1 <= Hkv <= H, H % Hkv == 0 (else FA_ERR_ARG).
 */
int fa_bwd_gqa(const void* q, const void* k, const void* v, const void* o, const void* dout,
               const float* lse, float* delta_ws, float* dq, float* dk, float* dv,
               int B, int H, int Hkv, int N, int d, float scale, int causal, int dtype,
               void* stream);

/*
 * Host copy of the head map fa_fwd_gqa / fa_bwd_gqa use: the flat K/V head
 * b * Hkv + h / (H / Hkv) that the flat query head bh = b * H + h reads.
 * Returns -1 unless 0 <= bh, 1 <= Hkv <= H, H % Hkv == 0.  Pure host
 * function (no HIP call).
 */
int fa_kv_head(int bh, int H, int Hkv);

/*
 * Decoding: the newest token of every sequence attends to its K/V cache
 * ("Flash Attention -- five lessons converging into 80 lines", "LLM-serving
 * translation": in decoding Q has one row per head).  With few K/V heads and
 * small batches one workgroup per head leaves most of the GPU idle ("Flash
 * Attention: IO-awareness principle", section on serving), so the cached
 * keys of the whole batch are shared out evenly among n_parts workgroups,
 * and results cut between workgroups are merged with the log-sum-exp form of
 * the softmax decomposition ("Paper review: FlashAttention ...", "Tiling").
 *
 * For every batch b and query head h, with L = kv_lens[b] (clamped to
 * [0, Nkv]; all Nkv when kv_lens is NULL) and K/V head g = h / (H / Hkv):
 *     s_j = scale * q[b,h] . k_cache[b,g,j]   for j < L
 *     o[b,h] = sum_j softmax(s)_j v_cache[b,g,j],  lse[b,h] = ln sum_j exp(s_j)
 * L = 0 gives o = 0 and lse = -inf (the empty sum).  Cache rows j >= L are
 * never read, so they may hold anything.
 *
 * q, o: dtype [B,H,d]; k_cache, v_cache: dtype [B,Hkv,Nkv,d] (Nkv is the
 * cache capacity, the row stride of a head); lse: float32 [B,H]; kv_lens:
 * NULL or a device int32 [B] (4-byte aligned).  dtype f16 or bf16 (f32 ->
 * FA_ERR_UNSUPPORTED); d in {64, 128}; Hkv divides H; 1 <= n_parts <= 1024.
 *
 * Partition (computed on the device from kv_lens).  A unit is one (batch,
 * K/V head, block of 32 query heads of that head's group), numbered
 * u = (b Hkv + g) QB + qb with QB = ceil((H / Hkv) / 32); it owns
 * ceil(L_b / 128) tiles of 128 keys.  The units' tiles, laid end to end (T
 * in all), are cut into n_parts ranges of P = ceil(T / n_parts) tiles: part
 * w (one workgroup) takes tiles [w P, (w + 1) P).  A unit held whole by one
 * part is written to o and lse directly; a unit cut between parts leaves
 * each piece's result in workspace slot w + u and a second launch merges
 * them.  n_parts = 1 needs no workspace (ws may be NULL) and is one launch.
 * n_parts > 1 needs ws (16-byte aligned, caller-owned) of at least
 * fa_decode_workspace_bytes(B, H, Hkv, d, n_parts) bytes; afterwards slot s
 * of a cut unit holds float32 O [32][d] (query columns of the unit, each
 * normalised within the piece) at float offset s * 32 * d, and float32 LSE
 * [32] at byte offset ceil256((n_parts + U) * 32 * d * 4) + s * 32 * 4,
 * U = B Hkv QB; other slots are left as they were.
 * Errors as fa_fwd; a missing or short workspace, a bad n_parts or a bad
 * grouping -> FA_ERR_ARG; more than 2^31 tiles -> FA_ERR_UNSUPPORTED.
 */
int fa_decode(const void* q, const void* k_cache, const void* v_cache, const int* kv_lens,
              void* o, float* lse, void* ws, size_t ws_bytes, int B, int H, int Hkv, int Nkv,
              int d, float scale, int n_parts, int dtype, void* stream);

/* Workspace bytes fa_decode needs for n_parts (0 for n_parts = 1 and for
 * invalid arguments). */
size_t fa_decode_workspace_bytes(int B, int H, int Hkv, int d, int n_parts);

/*
 * fa_decode for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  It
 * computes exactly what fa_decode computes (same kernels, same partition)
 * but keeps the pieces of cut units in a fixed scratch buffer the library
 * holds on each device, instead of a caller workspace; the caller still
 * passes q, the caches, kv_lens, o and lse.  No hipMalloc, hipFree or
 * allocating library routine is called.
 *
 * Limit: fa_decode_workspace_bytes(B, H, Hkv, d, n_parts) must not exceed
 * FA_DECODE_SCRATCH_BYTES (16 MiB), else FA_ERR_SCRATCH (checked on the host
 * before any HIP call).  n_parts = 1 uses no scratch.  The buffer lives on
 * every device the library runs on until the process ends; its address is
 * looked up once per device, on the first call there (FA_ERR_HIP if that
 * fails).  Nothing in it needs to start at zero: every piece the merge reads
 * was written earlier in the same call.  All calls on one device share the
 * buffer, so calls that overlap on one device (different streams, or
 * threads) race and must be serialised by the caller.  Other arguments,
 * checks and errors as fa_decode.
 */
#define FA_DECODE_SCRATCH_BYTES ((size_t)16 << 20)
int fa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, const int* kv_lens,
                      void* o, float* lse, int B, int H, int Hkv, int Nkv, int d, float scale,
                      int n_parts, int dtype, void* stream);

/*
 * The part count the library suggests for a decode step on the current
 * device: one per CU, at most the number of tiles at full length (and at
 * most 1024).  Queries the device's CU count (a HIP call; FA_ERR_HIP if that
 * fails).
 */
int fa_decode_plan(int B, int H, int Hkv, int Nkv, int d, int* n_parts);

/*
 * FP8 forward ("Flash Attention: IO-awareness principle", section
 * "FA2/FA3": FA3's FP8 mode), on gfx950's 8-bit matrix product.  q, k, v
 * hold OCP E4M3 codes (1 byte each; q [B,H,N,d], k and v [B,Hkv,N,d]) with
 * one dequantisation factor per tensor: value = code value * descale.
 * Computes fa_fwd_gqa's result for the dequantised inputs: scores and the
 * softmax statistics in fp32; the weights P (<= 1) are multiplied by 2^8
 * and rounded to E4M3 for the P V product, so O carries that rounding
 * (relative 2^-4 per weight in E4M3's normal range); the row sums and lse
 * use unrounded P.  o: bf16 [B,H,N,d]; lse: float32 [B,H,N], natural log.
 * d in {64, 128}; descales finite; other checks and errors as fa_fwd_gqa.
 */
int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
               int Hkv, int N, int d, float scale, float q_descale, float k_descale,
               float v_descale, int causal, void* stream);

/*
 * FlashAttention-1 loop order, kept to measure what the FA2 loop swap buys
 * ("Paper review: FlashAttention ...", Algorithm 1; "Flash Attention:
 * IO-awareness principle", section "FA2/FA3").  Same result as fa_fwd: o
 * (dtype [B,H,N,d]) and lse (float32 [B,H,N], natural log).  One
 * workgroup per (batch, head); K/V blocks of 64 keys in the outer loop,
 * query blocks of 128 rows inside, and at every step the block's running O,
 * l, m are read from and written back to ws.  ws (16-byte aligned, caller
 * owned, fa_fa1_workspace_bytes() bytes) holds afterwards: float32 O
 * [B,H,N,d] (normalised), then at ceil256 offsets float32 m [B,H,N] (row
 * max of scale * S in log2 units) and float32 l [B,H,N], with
 * lse = (m + log2 l) ln 2.  dtype f16 or bf16 (f32 -> FA_ERR_UNSUPPORTED);
 * other checks and errors as fa_fwd, a missing or short ws -> FA_ERR_ARG.
 */
int fa_fwd_fa1(const void* q, const void* k, const void* v, void* o, float* lse, void* ws,
               size_t ws_bytes, int B, int H, int N, int d, float scale, int causal, int dtype,
               void* stream);

/* Workspace bytes of fa_fwd_fa1 (0 for invalid arguments). */
size_t fa_fa1_workspace_bytes(int B, int H, int N, int d);

/*
 * Naive three-kernel forward ("Flash Attention -- five lessons converging
 * into 80 lines", "Two implementations"; Algorithm 0 of the FlashAttention
 * paper review): kernel 1 writes S = scale * Q K^T for all N x N into
 * s_ws; kernel 2 reads S, applies the causal mask if asked, and writes the
 * row softmax P into p_ws plus lse; kernel 3 reads P and V and writes o.
 * s_ws and p_ws are caller-owned, fa_naive_workspace_bytes() bytes each.
 * Kept to measure the N^2 memory traffic that fa_fwd avoids.
 */
int fa_naive_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                 void* s_ws, void* p_ws, int B, int H, int N, int d, float scale,
                 int causal, int dtype, void* stream);

/* Bytes of ONE of the naive S, P workspaces: B*H*N*N elements of float16
 * (dtype f16/bf16) or float32 (dtype f32).  0 for invalid arguments. */
size_t fa_naive_workspace_bytes(int B, int H, int N, int dtype);

/* Static English text for an fa_status value (never NULL). */
const char* fa_strerror(int status);

/* hipError_t of the most recent FA_ERR_HIP on the calling thread (0 if none). */
int fa_last_hip_error(void);

/*
 * Host copy of the causal key-block plan the kernels use ("Triton 06: Flash
 * Attention v2", Improvement 3).  For the query rows [row0, row_end) and key
 * blocks of `bn` keys: blocks [0, *s1_end) lie at or left of row0 and run
 * without a mask; blocks [*s1_end, *s2_end) straddle the diagonal and are
 * masked; later blocks are skipped.  Requires 0 <= row0 < row_end <= n,
 * bn >= 1; returns FA_ERR_ARG otherwise.  Pure host function (no HIP call).
 */
int fa_causal_stages(int row0, int row_end, int bn, int n, int* s1_end, int* s2_end);

/*
 * The forward's tile for (d, dtype): *bm query rows per workgroup,
 * *bn keys per K/V block, *waves wavefronts of 64 lanes per workgroup, as
 * the persistent kernel runs it when its work items fill the CUs.  (16-bit
 * problems whose items would fill at most half the CUs run half as many
 * waves and query rows per workgroup; short square ones the key-split
 * kernel, 64 query rows per workgroup.)  Pure host function;
 * FA_ERR_UNSUPPORTED for unsupported d/dtype.
 */
int fa_fwd_tile(int d, int dtype, int* bm, int* bn, int* waves);

/*
 * Measured ceilings of the chip, for reporting attention kernels against what
 * the hardware sustains as well as against its published peaks ("Flash
 * Attention -- five lessons converging into 80 lines", brianyu43.github.io,
 * Lesson 3: bandwidth as a fraction of what the memory delivers).  They
 * compute nothing of attention.
 *
 * fa_ceiling_mfma: `workgroups` workgroups of `waves` (4 or 8) wavefronts;
 * every wave issues iters x 8 independent v_mfma_f32_32x32x16_bf16 products
 * (32768 flops each), so the launch performs
 * workgroups * waves * iters * 8 * 32768 flops.  sink: caller-owned float
 * [workgroups * waves * 64] (one value per lane, so no product is dead).
 * clocks: NULL or caller-owned uint64 [2 * workgroups]; per workgroup, the
 * shader-clock counter (s_memtime) and the 100 MHz constant clock
 * (s_memrealtime) elapsed over its loop.  FA_ERR_ARG for null sink, sizes
 * < 1 or waves not 4/8; FA_ERR_ALIGN for unaligned pointers.
 *
 * fa_ceiling_copy: copies `bytes` (a multiple of 16, > 0) from src to dst
 * with 16-byte accesses over a fixed grid (8 workgroups per CU); HBM traffic
 * 2 * bytes.  fa_ceiling_read: reads `bytes` once and writes
 * fa_ceiling_read_sink_bytes() bytes of per-lane results to sink.  Both
 * return FA_ERR_ARG / FA_ERR_ALIGN like the attention entry points.
 */
int fa_ceiling_mfma(float* sink, unsigned long long* clocks, int workgroups, int waves, int iters, void* stream);
int fa_ceiling_copy(const void* src, void* dst, size_t bytes, void* stream);
int fa_ceiling_read(const void* src, size_t bytes, void* sink, void* stream);
size_t fa_ceiling_read_sink_bytes(void);

/*
 * fa_ceiling_valu: the issue cost of the softmax's two kinds of vector
 * instruction, one wavefront on one SIMD, timed with the shader clock.  Per
 * loop iteration mode 0 issues 32 v_exp_f32 (each after a v_mul_f32) on 8
 * independent chains, mode 1 issues 96 v_fma_f32 on 24 independent chains,
 * mode 2 issues both sets.  cycles: caller-owned uint64 [1] (8-byte
 * aligned), the shader-clock cycles (s_memtime) of iters iterations.  sink:
 * caller-owned float [64] (16-byte aligned).  FA_ERR_ARG for a bad mode,
 * iters < 1 or a null pointer.
 */
int fa_ceiling_valu(int mode, float* sink, unsigned long long* cycles, int iters, void* stream);

/*
 * fa_ceiling_mix: the 16-bit forward's inner step without HBM traffic, to
 * show what its mix of instructions sustains on the matrix cores.
 * workgroups x 512 threads (eight waves, two per SIMD, as the forward); per
 * wave iters x 2 steps of 8 slots, a slot being one 32x32x16 bf16 score
 * product (a dependent chain), the weights of two keys (fma, exp2, bf16
 * pack, add) and one 32x32x16 PV product (four accumulators).  Mode 0:
 * operands from registers; mode 1: each slot's A operands read from LDS as
 * the forward reads them (a 16-byte row read, two transposing 8-byte
 * reads), three slots ahead; mode 2: mode 1 plus a workgroup barrier every
 * two steps.  One launch performs workgroups * 8 * iters * 32 * 32768
 * matrix flops.  sink: caller-owned float [workgroups * 512] (16-byte
 * aligned), written so no product is dead.  clocks: null, or caller-owned
 * uint64 [2 * workgroups] (16-byte aligned) that receives per workgroup the
 * shader-clock (s_memtime) and 100 MHz constant-clock (s_memrealtime)
 * ticks of its loop, whose ratio gives the clock the chip held.
 * FA_ERR_ARG for a bad mode, workgroups or iters < 1, or a null sink.
 */
int fa_ceiling_mix(int mode, float* sink, unsigned long long* clocks, int workgroups, int iters,
                   void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
