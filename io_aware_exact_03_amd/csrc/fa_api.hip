// fa_api.hip -- the C ABI declared in include/fa.h: argument validation on the
// host (before any HIP call), kernel dispatch, error mapping.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "../../include/fa.h"
#include "fa_kernels.hpp"
#include "fa_plan.hpp"

namespace {

thread_local int g_last_hip_error = 0;

int hip_status(hipError_t e) {
  if (e == hipSuccess) return FA_OK;
  g_last_hip_error = (int)e;
  return FA_ERR_HIP;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int elem_bytes(int dtype) { return dtype == FA_F32 ? 4 : 2; }

// Shape checks shared by every entry point.  Sizes must fit the kernels'
// index arithmetic: int for row/column indices, 64-bit for element offsets.
int check_shape(int B, int H, int N, int d, int dtype, int causal, float scale) {
  if (B < 1 || H < 1 || N < 1) return FA_ERR_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_ARG;
  if (!isfinite(scale)) return FA_ERR_ARG;
  if (dtype != FA_F32 && dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  const long long bh = (long long)B * H;
  if (bh > 0x7fffffffLL) return FA_ERR_ARG;
  // bytes of one [B,H,N,d] tensor must fit in int64 (and then some)
  const long double bytes = (long double)bh * N * d * elem_bytes(dtype);
  if (bytes > (long double)(1LL << 62)) return FA_ERR_ARG;
  // the kernels address one (batch, head) slice with 32-bit buffer offsets
  if ((long long)N * d * elem_bytes(dtype) >= (1LL << 31)) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

}  // namespace

namespace fa {
void record_hip_error(int e) { g_last_hip_error = e; }
}  // namespace fa

// The allocation-free decode keeps the pieces of cut units here: one fixed
// buffer per device, present for the life of the process.  In host code the
// array's name is only a stand-in for the symbol; its device address comes
// from hipGetSymbolAddress, looked up once per device with that device
// current, and only that address is ever passed to kernels.
static __device__ __align__(256) unsigned char scratch[FA_DECODE_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_of_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) return FA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e);
    if (p == nullptr) return FA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return FA_OK;
}
}  // namespace

extern "C" {

const char* fa_strerror(int status) {
  switch (status) {
    case FA_OK: return "success";
    case FA_ERR_ARG: return "invalid argument (null pointer, bad size or flag, non-finite scale, or overflow)";
    case FA_ERR_UNSUPPORTED: return "unsupported head dimension or dtype";
    case FA_ERR_ALIGN: return "pointer not 16-byte aligned";
    case FA_ERR_HIP: return "HIP launch error (see fa_last_hip_error)";
    case FA_ERR_SCRATCH: return "request needs more than the library's fixed allocation-free scratch buffer holds";
    default: return "unknown fa_status";
  }
}

int fa_last_hip_error(void) { return g_last_hip_error; }

int fa_causal_stages(int row0, int row_end, int bn, int n, int* s1_end, int* s2_end) {
  if (!s1_end || !s2_end || bn < 1 || row0 < 0 || row_end <= row0 || row_end > n) return FA_ERR_ARG;
  fa::causal_stages(row0, row_end, bn, s1_end, s2_end);
  return FA_OK;
}

int fa_fwd_tile(int d, int dtype, int* bm, int* bn, int* waves) {
  if (!bm || !bn || !waves) return FA_ERR_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (dtype != FA_F32 && dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  const fa::FwdTile t = fa::fwd_tile(d, dtype == FA_F32);
  *bm = t.bm;
  *bn = t.bn;
  *waves = t.waves;
  return FA_OK;
}

size_t fa_naive_workspace_bytes(int B, int H, int N, int dtype) {
  if (B < 1 || H < 1 || N < 1) return 0;
  if (dtype != FA_F32 && dtype != FA_F16 && dtype != FA_BF16) return 0;
  const long double b = (long double)B * H * N * N * (dtype == FA_F32 ? 4 : 2);
  if (b > (long double)(1LL << 62)) return 0;
  return (size_t)B * H * (size_t)N * (size_t)N * (dtype == FA_F32 ? 4 : 2);
}

int fa_fwd_chunk(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Hkv,
                 int Nq, int Nk, int d, float scale, int causal, int dtype, void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_ARG;
  int st = check_shape(B, H, Nq, d, dtype, causal, scale);
  if (st != FA_OK) return st;
  st = check_shape(B, H, Nk, d, dtype, causal, scale);
  if (st != FA_OK) return st;
  if (Hkv < 1 || Hkv > H || H % Hkv != 0) return FA_ERR_ARG;
  if (causal && Nq > Nk) return FA_ERR_ARG;
  if (Nq != Nk && dtype == FA_F32) return FA_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse)) return FA_ERR_ALIGN;
  fa::FwdArgs a;
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
  a.BH = B * H; a.G = H / Hkv; a.N = Nq; a.Nk = Nk; a.d = d; a.dtype = dtype; a.causal = causal != 0;
  a.qk_scale = fabsf(scale) * fa::kLog2eHost;
  a.neg = scale < 0.f;
  a.stream = static_cast<hipStream_t>(stream);
  return hip_status(fa::launch_fwd(a));
}

int fa_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Hkv, int N,
               int d, float scale, int causal, int dtype, void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_ARG;
  const int st = check_shape(B, H, N, d, dtype, causal, scale);
  if (st != FA_OK) return st;
  if (Hkv < 1 || Hkv > H || H % Hkv != 0) return FA_ERR_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse)) return FA_ERR_ALIGN;
  fa::FwdArgs a;
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
  a.BH = B * H; a.G = H / Hkv; a.N = N; a.Nk = N; a.d = d; a.dtype = dtype; a.causal = causal != 0;
  a.qk_scale = fabsf(scale) * fa::kLog2eHost;
  a.neg = scale < 0.f;
  a.stream = static_cast<hipStream_t>(stream);
  return hip_status(fa::launch_fwd(a));
}

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
           float scale, int causal, int dtype, void* stream) {
  return fa_fwd_gqa(q, k, v, o, lse, B, H, H, N, d, scale, causal, dtype, stream);
}

static int bwd_common(int stage, const void* q, const void* k, const void* v, const void* o, const void* dout,
                      const float* lse, float* delta_ws, float* dq, float* dk, float* dv, int B, int H, int Hkv,
                      int N, int d, float scale, int causal, int dtype, void* stream) {
  if (stage < 0 || stage > 3) return FA_ERR_ARG;
  if (!q || !k || !v || !o || !dout || !lse || !delta_ws || !dq || !dk || !dv) return FA_ERR_ARG;
  const int st = check_shape(B, H, N, d, dtype, causal, scale);
  if (st != FA_OK) return st;
  if (Hkv < 1 || Hkv > H || H % Hkv != 0) return FA_ERR_ARG;
  if (dtype == FA_F32) return FA_ERR_UNSUPPORTED;  // the backward kernels are 16-bit MFMA only
  // dQ, dK, dV are fp32: one head of them is twice the bytes of a 16-bit
  // head, and the kernels' 32-bit buffer offsets also cover the padded rows
  // of the last block (up to 255 past N) before the range check drops them.
  if ((long long)(N + 255) * d * 4 >= (1LL << 31)) return FA_ERR_UNSUPPORTED;
  const void* ptrs[] = {q, k, v, o, dout, lse, delta_ws, dq, dk, dv};
  for (const void* p : ptrs)
    if (!aligned16(p)) return FA_ERR_ALIGN;
  fa::BwdArgs a;
  a.q = q; a.k = k; a.v = v; a.o = o; a.dout = dout; a.lse = lse;
  a.delta = delta_ws; a.dq = dq; a.dk = dk; a.dv = dv;
  a.BH = B * H; a.G = H / Hkv; a.N = N; a.d = d; a.dtype = dtype; a.causal = causal != 0;
  a.scale = scale;
  a.stream = static_cast<hipStream_t>(stream);
  return hip_status(fa::launch_bwd(a, stage));
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
           float* delta_ws, float* dq, float* dk, float* dv, int B, int H, int N, int d, float scale, int causal,
           int dtype, void* stream) {
  return bwd_common(0, q, k, v, o, dout, lse, delta_ws, dq, dk, dv, B, H, H, N, d, scale, causal, dtype, stream);
}

int fa_bwd_gqa(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
               float* delta_ws, float* dq, float* dk, float* dv, int B, int H, int Hkv, int N, int d, float scale,
               int causal, int dtype, void* stream) {
  return bwd_common(0, q, k, v, o, dout, lse, delta_ws, dq, dk, dv, B, H, Hkv, N, d, scale, causal, dtype, stream);
}

int fa_bwd_stage(int stage, const void* q, const void* k, const void* v, const void* o, const void* dout,
                 const float* lse, float* delta_ws, float* dq, float* dk, float* dv, int B, int H, int N, int d,
                 float scale, int causal, int dtype, void* stream) {
  if (stage < 1) return FA_ERR_ARG;
  return bwd_common(stage, q, k, v, o, dout, lse, delta_ws, dq, dk, dv, B, H, H, N, d, scale, causal, dtype,
                    stream);
}

int fa_kv_head(int bh, int H, int Hkv) {
  if (bh < 0 || H < 1 || Hkv < 1 || Hkv > H || H % Hkv != 0) return -1;
  return fa::kv_head_of(bh, H / Hkv);
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static long long decode_units(int B, int H, int Hkv) {
  return (long long)B * Hkv * fa::decode_query_blocks(H / Hkv);
}

size_t fa_decode_workspace_bytes(int B, int H, int Hkv, int d, int n_parts) {
  if (B < 1 || H < 1 || Hkv < 1 || Hkv > H || H % Hkv != 0 || (d != 64 && d != 128)) return 0;
  if (n_parts < 1 || n_parts > fa::kDecodeMaxParts) return 0;
  if (n_parts == 1) return 0;
  const size_t slots = (size_t)n_parts + (size_t)decode_units(B, H, Hkv);
  return align256(slots * 32 * d * 4) + align256(slots * 32 * 4);
}

int fa_decode_plan(int B, int H, int Hkv, int Nkv, int d, int* n_parts) {
  if (!n_parts) return FA_ERR_ARG;
  if (B < 1 || H < 1 || Hkv < 1 || Hkv > H || H % Hkv != 0 || Nkv < 1) return FA_ERR_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_status(e);
  // One part per CU (a part's LDS ring fills a CU), never more parts than
  // tiles at full length.
  const long long tiles = decode_units(B, H, Hkv) * fa::decode_tiles(Nkv);
  long long P = cus < 1 ? 1 : cus;
  if (P > tiles) P = tiles;
  if (P > fa::kDecodeMaxParts) P = fa::kDecodeMaxParts;
  *n_parts = (int)(P < 1 ? 1 : P);
  return FA_OK;
}

// Host checks shared by fa_decode and fa_decode_noalloc (no HIP call).
static int decode_check(const void* q, const void* k_cache, const void* v_cache, const int* kv_lens, void* o,
                        float* lse, int B, int H, int Hkv, int Nkv, int d, float scale, int n_parts, int dtype) {
  if (!q || !k_cache || !v_cache || !o || !lse) return FA_ERR_ARG;
  if (Hkv < 1 || H < 1 || Hkv > H || H % Hkv != 0) return FA_ERR_ARG;
  if (n_parts < 1 || n_parts > fa::kDecodeMaxParts) return FA_ERR_ARG;
  const int st = check_shape(B, H, Nkv, d, dtype, 0, scale);
  if (st != FA_OK) return st;
  if (dtype == FA_F32) return FA_ERR_UNSUPPORTED;
  if (decode_units(B, H, Hkv) * fa::decode_tiles(Nkv) >= (1LL << 31) ||
      (decode_units(B, H, Hkv) + n_parts) * 32 >= (1LL << 31))
    return FA_ERR_UNSUPPORTED;
  const void* ptrs[] = {q, k_cache, v_cache, o, lse};
  for (const void* p : ptrs)
    if (!aligned16(p)) return FA_ERR_ALIGN;
  if (kv_lens && ((uintptr_t)kv_lens & 3u)) return FA_ERR_ALIGN;
  return FA_OK;
}

// Launch with a validated workspace (ignored for n_parts = 1).
static int decode_launch(const void* q, const void* k_cache, const void* v_cache, const int* kv_lens, void* o,
                         float* lse, void* ws, int B, int H, int Hkv, int Nkv, int d, float scale, int n_parts,
                         int dtype, void* stream) {
  fa::DecodeArgs a;
  a.q = q; a.k = k_cache; a.v = v_cache; a.kv_lens = kv_lens; a.o = o; a.lse = lse;
  const size_t slots = (size_t)n_parts + (size_t)decode_units(B, H, Hkv);
  a.opart = n_parts > 1 ? static_cast<float*>(ws) : nullptr;
  a.lpart = n_parts > 1 ? reinterpret_cast<float*>(static_cast<char*>(ws) + align256(slots * 32 * d * 4)) : nullptr;
  a.B = B; a.H = H; a.G = H / Hkv; a.Nkv = Nkv; a.d = d; a.dtype = dtype;
  a.parts = n_parts;
  a.scale = scale;
  a.stream = static_cast<hipStream_t>(stream);
  return hip_status(fa::launch_decode(a));
}

int fa_decode(const void* q, const void* k_cache, const void* v_cache, const int* kv_lens, void* o, float* lse,
              void* ws, size_t ws_bytes, int B, int H, int Hkv, int Nkv, int d, float scale, int n_parts,
              int dtype, void* stream) {
  if (!q || !k_cache || !v_cache || !o || !lse) return FA_ERR_ARG;
  if (Hkv < 1 || H < 1 || Hkv > H || H % Hkv != 0) return FA_ERR_ARG;
  if (n_parts < 1 || n_parts > fa::kDecodeMaxParts) return FA_ERR_ARG;
  const int st = check_shape(B, H, Nkv, d, dtype, 0, scale);
  if (st != FA_OK) return st;
  if (dtype == FA_F32) return FA_ERR_UNSUPPORTED;
  // tile and slot counts are int in the kernels
  if (decode_units(B, H, Hkv) * fa::decode_tiles(Nkv) >= (1LL << 31) ||
      (decode_units(B, H, Hkv) + n_parts) * 32 >= (1LL << 31))
    return FA_ERR_UNSUPPORTED;
  const size_t need = fa_decode_workspace_bytes(B, H, Hkv, d, n_parts);
  if (n_parts > 1 && (!ws || ws_bytes < need)) return FA_ERR_ARG;
  const void* ptrs[] = {q, k_cache, v_cache, o, lse};
  for (const void* p : ptrs)
    if (!aligned16(p)) return FA_ERR_ALIGN;
  if (kv_lens && ((uintptr_t)kv_lens & 3u)) return FA_ERR_ALIGN;
  if (n_parts > 1 && !aligned16(ws)) return FA_ERR_ALIGN;
  return decode_launch(q, k_cache, v_cache, kv_lens, o, lse, ws, B, H, Hkv, Nkv, d, scale, n_parts, dtype, stream);
}

int fa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, const int* kv_lens, void* o,
                      float* lse, int B, int H, int Hkv, int Nkv, int d, float scale, int n_parts, int dtype,
                      void* stream) {
  const int st = decode_check(q, k_cache, v_cache, kv_lens, o, lse, B, H, Hkv, Nkv, d, scale, n_parts, dtype);
  if (st != FA_OK) return st;
  if (fa_decode_workspace_bytes(B, H, Hkv, d, n_parts) > FA_DECODE_SCRATCH_BYTES) return FA_ERR_SCRATCH;
  void* ws = nullptr;
  if (n_parts > 1) {
    const int e = scratch_of_current_device(&ws);
    if (e != FA_OK) return e;
  }
  return decode_launch(q, k_cache, v_cache, kv_lens, o, lse, ws, B, H, Hkv, Nkv, d, scale, n_parts, dtype, stream);
}

int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Hkv, int N,
               int d, float scale, float q_descale, float k_descale, float v_descale, int causal, void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_ARG;
  const int st = check_shape(B, H, N, d, FA_BF16, causal, scale);  // bf16 output; 1-byte inputs are smaller
  if (st != FA_OK) return st;
  if (Hkv < 1 || Hkv > H || H % Hkv != 0) return FA_ERR_ARG;
  if (!isfinite(q_descale) || !isfinite(k_descale) || !isfinite(v_descale)) return FA_ERR_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse)) return FA_ERR_ALIGN;
  fa::Fp8Args a;
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
  a.BH = B * H; a.G = H / Hkv; a.N = N; a.d = d; a.causal = causal != 0;
  a.scale = scale; a.q_descale = q_descale; a.k_descale = k_descale; a.v_descale = v_descale;
  a.stream = static_cast<hipStream_t>(stream);
  return hip_status(fa::launch_fwd_fp8(a));
}

size_t fa_fa1_workspace_bytes(int B, int H, int N, int d) {
  if (B < 1 || H < 1 || N < 1 || (d != 64 && d != 128)) return 0;
  const size_t rows = (size_t)B * H * N;
  return align256(rows * d * 4) + 2 * align256(rows * 4);
}

int fa_fwd_fa1(const void* q, const void* k, const void* v, void* o, float* lse, void* ws, size_t ws_bytes, int B,
               int H, int N, int d, float scale, int causal, int dtype, void* stream) {
  if (!q || !k || !v || !o || !lse || !ws) return FA_ERR_ARG;
  const int st = check_shape(B, H, N, d, dtype, causal, scale);
  if (st != FA_OK) return st;
  if (dtype == FA_F32) return FA_ERR_UNSUPPORTED;
  if (ws_bytes < fa_fa1_workspace_bytes(B, H, N, d)) return FA_ERR_ARG;
  const void* ptrs[] = {q, k, v, o, lse, ws};
  for (const void* p : ptrs)
    if (!aligned16(p)) return FA_ERR_ALIGN;
  fa::Fa1Args a;
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
  const size_t rows = (size_t)B * H * N;
  a.ows = static_cast<float*>(ws);
  a.mws = reinterpret_cast<float*>(static_cast<char*>(ws) + align256(rows * d * 4));
  a.lws = reinterpret_cast<float*>(static_cast<char*>(ws) + align256(rows * d * 4) + align256(rows * 4));
  a.BH = B * H; a.N = N; a.d = d; a.dtype = dtype; a.causal = causal != 0; a.scale = scale;
  a.stream = static_cast<hipStream_t>(stream);
  return hip_status(fa::launch_fa1(a));
}

int fa_naive_fwd(const void* q, const void* k, const void* v, void* o, float* lse, void* s_ws, void* p_ws, int B,
                 int H, int N, int d, float scale, int causal, int dtype, void* stream) {
  if (!q || !k || !v || !o || !lse || !s_ws || !p_ws) return FA_ERR_ARG;
  const int st = check_shape(B, H, N, d, dtype, causal, scale);
  if (st != FA_OK) return st;
  if (fa_naive_workspace_bytes(B, H, N, dtype) == 0) return FA_ERR_ARG;
  const void* ptrs[] = {q, k, v, o, lse, s_ws, p_ws};
  for (const void* p : ptrs)
    if (!aligned16(p)) return FA_ERR_ALIGN;
  fa::NaiveArgs a;
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse; a.s = s_ws; a.p = p_ws;
  a.BH = B * H; a.N = N; a.d = d; a.dtype = dtype; a.causal = causal != 0; a.scale = scale;
  a.stream = static_cast<hipStream_t>(stream);
  return hip_status(fa::launch_naive(a));
}

}  // extern "C"
