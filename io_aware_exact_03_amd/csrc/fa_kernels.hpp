// fa_kernels.hpp -- internal launch interface between the C ABI (fa_api.hip)
// and the kernel translation units.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace fa {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int BH;          // batch * query heads
  int G;           // query heads per K/V head (1: one K/V head per query head); K/V head = bh / G
  int N;           // queries per head
  int Nk;          // keys per head (N for square attention)
  int d;           // 64 or 128
  int dtype;       // 0 f32, 1 f16, 2 bf16
  bool causal;     // query i sees keys j <= i + (Nk - N)
  float qk_scale;  // |scale| * log2(e)
  bool neg;        // scale < 0: the kernels negate Q on load
  hipStream_t stream;
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  float* delta;
  float* dq;
  float* dk;
  float* dv;
  int BH;          // batch * query heads (dK, dV: batch * K/V heads = BH / G)
  int G;           // query heads per K/V head
  int N;
  int d;
  int dtype;
  bool causal;
  float scale;     // signed
  hipStream_t stream;
};

struct NaiveArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  void* s;
  void* p;
  int BH;
  int N;
  int d;
  int dtype;
  bool causal;
  float scale;
  hipStream_t stream;
};

struct DecodeArgs {
  const void* q;        // [B, H, d]
  const void* k;        // [B, Hkv, Nkv, d]
  const void* v;
  const int* kv_lens;   // [B] on the device, or null (all Nkv)
  void* o;              // [B, H, d]
  float* lse;           // [B, H]
  float* opart;         // [parts + units][32][d] segment outputs (parts > 1)
  float* lpart;         // [parts + units][32] segment LSEs (parts > 1)
  int B, H, G, Nkv, d, dtype;
  int parts;            // workgroups sharing the key tiles
  float scale;
  hipStream_t stream;
};

struct Fa1Args {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  float* ows;      // [BH, N, d] running O (fp32)
  float* mws;      // [BH, N] running max, log2 units
  float* lws;      // [BH, N] running sum
  int BH, N, d, dtype;
  bool causal;
  float scale;
  hipStream_t stream;
};

struct Fp8Args {
  const void* q;   // E4M3 codes [BH, N, d]
  const void* k;   // [BH / G, N, d]
  const void* v;
  void* o;         // bf16 [BH, N, d]
  float* lse;      // [BH, N]
  int BH, G, N, d;
  bool causal;
  float scale, q_descale, k_descale, v_descale;
  hipStream_t stream;
};

// Keep a failed launch's hipError_t for fa_last_hip_error() (calling thread).
void record_hip_error(int e);

hipError_t launch_fwd(const FwdArgs& a);
// stage 0 = all three launches in order; 1 = Delta, 2 = dK/dV, 3 = dQ.
hipError_t launch_bwd(const BwdArgs& a, int stage);
hipError_t launch_naive(const NaiveArgs& a);
hipError_t launch_decode(const DecodeArgs& a);
hipError_t launch_fa1(const Fa1Args& a);
hipError_t launch_fwd_fp8(const Fp8Args& a);

}  // namespace fa
