// Launch descriptors passed from the C-ABI layer to the kernels.
#pragma once
#include <hip/hip_runtime.h>

namespace fa {

// One forward (prefill) call.  Tensors are contiguous [B,H,T,d].
struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;      // may be null
  int B, Hq, Hkv, Tq, Tk;
  int g;           // Hq / Hkv: query heads per kv head
  int groups;      // g / hg: workgroups that share one kv head along x
  float c;         // |scale| * log2(e), the factor that turns scores into base-2 exponents
  int negate_q;    // scale < 0: queries are sign-flipped on load, c uses |scale|
};

// One decode call.  q,o: [B,Hq,d]; caches: [B,Hkv,Tk_max,d].
struct DecodeParams {
  const void* q;
  const void* kcache;
  const void* vcache;
  const int* seqlens;
  void* o;
  float* part_m;   // [B, Hq, S] running max (base-2 scaled), -inf for empty pieces
  float* part_l;   // [B, Hq, S] sum of 2^(s*c - m)
  float* part_o;   // [B, Hq, S, d] unnormalised weighted value sums
  int B, Hq, Hkv, Tk_max;
  int g;
  int splits;
  float c;         // log2(e) / sqrt(d)
};

hipError_t launch_fwd_bf16(const FwdParams& p, int d, bool causal, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdParams& p, int d, bool causal, hipStream_t stream);
hipError_t launch_decode(const DecodeParams& p, int d, hipStream_t stream);

// Key granularity of decode pieces: a piece covers a multiple of this many keys.
constexpr int kDecodeTile = 64;

}  // namespace fa
