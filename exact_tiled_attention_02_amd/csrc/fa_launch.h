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
  int pair;        // causal: workgroups pair mirrored light/heavy half-tiles
  int causal_off;  // causal: row i sees key j iff j <= i + causal_off (0 or Tk - Tq)
  // 8-bit inputs only (E4M3 codes): q row scales [B,Hq,Tq], k and v scales
  // per (batch, kv head) [B,Hkv].
  const float* qscale;
  const float* kscale;
  const float* vscale;
};

// One decode call.  q,o: [B,Hq,d]; caches: [B,Hkv,Tk_max,d].
//
// The valid keys of all (sequence, kv head, head group) segments, laid end to
// end in that order, form one key space of sum_b n_b * Hkv * groups keys.
// Workgroup w takes the contiguous range [w * per, (w + 1) * per) of it and
// writes one partial (m, l, o) for every segment the range touches, into slot
// w + segment.  The merge kernel combines the slots of each segment.
struct DecodeParams {
  const void* q;
  const void* kcache;   // bf16, or 8-bit codes (one byte per element)
  const void* vcache;
  const float* kscale;  // 8-bit cache: one scale per row, [B, Hkv, Tk_max]; else null
  const float* vscale;
  const int* seqlens;
  void* o;
  long long* cum;  // [B + 1] exclusive prefix sums of the clamped sequence lengths
  float* part_m;   // [slots, hpw] running max (base-2 scaled)
  float* part_l;   // [slots, hpw] sum of 2^(s*c - m)
  float* part_o;   // [slots, hpw, d] unnormalised weighted value sums
  int B, Hq, Hkv, Tk_max;
  int g;           // Hq / Hkv
  int hpw;         // query heads per workgroup (a divisor of g)
  int W;           // workgroups sharing the key space
  float c;         // log2(e) / sqrt(d)
};

// One backward call.  q, o, dout, dq: [B,Hq,Tq,d]; k, v, dk, dv: [B,Hkv,Tk,d];
// all bf16.  l2 and delta are library workspace, [B*Hq, Tqp] fp32 each.
struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;  // [B,Hq,Tq] natural-log row log-sum-exp of the forward
  void* dq;
  void* dk;
  void* dv;
  float* l2;         // lse * log2(e) per query row; 0 on padding rows
  float* delta;      // dO_i . O_i per query row; 0 on padding rows
  int B, Hq, Hkv, Tq, Tk;
  int causal_off;    // causal: row i sees key j iff j <= i + causal_off
  int Tqp;           // Tq rounded up to a multiple of kBwdRowPad
  int g;             // Hq / Hkv
  float c;           // scale * log2(e) (signed)
  float scale;
  // Small causal grids: each key block's (query head, query tile) items are
  // split into kparts contiguous parts, one workgroup each, which write fp32
  // partial dK and dV [kparts, B*Hkv, Tk, d] that a merge kernel sums in
  // part order.  kparts = 1: dK and dV are written directly.
  int kparts;
  float* part_dk;
  float* part_dv;
};

// Rows of each (batch, head) plane of the backward workspace are padded to a
// multiple of this, so that whole query tiles of it can be read unchecked.
constexpr int kBwdRowPad = 256;

// Compute units of the current device (cached per device; 256 if the query
// fails).
int compute_units();

// Item parts per dK/dV key block for a backward call (see BwdParams::kparts).
int bwd_key_parts(int B, int Hkv, int Tk, bool causal);

hipError_t launch_fwd_bf16(const FwdParams& p, int d, bool causal, hipStream_t stream);
hipError_t launch_bwd(const BwdParams& p, int d, bool causal, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdParams& p, int d, bool causal, hipStream_t stream);
hipError_t launch_fwd_fp8(const FwdParams& p, int d, bool causal, hipStream_t stream);
// Element type of a decode KV cache.
enum KvKind : int {
  kKvBf16 = 0,   // bf16 elements
  kKvE4m3 = 1,   // E4M3 codes with one fp32 scale per row
  kKvInt8 = 2,   // two's-complement int8 codes with one fp32 scale per row
};
hipError_t launch_decode(const DecodeParams& p, int d, int kv, hipStream_t stream);
// Workgroups that the decode kernel for (d, hpw, cache type) keeps resident
// on the current device at once; 0 if the device cannot be queried.
int decode_resident_workgroups(int d, int hpw, int kv);
// Streams `bytes` (a multiple of 16) from src once, XOR-folding them into
// *sink (which the caller zeroes).
hipError_t launch_read_probe(const void* src, size_t bytes, unsigned* sink, hipStream_t stream);

// Query heads one decode workgroup serves (a divisor of the group size g).
inline int decode_heads_per_workgroup(int g) {
  return (g % 8 == 0) ? 8 : (g % 4 == 0) ? 4 : (g % 2 == 0) ? 2 : 1;
}

// Partial slots a decode call with W workgroups needs.
inline size_t decode_slots(int W, int B, int Hkv, int g, int hpw) {
  return (size_t)W + (size_t)B * Hkv * (g / hpw);
}

// Keys per workgroup range: ceil(total / W) rounded up to 16.  The decode
// and merge kernels both evaluate exactly this.
__host__ __device__ inline long long decode_range(long long total, int W) {
  const long long per = (total + W - 1) / W;
  return ((per + 15) / 16) * 16;
}

}  // namespace fa
