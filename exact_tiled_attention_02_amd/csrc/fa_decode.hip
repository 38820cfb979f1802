// Split-KV flash-decoding kernels for gfx950: one query token per sequence
// attending over a long KV cache.
//
// Sources (web pages; sections named as headed there):
//   [NOTE]  "Atencja od strony jądra: FlashAttention, softmax online i
//           połączona dekwantyzacja" (trefon.com), section "Prefill i
//           dekodowanie to różne problemy": decode is a stream over the
//           cache at memory speed; GQA lets one K/V load serve the g query
//           heads of its group; flash-decoding cuts the key sequence into
//           pieces whose partial (m, l, o) are merged by the rescale rule.
//   [BOOK5] "Глава 5. Операторы и среда выполнения" (bojieli.github.io),
//           section 5.3.3 (Example 5-6: merging block results needs the
//           block statistics m and l, not only normalised outputs) and
//           section 5.2.4 (a fixed merge order keeps split results
//           reproducible).
//
// This work is bound by HBM bandwidth (about 4 FLOP per cache byte with a
// group of 4; 8 with an 8-bit cache): the design goal is to stream every
// cache byte exactly once with coalesced loads and enough of them in
// flight, while spending as few vector instructions per key as possible so
// that the arithmetic hides under the memory time.
//
// W workgroups (as many as the device keeps resident) each take an equal
// contiguous range of the key space of all (sequence, kv head group)
// segments laid end to end, so every workgroup carries the same number of
// keys whatever the sequence lengths; a range that crosses segments emits
// one partial per segment it touches.  Within a range (packed-dot loop):
//  * 4 wavefronts march through the range's keys.  A key row is read by LPR
//    lanes (8 at d = 128 with up to 4 heads per workgroup, else 16 at
//    d = 128 and 8 at d = 64), each lane holding EPL = d / LPR elements, so
//    one load step of a wavefront covers 64 / LPR consecutive keys and every
//    16-byte load instruction reads whole 128-byte lines.
//  * Scores of the HPW query heads: each lane forms a partial dot product
//    over its elements (packed bf16 dot instructions, fp32 sums), then a
//    reduction across the LPR lanes of the row (DPP quad permutes and
//    mirrors) leaves the full score in every lane of the row.
//  * Every key row keeps its own running max, sum and accumulator per head,
//    so the online softmax needs no cross-lane traffic inside the loop; the
//    accumulator is rescaled only when some row's max grew.
//  * P.V pairs two keys of the same lane: probabilities are rounded to bf16
//    and packed (p_a, p_b), the value elements of the two keys are packed
//    the same way with byte permutes, and one packed dot instruction adds
//    p_a v_a + p_b v_b to an fp32 accumulator.  The row sum l is formed from
//    the unrounded fp32 probabilities.
//  * At the end the rows of a wavefront are merged with the rescale rule
//    (lane shuffles), then the 4 wavefronts through LDS, and the range's
//    (m, l, o) for the segment is written to the workspace.
// An 8-bit cache (E4M3 or int8 codes, one fp32 scale per row: [NOTE]'s fused
// dequantisation, the cache expanded inside the tile load) widens the codes
// exactly to bf16 in registers right after the load.  At d = 128 with 4 or 8
// heads per workgroup it runs a matrix-core loop (decode_range_mfma): the
// scores and P.V on the 16x16x32 bf16 matrix core, V^T through LDS;
// otherwise the packed-dot loop above.
// Merge kernel, one wavefront per (sequence, query head): fixed-order pass
// over the pieces, O = sum 2^(m_s - M) o_s / sum 2^(m_s - M) l_s.
#include "fa_device.h"
#include "fa_lds.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kDecThreads = 256;
constexpr int kDecKU = 4;   // load steps per wavefront per iteration (even)

// All-reduce (sum) over aligned groups of 8 lanes: swap neighbours, swap
// pairs, then mirror within each half-row of 8.
__device__ __forceinline__ float group8_sum(float x) {
  x += __builtin_amdgcn_update_dpp(0.f, x, 0xB1, 0xf, 0xf, false);    // quad_perm [1,0,3,2]
  x += __builtin_amdgcn_update_dpp(0.f, x, 0x4E, 0xf, 0xf, false);    // quad_perm [2,3,0,1]
  x += __builtin_amdgcn_update_dpp(0.f, x, 0x141, 0xf, 0xf, false);   // row_half_mirror
  return x;
}
// All-reduce (sum) over aligned groups of 16 lanes (one DPP row).
__device__ __forceinline__ float group16_sum(float x) {
  x = group8_sum(x);
  return x + __builtin_amdgcn_update_dpp(0.f, x, 0x140, 0xf, 0xf, false);   // row_mirror
}

// Combine the values held by the key rows of a wavefront (lanes that differ
// in the bits at or above log2(LPR)).
template <int LPR>
__device__ __forceinline__ float rows_max(float x) {
  if constexpr (LPR == 8) x = fmaxf(x, __builtin_amdgcn_update_dpp(0.f, x, 0x128, 0xf, 0xf, false));
  x = fmaxf(x, __shfl_xor(x, 16, 64));
  return fmaxf(x, __shfl_xor(x, 32, 64));
}
template <int LPR>
__device__ __forceinline__ float rows_sum(float x) {
  if constexpr (LPR == 8) x += __builtin_amdgcn_update_dpp(0.f, x, 0x128, 0xf, 0xf, false);
  x += __shfl_xor(x, 16, 64);
  return x + __shfl_xor(x, 32, 64);
}

// Pack the low (sel 0x05040100) or high (0x07060302) bf16 halves of two
// words: result = (lo-or-hi of a, lo-or-hi of b).
__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}
__device__ __forceinline__ uint32_t bf16_pair_bits(float a, float b) {
  const bf16x2 v = to_bf16x2(a, b);
  uint32_t w;
  __builtin_memcpy(&w, &v, sizeof(w));
  return w;
}

// a.x * b.x + a.y * b.y in fp32 (bf16 pairs).  The three-operand form with
// an inline zero addend starts a dot chain without first zeroing the
// accumulator register, which the two-operand form would need.
__device__ __forceinline__ float dot2_from_zero(bf16x2 a, bf16x2 b) {
  float r;
  asm("v_dot2_f32_bf16 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// Elements held by a lane: EPL = 8 * NV values, vector j (16 bytes) being
// elements [j * d / NV + dl * 8, +8) of the row, dl = lane % LPR.
template <int D, int HPW>
struct DecodeShape {
  static constexpr int EPL = (D == 128 && HPW <= 4) ? 16 : 8;
  static constexpr int LPR = D / EPL;
  static constexpr int RPW = 64 / LPR;   // key rows per load step of a wavefront
  static constexpr int NV = EPL / 8;
};

// Widen 4 E4M3 codes (one word) to two words of bf16 pairs, in order; the
// conversion is exact (every E4M3 value is a bf16 value).
__device__ __forceinline__ u32x2 e4m3x4_to_bf16(uint32_t w) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
  uint32_t lo, hi;
  __builtin_memcpy(&lo, &a, 4);
  __builtin_memcpy(&hi, &b, 4);
  return u32x2{lo, hi};
}
// Widen 8 E4M3 codes (two words) to one 16-byte vector of bf16 pairs.
__device__ __forceinline__ u32x4 e4m3x8_to_bf16(uint32_t w0, uint32_t w1) {
  const u32x2 a = e4m3x4_to_bf16(w0);
  const u32x2 b = e4m3x4_to_bf16(w1);
  return u32x4{a[0], a[1], b[0], b[1]};
}

// Int8 code k (byte k, two's complement) of a word as a float.
__device__ __forceinline__ float int8_at(uint32_t w, int k) {
  return (float)((int32_t)(w << (24 - 8 * k)) >> 24);
}
// Widen 8 int8 codes (two words) to one 16-byte vector of bf16 pairs, in
// order; exact (every integer in [-128, 127] is a bf16 value).
__device__ __forceinline__ u32x4 int8x8_to_bf16(uint32_t w0, uint32_t w1) {
  return u32x4{bf16_pair_bits(int8_at(w0, 0), int8_at(w0, 1)), bf16_pair_bits(int8_at(w0, 2), int8_at(w0, 3)),
               bf16_pair_bits(int8_at(w1, 0), int8_at(w1, 1)), bf16_pair_bits(int8_at(w1, 2), int8_at(w1, 3))};
}
// 8 codes (two words) of an 8-bit cache of kind KV as 8 bf16 values, in order.
template <int KV>
__device__ __forceinline__ u32x4 widen8(uint32_t w0, uint32_t w1) {
  if constexpr (KV == kKvInt8) return int8x8_to_bf16(w0, w1);
  else return e4m3x8_to_bf16(w0, w1);
}
// Codes k = 0..3 of the words wa and wb (two keys) as (v_a, v_b) bf16 pairs.
// E4M3: byte-interleave first (a0 b0 a1 b1, a2 b2 a3 b3), so that each
// widening gives one pair directly.
template <int KV>
__device__ __forceinline__ void pairs4(uint32_t wa, uint32_t wb, bf16x2 (&v2)[4]) {
  if constexpr (KV == kKvInt8) {
#pragma unroll
    for (int k = 0; k < 4; ++k) v2[k] = to_bf16x2(int8_at(wa, k), int8_at(wb, k));
  } else {
    const uint32_t x0 = __builtin_amdgcn_perm(wb, wa, 0x05010400u);
    const uint32_t x1 = __builtin_amdgcn_perm(wb, wa, 0x07030602u);
    v2[0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x0, 1.0f, false);
    v2[1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x0, 1.0f, true);
    v2[2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x1, 1.0f, false);
    v2[3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x1, 1.0f, true);
  }
}

// Attention of the HPW query heads hq0.. over keys [lo, hi) of kv head
// (b, kvh); the partial (m, l, o) goes to `slot`.  Every thread of the
// workgroup calls this with the same arguments.  FP8: the cache holds E4M3
// codes with one fp32 scale per row; a lane loads its EPL codes with one
// load, widens them to bf16 in registers and the rest of the loop is the
// bf16 one, with the K row scale applied to the row's score and the V row
// scale to its probability (after the row sum l is formed).
template <int D, int HPW, int KU, int KV>
__device__ __forceinline__ void decode_range_keys(const DecodeParams& p, int b, int kvh, int hq0,
                                                  int lo, int hi, size_t slot, float (*red_m)[HPW],
                                                  float (*red_l)[HPW], float (*red_o)[HPW][D]) {
  typedef DecodeShape<D, HPW> S;
  constexpr int EPL = S::EPL, LPR = S::LPR, RPW = S::RPW, NV = S::NV;
  constexpr bool FP8 = KV != kKvBf16;   // an 8-bit cache (E4M3 or int8 codes)
  constexpr int STEP = 4 * RPW * KU;   // keys per workgroup iteration
  static_assert(KU % 2 == 0, "keys are paired within a lane");
  // The range is the same for the whole workgroup; keep it in scalar
  // registers so that the buffer resources built from it are scalar too.
  b = __builtin_amdgcn_readfirstlane(b);
  kvh = __builtin_amdgcn_readfirstlane(kvh);
  hq0 = __builtin_amdgcn_readfirstlane(hq0);
  lo = __builtin_amdgcn_readfirstlane(lo);
  hi = __builtin_amdgcn_readfirstlane(hi);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int row = lane / LPR;
  const int dl = lane % LPR;
  const float c = p.c;

  // Element offset of vector j of this lane inside a row (FP8: the lane's
  // EPL elements are contiguous so that one load fetches them).
  auto eoff = [&](int j) { return FP8 ? dl * EPL + 8 * j : j * (D / NV) + dl * 8; };

  u32x4 qv[HPW][NV];
#pragma unroll
  for (int h = 0; h < HPW; ++h)
#pragma unroll
    for (int j = 0; j < NV; ++j)
      qv[h][j] = *(const u32x4*)((const bf16*)p.q + ((size_t)b * p.Hq + hq0 + h) * D + eoff(j));

  const size_t head_off = ((size_t)b * p.Hkv + kvh) * p.Tk_max * D;
  const size_t srow = ((size_t)b * p.Hkv + kvh) * p.Tk_max;   // row-scale index of key 0
  constexpr int ESZ = FP8 ? 1 : 2;                           // bytes per cache element
  const char* Kb = (const char*)p.kcache + head_off * ESZ;
  const char* Vb = (const char*)p.vcache + head_off * ESZ;

  float m[HPW], l[HPW], o[HPW][EPL];
#pragma unroll
  for (int h = 0; h < HPW; ++h) {
    m[h] = kNegInf;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[h][e] = 0.f;
  }

  // Loads go through buffer resources based at the iteration's first key
  // whose size ends at key hi: a row at or past hi reads zeros (its score
  // is masked below), with no branch per load.  The per-lane byte offsets
  // inside an iteration are loop invariants.  Cache rows are streamed with
  // the nontemporal policy (read exactly once).
  constexpr int kNT = 2;   // buffer-load cache policy: nt
  uint32_t roff[KU];       // row of load step u inside the iteration
#pragma unroll
  for (int u = 0; u < KU; ++u) roff[u] = (uint32_t)(wave * RPW * KU + u * RPW + row);

  for (int base = lo; base < hi; base += STEP) {
    const uint32_t rows_left = (uint32_t)min(hi - base, STEP);
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(Kb + (size_t)base * D * ESZ), 0, rows_left * D * ESZ, 0x00020000);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(Vb + (size_t)base * D * ESZ), 0, rows_left * D * ESZ, 0x00020000);
    // Key of load step u of this lane: base + roff[u].
    const int k0 = base + wave * RPW * KU + row;
    u32x4 kr[KU][NV], vr[KU][NV];
    float ks[KU], vs[KU];   // FP8: row scales (0 past the range)
    // FP8: EPL codes per lane and row, widened to bf16 only where used.
    typedef uint32_t raw_t __attribute__((ext_vector_type(EPL / 4)));
    raw_t kb[KU], vb[KU];
    if constexpr (FP8) {
      const __amdgpu_buffer_rsrc_t ksr = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(p.kscale + srow + base), 0, rows_left * 4, 0x00020000);
      const __amdgpu_buffer_rsrc_t vsr = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(p.vscale + srow + base), 0, rows_left * 4, 0x00020000);
      // EPL codes per lane: one 16- or 8-byte load per row and tensor.
#pragma unroll
      for (int u = 0; u < KU; ++u) {
        const uint32_t off = roff[u] * D + dl * EPL;
        if constexpr (EPL == 16) kb[u] = __builtin_amdgcn_raw_buffer_load_b128(krs, off, 0, kNT);
        else kb[u] = __builtin_amdgcn_raw_buffer_load_b64(krs, off, 0, kNT);
        ks[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ksr, roff[u] * 4, 0, kNT));
      }
#pragma unroll
      for (int u = 0; u < KU; ++u) {
        const uint32_t off = roff[u] * D + dl * EPL;
        if constexpr (EPL == 16) vb[u] = __builtin_amdgcn_raw_buffer_load_b128(vrs, off, 0, kNT);
        else vb[u] = __builtin_amdgcn_raw_buffer_load_b64(vrs, off, 0, kNT);
        vs[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(vsr, roff[u] * 4, 0, kNT));
      }
    } else {
#pragma unroll
      for (int u = 0; u < KU; ++u)
#pragma unroll
        for (int j = 0; j < NV; ++j)
          kr[u][j] = __builtin_amdgcn_raw_buffer_load_b128(krs, (roff[u] * D + eoff(j)) * 2, 0, kNT);
#pragma unroll
      for (int u = 0; u < KU; ++u)
#pragma unroll
        for (int j = 0; j < NV; ++j)
          vr[u][j] = __builtin_amdgcn_raw_buffer_load_b128(vrs, (roff[u] * D + eoff(j)) * 2, 0, kNT);
    }

    // Scores, reduced over the LPR lanes of each row.  FP8: each 16-byte
    // chunk of K is widened right where the HPW dot chains consume it, so
    // that the widened row is never held whole.
    float sc[KU][HPW];
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      float acc[HPW];
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const u32x4 k4 = FP8 ? widen8<KV>(kb[u][2 * j], kb[u][2 * j + 1]) : kr[u][j];
#pragma unroll
        for (int h = 0; h < HPW; ++h) {
          if (j == 0) acc[h] = dot2_from_zero(as_bf16x2(k4[0]), as_bf16x2(qv[h][0][0]));
#pragma unroll
          for (int w = j == 0 ? 1 : 0; w < 4; ++w)
            acc[h] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(k4[w]), as_bf16x2(qv[h][j][w]),
                                                     acc[h], false);
        }
      }
#pragma unroll
      for (int h = 0; h < HPW; ++h) {
        sc[u][h] = LPR == 8 ? group8_sum(acc[h]) : group16_sum(acc[h]);
        if constexpr (FP8) sc[u][h] *= ks[u];
      }
    }
    if (base + STEP > hi) {   // last iteration: keys past the range get -inf
#pragma unroll
      for (int u = 0; u < KU; ++u)
#pragma unroll
        for (int h = 0; h < HPW; ++h)
          if (k0 + u * RPW >= hi) sc[u][h] = kNegInf;
    }

    // Online softmax per (row, head).
    uint32_t pp[KU / 2][HPW];   // bf16 probabilities of key pairs (2t, 2t+1)
#pragma unroll
    for (int h = 0; h < HPW; ++h) {
      float mt = sc[0][h];
#pragma unroll
      for (int u = 1; u < KU; ++u) mt = fmaxf(mt, sc[u][h]);
      const float m_new = fmaxf(m[h], mt);
      // A row that has not met a visible key yet keeps everything at zero;
      // subtract 0 instead of -inf so no inf - inf appears.
      const float mref = m_new == kNegInf ? 0.f : m_new;
      if (__builtin_amdgcn_ballot_w64(m_new > m[h]) != 0) {
        const float corr = exp2_fast((m[h] - mref) * c);
        l[h] *= corr;
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[h][e] *= corr;
      }
      m[h] = m_new;
      const float mc = mref * c;
      float pe[KU];
#pragma unroll
      for (int u = 0; u < KU; ++u) {
        pe[u] = exp2_fast(fmaf(sc[u][h], c, -mc));
        l[h] += pe[u];
      }
      if constexpr (FP8) {
#pragma unroll
        for (int u = 0; u < KU; ++u) pe[u] *= vs[u];
      }
#pragma unroll
      for (int t = 0; t < KU / 2; ++t) pp[t][h] = bf16_pair_bits(pe[2 * t], pe[2 * t + 1]);
    }

    // O += P V, two keys per packed dot.
    if constexpr (FP8) {
      // Byte-interleave the codes of the two keys first (a0 b0 a1 b1 and
      // a2 b2 a3 b3), so that each widening gives a (v_a, v_b) pair of one
      // element directly.
#pragma unroll
      for (int t = 0; t < KU / 2; ++t)
#pragma unroll
        for (int i = 0; i < EPL / 4; ++i) {
          bf16x2 v2[4];
          pairs4<KV>(vb[2 * t][i], vb[2 * t + 1][i], v2);
#pragma unroll
          for (int k = 0; k < 4; ++k)
#pragma unroll
            for (int h = 0; h < HPW; ++h)
              o[h][4 * i + k] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(pp[t][h]), v2[k],
                                                                o[h][4 * i + k], false);
        }
    } else {
#pragma unroll
    for (int t = 0; t < KU / 2; ++t)
#pragma unroll
      for (int j = 0; j < NV; ++j)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t va = vr[2 * t][j][w], vb = vr[2 * t + 1][j][w];
          const bf16x2 lo2 = as_bf16x2(pack_lo(va, vb));
          const bf16x2 hi2 = as_bf16x2(pack_hi(va, vb));
          const int e = j * 8 + 2 * w;
#pragma unroll
          for (int h = 0; h < HPW; ++h) {
            const bf16x2 ph = as_bf16x2(pp[t][h]);
            o[h][e] = __builtin_amdgcn_fdot2_f32_bf16(ph, lo2, o[h][e], false);
            o[h][e + 1] = __builtin_amdgcn_fdot2_f32_bf16(ph, hi2, o[h][e + 1], false);
          }
        }
    }
  }

  // Merge the rows of the wavefront (rescale rule), then hand the wavefront
  // result to LDS.
#pragma unroll
  for (int h = 0; h < HPW; ++h) {
    const float M = rows_max<LPR>(m[h]);
    const float Mref = M == kNegInf ? 0.f : M;
    const float wr = exp2_fast((m[h] - Mref) * c);
    const float lw = rows_sum<LPR>(l[h] * wr);
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[h][e] = rows_sum<LPR>(o[h][e] * wr);
    if (lane == 0) {
      red_m[wave][h] = M;
      red_l[wave][h] = lw;
    }
    if (row == 0) {
#pragma unroll
      for (int j = 0; j < NV; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) red_o[wave][h][eoff(j) + e] = o[h][j * 8 + e];
    }
  }
  __syncthreads();

  // Merge the 4 wavefronts (fixed order) and write the partial.
  for (int i = tid; i < HPW * D; i += kDecThreads) {
    const int h = i / D;
    const int d = i % D;
    float M = red_m[0][h];
#pragma unroll
    for (int w = 1; w < 4; ++w) M = fmaxf(M, red_m[w][h]);
    const float Mref = M == kNegInf ? 0.f : M;
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float wt = exp2_fast((red_m[w][h] - Mref) * c);
      L = fmaf(wt, red_l[w][h], L);
      O = fmaf(wt, red_o[w][h][d], O);
    }
    const size_t pi = slot * HPW + h;
    p.part_o[pi * D + d] = O;
    if (d == 0) {
      p.part_m[pi] = M * c;   // stored in base-2 exponent units
      p.part_l[pi] = L;
    }
  }
  __syncthreads();   // LDS is reused by the next range
}

// ---- Matrix-core loop for the E4M3 cache: d = 128, 4 or 8 heads per workgroup ----
//
// With one byte per cached element the packed-dot loop above spends more
// vector instructions per byte than the memory time covers, so the 8-bit
// cache takes this loop instead.  A wavefront takes blocks of 32
// consecutive keys.  The scores of a block come from the 16x16x32 bf16
// matrix core, S' = K Q^T, with the 16 keys of a half-block as rows and the
// workgroup's query heads as columns: lane l then holds the scores of keys
// 4*(l/16) + 0..3 of both half-blocks for head l % 16, which is exactly the
// operand layout that O^T += V^T P^T takes for its probabilities, so no
// lane exchange sits between the two products.  V^T (keys packed per lane)
// is gathered from a per-wavefront LDS copy of the block with the gfx950
// 8-bit transposing read.  The online softmax runs on 8 scores per lane,
// with one running max per head shared by the four lane groups.  (The bf16
// cache measured 1% faster on the packed-dot loop and stays there.)
constexpr int kMB = 32;   // keys per wavefront block
constexpr int kMfRowB = 128;   // bytes per cached E4M3 row at d = 128

// First head-dimension index of the 8 elements that lane group grp holds in
// k-step kk (four k-steps of 32 cover d = 128).  Any permutation works as
// long as K and Q use the same one; this one lets each 16-byte K load serve
// two k-steps.
__device__ __forceinline__ int mf_dim0(int grp, int kk) {
  return 64 * (kk >> 1) + 16 * grp + 8 * (kk & 1);
}
// LDS swizzle of the 16-byte chunks of V row `row`: within 32 lanes, the 8
// bytes of every lane of a transposing read fall in distinct banks.
__device__ __forceinline__ int mf_vswz(int row) {
  return ((row >> 1) & 1) | (((row >> 4) & 1) << 1) | (((row >> 2) & 1) << 2);
}
__device__ __forceinline__ f32x4 mma_16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// Max / sum over the four lane groups (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float groups_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float groups_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Same contract as decode_range_keys for the E4M3 cache (d = 128, HPW of 4
// or 8); `vlds` holds 2 * 4 * kMB rows (two blocks per wavefront).
template <int HPW, int KV>
__device__ __forceinline__ void decode_range_mfma(const DecodeParams& p, int b, int kvh, int hq0,
                                                  int lo, int hi, size_t slot, float (*red_m)[HPW],
                                                  float (*red_l)[HPW], float (*red_o)[HPW][128],
                                                  uint8_t* vlds) {
  constexpr int D = 128;
  constexpr int ROWB = kMfRowB;
  constexpr int STEP = 4 * kMB;                 // keys per workgroup iteration
  constexpr int NCOPY = kMB * ROWB / 1024;      // 1 KiB LDS copies per block
  constexpr int RPC = 1024 / ROWB;              // rows per copy instruction
  constexpr int CPR = ROWB / 16;                // 16-byte chunks per row
  constexpr int kNT = 2;                        // buffer-load cache policy: nt
  static_assert(HPW == 4 || HPW == 8, "matrix-core decode takes 4 or 8 heads");
  b = __builtin_amdgcn_readfirstlane(b);
  kvh = __builtin_amdgcn_readfirstlane(kvh);
  hq0 = __builtin_amdgcn_readfirstlane(hq0);
  lo = __builtin_amdgcn_readfirstlane(lo);
  hi = __builtin_amdgcn_readfirstlane(hi);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 15;    // head column (>= HPW: unused)
  const int grp = lane >> 4;    // lane group
  const float c = p.c;

  // Q as the B operand of S' = K Q^T: qb[kk] = q[hq0 + col][mf_dim0(grp, kk) .. +8].
  bf16x8 qb[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    u32x4 w = {0u, 0u, 0u, 0u};
    if (col < HPW)
      w = *(const u32x4*)((const bf16*)p.q + ((size_t)b * p.Hq + hq0 + col) * D + mf_dim0(grp, kk));
    __builtin_memcpy(&qb[kk], &w, sizeof(w));
  }

  const size_t row0 = ((size_t)b * p.Hkv + kvh) * p.Tk_max;   // cache row of key 0
  const uint8_t* Kb = (const uint8_t*)p.kcache + row0 * ROWB;
  const uint8_t* Vb = (const uint8_t*)p.vcache + row0 * ROWB;
  uint8_t* vbuf = vlds + __builtin_amdgcn_readfirstlane(wave) * 2 * kMB * ROWB;

  // Loop-invariant offsets, relative to the first key of a workgroup step.
  // K: lane (col, grp) loads 16-byte chunks grp and 4 + grp of row
  // kMB*wave + 16*hb + col.
  const uint32_t koff = (uint32_t)((kMB * wave + col) * ROWB + 16 * grp);
  // Row scales: lane (grp, n) loads the scale of key kappa(grp, n % 8) =
  // 16*(n%8/4) + 4*grp + n%4 of the block (one coalesced 4-byte load per
  // tensor and block, every key range-checked alone); each lane then takes
  // the 8 values of its row by broadcast within the row.
  const uint32_t soff = (uint32_t)((kMB * wave + 16 * ((lane & 7) >> 2) + 4 * grp + (lane & 3)) * 4);
  // V copies: instruction n puts rows RPC*n .. into LDS, lane -> (row, chunk').
  uint32_t vsrc[NCOPY];
#pragma unroll
  for (int n = 0; n < NCOPY; ++n) {
    const int row = RPC * n + lane / CPR;
    const int chunk = (lane % CPR) ^ mf_vswz(row);
    vsrc[n] = (uint32_t)((kMB * wave + row) * ROWB + 16 * chunk);
  }
  // Transposing reads of V^T (ds_read_b64_tr_b8), one address per 16-dim
  // block db: input lane 2e + h of a group addresses row
  // kappa(grp, e) = 16*(e/4) + 4*grp + e%4, bytes 16*db + 8*h .. +8.
  uint32_t vaddr[8];
  {
    const int gl = lane & 15;
    const int e = gl >> 1, h = gl & 1;
    const int row = 16 * (e >> 2) + 4 * grp + (e & 3);
    const uint32_t vb0 = lds_addr(vbuf);
#pragma unroll
    for (int db = 0; db < 8; ++db) vaddr[db] = vb0 + row * ROWB + 16 * (db ^ mf_vswz(row)) + 8 * h;
  }

  float m_run = kNegInf, l_run = 0.f;
  f32x4 oacc[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Two blocks in flight per wavefront: the loads of the next block (K rows
  // into registers, row scales, V rows into the other LDS buffer) are issued
  // before the current block is computed.
  u32x4 kc[2][2][2];
  uint32_t ksr_[2], vsr_[2];   // this lane's loaded row scales (see soff)
  auto issue = [&](int bs, auto buf_c) __attribute__((always_inline)) {
    constexpr int BUF = decltype(buf_c)::value;
    // Resources end at key hi; past the range (bs >= hi) they are empty and
    // every load reads zeros without a memory access.
    const uint32_t rows_left = (uint32_t)__builtin_amdgcn_readfirstlane(max(0, min(hi - bs, STEP)));
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(Kb + (size_t)bs * ROWB), 0, rows_left * ROWB, 0x00020000);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(Vb + (size_t)bs * ROWB), 0, rows_left * ROWB, 0x00020000);
    const __amdgpu_buffer_rsrc_t ksr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.kscale + row0 + bs), 0, rows_left * 4, 0x00020000);
    const __amdgpu_buffer_rsrc_t vsr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.vscale + row0 + bs), 0, rows_left * 4, 0x00020000);
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int i = 0; i < 2; ++i)
        kc[BUF][hb][i] = __builtin_amdgcn_raw_buffer_load_b128(krs, koff + 16 * hb * ROWB + 64 * i, 0, kNT);
    ksr_[BUF] = __builtin_amdgcn_raw_buffer_load_b32(ksr, soff, 0, kNT);
    vsr_[BUF] = __builtin_amdgcn_raw_buffer_load_b32(vsr, soff, 0, kNT);
    // V rows into LDS buffer BUF of this wavefront (that buffer's previous
    // transposing reads have all completed: each was waited for before its
    // product).
    asm volatile("" ::: "memory");
#pragma unroll
    for (int n = 0; n < NCOPY; ++n)
      copy16_buf_to_lds(vrs, vbuf + BUF * kMB * ROWB + 1024 * n, vsrc[n], 0);
  };
  constexpr int NVM = 4 + 2 + NCOPY;   // vector-memory operations per block

  auto compute = [&](int bs, auto buf_c) __attribute__((always_inline)) {
    constexpr int BUF = decltype(buf_c)::value;
    // The block's loads have landed once at most the next block's are
    // outstanding.
    __builtin_amdgcn_s_waitcnt(vmcnt_imm<NVM>());

    // S' = K Q^T per half-block: lane holds keys 16*hb + 4*grp + r, head col.
    f32x4 sacc[2];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      sacc[hb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const u32x4 a = widen8<KV>(kc[BUF][hb][kk >> 1][2 * (kk & 1)], kc[BUF][hb][kk >> 1][2 * (kk & 1) + 1]);
        bf16x8 ab;
        __builtin_memcpy(&ab, &a, sizeof(ab));
        sacc[hb] = mma_16x16x32(ab, qb[kk], sacc[hb]);
      }
    }

    // Row scales of the lane's keys kappa(grp, j): lane j of its row holds
    // them (DPP row_newbcast:j).
    float ksv[8], vsv[8];
    static_for<0, 8>([&](auto j_c) {
      constexpr int J = decltype(j_c)::value;
      ksv[J] = __uint_as_float(__builtin_amdgcn_update_dpp(0u, ksr_[BUF], 0x150 + J, 0xf, 0xf, false));
      vsv[J] = __uint_as_float(__builtin_amdgcn_update_dpp(0u, vsr_[BUF], 0x150 + J, 0xf, 0xf, false));
    });

    // Online softmax over the block (raw score units; K row scale applied).
    float sc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) sc[j] = sacc[j >> 2][j & 3] * ksv[j];
    if (bs + STEP > hi) {   // last block: keys past the range get -inf
      const int k0 = bs + kMB * wave + 4 * grp;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (k0 + 16 * (j >> 2) + (j & 3) >= hi) sc[j] = kNegInf;
    }
    float mt = fmaxf(fmaxf(sc[0], sc[1]), sc[2]);
    mt = fmaxf(fmaxf(mt, sc[3]), sc[4]);
    mt = fmaxf(fmaxf(mt, sc[5]), sc[6]);
    mt = groups_max(fmaxf(mt, sc[7]));
    const float m_new = fmaxf(m_run, mt);
    const float mref = m_new == kNegInf ? 0.f : m_new;
    if (__builtin_amdgcn_ballot_w64(m_new > m_run) != 0) {
      const float corr = exp2_fast((m_run - mref) * c);
      l_run *= corr;
#pragma unroll
      for (int db = 0; db < 8; ++db) oacc[db] *= corr;
    }
    m_run = m_new;
    const float mc = mref * c;
    float pe[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      pe[j] = exp2_fast(fmaf(sc[j], c, -mc));
      l_run += pe[j];
      pe[j] *= vsv[j];   // V row scale, after the row sum
    }
    bf16x8 pb;
    {
      const u32x4 w = {bf16_pair_bits(pe[0], pe[1]), bf16_pair_bits(pe[2], pe[3]),
                       bf16_pair_bits(pe[4], pe[5]), bf16_pair_bits(pe[6], pe[7])};
      __builtin_memcpy(&pb, &w, sizeof(pb));
    }

    // O^T += V^T P^T with V^T from LDS buffer BUF.
    constexpr int VOFF = BUF * kMB * ROWB;
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      u32x2 t = lds_read_tr8<VOFF>(vaddr[db]);
      lgkm_wait<0>();
      tie(t);
      const u32x4 w = widen8<KV>(t[0], t[1]);
      bf16x8 va;
      __builtin_memcpy(&va, &w, sizeof(va));
      oacc[db] = mma_16x16x32(va, pb, oacc[db]);
    }
  };

  // The next block is always issued (an empty one past the range), so that
  // every path through the loop has the same loads in flight.
  if (lo < hi) {
    issue(lo, IC<0>{});
    for (int bs = lo;; bs += 2 * STEP) {
      issue(bs + STEP, IC<1>{});
      compute(bs, IC<0>{});
      if (bs + STEP >= hi) break;
      issue(bs + 2 * STEP, IC<0>{});
      compute(bs + STEP, IC<1>{});
      if (bs + 2 * STEP >= hi) break;
    }
    // No copy into LDS may still be in flight once the loop is left.
    __builtin_amdgcn_s_waitcnt(vmcnt_imm<0>());
  }

  // Wavefront result per head: l summed over the lane groups, O^T element
  // (16*db + 4*grp + r, col) in register r of block db.
  const float lt = groups_sum(l_run);
  if (col < HPW) {
    if (grp == 0) {
      red_m[wave][col] = m_run;
      red_l[wave][col] = lt;
    }
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) red_o[wave][col][16 * db + 4 * grp + r] = oacc[db][r];
  }
  __syncthreads();

  // Merge the 4 wavefronts (fixed order) and write the partial.
  for (int i = tid; i < HPW * D; i += kDecThreads) {
    const int h = i / D;
    const int d = i % D;
    float M = red_m[0][h];
#pragma unroll
    for (int w = 1; w < 4; ++w) M = fmaxf(M, red_m[w][h]);
    const float Mref = M == kNegInf ? 0.f : M;
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float wt = exp2_fast((red_m[w][h] - Mref) * c);
      L = fmaf(wt, red_l[w][h], L);
      O = fmaf(wt, red_o[w][h][d], O);
    }
    const size_t pi = slot * HPW + h;
    p.part_o[pi * D + d] = O;
    if (d == 0) {
      p.part_m[pi] = M * c;   // stored in base-2 exponent units
      p.part_l[pi] = L;
    }
  }
  __syncthreads();   // LDS is reused by the next range
}

__device__ __forceinline__ int clamp_len(const DecodeParams& p, int b) {
  return min(max(p.seqlens[b], 0), p.Tk_max);
}

// Workgroup w of W: balanced share of the key space of all segments.
template <int D, int HPW, int KU, int KV>
__global__ void __launch_bounds__(kDecThreads) decode_kernel(const DecodeParams p) {
  __shared__ float red_m[4][HPW];
  __shared__ float red_l[4][HPW];
  __shared__ float red_o[4][HPW][D];
  constexpr bool MF = KV != kKvBf16 && D == 128 && HPW >= 4;   // matrix-core range loop
  __shared__ __attribute__((aligned(16))) uint8_t vlds[MF ? 2 * 4 * kMB * kMfRowB : 16];
  __shared__ long long wave_tot[4];
  __shared__ int start[3];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int w = blockIdx.x;
  const int groups = p.g / HPW;
  const int G = p.Hkv * groups;   // segments per sequence

  // Prefix sums of the sequence lengths: thread t owns the sequences
  // [t * cpt, (t + 1) * cpt); a wavefront scan plus the wavefront totals
  // give each thread the number of keys before its block.
  const int cpt = (p.B + kDecThreads - 1) / kDecThreads;
  const int b0 = min(p.B, tid * cpt), b1 = min(p.B, b0 + cpt);
  long long own = 0;
  for (int bb = b0; bb < b1; ++bb) own += clamp_len(p, bb);
  long long incl = own;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const long long v = __shfl_up(incl, off, 64);
    if (lane >= off) incl += v;
  }
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  long long before = 0, total = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    before += i < wave ? wave_tot[i] : 0;
    total += wave_tot[i];
  }
  const long long excl = before + incl - own;   // keys of sequences before b0

  if (w == 0) {   // the merge kernel reads the prefix sums
    long long run = excl;
    for (int bb = b0; bb < b1; ++bb) {
      p.cum[bb] = run;
      run += clamp_len(p, bb);
    }
    if (tid == 0) p.cum[p.B] = total;
  }

  const long long ktot = total * G;
  const long long per = decode_range(ktot, p.W);
  const long long pos0 = (long long)w * per;
  if (pos0 >= ktot) return;
  const long long pend = min(pos0 + per, ktot);

  // Locate the segment holding pos0: sequence b covers the positions
  // [cum_b * G, cum_{b+1} * G), its segment j the n_b keys from cum_b * G + j * n_b.
  if (excl * G <= pos0 && pos0 < (excl + own) * G) {
    long long run = excl;
    for (int bb = b0; bb < b1; ++bb) {
      const int n = clamp_len(p, bb);
      if (pos0 < (run + n) * G) {
        const long long off = pos0 - run * G;
        start[0] = bb;
        start[1] = (int)(off / n);
        start[2] = (int)(off % n);
        break;
      }
      run += n;
    }
  }
  __syncthreads();
  int b = start[0], j = start[1], key = start[2];
  int n = clamp_len(p, b);

  long long pos = pos0;
  while (true) {
    const int cnt = (int)min((long long)(n - key), pend - pos);
    const int kvh = j / groups;
    const int hq0 = kvh * p.g + (j % groups) * HPW;
    if constexpr (MF)
      decode_range_mfma<HPW, KV>(p, b, kvh, hq0, key, key + cnt, (size_t)w + (size_t)b * G + j,
                                  red_m, red_l, red_o, vlds);
    else
      decode_range_keys<D, HPW, KU, KV>(p, b, kvh, hq0, key, key + cnt,
                                         (size_t)w + (size_t)b * G + j, red_m, red_l, red_o);
    pos += cnt;
    if (pos >= pend) break;
    key = 0;
    if (++j == G) {   // next sequence with keys (one exists: pos < ktot)
      j = 0;
      do {
        ++b;
        n = clamp_len(p, b);
      } while (n == 0 && b + 1 < p.B);
    }
  }
}

// Merge, one wavefront per (sequence, query head): fixed-order combination
// of the slots of the head's segment, O = sum_s 2^(m_s - M) o_s / sum_s
// 2^(m_s - M) l_s.  Every slot of the segment holds at least one key.  Lane
// t holds slot t's statistics (64 slots per pass, passes combined by the
// same rule); the output rows of the first 8 slots are loaded together with
// the statistics so that the merge costs about two memory latencies.
template <int D>
__global__ void __launch_bounds__(64) decode_merge_kernel(const DecodeParams p) {
  constexpr int E = D / 64;
  constexpr int PRE = 8;
  const int lane = threadIdx.x;
  const int bh = blockIdx.x;   // b * Hq + hq
  const int b = bh / p.Hq;
  const int hq = bh % p.Hq;
  const int groups = p.g / p.hpw;
  const int G = p.Hkv * groups;
  const int kvh = hq / p.g;
  const int r = hq % p.g;
  const int j = kvh * groups + r / p.hpw;
  const int h = r % p.hpw;

  const long long c0 = p.cum[b];
  const long long n = p.cum[b + 1] - c0;
  const long long ktot = p.cum[p.B] * G;
  float O[E];
#pragma unroll
  for (int e = 0; e < E; ++e) O[e] = 0.f;
  float L = 0.f;
  if (n > 0) {
    const long long per = decode_range(ktot, p.W);
    const long long s0 = c0 * G + (long long)j * n;
    const int w0 = (int)(s0 / per);
    const int cnt = (int)((s0 + n - 1) / per) - w0 + 1;
    const size_t first = ((size_t)w0 + (size_t)b * G + j) * p.hpw + h;   // slot stride: hpw
    const size_t st = p.hpw;
    const float* pm = p.part_m + first;
    const float* pl = p.part_l + first;
    const float* po = p.part_o + first * D + lane * E;

    float pre[PRE][E];
#pragma unroll
    for (int t = 0; t < PRE; ++t)
#pragma unroll
      for (int e = 0; e < E; ++e) pre[t][e] = t < cnt ? po[t * st * D + e] : 0.f;

    float M = kNegInf;
    for (int t0 = 0; t0 < cnt; t0 += 64) {
      const int nc = min(64, cnt - t0);
      const float mt = lane < nc ? pm[(t0 + lane) * st] : kNegInf;
      const float lt = lane < nc ? pl[(t0 + lane) * st] : 0.f;
      float Mc = mt;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) Mc = fmaxf(Mc, __shfl_xor(Mc, off, 64));
      const float Mn = fmaxf(M, Mc);
      const float scale = exp2_fast(M - Mn);   // 0 on the first pass
      const float wt = lane < nc ? exp2_fast(mt - Mn) : 0.f;
      float lw = wt * lt;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) lw += __shfl_xor(lw, off, 64);
      L = L * scale + lw;
#pragma unroll
      for (int e = 0; e < E; ++e) O[e] *= scale;
      int t = 0;
      if (t0 == 0) {
#pragma unroll
        for (; t < PRE; ++t) {
          if (t >= nc) break;
          const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wt), t));
#pragma unroll
          for (int e = 0; e < E; ++e) O[e] = fmaf(wj, pre[t][e], O[e]);
        }
      }
      for (; t < nc; ++t) {
        const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wt), t));
#pragma unroll
        for (int e = 0; e < E; ++e) O[e] = fmaf(wj, po[(t0 + t) * st * D + e], O[e]);
      }
      M = Mn;
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  bf16* og = (bf16*)p.o + (size_t)bh * D + lane * E;
  if constexpr (E == 2) {
    *(bf16x2*)og = to_bf16x2(O[0] * inv, O[1] * inv);
  } else {
    og[0] = to_bf16x2(O[0] * inv, 0.f)[0];
  }
}

template <int D, int HPW, int KV>
const void* decode_kernel_ptr() {
  return (const void*)decode_kernel<D, HPW, kDecKU, KV>;
}

template <int D, int KV>
const void* decode_kernel_for(int hpw) {
  switch (hpw) {
    case 8: return decode_kernel_ptr<D, 8, KV>();
    case 4: return decode_kernel_ptr<D, 4, KV>();
    case 2: return decode_kernel_ptr<D, 2, KV>();
    default: return decode_kernel_ptr<D, 1, KV>();
  }
}

template <int KV>
const void* decode_kernel_dk(int d, int hpw) {
  return d == 64 ? decode_kernel_for<64, KV>(hpw) : decode_kernel_for<128, KV>(hpw);
}

template <int D, int KV>
hipError_t launch_decode_d(const DecodeParams& p, hipStream_t stream) {
  const dim3 grid((unsigned)p.W);
  switch (p.hpw) {
    case 8: hipLaunchKernelGGL((decode_kernel<D, 8, kDecKU, KV>), grid, dim3(kDecThreads), 0, stream, p); break;
    case 4: hipLaunchKernelGGL((decode_kernel<D, 4, kDecKU, KV>), grid, dim3(kDecThreads), 0, stream, p); break;
    case 2: hipLaunchKernelGGL((decode_kernel<D, 2, kDecKU, KV>), grid, dim3(kDecThreads), 0, stream, p); break;
    default: hipLaunchKernelGGL((decode_kernel<D, 1, kDecKU, KV>), grid, dim3(kDecThreads), 0, stream, p); break;
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL((decode_merge_kernel<D>), dim3((unsigned)(p.B * p.Hq)), dim3(64), 0, stream, p);
  return hipGetLastError();
}

template <int KV>
hipError_t launch_decode_k(const DecodeParams& p, int d, hipStream_t stream) {
  return d == 64 ? launch_decode_d<64, KV>(p, stream) : launch_decode_d<128, KV>(p, stream);
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, int d, int kv, hipStream_t stream) {
  switch (kv) {
    case kKvE4m3: return launch_decode_k<kKvE4m3>(p, d, stream);
    case kKvInt8: return launch_decode_k<kKvInt8>(p, d, stream);
    default: return launch_decode_k<kKvBf16>(p, d, stream);
  }
}

int decode_resident_workgroups(int d, int hpw, int kv) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  const void* k = kv == kKvE4m3   ? decode_kernel_dk<kKvE4m3>(d, hpw)
                  : kv == kKvInt8 ? decode_kernel_dk<kKvInt8>(d, hpw)
                                  : decode_kernel_dk<kKvBf16>(d, hpw);
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, kDecThreads, 0) != hipSuccess) return 0;
  return cus * per_cu;
}

}  // namespace fa
