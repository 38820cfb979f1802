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
// group of 4; 8 with an 8-bit cache), so it runs on the vector ALUs; the design goal is to stream
// every cache byte exactly once with coalesced 16-byte loads and enough
// loads in flight, while spending as few vector instructions per key as
// possible so that the arithmetic hides under the memory time.
//
// One workgroup per (piece s, kv head group, sequence b); pieces have the
// same size for every sequence (the cache capacity divided by the split
// count, rounded up to 64 keys), so workgroups carry equal work whatever the
// sequence lengths:
//  * 4 wavefronts march through the piece's keys.  A key row is read by LPR
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
//    (lane shuffles), then the 4 wavefronts through LDS, and the piece's
//    (m, l, o) is written to the workspace.
// An 8-bit cache (E4M3 codes, one fp32 scale per row: [NOTE]'s fused
// dequantisation, the cache expanded inside the tile load) runs the same
// loop: the codes are widened to bf16 in registers right after the load.
// Merge kernel, one wavefront per (sequence, query head): fixed-order pass
// over the pieces, O = sum 2^(m_s - M) o_s / sum 2^(m_s - M) l_s.
#include "fa_device.h"
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

// Attention of the HPW query heads hq0.. over keys [lo, hi) of kv head
// (b, kvh); the partial (m, l, o) goes to `slot`.  Every thread of the
// workgroup calls this with the same arguments.  FP8: the cache holds E4M3
// codes with one fp32 scale per row; a lane loads its EPL codes with one
// load, widens them to bf16 in registers and the rest of the loop is the
// bf16 one, with the K row scale applied to the row's score and the V row
// scale to its probability (after the row sum l is formed).
template <int D, int HPW, int KU, bool FP8>
__device__ __forceinline__ void decode_range_keys(const DecodeParams& p, int b, int kvh, int hq0,
                                                  int lo, int hi, size_t slot, float (*red_m)[HPW],
                                                  float (*red_l)[HPW], float (*red_o)[HPW][D]) {
  typedef DecodeShape<D, HPW> S;
  constexpr int EPL = S::EPL, LPR = S::LPR, RPW = S::RPW, NV = S::NV;
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
    if constexpr (FP8) {
      const __amdgpu_buffer_rsrc_t ksr = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(p.kscale + srow + base), 0, rows_left * 4, 0x00020000);
      const __amdgpu_buffer_rsrc_t vsr = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(p.vscale + srow + base), 0, rows_left * 4, 0x00020000);
      // EPL codes per lane: one 16- or 8-byte load per row and tensor.
      typedef uint32_t raw_t __attribute__((ext_vector_type(EPL / 4)));
      raw_t kb[KU], vb[KU];
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
#pragma unroll
      for (int u = 0; u < KU; ++u)
#pragma unroll
        for (int j = 0; j < NV; ++j) {
          kr[u][j] = e4m3x8_to_bf16(kb[u][2 * j], kb[u][2 * j + 1]);
          vr[u][j] = e4m3x8_to_bf16(vb[u][2 * j], vb[u][2 * j + 1]);
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

    // Scores, reduced over the LPR lanes of each row.
    float sc[KU][HPW];
#pragma unroll
    for (int u = 0; u < KU; ++u)
#pragma unroll
      for (int h = 0; h < HPW; ++h) {
        float acc = dot2_from_zero(as_bf16x2(kr[u][0][0]), as_bf16x2(qv[h][0][0]));
#pragma unroll
        for (int j = 0; j < NV; ++j)
#pragma unroll
          for (int w = j == 0 ? 1 : 0; w < 4; ++w)
            acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(kr[u][j][w]), as_bf16x2(qv[h][j][w]),
                                                  acc, false);
        sc[u][h] = LPR == 8 ? group8_sum(acc) : group16_sum(acc);
        if constexpr (FP8) sc[u][h] *= ks[u];
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

__device__ __forceinline__ int clamp_len(const DecodeParams& p, int b) {
  return min(max(p.seqlens[b], 0), p.Tk_max);
}

// Workgroup w of W: balanced share of the key space of all segments.
template <int D, int HPW, int KU, bool FP8>
__global__ void __launch_bounds__(kDecThreads) decode_kernel(const DecodeParams p) {
  __shared__ float red_m[4][HPW];
  __shared__ float red_l[4][HPW];
  __shared__ float red_o[4][HPW][D];
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
    decode_range_keys<D, HPW, KU, FP8>(p, b, kvh, hq0, key, key + cnt,
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

template <int D, int HPW, bool FP8>
const void* decode_kernel_ptr() {
  return (const void*)decode_kernel<D, HPW, kDecKU, FP8>;
}

template <int D, bool FP8>
const void* decode_kernel_for(int hpw) {
  switch (hpw) {
    case 8: return decode_kernel_ptr<D, 8, FP8>();
    case 4: return decode_kernel_ptr<D, 4, FP8>();
    case 2: return decode_kernel_ptr<D, 2, FP8>();
    default: return decode_kernel_ptr<D, 1, FP8>();
  }
}

template <int D, bool FP8>
hipError_t launch_decode_d(const DecodeParams& p, hipStream_t stream) {
  const dim3 grid((unsigned)p.W);
  switch (p.hpw) {
    case 8: hipLaunchKernelGGL((decode_kernel<D, 8, kDecKU, FP8>), grid, dim3(kDecThreads), 0, stream, p); break;
    case 4: hipLaunchKernelGGL((decode_kernel<D, 4, kDecKU, FP8>), grid, dim3(kDecThreads), 0, stream, p); break;
    case 2: hipLaunchKernelGGL((decode_kernel<D, 2, kDecKU, FP8>), grid, dim3(kDecThreads), 0, stream, p); break;
    default: hipLaunchKernelGGL((decode_kernel<D, 1, kDecKU, FP8>), grid, dim3(kDecThreads), 0, stream, p); break;
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL((decode_merge_kernel<D>), dim3((unsigned)(p.B * p.Hq)), dim3(64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, int d, bool fp8, hipStream_t stream) {
  if (fp8) return d == 64 ? launch_decode_d<64, true>(p, stream) : launch_decode_d<128, true>(p, stream);
  return d == 64 ? launch_decode_d<64, false>(p, stream) : launch_decode_d<128, false>(p, stream);
}

int decode_resident_workgroups(int d, int hpw, bool fp8) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  const void* k = fp8 ? (d == 64 ? decode_kernel_for<64, true>(hpw) : decode_kernel_for<128, true>(hpw))
                      : (d == 64 ? decode_kernel_for<64, false>(hpw) : decode_kernel_for<128, false>(hpw));
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, kDecThreads, 0) != hipSuccess) return 0;
  return cus * per_cu;
}

}  // namespace fa
