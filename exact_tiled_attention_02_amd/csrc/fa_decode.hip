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
// group of 4), so it runs on the vector ALUs; the design goal is to stream
// every cache byte exactly once with coalesced 16-byte loads and enough
// loads in flight.
//
// Split kernel, one workgroup per (piece s, kv head group, sequence b):
//  * 4 wavefronts march through the piece's keys; per load step a
//    wavefront reads 4 consecutive key rows, 16 lanes per row, each lane
//    d/16 consecutive elements (16 B at d = 128).
//  * Scores of the HPW query heads: each lane forms a partial dot product
//    over its d-slice (packed bf16 dot instructions, fp32 sums), then a
//    16-lane rotate-and-add reduction (DPP row rotations) leaves the full
//    score in every lane of the row.
//  * Online softmax per head with a wavefront-wide running max; the value
//    rows are multiplied in the same lane layout, so probabilities never
//    move between lanes.
//  * At the end the 4 rows and 4 wavefronts are merged (rescale rule) and
//    the piece's (m, l, o) is written to the workspace.
// Merge kernel, one wavefront per (sequence, query head): fixed-order pass
// over the pieces, O = sum 2^(m_s - M) o_s / sum 2^(m_s - M) l_s.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kDecThreads = 256;
constexpr int kU = 8;  // load steps (of 4 keys) per wavefront per iteration

__device__ __forceinline__ float row16_sum(float x) {
  // All-reduce over the 16 lanes of a DPP row by rotations 8, 4, 2, 1.
  x += __builtin_amdgcn_update_dpp(0.f, x, 0x128, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0.f, x, 0x124, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0.f, x, 0x122, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0.f, x, 0x121, 0xf, 0xf, false);
  return x;
}

__device__ __forceinline__ float wave_rows_max(float x) {
  x = fmaxf(x, __shfl_xor(x, 16, 64));
  return fmaxf(x, __shfl_xor(x, 32, 64));
}
__device__ __forceinline__ float wave_rows_sum(float x) {
  x += __shfl_xor(x, 16, 64);
  return x + __shfl_xor(x, 32, 64);
}

template <int D>
struct Slice;  // the per-lane share of one key row
template <>
struct Slice<128> {
  typedef u32x4 T;  // 8 bf16
  static constexpr int W = 4;
};
template <>
struct Slice<64> {
  typedef u32x2 T;  // 4 bf16
  static constexpr int W = 2;
};

template <int D, int HPW>
__global__ void __launch_bounds__(kDecThreads) decode_split_kernel(const DecodeParams p) {
  typedef typename Slice<D>::T SliceT;
  constexpr int W = Slice<D>::W;   // dwords per lane per key row
  constexpr int DPL = 2 * W;       // d elements per lane
  __shared__ float red_m[4][HPW];
  __shared__ float red_l[4][HPW];
  __shared__ float red_o[4][HPW][D];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int row = lane >> 4;   // which of the 4 keys of a load step
  const int dl = lane & 15;    // d-slice index

  const int s = blockIdx.x;
  const int groups = p.g / HPW;
  const int kvh = blockIdx.y / groups;
  const int hq0 = kvh * p.g + (blockIdx.y % groups) * HPW;
  const int b = blockIdx.z;

  const int n = min(max(p.seqlens[b], 0), p.Tk_max);
  const int per = (n + p.splits - 1) / p.splits;
  const int chunk = n > 0 ? ((per + kDecodeTile - 1) / kDecodeTile) * kDecodeTile : kDecodeTile;
  const int lo = s * chunk;
  const int hi = min(n, lo + chunk);

  const size_t pidx0 = ((size_t)b * p.Hq + hq0) * p.splits + s;   // head stride: splits
  if (lo >= hi) {  // empty piece: weight zero in the merge
    if (tid < HPW) {
      p.part_m[pidx0 + (size_t)tid * p.splits] = kNegInf;
      p.part_l[pidx0 + (size_t)tid * p.splits] = 0.f;
    }
    return;
  }

  // This lane's d-slice of each query head, as packed bf16 pairs.
  SliceT qv[HPW];
#pragma unroll
  for (int h = 0; h < HPW; ++h)
    qv[h] = *(const SliceT*)((const bf16*)p.q + ((size_t)b * p.Hq + hq0 + h) * D + dl * DPL);

  const bf16* Kg = (const bf16*)p.kcache + ((size_t)b * p.Hkv + kvh) * p.Tk_max * D + dl * DPL;
  const bf16* Vg = (const bf16*)p.vcache + ((size_t)b * p.Hkv + kvh) * p.Tk_max * D + dl * DPL;

  const float c = p.c;
  float m[HPW], l[HPW], o[HPW][DPL];
#pragma unroll
  for (int h = 0; h < HPW; ++h) {
    m[h] = kNegInf;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) o[h][e] = 0.f;
  }

  SliceT zero;
#pragma unroll
  for (int w = 0; w < W; ++w) zero[w] = 0u;

  for (int base = lo; base < hi; base += 4 * 4 * kU) {
    const int kbase = base + wave * 4 * kU + row;   // key of load step u: kbase + 4u
    SliceT kr[kU], vr[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int key = kbase + 4 * u;
      kr[u] = key < hi ? *(const SliceT*)(Kg + (size_t)key * D) : zero;
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int key = kbase + 4 * u;
      vr[u] = key < hi ? *(const SliceT*)(Vg + (size_t)key * D) : zero;
    }

    float sc[kU][HPW];
#pragma unroll
    for (int u = 0; u < kU; ++u)
#pragma unroll
      for (int h = 0; h < HPW; ++h) {
        float acc = 0.f;
#pragma unroll
        for (int w = 0; w < W; ++w)
          acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(kr[u][w]), as_bf16x2(qv[h][w]), acc,
                                                false);
        acc = row16_sum(acc);
        sc[u][h] = (kbase + 4 * u < hi) ? acc : kNegInf;
      }

#pragma unroll
    for (int h = 0; h < HPW; ++h) {
      float mt = sc[0][h];
#pragma unroll
      for (int u = 1; u < kU; ++u) mt = fmaxf(mt, sc[u][h]);
      mt = wave_rows_max(mt);
      const float m_new = fmaxf(m[h], mt);
      // A wavefront that has not met a visible key yet keeps everything at
      // zero; subtract 0 instead of -inf so no inf - inf appears.
      const float mref = m_new == kNegInf ? 0.f : m_new;
      const float corr = exp2_fast((m[h] - mref) * c);
      const float mc = mref * c;
      float ls = 0.f;
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const float e = exp2_fast(fmaf(sc[u][h], c, -mc));
        sc[u][h] = e;
        ls += e;
      }
      l[h] = l[h] * corr + ls;
      m[h] = m_new;
#pragma unroll
      for (int e = 0; e < DPL; ++e) o[h][e] *= corr;
    }

#pragma unroll
    for (int u = 0; u < kU; ++u) {
      float vf[DPL];
#pragma unroll
      for (int w = 0; w < W; ++w) {
        vf[2 * w] = bf16_lo(vr[u][w]);
        vf[2 * w + 1] = bf16_hi(vr[u][w]);
      }
#pragma unroll
      for (int h = 0; h < HPW; ++h)
#pragma unroll
        for (int e = 0; e < DPL; ++e) o[h][e] = fmaf(sc[u][h], vf[e], o[h][e]);
    }
  }

  // The 4 rows of a wavefront share m: add their sums.
#pragma unroll
  for (int h = 0; h < HPW; ++h) {
    const float lw = wave_rows_sum(l[h]);
#pragma unroll
    for (int e = 0; e < DPL; ++e) o[h][e] = wave_rows_sum(o[h][e]);
    if (lane == 0) {
      red_m[wave][h] = m[h];
      red_l[wave][h] = lw;
    }
    if (row == 0) {
#pragma unroll
      for (int e = 0; e < DPL; ++e) red_o[wave][h][dl * DPL + e] = o[h][e];
    }
  }
  __syncthreads();

  // Merge the 4 wavefronts (fixed order) and write the piece's partials.
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
    const size_t pi = pidx0 + (size_t)h * p.splits;
    p.part_o[pi * D + d] = O;
    if (d == 0) {
      p.part_m[pi] = M * c;   // stored in base-2 exponent units
      p.part_l[pi] = L;
    }
  }
}

// One wavefront per (sequence, query head).
template <int D>
__global__ void __launch_bounds__(64) decode_merge_kernel(const DecodeParams p) {
  constexpr int E = D / 64;
  const int lane = threadIdx.x;
  const size_t bh = blockIdx.x;   // b * Hq + hq
  const float* pm = p.part_m + bh * p.splits;
  const float* pl = p.part_l + bh * p.splits;
  const float* po = p.part_o + bh * p.splits * D;

  float M = kNegInf;
  for (int s = 0; s < p.splits; ++s) M = fmaxf(M, pm[s]);
  float L = 0.f;
  float O[E];
#pragma unroll
  for (int e = 0; e < E; ++e) O[e] = 0.f;
  if (M != kNegInf) {
    for (int s = 0; s < p.splits; ++s) {
      const float ms = pm[s];
      if (ms == kNegInf) continue;   // empty piece
      const float wt = exp2_fast(ms - M);
      L = fmaf(wt, pl[s], L);
#pragma unroll
      for (int e = 0; e < E; ++e) O[e] = fmaf(wt, po[(size_t)s * D + lane * E + e], O[e]);
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  bf16* og = (bf16*)p.o + bh * D + lane * E;
  if constexpr (E == 2) {
    *(bf16x2*)og = to_bf16x2(O[0] * inv, O[1] * inv);
  } else {
    const bf16x2 two = to_bf16x2(O[0] * inv, 0.f);
    og[0] = two[0];
  }
}

template <int D>
hipError_t launch_decode_d(const DecodeParams& p, hipStream_t stream) {
  const int hpw = (p.g % 8 == 0) ? 8 : (p.g % 4 == 0) ? 4 : (p.g % 2 == 0) ? 2 : 1;
  dim3 grid((unsigned)p.splits, (unsigned)(p.Hkv * (p.g / hpw)), (unsigned)p.B);
  switch (hpw) {
    case 8: hipLaunchKernelGGL((decode_split_kernel<D, 8>), grid, dim3(kDecThreads), 0, stream, p); break;
    case 4: hipLaunchKernelGGL((decode_split_kernel<D, 4>), grid, dim3(kDecThreads), 0, stream, p); break;
    case 2: hipLaunchKernelGGL((decode_split_kernel<D, 2>), grid, dim3(kDecThreads), 0, stream, p); break;
    default: hipLaunchKernelGGL((decode_split_kernel<D, 1>), grid, dim3(kDecThreads), 0, stream, p); break;
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL((decode_merge_kernel<D>), dim3((unsigned)(p.B * p.Hq)), dim3(64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, int d, hipStream_t stream) {
  return d == 64 ? launch_decode_d<64>(p, stream) : launch_decode_d<128>(p, stream);
}

}  // namespace fa
