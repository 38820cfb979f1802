// FlashAttention forward (prefill) kernels for gfx950.
//
// Sources (web pages; sections named as headed there):
//   [FUSED07] "Модуль 07: Fused-операторы и FlashAttention" (hermes-agent.ru)
//   [LESSON]  "FlashAttention: внимание без матрицы n×n" (ai.flicky.cc)
//   [NOTE]    "Atencja od strony jądra: FlashAttention, softmax online i
//             połączona dekwantyzacja" (trefon.com)
//   [BOOK5]   "Глава 5. Операторы и среда выполнения" (bojieli.github.io)
//
// Algorithm ([LESSON] "Прямой проход FlashAttention"; [FUSED07] "Online
// softmax: вывод" and "FlashAttention-2"): a workgroup owns a block of query
// rows and streams the key/value sequence past it in tiles of 64 keys.  Per
// tile and row it keeps the running max m, the running sum l and the
// unnormalised output accumulator; when the max grows the old l and
// accumulator are multiplied by 2^((m_old - m_new) * c).  O = acc / l is
// written once at the end together with lse = m + log l.  Neither scores nor
// probabilities ever leave the chip.
//
// Mapping onto CDNA4:
//  * 256 threads = 4 wavefronts; each wavefront owns 32 query rows of one
//    query head.  A workgroup holds HG query heads of one grouped-query
//    group (HG = 4, 2 or 1) so every K/V tile staged in LDS serves all of
//    them ([NOTE] "Prefill i dekodowanie to różne problemy": GQA reuses
//    each K/V tile g times).
//  * Scores are computed transposed, S^T = K Q^T, with the 32x32x16 bf16
//    matrix instruction: every lane then holds one query row's scores for 16
//    keys, so the row max and row sum are in-lane reductions plus one
//    exchange between the two wave halves.  The output is accumulated
//    transposed as well, O^T += V^T P^T, so the rescale factor of a row is
//    the lane's own value and the probabilities feed the next matrix
//    instruction straight from the score registers (a consistent permutation
//    of the reduction index; no LDS round trip).
//  * K tiles are stored row-major in LDS with XOR-swizzled 16-byte chunks;
//    V tiles are stored transposed (V^T, head-dim rows, key columns) with
//    XOR-swizzled 8-byte slots, so both operand reads avoid bank conflicts
//    ([BOOK5] section 5.2.3 on spreading simultaneous requests over banks).
//  * Two LDS stages: tile t+1 is fetched into registers while tile t is
//    computed, then written to the other stage ([BOOK5] section 5.3.2,
//    double buffering, Example 5-5).
//  * Causal: key tiles starting after the workgroup's last row are never
//    visited; only tiles crossing the diagonal (or the key tail) are masked,
//    with -inf before the max ([FUSED07] task 07.2 pitfalls).  Workgroups
//    are issued heaviest query tile first.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kThreads = 256;
constexpr int kBN = 64;  // keys per tile (bf16 kernel)

// ---------------------------------------------------------------------------
// LDS layouts of the bf16 kernel
// ---------------------------------------------------------------------------

// K tile: 64 key rows x D bf16; the 16-byte chunks of a row are XOR-permuted
// so the 32 rows read by one half-wavefront land in distinct banks.
template <int D>
__device__ __forceinline__ int k_off(int row, int chunk) {
  constexpr int CPR = D / 8;
  constexpr int R = CPR >= 16 ? 1 : 16 / CPR;
  return row * D + ((chunk ^ ((row / R) % CPR)) << 3);
}

// V^T tile: D rows (head dimension) x 64 keys; 8-byte slots of 4 keys are
// XOR-permuted by the row index.
__device__ __forceinline__ int vt_off(int drow, int slot) {
  return drow * kBN + ((slot ^ ((drow >> 1) & 15)) << 2);
}

__device__ __forceinline__ uint32_t pick16(const u32x4& w, int e) {
  const uint32_t x = w[e >> 1];
  return (e & 1) ? (x >> 16) : (x & 0xffffu);
}

// ---------------------------------------------------------------------------
// bf16 forward kernel
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL, int HG>
__global__ void __launch_bounds__(kThreads, 2) fwd_bf16_kernel(const FwdParams p) {
  constexpr int WPH = 4 / HG;        // wavefronts per query head
  constexpr int BMPOS = 32 * WPH;    // query positions per workgroup
  constexpr int KT = kBN * D;        // elements of one K tile
  constexpr int VT = D * kBN;        // elements of one V^T tile
  constexpr int NC = D / 16;         // 16-deep steps of the Q.K product
  constexpr int ND = D / 32;         // 32-wide blocks of the output
  constexpr int CPR = D / 8;         // 16-byte chunks per K/V row
  constexpr int NLD = kBN * CPR / kThreads;  // 16-byte loads per thread per tile
  constexpr int RPL = kThreads / CPR;        // K rows covered by one load step
  __shared__ __attribute__((aligned(16))) bf16 lds[2 * (KT + VT)];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int col = lane & 31;

  int x = blockIdx.x;
  const int grp = x % p.groups;
  x /= p.groups;
  const int kvh = x % p.Hkv;
  const int b = x / p.Hkv;
  const int qt = CAUSAL ? (int)(gridDim.y - 1 - blockIdx.y) : (int)blockIdx.y;
  const int q0 = qt * BMPOS;
  const int hq = kvh * p.g + grp * HG + wave / WPH;
  const int q0w = q0 + (wave % WPH) * 32;
  const int my_q = q0w + col;

  const bf16* Qg = (const bf16*)p.q + (size_t)(b * p.Hq + hq) * p.Tq * D;
  const bf16* Kg = (const bf16*)p.k + (size_t)(b * p.Hkv + kvh) * p.Tk * D;
  const bf16* Vg = (const bf16*)p.v + (size_t)(b * p.Hkv + kvh) * p.Tk * D;

  // This lane's query row as the B operand of S^T = K Q^T:
  // qf[c] = q[my_q][16c + 8*half .. +8].
  bf16x8 qf[NC];
  {
    const uint32_t sgn = p.negate_q ? 0x80008000u : 0u;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (my_q < p.Tq) w = *(const u32x4*)(Qg + (size_t)my_q * D + 16 * c + 8 * half);
      w ^= sgn;
      __builtin_memcpy(&qf[c], &w, sizeof(w));
    }
  }

  // Keys this workgroup needs: all, or under the causal mask those at or
  // before its last (real) query row.
  const int q_last = min(p.Tq, q0 + BMPOS);
  const int kend = CAUSAL ? min(p.Tk, q_last) : p.Tk;
  const int ntiles = (kend + kBN - 1) / kBN;

  u32x4 kreg[NLD], vreg[NLD];
  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  auto fetch = [&](int t0) {
#pragma unroll
    for (int r = 0; r < NLD; ++r) {
      const int key = t0 + r * RPL + tid / CPR;
      kreg[r] = key < p.Tk ? *(const u32x4*)(Kg + (size_t)key * D + (tid % CPR) * 8) : zero4;
    }
#pragma unroll
    for (int r = 0; r < NLD; ++r) {
      const int key = t0 + (tid / CPR) * NLD + r;
      vreg[r] = key < p.Tk ? *(const u32x4*)(Vg + (size_t)key * D + (tid % CPR) * 8) : zero4;
    }
  };
  auto stash = [&](int stage) {
    bf16* Ks = lds + stage * (KT + VT);
    bf16* Vs = Ks + KT;
#pragma unroll
    for (int r = 0; r < NLD; ++r)
      *(u32x4*)(Ks + k_off<D>(r * RPL + tid / CPR, tid % CPR)) = kreg[r];
    // V^T: this thread holds NLD consecutive keys of one 8-wide d chunk.
    const int kg = tid / CPR;
    const int dch = (tid % CPR) * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if constexpr (NLD == 4) {
        const uint32_t w0 = pick16(vreg[0], e) | (pick16(vreg[1], e) << 16);
        const uint32_t w1 = pick16(vreg[2], e) | (pick16(vreg[3], e) << 16);
        const u32x2 w = {w0, w1};
        *(u32x2*)(Vs + vt_off(dch + e, kg)) = w;
      } else {
        static_assert(NLD == 2, "unexpected tile shape");
        const uint32_t w0 = pick16(vreg[0], e) | (pick16(vreg[1], e) << 16);
        *(uint32_t*)(Vs + vt_off(dch + e, kg >> 1) + ((kg & 1) << 1)) = w0;
      }
    }
  };

  const float c = p.c;
  float m = kNegInf;   // running max of this row's raw scores
  float l = 0.f;       // this half-wave's share of the running sum
  f32x16 acc[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;

  if (ntiles > 0) {
    fetch(0);
    stash(0);
  }
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int t0 = t * kBN;
    if (t + 1 < ntiles) fetch(t0 + kBN);
    const bf16* Ks = lds + (t & 1) * (KT + VT);
    const bf16* Vs = Ks + KT;

    // S^T for the tile's two 32-key blocks.  Under the causal mask a block
    // whose first key lies after this wavefront's last row is all masked.
    f32x16 s[2];
    bool act[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      act[kb] = !CAUSAL || (t0 + 32 * kb <= q0w + 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
      if (act[kb]) {
#pragma unroll
        for (int cc = 0; cc < NC; ++cc) {
          const bf16x8 a = *(const bf16x8*)(Ks + k_off<D>(32 * kb + col, 2 * cc + half));
          s[kb] = mma_32x32x16(a, qf[cc], s[kb]);
        }
      }
    }

    // Mask (only tiles that cross the diagonal or the key tail): -inf
    // before the max, so masked keys get probability exactly 0.
    const bool need_mask = (t0 + kBN > p.Tk) || (CAUSAL && t0 + kBN - 1 > q0w);
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = t0 + 32 * kb + 8 * (r >> 2) + 4 * half + (r & 3);
          const bool vis = act[kb] && key < p.Tk && (!CAUSAL || key <= my_q);
          s[kb][r] = vis ? s[kb][r] : kNegInf;
        }
    }

    // Online softmax update for this row.
    float mt = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[kb][r]);
    mt = fmaxf(mt, swap_halves(mt));
    const float m_new = fmaxf(m, mt);
    const float corr = exp2_fast((m - m_new) * c);
    const float mc = m_new * c;
    float ls = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = exp2_fast(fmaf(s[kb][r], c, -mc));
        s[kb][r] = e;
        ls += e;
      }
    l = l * corr + ls;
    m = m_new;
#pragma unroll
    for (int i = 0; i < ND; ++i) acc[i] *= corr;

    // O^T += V^T P^T.  The B operand for keys {16*j2 + 4*half + 0..3,
    // 16*j2 + 8 + 4*half + 0..3} of block kb is s[kb][8*j2 .. 8*j2+7];
    // the A operand reads V^T at the same keys.
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if (!act[kb]) continue;
#pragma unroll
      for (int j2 = 0; j2 < 2; ++j2) {
        bf16x8 pb;
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
          const bf16x2 two = to_bf16x2(s[kb][8 * j2 + i], s[kb][8 * j2 + i + 1]);
          pb[i] = two[0];
          pb[i + 1] = two[1];
        }
        const int slot = 8 * kb + 4 * j2 + half;
#pragma unroll
        for (int db = 0; db < ND; ++db) {
          const int drow = 32 * db + col;
          const bf16x4 lo = *(const bf16x4*)(Vs + vt_off(drow, slot));
          const bf16x4 hi = *(const bf16x4*)(Vs + vt_off(drow, slot + 2));
          const bf16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          acc[db] = mma_32x32x16(a, pb, acc[db]);
        }
      }
    }

    if (t + 1 < ntiles) stash((t + 1) & 1);
    __syncthreads();
  }

  // Finalise: one division per row; lse in natural log.
  const float lt = l + swap_halves(l);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (my_q < p.Tq) {
    bf16* Og = (bf16*)p.o + ((size_t)(b * p.Hq + hq) * p.Tq + my_q) * D;
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x2 lo = to_bf16x2(acc[db][4 * j] * inv, acc[db][4 * j + 1] * inv);
        const bf16x2 hi = to_bf16x2(acc[db][4 * j + 2] * inv, acc[db][4 * j + 3] * inv);
        *(bf16x4*)(Og + 32 * db + 8 * j + 4 * half) = __builtin_shufflevector(lo, hi, 0, 1, 2, 3);
      }
    if (p.lse != nullptr && half == 0)
      p.lse[(size_t)(b * p.Hq + hq) * p.Tq + my_q] =
          lt > 0.f ? (m * c + __builtin_amdgcn_logf(lt)) * kLn2 : kNegInf;
  }
}

// ---------------------------------------------------------------------------
// fp32 forward kernel (fp32 matrix cores, fp32 probabilities)
// ---------------------------------------------------------------------------
// Same loop; 32-key tiles, single LDS stage, one query head per workgroup.
template <int D, bool CAUSAL>
__global__ void __launch_bounds__(kThreads) fwd_f32_kernel(const FwdParams p) {
  constexpr int BN = 32;
  constexpr int KS = D + 1;   // padded K row: the 32 rows read together hit distinct banks
  constexpr int VS = D + 4;
  constexpr int ND = D / 32;
  __shared__ float Ks[BN * KS];
  __shared__ float Vs[BN * VS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int col = lane & 31;

  const int hq = blockIdx.x % p.Hq;
  const int b = blockIdx.x / p.Hq;
  const int kvh = hq / p.g;
  const int qt = CAUSAL ? (int)(gridDim.y - 1 - blockIdx.y) : (int)blockIdx.y;
  const int q0 = qt * 128;
  const int q0w = q0 + wave * 32;
  const int my_q = q0w + col;

  const float* Qg = (const float*)p.q + (size_t)(b * p.Hq + hq) * p.Tq * D;
  const float* Kg = (const float*)p.k + (size_t)(b * p.Hkv + kvh) * p.Tk * D;
  const float* Vg = (const float*)p.v + (size_t)(b * p.Hkv + kvh) * p.Tk * D;

  float qf[D / 2];
  const float sgn = p.negate_q ? -1.f : 1.f;
#pragma unroll
  for (int i = 0; i < D / 2; ++i)
    qf[i] = my_q < p.Tq ? sgn * Qg[(size_t)my_q * D + 2 * i + half] : 0.f;

  const int q_last = min(p.Tq, q0 + 128);
  const int kend = CAUSAL ? min(p.Tk, q_last) : p.Tk;
  const int ntiles = (kend + BN - 1) / BN;

  const float c = p.c;
  float m = kNegInf, l = 0.f;
  f32x16 acc[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;

  for (int t = 0; t < ntiles; ++t) {
    const int t0 = t * BN;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < BN * D / kThreads; ++i) {
      const int idx = i * kThreads + tid;
      const int row = idx / D, cc = idx % D;
      const int key = t0 + row;
      Ks[row * KS + cc] = key < p.Tk ? Kg[(size_t)key * D + cc] : 0.f;
      Vs[row * VS + cc] = key < p.Tk ? Vg[(size_t)key * D + cc] : 0.f;
    }
    __syncthreads();

    const bool act = !CAUSAL || t0 <= q0w + 31;
    if (!act) continue;
    f32x16 s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
    for (int i = 0; i < D / 2; ++i) s = mma_32x32x2_f32(Ks[col * KS + 2 * i + half], qf[i], s);

    const bool need_mask = (t0 + BN > p.Tk) || (CAUSAL && t0 + BN - 1 > q0w);
    if (need_mask) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = t0 + 8 * (r >> 2) + 4 * half + (r & 3);
        const bool vis = key < p.Tk && (!CAUSAL || key <= my_q);
        s[r] = vis ? s[r] : kNegInf;
      }
    }
    float mt = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mt = fmaxf(mt, s[r]);
    mt = fmaxf(mt, swap_halves(mt));
    const float m_new = fmaxf(m, mt);
    const float corr = exp2_fast((m - m_new) * c);
    const float mc = m_new * c;
    float ls = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s[r] = exp2_fast(fmaf(s[r], c, -mc));
      ls += s[r];
    }
    l = l * corr + ls;
    m = m_new;
#pragma unroll
    for (int i = 0; i < ND; ++i) acc[i] *= corr;
    // O^T += V^T P^T, two keys per instruction: lane half h contributes key
    // 8*(r/4) + 4*h + r%4 from its score register r.
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kl = 8 * (r >> 2) + 4 * half + (r & 3);
        acc[db] = mma_32x32x2_f32(Vs[kl * VS + 32 * db + col], s[r], acc[db]);
      }
  }

  const float lt = l + swap_halves(l);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (my_q < p.Tq) {
    float* Og = (float*)p.o + ((size_t)(b * p.Hq + hq) * p.Tq + my_q) * D;
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f32x4 v4 = {acc[db][4 * j] * inv, acc[db][4 * j + 1] * inv, acc[db][4 * j + 2] * inv,
                    acc[db][4 * j + 3] * inv};
        *(f32x4*)(Og + 32 * db + 8 * j + 4 * half) = v4;
      }
    if (p.lse != nullptr && half == 0)
      p.lse[(size_t)(b * p.Hq + hq) * p.Tq + my_q] =
          lt > 0.f ? (m * c + __builtin_amdgcn_logf(lt)) * kLn2 : kNegInf;
  }
}

template <int D, bool CAUSAL>
hipError_t launch_bf16_hg(const FwdParams& p0, hipStream_t stream) {
  FwdParams p = p0;
  const int hg = (p.g % 4 == 0) ? 4 : (p.g % 2 == 0) ? 2 : 1;
  p.groups = p.g / hg;
  const int bmpos = 128 / hg;
  dim3 grid((unsigned)(p.B * p.Hkv * p.groups), (unsigned)((p.Tq + bmpos - 1) / bmpos));
  if (hg == 4)
    hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, 4>), grid, dim3(kThreads), 0, stream, p);
  else if (hg == 2)
    hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, 2>), grid, dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, 1>), grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_f32_impl(const FwdParams& p0, hipStream_t stream) {
  FwdParams p = p0;
  p.groups = p.g;
  dim3 grid((unsigned)(p.B * p.Hq), (unsigned)((p.Tq + 127) / 128));
  hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL>), grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdParams& p, int d, bool causal, hipStream_t stream) {
  if (d == 64) return causal ? launch_bf16_hg<64, true>(p, stream) : launch_bf16_hg<64, false>(p, stream);
  return causal ? launch_bf16_hg<128, true>(p, stream) : launch_bf16_hg<128, false>(p, stream);
}

hipError_t launch_fwd_f32(const FwdParams& p, int d, bool causal, hipStream_t stream) {
  if (d == 64) return causal ? launch_f32_impl<64, true>(p, stream) : launch_f32_impl<64, false>(p, stream);
  return causal ? launch_f32_impl<128, true>(p, stream) : launch_f32_impl<128, false>(p, stream);
}

}  // namespace fa
