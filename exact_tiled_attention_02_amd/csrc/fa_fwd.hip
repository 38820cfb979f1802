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
// unnormalised output accumulator; when the reference max moves the old l
// and accumulator are multiplied by 2^((ref_old - ref_new) * c).  The bf16
// kernel moves its reference only when a row's max has outgrown it by more
// than a factor 2^16 and undoes the bf16 rounding of the largest probability
// (top_fix), which keeps the exact-max result.  O = acc / l is written once
// at the end together with lse = ref + log l.  Neither scores nor
// probabilities ever leave the chip.
//
// Mapping onto CDNA4:
//  * The bf16 kernel's workgroup is 512 threads = 8 wavefronts, two per
//    SIMD; each wavefront owns 32 query rows of one query head.  A
//    workgroup holds HG query heads of one grouped-query group (HG = 4, 2
//    or 1) so every K/V tile staged in LDS serves all of them ([NOTE]
//    "Prefill i dekodowanie to różne problemy": GQA reuses each K/V tile g
//    times).
//  * Scores are computed transposed, S^T = K Q^T, with the 32x32x16 bf16
//    matrix instruction: every lane then holds one query row's scores for 16
//    keys, so the row max and row sum are in-lane reductions plus one
//    exchange between the two wave halves.  The output is accumulated
//    transposed as well, O^T += V^T P^T, so the rescale factor of a row is
//    the lane's own value and the probabilities feed the next matrix
//    instruction straight from the score registers (a consistent permutation
//    of the reduction index; no LDS round trip).
//  * K and V tiles are copied from HBM straight into LDS (buffer-resource
//    loads with an LDS destination; keys past the end read as zeros) into
//    four stages, the copy of tile t+3 being issued while tile t is
//    computed ([BOOK5] section 5.3.2, double buffering, Example 5-5).  Both
//    tiles are row-major with XOR-swizzled chunks: K is read 16 bytes per
//    lane, V through the transposing LDS read, and neither read has bank
//    conflicts ([BOOK5] section 5.2.3 on spreading simultaneous requests
//    over banks).
//  * Causal: key tiles starting after the workgroup's last row are never
//    visited; only tiles crossing the diagonal (or the key tail) are masked,
//    with -inf before the max ([FUSED07] task 07.2 pitfalls).  The diagonal
//    is top-left (row i sees keys j <= i) or, for a chunk of queries at the
//    end of a cached sequence, bottom-right (j <= i + Tk - Tq).  On small
//    causal grids a workgroup pairs a light and the mirrored heavy half-tile
//    of query rows so that all workgroups carry the same work, splitting
//    the keys of every tile between wavefront pairs when the grid holds
//    about one workgroup per compute unit.
#include <type_traits>

#include "fa_device.h"
#include "fa_launch.h"
#include "fa_lds.h"

namespace fa {
namespace {

constexpr int kThreads = 256;
constexpr int kBN = 64;  // keys per tile (bf16 kernel)

// ---------------------------------------------------------------------------
// LDS layouts of the bf16 kernel
// ---------------------------------------------------------------------------
// LDS holds [K stage 0 | K stage 1 | V stage 0 | V stage 1], each tile 64 key
// rows x D bf16, row-major exactly as in HBM, filled by direct global->LDS
// copies (16 bytes per lane).  Only the order of the 16-byte chunks inside a
// row is permuted (XOR swizzle), differently for the two tiles because they
// are read in different patterns:
//  * K is read 16 bytes per lane, 32 rows at one chunk position; the swizzle
//    spreads 16 consecutive rows over all banks.
//  * V is read through the transposing LDS read, 8 bytes per lane from 4
//    consecutive rows; the swizzle moves those 4 rows to distinct banks.
// Both swizzles depend on row bits that are the same for every row a given
// lane reads, so each lane's operand addresses are a fixed base plus
// compile-time offsets.
template <int D>
__device__ __forceinline__ int k_swz(int row) {
  return D == 128 ? (row & 15) : ((row >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int v_swz(int row) {
  return D == 128 ? ((row & 3) << 2) : (((row >> 1) & 1) << 2);
}


// Wait until at most N LDS reads of this wavefront are outstanding (they
// complete in issue order); the operand group passed in is tied to the wait
// so its uses cannot be scheduled before it.
template <int N, int ND>
__device__ __forceinline__ void lds_tr_wait(u32x2 (&v)[ND][2]) {
  static_assert(ND == 2 || ND == 4, "unexpected operand group");
  if constexpr (ND == 4)
    asm volatile("s_waitcnt lgkmcnt(%8)"
                 : "+v"(v[0][0]), "+v"(v[0][1]), "+v"(v[1][0]), "+v"(v[1][1]), "+v"(v[2][0]),
                   "+v"(v[2][1]), "+v"(v[3][0]), "+v"(v[3][1])
                 : "n"(N));
  else
    asm volatile("s_waitcnt lgkmcnt(%4)"
                 : "+v"(v[0][0]), "+v"(v[0][1]), "+v"(v[1][0]), "+v"(v[1][1])
                 : "n"(N));
}



__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Lazy reference of the bf16 kernel: the accumulator is rescaled only when a
// row's max has grown past its reference by more than this many powers of 2.
// fp32 and bf16 have the same relative precision at any magnitude, so the
// bound only keeps the sums far from overflow: probabilities stay below
// 2^16, row sums below 2^16 per key.
constexpr float kLazyLog2 = 16.f;

// x / bf16(x).  The accumulator holds bf16-rounded probabilities times V
// while l sums them unrounded, so a row dominated by one key would come out
// scaled by that key's rounding ratio.  Against an exact running max the
// largest probability is exactly 1 and has no rounding; against a lazy
// reference it is 2^(m*c + nmc) in [1, 2^kLazyLog2], computed by the same
// expression as in the tile, and multiplying the accumulator by this
// ratio (at each move of the reference and at the end) undoes its rounding.
__device__ __forceinline__ float top_fix(float x) {
  const float r = (float)to_bf16x2(x, x)[0];
  return x / r;
}

// ---------------------------------------------------------------------------
// bf16 forward kernel
// ---------------------------------------------------------------------------
// A workgroup is 8 wavefronts (two per SIMD); each wavefront owns 32 query
// rows of one query head and all 8 share every K/V tile staged in LDS.  LDS
// holds kStages K tiles and kStages V tiles; the copy of tile t+3 is issued
// while tile t is computed, so a copy has three iterations to land.
constexpr int kFwdThreads = 512;
constexpr int kStages = 4;

template <int D, bool CAUSAL, int HG, bool KSPLIT>
__global__ void __launch_bounds__(kFwdThreads, 1) fwd_bf16_kernel(const FwdParams p) {
  static_assert(!KSPLIT || CAUSAL, "the key split only balances causal work");
  constexpr int NW = kFwdThreads / 64;
  constexpr int WPH = NW / HG;       // wavefronts per query head
  constexpr int BMPOS = 32 * WPH;    // query positions per workgroup
  // Key split: wavefronts w and w + NW/2 own the same 32 query rows and take
  // the first and the second 64 keys of every 128-key tile; their partial
  // (m, l, acc) are merged at the end of each pass.  Two LDS stages of
  // 128-key tiles take the place of four stages of 64-key tiles.
  constexpr int BN = KSPLIT ? 2 * kBN : kBN;             // keys per tile
  constexpr int STAGES = KSPLIT ? kStages / 2 : kStages;
  constexpr int RPH = KSPLIT ? WPH / 2 : WPH;             // 32-row blocks per query head
  constexpr int NPASS = KSPLIT ? 2 : 1;                   // passes over the keys
  constexpr int TILE = BN * D;       // elements of one K or V tile
  constexpr int NC = D / 16;         // 16-deep steps of the Q.K product
  constexpr int ND = D / 32;         // 32-wide blocks of the output
  constexpr int CPR = D / 8;         // 16-byte chunks per row
  constexpr int NCOPY = TILE / 8 / kFwdThreads;   // 16-byte copies per thread per tile and tensor
  static_assert(NCOPY >= 1 && TILE / 8 % kFwdThreads == 0, "tile does not split over the workgroup");
  __shared__ __attribute__((aligned(16))) bf16 lds[2 * STAGES * TILE];   // K stages | V stages
  // Key split: (m, reference, l) of the second key half, handed over at the
  // end of a pass.
  __shared__ f32x4 xch_sc[KSPLIT ? (NW / 2) * 64 : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int col = lane & 31;
  const int kh = KSPLIT ? wave / (NW / 2) : 0;     // key half of every tile
  const int rw = KSPLIT ? wave % (NW / 2) : wave;  // row block

  int x = blockIdx.x;
  const int grp = x % p.groups;
  x /= p.groups;
  const int kvh = x % p.Hkv;
  const int b = x / p.Hkv;
  const int hq = kvh * p.g + grp * HG + rw / RPH;

  const bf16* Qg = (const bf16*)p.q + (size_t)(b * p.Hq + hq) * p.Tq * D;
  const bf16* Kg = (const bf16*)p.k + (size_t)(b * p.Hkv + kvh) * p.Tk * D;
  const bf16* Vg = (const bf16*)p.v + (size_t)(b * p.Hkv + kvh) * p.Tk * D;

  // Rows of this wavefront in pass `pass`: q0w .. q0w + 31; q_end is one past
  // the workgroup's last row in that pass.
  //  * Causal with many workgroups per compute unit: one pass; the hardware
  //    dispatcher evens out the triangle, heaviest query tile first.
  //  * Causal grids under 4 workgroups per compute unit (p.pair): a
  //    workgroup owns, per query head, two half-tiles of BMPOS/2 rows, light
  //    half-tile i (few visible keys) and the mirrored heavy half-tile
  //    nh-1-i, so every workgroup carries the same work.
  //    - Key split (up to about one such workgroup per compute unit): the
  //      heavy half-tile in one pass and the light one in the other
  //      (skipped when both are the middle one), both wavefronts of a SIMD
  //      busy through both passes.
  //    - Otherwise one pass; the two wavefronts that share a SIMD (w and
  //      w+4) get one light and one heavy block.
  int q0w = 0, q_end = 0;
  bool active = true;  // false: nothing to compute in this pass
  auto rows_of = [&](int pass, int& q0w, int& q_end, bool& active) {
    if constexpr (KSPLIT) {
      constexpr int HALF = BMPOS / 2;
      const int nh = (p.Tq + HALF - 1) / HALF;
      const int i = blockIdx.y;
      // Odd workgroups take the light half-tile first, so that the passes
      // of different workgroups end at different times and the loads and
      // stores between them do not all compete at once.
      const bool light_first = i & 1;
      const int first = light_first ? i : nh - 1 - i;
      const int second = light_first ? nh - 1 - i : i;
      const int ht = pass == 0 ? first : second;
      active = pass == 0 || first != second;
      q0w = ht * HALF + (rw % RPH) * 32;
      q_end = min(p.Tq, (ht + 1) * HALF);
    } else if (CAUSAL && p.pair) {
      constexpr int HALF = BMPOS / 2;
      const int nh = (p.Tq + HALF - 1) / HALF;
      const int i = blockIdx.y;
      const int hh = wave % WPH;
      const bool heavy = (wave >= 4) != ((WPH < 8) && (hh >= WPH / 2));
      const int ht = heavy ? nh - 1 - i : i;
      active = !(heavy && ht == i);
      q0w = ht * HALF + (hh % (WPH / 2)) * 32;
      q_end = min(p.Tq, (nh - i) * HALF);
    } else {
      const int qt = CAUSAL ? (int)(gridDim.y - 1 - blockIdx.y) : (int)blockIdx.y;
      q0w = qt * BMPOS + (wave % WPH) * 32;
      q_end = min(p.Tq, (qt + 1) * BMPOS);
    }
  };
  const int off = p.causal_off;   // causal: row i sees key j iff j <= i + off
  // Key tiles a pass over rows ending before q_end needs: all, or under the
  // causal mask those at or before its last (real) query row's limit.
  auto tiles_of = [&](int q_end) {
    const int kend = CAUSAL ? max(0, min(p.Tk, q_end + off)) : p.Tk;
    return (kend + BN - 1) / BN;
  };

  // Global->LDS copies through buffer resources covering this head's K and
  // V: reads past the last key return zeros (finite; those keys are masked).
  // Copy r of wavefront w fills LDS chunks [(r*NW + w)*64, +64) of a tile;
  // chunk L is row L / CPR, physical chunk L % CPR, which holds logical
  // chunk (L % CPR) ^ swizzle(row).  Lane byte offsets within a tile are
  // constants; the tile start is added to them (not passed as the scalar
  // offset, which the buffer range check does not include).
  const int nbytes = p.Tk * D * 2;
  const __amdgpu_buffer_rsrc_t krsrc = __builtin_amdgcn_make_buffer_rsrc((void*)Kg, 0, nbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrsrc = __builtin_amdgcn_make_buffer_rsrc((void*)Vg, 0, nbytes, 0x00020000);
  uint32_t ksrc[NCOPY], vsrc[NCOPY];
#pragma unroll
  for (int r = 0; r < NCOPY; ++r) {
    const int L = (r * NW + wave) * 64 + lane;
    const int row = L / CPR;
    const int pc = L % CPR;
    ksrc[r] = (uint32_t)(row * D + ((pc ^ k_swz<D>(row)) << 3)) * 2u;
    vsrc[r] = (uint32_t)(row * D + ((pc ^ v_swz<D>(row)) << 3)) * 2u;
  }
  auto issue_copies = [&](int t) {   // tile t into stage t % STAGES
    const int st = t % STAGES;
    const uint32_t soff = (uint32_t)t * BN * D * 2;
    bf16* Kd = lds + st * TILE;
    bf16* Vd = lds + (STAGES + st) * TILE;
#pragma unroll
    for (int r = 0; r < NCOPY; ++r) {
      copy16_buf_to_lds(krsrc, Kd + (r * NW + wave) * 512, ksrc[r] + soff, 0);
      copy16_buf_to_lds(vrsrc, Vd + (r * NW + wave) * 512, vsrc[r] + soff, 0);
    }
  };
  // Wait until the copies of tile t (issued `later` tiles before the newest
  // ones) have landed: the vector-memory counter counts 2*NCOPY per tile.
  auto wait_copies = [&](int later) {
    if (later >= 2)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm<4 * NCOPY>());
    else if (later == 1)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm<2 * NCOPY>());
    else
      __builtin_amdgcn_s_waitcnt(vmcnt_imm<0>());
  };

  // K operand read bases (stage 0, key block 0 of this wavefront's keys):
  // stage s adds s*TILE and key block kb adds 32*kb*D elements.  k_swz of
  // rows 64*kh + 32*kb + col is k_swz(col).
  uint32_t kread[NC];
  {
    const int sw = k_swz<D>(col);
#pragma unroll
    for (int cc = 0; cc < NC; ++cc)
      kread[cc] = lds_addr(lds + (64 * kh + col) * D + (((2 * cc + half) ^ sw) << 3));
  }
  // V operand bases for the transposing reads: input lane 4j + q of 16-lane
  // group G addresses 4 head-dim values starting at 32*db + 16*(G%2) + 4q
  // of key row 64*kh + 4*half + j (+ 32*kb + 16*j2 + 8*hi, a compile-time
  // offset); v_swz is the same for all of those rows.
  uint32_t vread[ND];
  {
    const int tr_j = (lane & 15) >> 2;
    const int tr_d = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    const int r0 = 4 * half + tr_j;
    const int sw = v_swz<D>(r0);
#pragma unroll
    for (int db = 0; db < ND; ++db) {
      const int dd = 32 * db + tr_d;
      vread[db] = lds_addr(lds + STAGES * TILE + (64 * kh + r0) * D + (((dd >> 3) ^ sw) << 3) + (dd & 7));
    }
  }

  const float c = p.c;
  const float lazy_raw = kLazyLog2 / c;
  // This lane's query row as the B operand of S^T = K Q^T:
  // qf[c] = q[row][16c + 8*half .. +8].  The sign flip (negative scale) sits
  // behind a uniform branch so that, without it, nothing waits for the
  // loads before the first product and the first key tile's copies are
  // issued while they are in flight.
  bf16x8 qf[NC];
  auto load_q = [&](int row) {
    u32x4 w[NC];
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
      w[cc] = u32x4{0u, 0u, 0u, 0u};
      if (row < p.Tq) w[cc] = *(const u32x4*)(Qg + (size_t)row * D + 16 * cc + 8 * half);
    }
    if (p.negate_q) {
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) w[cc] ^= 0x80008000u;
    }
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) __builtin_memcpy(&qf[cc], &w[cc], sizeof(w[cc]));
  };

  // Key split: the next pass's query rows and first key tile are loaded
  // while this pass's halves merge and its output is written.
  bool prefetched = false;
  for (int pass = 0; pass < NPASS; ++pass) {
    rows_of(pass, q0w, q_end, active);
    if (KSPLIT && !active) break;   // the same for the whole workgroup
    const int my_q = q0w + col;
    if (!prefetched) load_q(my_q);

    const int ntiles = tiles_of(q_end);
    // Last tile this wavefront computes: its rows see none of its keys
    // after it.
    const int lim = q0w + 31 + off - 64 * kh;
    const int my_tiles = !active ? 0 : CAUSAL ? (lim < 0 ? 0 : min(ntiles, lim / BN + 1)) : ntiles;

    // Probabilities are taken against a reference max that moves only when
    // some row's max exceeds its reference by more than 2^kLazyLog2 in
    // probability (see the update below).  nmc = -reference * c (0 until
    // the row has seen a key), and thr is the raw score past which the
    // reference must move.
    float m = kNegInf;   // running max of this row's raw scores
    float nmc = 0.f;
    float thr = kNegInf;
    // At d = 128 the score products start from minus the reference (raw
    // units; 0 until the row has seen a key) instead of 0, so that the
    // exponent argument is one multiplication, s' * c, rather than an FMA.
    constexpr bool SHIFT = D == 128;
    float nref = 0.f;
    f32x16 sinit;
#pragma unroll
    for (int r = 0; r < 16; ++r) sinit[r] = 0.f;
    float l = 0.f;       // this half-wave's share of the running sum
    f32x16 acc[ND];
#pragma unroll
    for (int i = 0; i < ND; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;

    if (!prefetched)
      for (int t = 0; t < min(ntiles, STAGES - 1); ++t) issue_copies(t);
    prefetched = false;

    // One key tile; ST = t % STAGES is a compile-time constant, so every
    // LDS operand address is a per-lane base plus an immediate offset.
    auto tile = [&](int t, auto st_c) {
      constexpr int ST = decltype(st_c)::value;
      const int t0 = t * BN + 64 * kh;   // this wavefront's first key
      wait_copies(min(ntiles - 1 - t, STAGES - 2));
      tile_barrier();   // tile t visible to all; stage (t-1) % STAGES free
      if (t + STAGES - 1 < ntiles) issue_copies(t + STAGES - 1);
      if (t >= my_tiles) return;   // still copies and meets the barriers

      // S^T for the wavefront's two 32-key blocks (on the diagonal tile a
      // block may be entirely masked; it is computed anyway and masked
      // below).  K operand I = 2*cc + kb is read PF operands ahead of its
      // instruction; the two key blocks alternate so that consecutive
      // instructions are independent.
      f32x16 s[2];
      {
        constexpr int NF = 2 * NC;
        constexpr int PF = NF < 8 ? NF : 8;
        bf16x8 kf[NF];
        auto read_k = [&](auto i_c) {
          constexpr int I = decltype(i_c)::value;
          kf[I] = lds_read_b128<(ST * TILE + (I & 1) * 32 * D) * 2>(kread[I >> 1]);
        };
        static_for<0, PF>(read_k);
        static_for<0, NF>([&](auto i_c) {
          constexpr int I = decltype(i_c)::value;
          constexpr int AFTER = I + PF <= NF ? PF - 1 : NF - 1 - I;
          lds_wait_tie<AFTER>(kf[I]);
          s[I & 1] = mma_32x32x16(kf[I], qf[I >> 1], I < 2 ? (SHIFT ? sinit : f32x16{}) : s[I & 1]);
          __builtin_amdgcn_sched_barrier(0);   // issued before the next wait, not sunk past it
          if constexpr (I + PF < NF) read_k(IC<I + PF>{});
        });
      }

      // Mask (only blocks that cross the diagonal or the key tail): -inf
      // before the max, so masked keys get probability exactly 0.
      const bool need_mask = (t0 + 64 > p.Tk) || (CAUSAL && t0 + 63 > q0w + off);
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = t0 + 32 * kb + 8 * (r >> 2) + 4 * half + (r & 3);
            const bool vis = key < p.Tk && (!CAUSAL || key <= my_q + off);
            s[kb][r] = vis ? s[kb][r] : kNegInf;
          }
      }

      // Row max of the tile: a chain of 3-input maxima in-lane, then across
      // the two wave halves.
      float mt = fmaxf(s[0][0], s[0][1]);
#pragma unroll
      for (int i = 2; i < 32; i += 2)
        mt = fmaxf(fmaxf(mt, s[i >> 4][i & 15]), s[(i + 1) >> 4][(i + 1) & 15]);
      mt = max_halves(mt);
      if constexpr (SHIFT) mt -= nref;   // back to raw units

      // Online update.  The running max m is exact; the reference the
      // probabilities are taken against moves to it only when some row of
      // the wavefront has outgrown its reference by more than 2^kLazyLog2
      // ([FUSED07] "FlashAttention-2": rescale only when the maximum has
      // increased; here only when it has increased by that much).  Between
      // moves a probability may exceed 1 (by at most 2^kLazyLog2), which
      // fp32 and bf16 represent with the same relative precision.  A row
      // that has seen no key keeps nmc = 0, so its masked scores give 0.
      const float m_prev = m;
      m = fmaxf(m, mt);
      if (__builtin_amdgcn_ballot_w64(m > thr) != 0) {
        const float nmc_new = m > kNegInf ? -m * c : 0.f;
        // Rows without a previous key hold acc = l = 0 and take factor 0;
        // the others also undo the bf16 rounding of their largest
        // probability so far (see top_fix).
        const bool seen = m_prev > kNegInf;
        const float corr = seen ? exp2_fast(nmc_new - nmc) : 0.f;
        const float fold = seen ? top_fix(exp2_fast(SHIFT ? (m_prev + nref) * c : fmaf(m_prev, c, nmc))) : 1.f;
        const float f = corr * fold;
        if (__builtin_amdgcn_ballot_w64(seen) != 0) {   // else acc is still 0
#pragma unroll
          for (int i = 0; i < ND; ++i) acc[i] *= f;
        }
        l *= corr;
        nmc = nmc_new;
        thr = m + lazy_raw;
        if constexpr (SHIFT) {
          // This tile's scores were shifted by the old reference: move them
          // to the new one, and start the next tiles' products from it.
          const float nref_new = m > kNegInf ? -m : 0.f;
          const float dlt = nref_new - nref;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) s[kb][r] += dlt;
          nref = nref_new;
#pragma unroll
          for (int r = 0; r < 16; ++r) sinit[r] = nref;
        }
      }
      float ls[4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          s[kb][r] = exp2_fast(SHIFT ? s[kb][r] * c : fmaf(s[kb][r], c, nmc));
          ls[r & 3] = kb == 0 && r < 4 ? s[kb][r] : ls[r & 3] + s[kb][r];   // four partial sums
        }
      l += (ls[0] + ls[1]) + (ls[2] + ls[3]);

      // O^T += V^T P^T in four groups g = (kb, j2).  The B operand for keys
      // {16*j2 + 4*half + 0..3, 16*j2 + 8 + 4*half + 0..3} of block kb is
      // s[kb][8*j2 .. 8*j2+7]; the A operand holds V at the same keys for
      // head-dim rows 32*db + col, read transposed from the row-major tile.
      // The reads of group g+1 are in flight while group g multiplies.  A
      // block that is entirely masked has probabilities 0 and is multiplied
      // anyway (this happens only on the diagonal tile).
      auto issue_v = [&](auto g_c, u32x2 (&v)[ND][2]) {
        constexpr int G = decltype(g_c)::value;
        constexpr int OFF = (ST * TILE + (32 * (G >> 1) + 16 * (G & 1)) * D) * 2;
        static_for<0, ND>([&](auto db_c) {
          constexpr int DB = decltype(db_c)::value;
          v[DB][0] = lds_read_tr<OFF>(vread[DB]);
          v[DB][1] = lds_read_tr<OFF + 8 * D * 2>(vread[DB]);
        });
      };
      auto multiply = [&](auto g_c, u32x2 (&v)[ND][2]) {
        constexpr int G = decltype(g_c)::value;
        constexpr int KB = G >> 1, J2 = G & 1;
        bf16x8 pb;
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
          const bf16x2 two = to_bf16x2(s[KB][8 * J2 + i], s[KB][8 * J2 + i + 1]);
          pb[i] = two[0];
          pb[i + 1] = two[1];
        }
#pragma unroll
        for (int db = 0; db < ND; ++db) {
          const u32x4 w = {v[db][0][0], v[db][0][1], v[db][1][0], v[db][1][1]};
          bf16x8 a;
          __builtin_memcpy(&a, &w, sizeof(a));
          acc[db] = mma_32x32x16(a, pb, acc[db]);
        }
      };
      {
        constexpr int NR = 2 * ND;   // LDS reads per group
        u32x2 va[ND][2], vb[ND][2];
        issue_v(IC<0>{}, va);
        issue_v(IC<1>{}, vb);
        lds_tr_wait<NR>(va);
        multiply(IC<0>{}, va);
        issue_v(IC<2>{}, va);
        lds_tr_wait<NR>(vb);
        multiply(IC<1>{}, vb);
        issue_v(IC<3>{}, vb);
        lds_tr_wait<NR>(va);
        multiply(IC<2>{}, va);
        lds_tr_wait<0>(vb);
        multiply(IC<3>{}, vb);
      }
    };
    for (int t = 0; t < ntiles; t += STAGES) {
      static_for<0, STAGES>([&](auto s_c) {
        if (t + decltype(s_c)::value < ntiles) tile(t + decltype(s_c)::value, s_c);
      });
    }

    // The bf16 rounding of the row's largest probability, undone (top_fix):
    // folded into the final scale, or applied before the key halves merge.
    const float fix = m > kNegInf ? top_fix(exp2_fast(SHIFT ? (m + nref) * c : fmaf(m, c, nmc))) : 1.f;
    if constexpr (KSPLIT) {
#pragma unroll
      for (int i = 0; i < ND; ++i) acc[i] *= fix;
    }

    if constexpr (KSPLIT) {
      // The two key halves of the same rows combine by the rescale rule
      // against the larger of their references: the second-half wavefront
      // hands its (m, nmc, l, acc) over through LDS (one 16-byte vector per
      // lane and slot, so the accesses are conflict-free).  Every tile of
      // the pass has been consumed and no copy is in flight (with two
      // stages each tile waits for all copies issued before it).
      tile_barrier();
      // Stage 0 is free from here on: the next pass's query rows and first
      // key tile start loading now.  The accumulators travel through the
      // stage-1 K and V tiles, which the next pass fills only after its
      // first tile's barrier, when every wavefront is past this exchange.
      if (pass + 1 < NPASS) {
        int nq0w = 0, nq_end = 0;
        bool nactive = false;
        rows_of(pass + 1, nq0w, nq_end, nactive);
        if (nactive && tiles_of(nq_end) > 0) {
          load_q(nq0w + col);
          issue_copies(0);
          prefetched = true;
        }
      }
      static_assert(2 * 4 * ND * 64 * 16 <= TILE * 2, "exchange exceeds a stage-1 tile");
      f32x4* xacc = (f32x4*)(lds + (rw < 2 ? 1 : STAGES + 1) * TILE) + (rw & 1) * 4 * ND * 64 + lane;
      f32x4* xsc = xch_sc + rw * 64 + lane;
      if (kh == 1) {
        xsc[0] = f32x4{m, nmc, l, 0.f};
#pragma unroll
        for (int db = 0; db < ND; ++db)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            xacc[(4 * db + j) * 64] = f32x4{acc[db][4 * j], acc[db][4 * j + 1], acc[db][4 * j + 2],
                                            acc[db][4 * j + 3]};
      }
      tile_barrier();
      if (kh == 0) {
        const f32x4 o = xsc[0];
        const bool la = m > kNegInf, lb = o[0] > kNegInf;
        const float nmc_r = la && lb ? fminf(nmc, o[1]) : la ? nmc : o[1];
        const float fa = la ? exp2_fast(nmc_r - nmc) : 0.f;
        const float fb = lb ? exp2_fast(nmc_r - o[1]) : 0.f;
        l = l * fa + o[2] * fb;
        m = fmaxf(m, o[0]);
        nmc = nmc_r;
#pragma unroll
        for (int db = 0; db < ND; ++db)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const f32x4 o2 = xacc[(4 * db + j) * 64];
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[db][4 * j + e] = acc[db][4 * j + e] * fa + o2[e] * fb;
          }
      }
    }

    // Finalise: one division per row; lse in natural log.
    const float lt = sum_halves(l);
    const float inv = lt > 0.f ? (KSPLIT ? 1.f : fix) / lt : 0.f;
    if (active && kh == 0 && my_q < p.Tq) {
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
            lt > 0.f ? (__builtin_amdgcn_logf(lt) - nmc) * kLn2 : kNegInf;
    }
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
  const int off = p.causal_off;   // causal: row i sees key j iff j <= i + off
  const int kend = CAUSAL ? max(0, min(p.Tk, q_last + off)) : p.Tk;
  const int ntiles = (kend + BN - 1) / BN;
  const bool has_keys = !CAUSAL || my_q + off >= 0;

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

    const bool act = !CAUSAL || t0 <= q0w + 31 + off;
    if (!act) continue;
    f32x16 s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
    for (int i = 0; i < D / 2; ++i) s = mma_32x32x2_f32(Ks[col * KS + 2 * i + half], qf[i], s);

    const bool need_mask = (t0 + BN > p.Tk) || (CAUSAL && t0 + BN - 1 > q0w + off);
    if (need_mask) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = t0 + 8 * (r >> 2) + 4 * half + (r & 3);
        const bool vis = key < p.Tk && (!CAUSAL || key <= my_q + off);
        s[r] = vis ? s[r] : kNegInf;
      }
    }
    float mt = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mt = fmaxf(mt, s[r]);
    mt = fmaxf(mt, swap_halves(mt));
    const float m_new = fmaxf(m, mt);
    const float corr = has_keys ? exp2_fast((m - m_new) * c) : 1.f;
    const float mc = has_keys ? m_new * c : 0.f;
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

template <int D, bool CAUSAL, bool KSPLIT>
void launch_bf16_grid(int hg, dim3 grid, const FwdParams& p, hipStream_t stream) {
  if (hg == 4)
    hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, 4, KSPLIT>), grid, dim3(kFwdThreads), 0, stream, p);
  else if (hg == 2)
    hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, 2, KSPLIT>), grid, dim3(kFwdThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, 1, KSPLIT>), grid, dim3(kFwdThreads), 0, stream, p);
}

template <int D, bool CAUSAL>
hipError_t launch_bf16_hg(const FwdParams& p0, hipStream_t stream) {
  FwdParams p = p0;
  const int hg = (p.g % 4 == 0) ? 4 : (p.g % 2 == 0) ? 2 : 1;
  p.groups = p.g / hg;
  const int bmpos = 32 * (kFwdThreads / 64) / hg;
  const int nx = p.B * p.Hkv * p.groups;
  const int ny = (p.Tq + bmpos - 1) / bmpos;
  // Causal work per query tile grows with its position.  With many
  // workgroups per compute unit the hardware dispatcher evens that out
  // (heaviest first); with fewer, each workgroup takes a light and the
  // mirrored heavy half-tile.  Up to about one such workgroup per compute
  // unit it does them one after the other with the key split (measured
  // 5-14% faster there, 3% slower at two per compute unit).
  p.pair = 0;
  if (CAUSAL && (long long)nx * ny < 4LL * compute_units()) {
    const int half = bmpos / 2;
    const int nyp = ((p.Tq + half - 1) / half + 1) / 2;
    const dim3 grid((unsigned)nx, (unsigned)nyp);
    p.pair = 1;
    if constexpr (CAUSAL) {
      if (2LL * nx * nyp <= 3LL * compute_units())
        launch_bf16_grid<D, true, true>(hg, grid, p, stream);
      else
        launch_bf16_grid<D, true, false>(hg, grid, p, stream);
    }
  } else {
    launch_bf16_grid<D, CAUSAL, false>(hg, dim3((unsigned)nx, (unsigned)ny), p, stream);
  }
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
