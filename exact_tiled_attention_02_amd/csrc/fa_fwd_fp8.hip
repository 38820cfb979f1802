// FlashAttention forward (prefill) over 8-bit inputs for gfx950.
//
// Sources (web pages; sections named as headed there):
//   [LESSON] "FlashAttention: внимание без матрицы n×n" (ai.flicky.cc),
//            section "Прямой проход FlashAttention" (the tiled loop) and
//            section "FlashAttention-2, -3 и дальше" (FA-3: FP8 with block
//            scaling).
//   [FA3QA]  "Как работает FlashAttention-3 математически?" (aivaro.ru),
//            section 6 (FP8 support: E4M3 inputs, higher-precision
//            accumulation).
//   [BOOK5]  "Глава 5. Операторы и среда выполнения" (bojieli.github.io),
//            section 5.4.3, Example 5-7 (a row scale is fixed by the whole
//            row's maximum before any element is quantised).
//
// Inputs are E4M3 codes with block scales: every query row has its own
// scale (q_i = qs_i * e4m3(q8_i)), and each (batch, kv head) has one scale
// for K and one for V.  The result is exact attention of those dequantised
// inputs up to the rounding stated here: q.k products of 8-bit values are
// exact; the matrix core (32x32x64 8-bit MFMA) adds the 64 of a block with
// terms far below the block's largest product partly dropped (measured:
// 448^2 plus 63 products of 1 came out 448^2 + 56) and the blocks in fp32;
// the online softmax runs in fp32 as in the bf16 kernel; the probabilities are
// rounded to E4M3 for the P.V product, which is the one rounding step that
// the 16-bit kernel does in bf16.  Each tile's probabilities are coded
// against their own power-of-two scale, so that the tile's largest lands
// between 224 and 448, within the largest code (see kF8Headroom); the scale
// goes to the P.V product as the matrix instruction's block scale of the P
// operand.  Codes below the normal range carry an absolute error of at most
// 2^-10, i.e. at most 2^(kF8Headroom-10) / 448 in units of the row's
// largest probability.
//
// Mapping onto CDNA4 (the bf16 kernel's design with 8-bit operands):
//  * 512 threads = 8 wavefronts of 32 query rows; HG query heads of a GQA
//    group share each K/V tile; 4 LDS stages filled by buffer-resource
//    copies three tiles ahead; causal pairing of light and heavy half-tiles
//    on small grids.
//  * S^T = K Q^T with one 32x32x64 MFMA per 64 head dimensions: lane l
//    supplies 32 bytes of its key row (A) or query row (B) for head
//    dimensions 64c + 32*(l/32) .. +32; the instruction sums over both lane
//    halves' bytes, so any byte order used alike on both sides is correct.
//  * O^T += V^T P^T with one MFMA per 64 keys and 32 head dimensions: the
//    probabilities come straight from the score registers (byte p of lane l
//    is key kappa(p) = 16*(p/8) + 8*((p%8)/4) + 4*(l/32) + p%4 of the tile),
//    and V^T is gathered with the gfx950 transposing 8-bit LDS read in the
//    same key order.
#include "fa_device.h"
#include "fa_launch.h"
#include "fa_lds.h"

namespace fa {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kF8Threads = 512;
constexpr int kF8Stages = 4;
constexpr int kF8BN = 64;                  // keys per tile
constexpr float kLog2E4M3Max = 8.807354922057604f;   // log2(448)
// Bits of probability between a tile's largest probability and the largest
// E4M3 value.  A row's reference m is the max of its first tile with a
// visible key.  The probabilities of a tile whose max is mt are coded as
// 448 * 2^-kF8Headroom * 2^((s - m) cq - k) with k = floor((mt - m) cq), so
// they never pass 448 and the tile's largest is at least 224; the factor 2^k
// is the P operand's block scale in P.V (exponent 127 + k) and multiplies
// the tile's share of the row sum.  Accumulator and row sum thus stay against
// m; m moves (and they are rescaled) only when a tile's max passes it by more
// than kF8MaxShift bits, which keeps them far from overflow.  Tiles more
// than 126 bits below m are coded with k = -126.
constexpr float kF8Headroom = 1.f;
constexpr float kF8MaxShift = 32.f;
constexpr float kF8Offset = kF8Headroom - kLog2E4M3Max;   // one constant in the exponent offset

// Byte tiles (rows x D codes, row-major): 16-byte chunk c of row r sits at
// position c ^ f8swz(r).  The function depends only on row bits that
// separate rows sharing an LDS bank line (1..3 at 128-byte rows, 2..3 at
// 64-byte rows): 16 consecutive rows read at one chunk hit distinct banks,
// and so do the 8 rows {0..3, 8..11} (+4) that one transposing read
// gathers, also together with the neighbouring 16-lane group that reads the
// adjacent chunk (at 128-byte rows those rows get even or odd values only).
// Rows r and r + 16i get the same value.
template <int D>
__device__ __forceinline__ int f8swz(int r) {
  return D == 128 ? ((((r >> 1) & 1) << 1) | (((r >> 3) & 1) << 2) | ((r >> 2) & 1)) : ((r >> 2) & 3);
}

// 32x32x64 MFMA on E4M3 operands with unit block scales.
__device__ __forceinline__ f32x16 mma_f8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}
// The same with B's block scale 2^(sb - 127) (E8M0 exponent byte sb, 1..254)
// given per lane: lane l scales column l % 32 over its 32 values of the
// contraction (probed on the device).
__device__ __forceinline__ f32x16 mma_f8_sb(i32x8 a, i32x8 b, f32x16 c, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, sb);
}

// Reference move and block-scale exponent for a tile whose max is mt (see
// kF8Headroom): on return m0 is the reference to use, mv whether it moved
// to mt (then acc and l need the factor 2^-x), k the exponent.  Written with
// selects only: a branch here would split the tile's code.
__device__ __forceinline__ void f8_plan(float m, float mt, float cq, float& m0, bool& mv, int& k,
                                        float& x) {
  const float r = m > kNegInf ? m : mt;   // the first tile with a key sets the reference
  x = (mt - r) * cq;                      // NaN when neither has a key
  mv = x > kF8MaxShift;
  m0 = mv ? mt : r;
  // Without a move x <= kF8MaxShift; a tile with no key (x = -inf or NaN)
  // gets -126, harmless since all its probabilities are 0.
  const int kf = (int)fmaxf(floorf(x), -126.f);
  k = mv ? 0 : kf;
}

// Four fp32 values (already within +-448) to E4M3 codes in one word, in order.
// The conversion writes one half of its destination and keeps the other;
// both halves are written here, so the word starts from an opaque value
// (an empty statement) rather than from a zero the compiler would have to
// move into it first.
__device__ __forceinline__ int pack_e4m3x4(float a, float b, float c, float d) {
  int w;
  asm volatile("" : "=v"(w));
  w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, w, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

__device__ __forceinline__ float max_halves8(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves8(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int D, bool CAUSAL, int HG, bool KSPLIT>
__global__ void __launch_bounds__(kF8Threads, 1) fwd_fp8_kernel(const FwdParams p) {
  static_assert(!KSPLIT || CAUSAL, "the key split only balances causal work");
  constexpr int NW = kF8Threads / 64;
  constexpr int WPH = NW / HG;           // wavefronts per query head
  constexpr int BMPOS = 32 * WPH;        // query positions per workgroup
  // Key split (small causal grids), as in the bf16 kernel: wavefronts w and
  // w + NW/2 own the same rows and take the first and the second 64 keys of
  // every 128-key tile, in two passes (heavy half-tile, then light), and
  // merge their (m, l, acc) at the end of each pass.
  constexpr int BN = KSPLIT ? 2 * kF8BN : kF8BN;            // keys per tile
  // Under the key split at d = 64 (the plain loop) two stages of 128-key
  // tiles; otherwise four, so that the pipelined loop below finds tile t+1
  // landed at tile t's barrier with tile t+2 still in flight.
  constexpr int STAGES = KSPLIT && D != 128 ? kF8Stages / 2 : kF8Stages;
  constexpr int RPH = KSPLIT ? WPH / 2 : WPH;               // 32-row blocks per query head
  constexpr int NPASS = KSPLIT ? 2 : 1;
  constexpr int TILE = BN * D;           // bytes of one K or V tile
  constexpr int NC8 = D / 64;            // 64-deep steps of the Q.K product
  constexpr int ND = D / 32;             // 32-wide blocks of the output
  constexpr int CPR = D / 16;            // 16-byte chunks per row
  constexpr int CW = TILE / 1024;        // 1 KiB copy blocks per tile and tensor
  constexpr int CWW = CW < NW ? CW : NW; // wavefronts that copy
  constexpr int NCP = CW / CWW;          // copies per copying wavefront, tile and tensor
  static_assert(CW >= 1 && CW % CWW == 0, "tile size and workgroup do not match");
  // K reads add up to (STAGES-1)*TILE + 32*D to their base, V reads (whose
  // base already points at the V stages) up to (STAGES-1)*TILE + 48*D.
  static_assert((STAGES - 1) * TILE + 48 * D < 65536, "operand offsets must fit the immediate");
  // Key split: the merge hands (m, l) and the accumulator of NW/2 row blocks
  // over through LDS, one 16-byte vector per lane and slot.
  constexpr int XCH = KSPLIT ? (NW / 2) * (4 * ND + 1) * 64 * 16 : 0;
  constexpr int LDS_BYTES = 2 * STAGES * TILE > XCH ? 2 * STAGES * TILE : XCH;
  __shared__ __attribute__((aligned(16))) char lds[LDS_BYTES];   // K stages | V stages

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
  // Rows of pass `pass`, with the same pairing of light and heavy half-tiles
  // as the bf16 kernel.
  int q0w = 0, q_end = 0;
  bool active = true;
  auto set_rows = [&](int pass) __attribute__((always_inline)) {
    if constexpr (KSPLIT) {
      constexpr int HALF = BMPOS / 2;
      const int nh = (p.Tq + HALF - 1) / HALF;
      const int i = blockIdx.y;
      const int ht = pass == 0 ? nh - 1 - i : i;
      active = pass == 0 || ht != nh - 1 - i;
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

  const size_t qplane = (size_t)b * p.Hq + hq;
  const size_t kvplane = (size_t)b * p.Hkv + kvh;
  const uint8_t* Qg = (const uint8_t*)p.q + qplane * p.Tq * D;
  const uint8_t* Kg = (const uint8_t*)p.k + kvplane * p.Tk * D;
  const uint8_t* Vg = (const uint8_t*)p.v + kvplane * p.Tk * D;

  const int off = p.causal_off;

  // Copies: copy r of wavefront w < CWW fills LDS bytes [(r*NW + w)*1024,
  // +1024) of a tile; chunk L is row L / CPR at position L % CPR, holding
  // chunk (L % CPR) ^ f8swz(row).
  const int nbytes = p.Tk * D;
  const __amdgpu_buffer_rsrc_t krsrc = __builtin_amdgcn_make_buffer_rsrc((void*)Kg, 0, nbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrsrc = __builtin_amdgcn_make_buffer_rsrc((void*)Vg, 0, nbytes, 0x00020000);
  uint32_t csrc[NCP];
#pragma unroll
  for (int r = 0; r < NCP; ++r) {
    const int L = (r * NW + wave) * 64 + lane;
    const int row = L / CPR;
    csrc[r] = (uint32_t)(row * D + (((L % CPR) ^ f8swz<D>(row)) << 4));
  }
  auto issue_copies = [&](int t) __attribute__((always_inline)) {
    if (wave >= CWW) return;
    const int st = t % STAGES;
    const uint32_t soff = (uint32_t)t * TILE;
#pragma unroll
    for (int r = 0; r < NCP; ++r) {
      copy16_buf_to_lds(krsrc, lds + st * TILE + (r * NW + wave) * 1024, csrc[r] + soff, 0);
      copy16_buf_to_lds(vrsrc, lds + (STAGES + st) * TILE + (r * NW + wave) * 1024, csrc[r] + soff, 0);
    }
  };
  // The vector-memory counter counts 2*NCP per tile on a copying wavefront.
  auto wait_copies = [&](int later) __attribute__((always_inline)) {
    if (later >= 2)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm<4 * NCP>());
    else if (later == 1)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm<2 * NCP>());
    else
      __builtin_amdgcn_s_waitcnt(vmcnt_imm<0>());
  };

  // K operand bases (stage 0, key block 0 of this wavefront's keys): row
  // 64*kh + col, chunks 4c + 2*half and 4c + 2*half + 1 (c < NC8); f8swz
  // does not see the 64-row offset.
  uint32_t kread[2 * NC8];
  {
    const int sw = f8swz<D>(col);
#pragma unroll
    for (int i = 0; i < 2 * NC8; ++i) {
      const int ch = 4 * (i >> 1) + 2 * half + (i & 1);
      kread[i] = lds_addr(lds) + (64 * kh + col) * D + ((ch ^ sw) << 4);
    }
  }
  // V^T operand bases for the transposing reads: input lane 2e + h of
  // 16-lane group G addresses 8 codes, head dimensions 32*db + 16*(G%2) +
  // 8h .. +8, of key row 64*kh + 8*(e/4) + 4*half + e%4 (plus 16j for read
  // j, a compile-time offset that f8swz does not see).
  uint32_t vread[ND];
  {
    const int t = lane & 15;
    const int e = t >> 1, h = t & 1;
    const int row = 8 * (e >> 2) + 4 * half + (e & 3);
    const int sw = f8swz<D>(row);
#pragma unroll
    for (int db = 0; db < ND; ++db) {
      const int ch = 2 * db + ((lane >> 4) & 1);
      vread[db] = lds_addr(lds + STAGES * TILE) + (64 * kh + row) * D + ((ch ^ sw) << 4) + 8 * h;
    }
  }
  const float vs = p.vscale[kvplane];
  for (int pass = 0; pass < NPASS; ++pass) {
    set_rows(pass);
    if (KSPLIT && !active) break;   // the same for the whole workgroup
    const int my_q = q0w + col;

    const int kend = CAUSAL ? max(0, min(p.Tk, q_end + off)) : p.Tk;
    const int ntiles = (kend + BN - 1) / BN;

    // This lane's query row as the B operand: 32 codes of head dimensions
    // 64c + 32*half .. +32 (sign bits flipped for a negative scale).  The
    // first key tiles' copies are issued before anything waits for these
    // loads; the sign flip sits behind a uniform branch for the same reason.
    u32x4 qw[2 * NC8];
#pragma unroll
    for (int c = 0; c < NC8; ++c) {
      qw[2 * c] = u32x4{0u, 0u, 0u, 0u};
      qw[2 * c + 1] = u32x4{0u, 0u, 0u, 0u};
      if (my_q < p.Tq) {
        const uint8_t* src = Qg + (size_t)my_q * D + 64 * c + 32 * half;
        qw[2 * c] = *(const u32x4*)src;
        qw[2 * c + 1] = *(const u32x4*)(src + 16);
      }
    }
    const float qs = my_q < p.Tq ? p.qscale[qplane * p.Tq + my_q] : 1.f;
    for (int t = 0; t < min(ntiles, STAGES - 1); ++t) issue_copies(t);
    if (p.negate_q) {
#pragma unroll
      for (int c = 0; c < 2 * NC8; ++c) qw[c] ^= 0x80808080u;
    }
    i32x8 qf[NC8];
#pragma unroll
    for (int c = 0; c < NC8; ++c)
      qf[c] = i32x8{(int)qw[2 * c][0], (int)qw[2 * c][1], (int)qw[2 * c][2], (int)qw[2 * c][3],
                    (int)qw[2 * c + 1][0], (int)qw[2 * c + 1][1], (int)qw[2 * c + 1][2], (int)qw[2 * c + 1][3]};
    // Base-2 exponent factor of this row: |scale| * log2(e) * qs_i * ks, and
    // the headroom in raw product units.
    const float cq = fmaxf(p.c * qs * p.kscale[kvplane], 1e-30f);

    const int lim = q0w + 31 + off - 64 * kh;   // last key its rows see, minus its block start
    const int my_tiles = !active ? 0 : CAUSAL ? (lim < 0 ? 0 : min(ntiles, lim / BN + 1)) : ntiles;
    // A row keeps m = -inf and offset 0 until a tile shows it a key.

    float m = kNegInf;   // reference max of this row's raw 8-bit products
    float l = 0.f;       // this half-wave's share of the running sum of 448 * P
    f32x16 acc[ND];
#pragma unroll
    for (int i = 0; i < ND; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;

    auto tile = [&](int t, auto st_c) __attribute__((always_inline)) {
      constexpr int ST = decltype(st_c)::value;
      constexpr int KT = ST * TILE;
      constexpr int VT = ST * TILE;   // vread already points at the V stages
      const int t0 = t * BN + 64 * kh;   // this wavefront's first key
      wait_copies(min(ntiles - 1 - t, STAGES - 2));
      tile_barrier();
      if (t + STAGES - 1 < ntiles) issue_copies(t + STAGES - 1);
      if (t >= my_tiles) return;
      // S^T for the two 32-key blocks: K reads in the order the products
      // consume them, each product waiting only for its own two.
      constexpr int NP = 2 * NC8;   // products
      u32x4 kr[2][2 * NC8];
      static_for<0, NP>([&](auto j_c) {
        constexpr int KB = decltype(j_c)::value & 1, C = decltype(j_c)::value >> 1;
        kr[KB][2 * C] = lds_read_u32x4<KT + KB * 32 * D>(kread[2 * C]);
        kr[KB][2 * C + 1] = lds_read_u32x4<KT + KB * 32 * D>(kread[2 * C + 1]);
      });
      // Products alternate between the two key blocks (no product waits on
      // the accumulator of the one just before it).
      f32x16 s[2];
      static_for<0, NP>([&](auto j_c) {
        constexpr int J = decltype(j_c)::value;
        constexpr int KB = J & 1, C = J >> 1;
        lgkm_wait<2 * (NP - 1 - J)>();
        tie(kr[KB][2 * C]);
        tie(kr[KB][2 * C + 1]);
        const u32x4 a0 = kr[KB][2 * C], a1 = kr[KB][2 * C + 1];
        const i32x8 a = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3],
                         (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
        s[KB] = mma_f8(a, qf[C], C == 0 ? f32x16{} : s[KB]);
        __builtin_amdgcn_sched_barrier(0);   // issued before the next wait
      });

      // V^T reads for the first half of the output blocks go out now; they do
      // not depend on the probabilities.
      constexpr int NDH = ND / 2;
      u32x2 va[ND][4];
      static_for<0, NDH>([&](auto db_c) {
        static_for<0, 4>([&](auto j_c) { va[db_c][j_c] = lds_read_tr8<VT + 16 * j_c * D>(vread[db_c]); });
      });

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
      float mt = fmaxf(s[0][0], s[0][1]);
#pragma unroll
      for (int i = 2; i < 32; i += 2)
        mt = fmaxf(fmaxf(mt, s[i >> 4][i & 15]), s[(i + 1) >> 4][(i + 1) & 15]);
      mt = max_halves8(mt);
      float m0;
      bool mv;
      int k;
      float x;
      f8_plan(m, mt, cq, m0, mv, k, x);
      if (__builtin_amdgcn_ballot_w64(mv) != 0) {
        const float corr = mv ? exp2_fast(-x) : 1.f;
#pragma unroll
        for (int i = 0; i < ND; ++i) acc[i] *= corr;
        l *= corr;
      }
      m = m0;
      // 448 * 2^-headroom * P * 2^-k = 2^(s*cq - m*cq - k + log2 448 - headroom).
      const float mc = m > kNegInf ? fmaf(m, cq, (float)k + kF8Offset) : 0.f;
      float ls[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          s[kb][r] = exp2_fast(fmaf(s[kb][r], cq, -mc));
          ls[r & 3] += s[kb][r];
        }
      l += ldexpf((ls[0] + ls[1]) + (ls[2] + ls[3]), k);
      const int sb = 127 + k;
      // B operand: byte 4w + i is key block w/4, register 4*(w%4) + i.
      i32x8 pb;
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const int kb = w >> 2, r = 4 * (w & 3);
        pb[w] = pack_e4m3x4(s[kb][r], s[kb][r + 1], s[kb][r + 2], s[kb][r + 3]);
      }

      lgkm_wait<0>();
      static_for<NDH, ND>([&](auto db_c) {
        static_for<0, 4>([&](auto j_c) { va[db_c][j_c] = lds_read_tr8<VT + 16 * j_c * D>(vread[db_c]); });
      });
#pragma unroll
      for (int db = 0; db < NDH; ++db) {
#pragma unroll
        for (int j = 0; j < 4; ++j) tie(va[db][j]);
        const i32x8 a = {(int)va[db][0][0], (int)va[db][0][1], (int)va[db][1][0], (int)va[db][1][1],
                         (int)va[db][2][0], (int)va[db][2][1], (int)va[db][3][0], (int)va[db][3][1]};
        acc[db] = mma_f8_sb(a, pb, acc[db], sb);
      }
      lgkm_wait<0>();
#pragma unroll
      for (int db = NDH; db < ND; ++db) {
#pragma unroll
        for (int j = 0; j < 4; ++j) tie(va[db][j]);
        const i32x8 a = {(int)va[db][0][0], (int)va[db][0][1], (int)va[db][1][0], (int)va[db][1][1],
                         (int)va[db][2][0], (int)va[db][2][1], (int)va[db][3][0], (int)va[db][3][1]};
        acc[db] = mma_f8_sb(a, pb, acc[db], sb);
      }
    };
    if constexpr (D != 128) {
      // (At d = 64 the pipelined loop's second score set would take the
      // kernel from 115 to 148 registers, one workgroup per CU instead of two.)
      for (int t = 0; t < ntiles; t += STAGES) {
        static_for<0, STAGES>([&](auto s_c) {
          if (t + decltype(s_c)::value < ntiles) tile(t + decltype(s_c)::value, s_c);
        });
      }
    } else {
      // Software-pipelined tile loop (d = 128): tile t+1's
      // scores go to the matrix core before tile t's exponentials and
      // packing, and tile t+1's mask and max follow tile t's P.V, so every
      // phase of VALU work has independent matrix-core work beside it in the
      // same wavefront.  Tile t+1 must have landed at tile t's barrier:
      // copies run two tiles ahead of it.
      f32x16 sbuf[2][2];                   // scores of tiles t (even/odd) and t+1
      int k_next = 0;                      // tile t+1's block-scale exponent
      auto scores = [&](auto st_c, f32x16 (&s)[2]) __attribute__((always_inline)) {
        constexpr int KT = decltype(st_c)::value * TILE;
        // K reads in the order the products consume them, each product
        // waiting only for its own two (the first product starts while the
        // other reads are still in flight).
        constexpr int NP = 2 * NC8;   // products
        u32x4 kr[2][2 * NC8];
        static_for<0, NP>([&](auto j_c) {
          constexpr int KB = decltype(j_c)::value & 1, C = decltype(j_c)::value >> 1;
          kr[KB][2 * C] = lds_read_u32x4<KT + KB * 32 * D>(kread[2 * C]);
          kr[KB][2 * C + 1] = lds_read_u32x4<KT + KB * 32 * D>(kread[2 * C + 1]);
        });
        // Products alternate between the two key blocks, so that no product
        // waits on the accumulator of the one just before it.
        static_for<0, NP>([&](auto j_c) {
          constexpr int J = decltype(j_c)::value;
          constexpr int KB = J & 1, C = J >> 1;
          lgkm_wait<2 * (NP - 1 - J)>();
          tie(kr[KB][2 * C]);
          tie(kr[KB][2 * C + 1]);
          const u32x4 a0 = kr[KB][2 * C], a1 = kr[KB][2 * C + 1];
          const i32x8 a = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3],
                           (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
          s[KB] = mma_f8(a, qf[C], C == 0 ? f32x16{} : s[KB]);
          __builtin_amdgcn_sched_barrier(0);   // issued before the next wait
        });
      };
      // Mask tile t's scores, take its max and decide the reference move.
      // Tiles past this wavefront's last (formed on stale stage data) are
      // masked whole and move nothing.
      auto decide = [&](int t, f32x16 (&s)[2]) __attribute__((always_inline)) {
        const int t0 = t * BN + 64 * kh;   // this wavefront's first key
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
        float mt = fmaxf(s[0][0], s[0][1]);
#pragma unroll
        for (int i = 2; i < 32; i += 2)
          mt = fmaxf(fmaxf(mt, s[i >> 4][i & 15]), s[(i + 1) >> 4][(i + 1) & 15]);
        mt = max_halves8(mt);
        // The reference for tile t+1, and its (rare) move, applied here:
        // after tile t's P.V, at the end of its step, so that no branch
        // splits the step's code.
        float m0, x;
        bool mv;
        f8_plan(m, mt, cq, m0, mv, k_next, x);
        if (__builtin_amdgcn_ballot_w64(mv) != 0) {
          const float corr = mv ? exp2_fast(-x) : 1.f;
#pragma unroll
          for (int i = 0; i < ND; ++i) acc[i] *= corr;
          l *= corr;
        }
        m = m0;
      };
      auto step = [&](int t, auto st_c) __attribute__((always_inline)) {
        constexpr int ST = decltype(st_c)::value;
        constexpr int VT = ST * TILE;   // vread already points at the V stages
        constexpr int CUR = ST & 1;
        // Issued so far: tiles up to t + STAGES - 2; tile t+1 must be in.
        wait_copies(max(0, min(ntiles - 2 - t, STAGES - 3)));
        tile_barrier();
        if (t + STAGES - 1 < ntiles) issue_copies(t + STAGES - 1);
        if (t >= my_tiles) return;
        const int k = k_next;
        scores(IC<(ST + 1) % STAGES>{}, sbuf[CUR ^ 1]);
        u32x2 va[ND][4];
        static_for<0, ND>([&](auto db_c) {
          static_for<0, 4>([&](auto j_c) { va[db_c][j_c] = lds_read_tr8<VT + 16 * j_c * D>(vread[db_c]); });
        });
        // 448 * 2^-headroom * P * 2^-k = 2^(s*cq - m*cq - k + log2 448 - headroom).
        const float mc = m > kNegInf ? fmaf(m, cq, (float)k + kF8Offset) : 0.f;
        f32x16 (&s)[2] = sbuf[CUR];
        float ls[4];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            s[kb][r] = exp2_fast(fmaf(s[kb][r], cq, -mc));
            ls[r & 3] = kb == 0 && r < 4 ? s[kb][r] : ls[r & 3] + s[kb][r];
          }
        l += ldexpf((ls[0] + ls[1]) + (ls[2] + ls[3]), k);
        const int sb = 127 + k;
        i32x8 pb;
#pragma unroll
        for (int w = 0; w < 8; ++w) {
          const int kb = w >> 2, r = 4 * (w & 3);
          pb[w] = pack_e4m3x4(s[kb][r], s[kb][r + 1], s[kb][r + 2], s[kb][r + 3]);
        }
        lgkm_wait<0>();
#pragma unroll
        for (int db = 0; db < ND; ++db) {
#pragma unroll
          for (int j = 0; j < 4; ++j) tie(va[db][j]);
          const i32x8 a = {(int)va[db][0][0], (int)va[db][0][1], (int)va[db][1][0], (int)va[db][1][1],
                           (int)va[db][2][0], (int)va[db][2][1], (int)va[db][3][0], (int)va[db][3][1]};
          acc[db] = mma_f8_sb(a, pb, acc[db], sb);
        }
        decide(t + 1, sbuf[CUR ^ 1]);
      };
      // Tile 0's scores, mask and max.
      if (ntiles > 0) {
        wait_copies(min(ntiles - 1, STAGES - 2));
        tile_barrier();
        if (my_tiles > 0) {
          scores(IC<0>{}, sbuf[0]);
          decide(0, sbuf[0]);
        }
      }
      for (int t = 0; t < ntiles; t += STAGES) {
        static_for<0, STAGES>([&](auto s_c) {
          if (t + decltype(s_c)::value < ntiles) step(t + decltype(s_c)::value, s_c);
        });
      }
    }

    if constexpr (KSPLIT) {
      // The two key halves of the same rows combine by the rescale rule:
      // the second-half wavefront hands its (m, l, acc) over through LDS (one
      // 16-byte vector per lane and slot).  No copy is in flight: the last
      // tile of a pass waits for every copy issued before it.
      tile_barrier();
      f32x4* xch = (f32x4*)lds + rw * (4 * ND + 1) * 64 + lane;
      if (kh == 1) {
        xch[0] = f32x4{m, l, 0.f, 0.f};
#pragma unroll
        for (int db = 0; db < ND; ++db)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            xch[(1 + 4 * db + j) * 64] = f32x4{acc[db][4 * j], acc[db][4 * j + 1], acc[db][4 * j + 2],
                                               acc[db][4 * j + 3]};
      }
      tile_barrier();
      if (kh == 0) {
        const f32x4 o = xch[0];
        const float m_new = fmaxf(m, o[0]);
        const bool live = m_new > kNegInf;
        const float fa = exp2_fast(live ? (m - m_new) * cq : 0.f);
        const float fb = exp2_fast(live ? (o[0] - m_new) * cq : 0.f);
        l = l * fa + o[1] * fb;
        m = m_new;
#pragma unroll
        for (int db = 0; db < ND; ++db)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const f32x4 o2 = xch[(1 + 4 * db + j) * 64];
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[db][4 * j + e] = acc[db][4 * j + e] * fa + o2[e] * fb;
          }
      }
      tile_barrier();   // the exchange slots are free before the next pass's copies
    }

    // O = acc * vs / l (the 448 * 2^-headroom of the probabilities cancels);
    // lse in natural log: (m*cq + log2(l) - log2 448 + headroom) * ln 2.
    const float lt = sum_halves8(l);
    const float inv = lt > 0.f ? vs / lt : 0.f;
    if (active && kh == 0 && my_q < p.Tq) {
      bf16* Og = (bf16*)p.o + (qplane * p.Tq + my_q) * D;
#pragma unroll
      for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bf16x2 lo = to_bf16x2(acc[db][4 * j] * inv, acc[db][4 * j + 1] * inv);
          const bf16x2 hi = to_bf16x2(acc[db][4 * j + 2] * inv, acc[db][4 * j + 3] * inv);
          *(bf16x4*)(Og + 32 * db + 8 * j + 4 * half) = __builtin_shufflevector(lo, hi, 0, 1, 2, 3);
        }
      if (p.lse != nullptr && half == 0)
        p.lse[qplane * p.Tq + my_q] =
            lt > 0.f ? (m * cq + __builtin_amdgcn_logf(lt) - kLog2E4M3Max + kF8Headroom) * kLn2 : kNegInf;
    }
  }
}

template <int D, bool CAUSAL, bool KSPLIT>
void launch_fp8_grid(int hg, dim3 grid, const FwdParams& p, hipStream_t stream) {
  if (hg == 4)
    hipLaunchKernelGGL((fwd_fp8_kernel<D, CAUSAL, 4, KSPLIT>), grid, dim3(kF8Threads), 0, stream, p);
  else if (hg == 2)
    hipLaunchKernelGGL((fwd_fp8_kernel<D, CAUSAL, 2, KSPLIT>), grid, dim3(kF8Threads), 0, stream, p);
  else
    hipLaunchKernelGGL((fwd_fp8_kernel<D, CAUSAL, 1, KSPLIT>), grid, dim3(kF8Threads), 0, stream, p);
}

template <int D, bool CAUSAL>
hipError_t launch_fp8_hg(const FwdParams& p0, hipStream_t stream) {
  FwdParams p = p0;
  const int hg = (p.g % 4 == 0) ? 4 : (p.g % 2 == 0) ? 2 : 1;
  p.groups = p.g / hg;
  const int bmpos = 32 * (kF8Threads / 64) / hg;
  const int nx = p.B * p.Hkv * p.groups;
  const int ny = (p.Tq + bmpos - 1) / bmpos;
  // The same grid choice as the bf16 kernel: light/heavy pairing under four
  // workgroups per compute unit, with the key split up to about one.
  p.pair = 0;
  if (CAUSAL && (long long)nx * ny < 4LL * compute_units()) {
    const int half = bmpos / 2;
    const int nyp = ((p.Tq + half - 1) / half + 1) / 2;
    const dim3 grid((unsigned)nx, (unsigned)nyp);
    p.pair = 1;
    if constexpr (CAUSAL) {
      if (2LL * nx * nyp <= 3LL * compute_units())
        launch_fp8_grid<D, true, true>(hg, grid, p, stream);
      else
        launch_fp8_grid<D, true, false>(hg, grid, p, stream);
    }
  } else {
    launch_fp8_grid<D, CAUSAL, false>(hg, dim3((unsigned)nx, (unsigned)ny), p, stream);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_fp8(const FwdParams& p, int d, bool causal, hipStream_t stream) {
  if (d == 64) return causal ? launch_fp8_hg<64, true>(p, stream) : launch_fp8_hg<64, false>(p, stream);
  return causal ? launch_fp8_hg<128, true>(p, stream) : launch_fp8_hg<128, false>(p, stream);
}

}  // namespace fa
