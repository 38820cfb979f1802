// Backward pass of exact attention (dQ, dK, dV) for gfx950.
//
// Sources (web pages; sections named as headed there):
//   [LESSON] "FlashAttention: внимание без матрицы n×n" (ai.flicky.cc),
//            section "Обратный проход: пересчитать дешевле, чем хранить".
//   [NOTE]   "Atencja od strony jądra: FlashAttention, softmax online i
//            połączona dekwantyzacja" (trefon.com), section "Prefill i
//            dekodowanie to różne problemy" (grouped-query attention).
//   [BOOK5]  "Глава 5. Операторы и среда выполнения" (bojieli.github.io),
//            section 5.3.2 (tiles double-buffered in on-chip memory).
//
// What is computed ([LESSON], backward section): the forward keeps only O
// and the row log-sum-exp L_i.  Score tiles S = scale * Q K^T are computed
// again and the probabilities recovered without any normalisation,
// P_ij = exp(S_ij - L_i); then
//     dV = P^T dO,   dP = dO V^T,   dS_ij = P_ij (dP_ij - D_i),
//     D_i = sum_j P_ij dP_ij = dO_i . O_i,
//     dQ = scale * dS K,   dK = scale * dS^T Q
// (the page has scale = 1/sqrt(d)).  With grouped-query attention the g
// query heads that share a kv head all add into that head's dK and dV.
//
// Three kernels; none writes anything of size Tq x Tk and none uses atomics
// (every output element is produced by exactly one lane):
//  1. bwd_prep: D_i = dO_i . O_i in fp32 from the bf16 O and dO, and
//     L_i * log2(e), into a workspace whose per-head planes are padded with
//     zero rows to a multiple of kBwdRowPad.
//  2. bwd_dkdv: a workgroup owns 128 keys of one kv head, 32 per wavefront.
//     K and V stay in registers and dK^T, dV^T in accumulators while tiles of
//     64 query rows (Q, dO, L, D) of every query head of the group stream
//     through LDS, the next tile copied while the current one is used.  Per
//     32 query rows a wavefront forms S = Q K^T and dP = dO V^T (lane = key,
//     registers = queries), P and dS in registers, then dV^T += dO^T P and
//     dK^T += Q^T dS with dO^T and Q^T read through the transposing LDS read.
//     Under the causal mask the query rows that see none of the workgroup's
//     keys are never visited and 32x32 blocks above the diagonal are skipped.
//  3. bwd_dq: a workgroup owns 32*NW query rows of one query head; Q and dO
//     stay in registers and dQ^T in accumulators while tiles of 64 keys (K,
//     V) stream through LDS.  Per 32 keys: S^T = K Q^T and dP^T = V dO^T
//     (lane = query), P^T and dS^T, then dQ^T += K^T dS^T with K^T read
//     transposed.  Key tiles after the workgroup's last row's limit are never
//     visited under the causal mask.
// The causal diagonal is top-left (row i sees keys j <= i) or bottom-right
// (j <= i + Tk - Tq, a chunk of queries at the end of a cached sequence).
// The probabilities and dS are rounded to bf16 for the matrix products that
// consume them; all sums are fp32.  Masked entries of P are set to 0
// explicitly (never through -inf), so any finite scale works.
#include "fa_device.h"
#include "fa_launch.h"
#include "fa_lds.h"

#include <type_traits>

namespace fa {
namespace {

constexpr int kDkdvThreads = 256;  // 4 wavefronts, 32 keys each
constexpr int kKeysPerWg = 128;    // keys per dK/dV workgroup
constexpr int kQTile = 64;         // query rows per LDS stage (dK/dV kernel)
constexpr int kKTile = 64;         // keys per LDS stage (dQ kernel)
constexpr int kPrepThreads = 256;

// ---------------------------------------------------------------------------
// LDS tile layout of the backward kernels
// ---------------------------------------------------------------------------
// A tile is rows x D bf16, row-major as in HBM, with the 16-byte chunks of
// each row permuted: chunk c of row r sits at position c ^ bswz(r).  Every
// tile here is read two ways, so the swizzle serves both:
//  * row reads (a matrix-core operand with one tile row per lane): 16 bytes
//    per lane from 32 consecutive rows at one chunk; bswz is a bijection on
//    the row bits that select a bank line, so 16 consecutive rows hit
//    distinct banks;
//  * transposing reads (one tile column per lane): 8 bytes per lane from 4
//    consecutive rows and 4 consecutive chunks; bswz gives those 4 rows
//    distinct values in the bits that select the chunk group, so the 16
//    chunks land on distinct banks.
// bswz depends only on the low 4 row bits, so a lane's read addresses for
// rows r + 16*i are one base plus compile-time offsets.
template <int D>
__device__ __forceinline__ int bswz(int row) {
  return D == 128 ? (((row & 3) << 2) | ((row >> 2) & 3))
                  : ((((row >> 1) & 1) << 2) | ((row >> 2) & 3));
}

// Byte offset of 16-byte chunk `chunk` of row `row` in a swizzled tile.
template <int D>
__device__ __forceinline__ uint32_t tile_off(int row, int chunk) {
  return (uint32_t)(row * D * 2 + ((chunk ^ bswz<D>(row)) << 4));
}

// Per-lane LDS read bases of one 32-row block of a swizzled tile at LDS
// address 0 (kernels add the tile's address as a compile-time offset).
//  row[s]:    A operand of a product over the tile's columns, one tile row
//             per lane: row `col`, columns 16s + 8*half .. +8.
//  tr[e][db]: A operand of a product over the tile's rows, one tile column
//             per lane: the transposing read, rows 4*half + 8e + 0..3 (plus
//             16*j added as an offset), columns 32*db + col.
template <int D>
struct TileReads {
  static constexpr int NC = D / 16;
  static constexpr int ND = D / 32;
  uint32_t row[NC];
  uint32_t tr[2][ND];

  __device__ __forceinline__ explicit TileReads(uint32_t base, int lane) {
    const int half = lane >> 5;
    const int col = lane & 31;
#pragma unroll
    for (int s = 0; s < NC; ++s) row[s] = base + tile_off<D>(col, 2 * s + half);
    // Input lane 4j + q of 16-lane group G addresses columns
    // 32*db + 16*(G%2) + 4q .. +3 of row 4*half + j (+ 8e).
    const int tj = (lane & 15) >> 2;
    const int tc = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int r = 4 * half + tj + 8 * e;
#pragma unroll
      for (int db = 0; db < ND; ++db) {
        const int cc = 32 * db + tc;
        tr[e][db] = base + tile_off<D>(r, cc >> 3) + (cc & 7) * 2;
      }
    }
  }
};

// Load 8 bf16 of global row `row` (if row < n, else zeros): the B operand
// slice columns 16s + 8*half .. +8 for s = 0 .. D/16-1.
template <int D>
__device__ __forceinline__ void load_row_operand(const bf16* base, int row, int n, int half,
                                                 bf16x8 (&out)[D / 16]) {
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    u32x4 w = {0u, 0u, 0u, 0u};
    if (row < n) w = *(const u32x4*)(base + (size_t)row * D + 16 * s + 8 * half);
    __builtin_memcpy(&out[s], &w, sizeof(w));
  }
}

// Pack accumulator registers 8j .. 8j+7 to bf16 (a B operand over 16 rows).
__device__ __forceinline__ bf16x8 pack8(const float* x) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; i += 2) {
    const bf16x2 two = to_bf16x2(x[i], x[i + 1]);
    r[i] = two[0];
    r[i + 1] = two[1];
  }
  return r;
}

// Two transposing reads (rows +0..3 and +8..11) as one A operand.
__device__ __forceinline__ bf16x8 join_tr(const u32x2 (&v)[2]) {
  const u32x4 w = {v[0][0], v[0][1], v[1][0], v[1][1]};
  bf16x8 a;
  __builtin_memcpy(&a, &w, sizeof(a));
  return a;
}

// Store a 32 x 32 accumulator block (dims x rows, lane = row) times f as
// bf16 into row `row` of a row-major [*, D] array, columns 32*db + ...
template <int D>
__device__ __forceinline__ void store_acc_row(bf16* dst_row, int db, int half, const f32x16& a,
                                              float f) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const bf16x2 lo = to_bf16x2(a[4 * j] * f, a[4 * j + 1] * f);
    const bf16x2 hi = to_bf16x2(a[4 * j + 2] * f, a[4 * j + 3] * f);
    *(bf16x4*)(dst_row + 32 * db + 8 * j + 4 * half) = __builtin_shufflevector(lo, hi, 0, 1, 2, 3);
  }
}

// The same row of an accumulator as fp32, unscaled (a partial sum).
template <int D>
__device__ __forceinline__ void store_acc_row_f32(float* dst_row, int db, int half, const f32x16& a) {
#pragma unroll
  for (int j = 0; j < 4; ++j)
    *(f32x4*)(dst_row + 32 * db + 8 * j + 4 * half) = f32x4{a[4 * j], a[4 * j + 1], a[4 * j + 2], a[4 * j + 3]};
}

// ---------------------------------------------------------------------------
// 1. Row terms: D_i = dO_i . O_i and L_i * log2(e)
// ---------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(kPrepThreads) bwd_prep_kernel(const BwdParams p) {
  constexpr int TPR = D / 8;                 // threads per row, 8 values each
  constexpr int RPB = kPrepThreads / TPR;    // rows per workgroup
  const long long row = (long long)blockIdx.x * RPB + threadIdx.x / TPR;
  const int sub = threadIdx.x % TPR;
  const long long nrows = (long long)p.B * p.Hq * p.Tqp;
  if (row >= nrows) return;   // whole row groups leave together
  const long long bh = row / p.Tqp;
  const int i = (int)(row - bh * p.Tqp);
  float dot = 0.f;
  if (i < p.Tq) {
    const size_t off = ((size_t)bh * p.Tq + i) * D + 8 * sub;
    const u32x4 a = *(const u32x4*)((const bf16*)p.o + off);
    const u32x4 g = *(const u32x4*)((const bf16*)p.dout + off);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      dot = fmaf(bf16_lo(a[k]), bf16_lo(g[k]), dot);
      dot = fmaf(bf16_hi(a[k]), bf16_hi(g[k]), dot);
    }
  }
#pragma unroll
  for (int m = TPR / 2; m >= 1; m >>= 1) dot += __shfl_xor(dot, m, 64);
  if (sub == 0) {
    p.delta[row] = dot;
    p.l2[row] = i < p.Tq ? p.lse[(size_t)bh * p.Tq + i] * kLog2e : 0.f;
  }
}

// ---------------------------------------------------------------------------
// 2. dK and dV
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ void __launch_bounds__(kDkdvThreads, 1) bwd_dkdv_kernel(const BwdParams p) {
  constexpr int NW = kDkdvThreads / 64;
  constexpr int NC = D / 16;                         // 16-deep steps over the head dim
  constexpr int ND = D / 32;                         // 32-wide output blocks
  constexpr int CPR = D / 8;                         // 16-byte chunks per row
  constexpr int TB = kQTile * D * 2;                 // bytes of a Q or dO tile
  constexpr int NCOPY = kQTile * CPR / kDkdvThreads; // copies per thread, tile and tensor
  constexpr int LDB = 2 * kQTile * 4;                // bytes of a tile's L and D rows
  constexpr int QOFF = 2 * LDB;                      // LDS: [L,D x2 | Q,dO stage 0 | Q,dO stage 1]
  constexpr int SB = 2 * TB;
  static_assert(NCOPY >= 1, "tile too small for the workgroup");
  static_assert(QOFF + SB + TB + 48 * D * 2 < 65536, "operand offsets must fit the immediate");
  __shared__ __attribute__((aligned(16))) char lds[QOFF + 2 * SB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int col = lane & 31;

  // Heaviest key blocks (the first ones, under the causal mask) first; the
  // kparts parts of a block are neighbours.
  const int nbkv = p.B * p.Hkv;
  const int bkv = blockIdx.x % nbkv;
  const int kblk = blockIdx.x / nbkv / p.kparts;
  const int part = blockIdx.x / nbkv % p.kparts;
  const int b = bkv / p.Hkv;
  const int kvh = bkv % p.Hkv;
  const int k0 = kblk * kKeysPerWg;
  const int kw = k0 + 32 * wave;   // this wavefront's keys kw .. kw + 31
  const int my_k = kw + col;

  // K and V rows of this lane's key as B operands (zeros past Tk; those
  // lanes' results are never stored).
  bf16x8 kf[NC], vf[NC];
  load_row_operand<D>((const bf16*)p.k + (size_t)bkv * p.Tk * D, my_k, p.Tk, half, kf);
  load_row_operand<D>((const bf16*)p.v + (size_t)bkv * p.Tk * D, my_k, p.Tk, half, vf);

  f32x16 dv[ND], dk[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dv[i][r] = 0.f;
      dk[i][r] = 0.f;
    }

  // Query tiles: rows qs .. Tq-1 of each of the g query heads.  Causal: row i
  // sees key j iff j <= i + off, so rows before k0 - off see none of these
  // keys (qs is kept a multiple of the tile height).
  const int off = p.causal_off;
  const int qs = CAUSAL ? max(0, k0 - off) / kQTile * kQTile : 0;
  const int ntq = qs < p.Tq ? (p.Tq - qs + kQTile - 1) / kQTile : 0;
  const int nit = p.g * ntq;
  // This workgroup's items (query head it / ntq, query tile it % ntq).
  const int i0 = (int)((long long)nit * part / p.kparts);
  const int i1 = (int)((long long)nit * (part + 1) / p.kparts);

  // Copy r of wavefront w fills LDS chunks [(r*NW + w)*64, +64) of a tile:
  // chunk L is row L / CPR at position L % CPR, holding chunk
  // (L % CPR) ^ bswz(row) of that row.
  uint32_t csrc[NCOPY];
#pragma unroll
  for (int r = 0; r < NCOPY; ++r) {
    const int L = (r * NW + wave) * 64 + lane;
    const int row = L / CPR;
    csrc[r] = (uint32_t)(row * D + (((L % CPR) ^ bswz<D>(row)) << 3)) * 2u;
  }
  const int qbytes = p.Tq * D * 2;
  auto issue = [&](int it, auto st_c) __attribute__((always_inline)) {
    constexpr int ST = decltype(st_c)::value;
    const int hq = kvh * p.g + it / ntq;
    const int q0 = qs + (it % ntq) * kQTile;
    const size_t plane = (size_t)b * p.Hq + hq;
    // Rows past Tq read as zeros (the whole offset is in the range-checked
    // lane offset).
    const __amdgpu_buffer_rsrc_t qr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((const bf16*)p.q + plane * p.Tq * D), 0, qbytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t gr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((const bf16*)p.dout + plane * p.Tq * D), 0, qbytes, 0x00020000);
    const uint32_t base = (uint32_t)q0 * D * 2;
    char* qd = lds + QOFF + ST * SB;
#pragma unroll
    for (int r = 0; r < NCOPY; ++r) {
      copy16_buf_to_lds(qr, qd + (r * NW + wave) * 1024, csrc[r] + base, 0);
      copy16_buf_to_lds(gr, qd + TB + (r * NW + wave) * 1024, csrc[r] + base, 0);
    }
    // L and D of the 64 rows (padded planes: always in bounds): wavefronts
    // 0,1 copy L, 2,3 copy D, 32 values each with 8 lanes.
    const float* src = (wave < 2 ? p.l2 : p.delta) + plane * p.Tqp + q0 + 32 * (wave & 1) + 4 * lane;
    if (lane < 8) copy16_to_lds(src, lds + ST * LDB + (wave >> 1) * 256 + (wave & 1) * 128);
  };

  const TileReads<D> rd(lds_addr(lds), lane);
  const uint32_t lrd = lds_addr(lds) + 16 * half;   // L/D rows 8j + 4*half .. +3
  const float c = p.c;

  // 32 query rows (half HF of the stage-ST tile whose first row is q0).
  // MK: 0 no mask, 1 mask, 2 decided at run time by mask_rt (one code path;
  // at d = 128 separate paths cost registers and were slower).
  auto rows32 = [&](int q0h, auto st_c, auto hf_c, auto mk_c, bool mask_rt) __attribute__((always_inline)) {
    constexpr int ST = decltype(st_c)::value;
    constexpr int HF = decltype(hf_c)::value;
    constexpr int MK = decltype(mk_c)::value;
    constexpr int QT = QOFF + ST * SB + HF * 32 * D * 2;   // Q rows of this half
    constexpr int GT = QT + TB;                            // dO rows
    constexpr int LT = ST * LDB + HF * 32 * 4;             // L rows; D at +256

    // S = Q K^T and dP = dO V^T: lane = key, register r = query row
    // 8*(r/4) + 4*half + r%4 of this half.
    bf16x8 a[NC];
    f32x4 lv[4], dl[4];
    static_for<0, NC>([&](auto s_c) { a[s_c] = lds_read_b128<QT>(rd.row[s_c]); });
    static_for<0, 4>([&](auto j_c) { lv[j_c] = lds_read_f32x4<LT + 32 * j_c>(lrd); });
    lgkm_wait<0>();
#pragma unroll
    for (int s = 0; s < NC; ++s) tie(a[s]);
    bf16x8 g[NC];
    static_for<0, NC>([&](auto s_c) { g[s_c] = lds_read_b128<GT>(rd.row[s_c]); });
    static_for<0, 4>([&](auto j_c) { dl[j_c] = lds_read_f32x4<LT + 256 + 32 * j_c>(lrd); });
    f32x16 sc = {};
#pragma unroll
    for (int s = 0; s < NC; ++s) sc = mma_32x32x16(a[s], kf[s], sc);
    lgkm_wait<0>();
#pragma unroll
    for (int s = 0; s < NC; ++s) tie(g[s]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      tie(lv[j]);
      tie(dl[j]);
    }
    f32x16 dp = {};
#pragma unroll
    for (int s = 0; s < NC; ++s) dp = mma_32x32x16(g[s], vf[s], dp);

    // P = exp(S*scale - L) (base 2), dS = P (dP - D).
    float pv[16], ds[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) pv[r] = exp2_fast(fmaf(sc[r], c, -lv[r >> 2][r & 3]));
    if (MK == 1 || (MK == 2 && mask_rt)) {
      // Row offsets 8*(r/4) + r%4 outside [lo, hi) are masked: rows past
      // Tq, and under the causal mask rows before this lane's key.
      const int base = q0h + 4 * half;
      const int lo = CAUSAL ? my_k - off - base : -64;
      const int hi = p.Tq - base;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int off = 8 * (r >> 2) + (r & 3);
        pv[r] = (off >= lo && off < hi) ? pv[r] : 0.f;
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) ds[r] = pv[r] * (dp[r] - dl[r >> 2][r & 3]);
    const bf16x8 pb[2] = {pack8(pv), pack8(pv + 8)};
    const bf16x8 sb[2] = {pack8(ds), pack8(ds + 8)};

    // dV^T += dO^T P and dK^T += Q^T dS over the 32 rows, in four groups
    // (tensor, 16-row step j); the reads of the next group are in flight
    // while the current one multiplies.
    auto tr_issue = [&](auto t_c, auto j_c, u32x2 (&v)[ND][2]) __attribute__((always_inline)) {
      constexpr int OFF = (decltype(t_c)::value == 0 ? GT : QT) + decltype(j_c)::value * 16 * D * 2;
      static_for<0, ND>([&](auto db_c) {
        v[db_c][0] = lds_read_tr<OFF>(rd.tr[0][db_c]);
        v[db_c][1] = lds_read_tr<OFF>(rd.tr[1][db_c]);
      });
    };
    auto tr_tie = [&](u32x2 (&v)[ND][2]) __attribute__((always_inline)) {
#pragma unroll
      for (int db = 0; db < ND; ++db) {
        tie(v[db][0]);
        tie(v[db][1]);
      }
    };
    auto tr_mul = [&](auto t_c, auto j_c, u32x2 (&v)[ND][2]) __attribute__((always_inline)) {
      constexpr int J = decltype(j_c)::value;
#pragma unroll
      for (int db = 0; db < ND; ++db) {
        if constexpr (decltype(t_c)::value == 0)
          dv[db] = mma_32x32x16(join_tr(v[db]), pb[J], dv[db]);
        else
          dk[db] = mma_32x32x16(join_tr(v[db]), sb[J], dk[db]);
      }
    };
    u32x2 va[ND][2], vb[ND][2];
    tr_issue(IC<0>{}, IC<0>{}, va);
    lgkm_wait<0>();
    tr_tie(va);
    tr_issue(IC<0>{}, IC<1>{}, vb);
    tr_mul(IC<0>{}, IC<0>{}, va);
    lgkm_wait<0>();
    tr_tie(vb);
    tr_issue(IC<1>{}, IC<0>{}, va);
    tr_mul(IC<0>{}, IC<1>{}, vb);
    lgkm_wait<0>();
    tr_tie(va);
    tr_issue(IC<1>{}, IC<1>{}, vb);
    tr_mul(IC<1>{}, IC<0>{}, va);
    lgkm_wait<0>();
    tr_tie(vb);
    tr_mul(IC<1>{}, IC<1>{}, vb);
  };

  auto step = [&](int it, auto st_c) __attribute__((always_inline)) {
    constexpr int ST = decltype(st_c)::value;
    // Tile `it` has landed (every wavefront waits for its own copies, then
    // all meet), and nobody reads stage ST^1 any more.
    __builtin_amdgcn_s_waitcnt(vmcnt_imm<0>());
    tile_barrier();
    if (it + 1 < i1) issue(it + 1, IC<ST ^ 1>{});
    const int q0 = qs + (it % ntq) * kQTile;
    static_for<0, 2>([&](auto hf_c) {
      const int q0h = q0 + 32 * hf_c;
      // Under the causal mask query i sees key j iff j <= i + off.  Blocks
      // with every key after every row's limit are skipped; only blocks that
      // cross the diagonal and the last rows need the mask.
      if (CAUSAL && q0h + 31 + off < kw) return;
      const bool mask = (CAUSAL && q0h + off < kw + 31) || q0h + 32 > p.Tq;
      if constexpr (D == 128)
        rows32(q0h, st_c, hf_c, IC<2>{}, mask);
      else if (mask)
        rows32(q0h, st_c, hf_c, IC<1>{}, true);
      else
        rows32(q0h, st_c, hf_c, IC<0>{}, false);
    });
  };
  if (i1 > i0) issue(i0, IC<0>{});
  for (int it = i0; it < i1; it += 2) {
    step(it, IC<0>{});
    if (it + 1 < i1) step(it + 1, IC<1>{});
  }

  if (my_k < p.Tk) {
    if (p.kparts == 1) {
      bf16* dkr = (bf16*)p.dk + ((size_t)bkv * p.Tk + my_k) * D;
      bf16* dvr = (bf16*)p.dv + ((size_t)bkv * p.Tk + my_k) * D;
#pragma unroll
      for (int db = 0; db < ND; ++db) {
        store_acc_row<D>(dkr, db, half, dk[db], p.scale);
        store_acc_row<D>(dvr, db, half, dv[db], 1.f);
      }
    } else {
      const size_t row = ((size_t)part * nbkv + bkv) * p.Tk + my_k;
#pragma unroll
      for (int db = 0; db < ND; ++db) {
        store_acc_row_f32<D>(p.part_dk + row * D, db, half, dk[db]);
        store_acc_row_f32<D>(p.part_dv + row * D, db, half, dv[db]);
      }
    }
  }
}

// dK = scale * sum of the parts, dV = sum of the parts, in part order; each
// thread handles 8 consecutive head dimensions of one key row.
template <int D>
__global__ void __launch_bounds__(256) bwd_dkdv_merge_kernel(const BwdParams p) {
  const size_t n8 = (size_t)p.B * p.Hkv * p.Tk * (D / 8);
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const size_t plane = (size_t)p.B * p.Hkv * p.Tk * D;   // floats per part
  f32x4 k0 = {0.f, 0.f, 0.f, 0.f}, k1 = k0, v0 = k0, v1 = k0;
  for (int q = 0; q < p.kparts; ++q) {
    const f32x4* ks = (const f32x4*)(p.part_dk + q * plane) + 2 * i;
    const f32x4* vs = (const f32x4*)(p.part_dv + q * plane) + 2 * i;
    k0 += ks[0];
    k1 += ks[1];
    v0 += vs[0];
    v1 += vs[1];
  }
  // 8-byte stores, as the kernels that write dK and dV directly.
  const float s = p.scale;
  bf16x4* dk = (bf16x4*)p.dk + 2 * i;
  bf16x4* dv = (bf16x4*)p.dv + 2 * i;
  dk[0] = __builtin_shufflevector(to_bf16x2(k0[0] * s, k0[1] * s), to_bf16x2(k0[2] * s, k0[3] * s), 0, 1, 2, 3);
  dk[1] = __builtin_shufflevector(to_bf16x2(k1[0] * s, k1[1] * s), to_bf16x2(k1[2] * s, k1[3] * s), 0, 1, 2, 3);
  dv[0] = __builtin_shufflevector(to_bf16x2(v0[0], v0[1]), to_bf16x2(v0[2], v0[3]), 0, 1, 2, 3);
  dv[1] = __builtin_shufflevector(to_bf16x2(v1[0], v1[1]), to_bf16x2(v1[2], v1[3]), 0, 1, 2, 3);
}

// ---------------------------------------------------------------------------
// 3. dQ
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL, int NW>
__global__ void __launch_bounds__(64 * NW, 1) bwd_dq_kernel(const BwdParams p) {
  constexpr int NT = 64 * NW;
  constexpr int BM = 32 * NW;                  // query rows per workgroup
  constexpr int NC = D / 16;
  constexpr int ND = D / 32;
  constexpr int CPR = D / 8;
  constexpr int TB = kKTile * D * 2;           // bytes of a K or V tile
  constexpr int NCOPY = kKTile * CPR / NT;
  constexpr int SB = 2 * TB;                   // LDS: [K,V stage 0 | K,V stage 1]
  static_assert(NCOPY >= 1, "tile too small for the workgroup");
  static_assert(SB + TB + 48 * D * 2 < 65536, "operand offsets must fit the immediate");
  static_assert(kBwdRowPad % BM == 0, "row padding must cover whole query tiles");
  __shared__ __attribute__((aligned(16))) char lds[2 * SB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int col = lane & 31;

  // Heaviest query tiles (the last ones, under the causal mask) first.
  const int nbh = p.B * p.Hq;
  const int bh = blockIdx.x % nbh;
  const int nqt = (p.Tq + BM - 1) / BM;
  const int qt = CAUSAL ? nqt - 1 - (int)(blockIdx.x / nbh) : (int)(blockIdx.x / nbh);
  const int b = bh / p.Hq;
  const int kvh = (bh % p.Hq) / p.g;
  const int q0w = qt * BM + 32 * wave;   // this wavefront's rows q0w .. q0w + 31
  const int my_q = q0w + col;
  const int q_end = min(p.Tq, (qt + 1) * BM);

  bf16x8 qf[NC], gf[NC];
  load_row_operand<D>((const bf16*)p.q + (size_t)bh * p.Tq * D, my_q, p.Tq, half, qf);
  load_row_operand<D>((const bf16*)p.dout + (size_t)bh * p.Tq * D, my_q, p.Tq, half, gf);
  // Padded planes: my_q < Tqp always.
  const float l2 = p.l2[(size_t)bh * p.Tqp + my_q];
  const float dl = p.delta[(size_t)bh * p.Tqp + my_q];

  f32x16 dq[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[i][r] = 0.f;

  const int off = p.causal_off;   // causal: row i sees key j iff j <= i + off
  const int kend = CAUSAL ? max(0, min(p.Tk, q_end + off)) : p.Tk;
  const int ntiles = (kend + kKTile - 1) / kKTile;
  // Key tiles this wavefront computes: none past its own last row.
  const int my_tiles = q0w >= p.Tq ? 0
                       : CAUSAL ? (q0w + 31 + off < 0 ? 0 : min(ntiles, (q0w + 31 + off) / kKTile + 1))
                                : ntiles;

  uint32_t csrc[NCOPY];
#pragma unroll
  for (int r = 0; r < NCOPY; ++r) {
    const int L = (r * NW + wave) * 64 + lane;
    const int row = L / CPR;
    csrc[r] = (uint32_t)(row * D + (((L % CPR) ^ bswz<D>(row)) << 3)) * 2u;
  }
  const size_t kvplane = (size_t)b * p.Hkv + kvh;
  const int kbytes = p.Tk * D * 2;
  const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const bf16*)p.k + kvplane * p.Tk * D), 0, kbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const bf16*)p.v + kvplane * p.Tk * D), 0, kbytes, 0x00020000);
  auto issue = [&](int t, auto st_c) __attribute__((always_inline)) {
    constexpr int ST = decltype(st_c)::value;
    const uint32_t base = (uint32_t)t * kKTile * D * 2;
    char* kd = lds + ST * SB;
#pragma unroll
    for (int r = 0; r < NCOPY; ++r) {
      copy16_buf_to_lds(kr, kd + (r * NW + wave) * 1024, csrc[r] + base, 0);
      copy16_buf_to_lds(vr, kd + TB + (r * NW + wave) * 1024, csrc[r] + base, 0);
    }
  };

  const TileReads<D> rd(lds_addr(lds), lane);
  const float c = p.c;

  // 32 keys (block KB of the stage-ST tile whose first key is t*kKTile).
  // MK as in the dK/dV kernel.
  auto keys32 = [&](int kb0, auto st_c, auto kb_c, auto mk_c, bool mask_rt) __attribute__((always_inline)) {
    constexpr int ST = decltype(st_c)::value;
    constexpr int KB = decltype(kb_c)::value;
    constexpr int MK = decltype(mk_c)::value;
    constexpr int KT = ST * SB + KB * 32 * D * 2;
    constexpr int VT = KT + TB;

    // S^T = K Q^T and dP^T = V dO^T: lane = query, register r = key
    // kb0 + 8*(r/4) + 4*half + r%4.
    bf16x8 a[NC], g[NC];
    static_for<0, NC>([&](auto s_c) { a[s_c] = lds_read_b128<KT>(rd.row[s_c]); });
    lgkm_wait<0>();
#pragma unroll
    for (int s = 0; s < NC; ++s) tie(a[s]);
    static_for<0, NC>([&](auto s_c) { g[s_c] = lds_read_b128<VT>(rd.row[s_c]); });
    f32x16 sc = {};
#pragma unroll
    for (int s = 0; s < NC; ++s) sc = mma_32x32x16(a[s], qf[s], sc);
    lgkm_wait<0>();
#pragma unroll
    for (int s = 0; s < NC; ++s) tie(g[s]);
    f32x16 dp = {};
#pragma unroll
    for (int s = 0; s < NC; ++s) dp = mma_32x32x16(g[s], gf[s], dp);

    // K^T reads for the first 16 keys go out while P and dS are formed.
    u32x2 va[ND][2], vb[ND][2];
    static_for<0, ND>([&](auto db_c) {
      va[db_c][0] = lds_read_tr<KT>(rd.tr[0][db_c]);
      va[db_c][1] = lds_read_tr<KT>(rd.tr[1][db_c]);
    });

    float pv[16], ds[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) pv[r] = exp2_fast(fmaf(sc[r], c, -l2));
    if (MK == 1 || (MK == 2 && mask_rt)) {
      // Key offsets 8*(r/4) + r%4 at or past hi are masked: keys past Tk,
      // and under the causal mask keys after this lane's row.
      const int base = kb0 + 4 * half;
      const int hi = CAUSAL ? max(0, min(p.Tk, my_q + off + 1)) - base : p.Tk - base;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int off = 8 * (r >> 2) + (r & 3);
        pv[r] = off < hi ? pv[r] : 0.f;
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) ds[r] = pv[r] * (dp[r] - dl);
    const bf16x8 sb[2] = {pack8(ds), pack8(ds + 8)};

    // dQ^T += K^T dS^T over the 32 keys in two 16-key steps.
    lgkm_wait<0>();
#pragma unroll
    for (int db = 0; db < ND; ++db) {
      tie(va[db][0]);
      tie(va[db][1]);
    }
    static_for<0, ND>([&](auto db_c) {
      vb[db_c][0] = lds_read_tr<KT + 16 * D * 2>(rd.tr[0][db_c]);
      vb[db_c][1] = lds_read_tr<KT + 16 * D * 2>(rd.tr[1][db_c]);
    });
#pragma unroll
    for (int db = 0; db < ND; ++db) dq[db] = mma_32x32x16(join_tr(va[db]), sb[0], dq[db]);
    lgkm_wait<0>();
#pragma unroll
    for (int db = 0; db < ND; ++db) {
      tie(vb[db][0]);
      tie(vb[db][1]);
    }
#pragma unroll
    for (int db = 0; db < ND; ++db) dq[db] = mma_32x32x16(join_tr(vb[db]), sb[1], dq[db]);
  };

  auto step = [&](int t, auto st_c) __attribute__((always_inline)) {
    constexpr int ST = decltype(st_c)::value;
    __builtin_amdgcn_s_waitcnt(vmcnt_imm<0>());
    tile_barrier();
    if (t + 1 < ntiles) issue(t + 1, IC<ST ^ 1>{});
    if (t < my_tiles) {
      static_for<0, 2>([&](auto kb_c) {
        const int kb0 = t * kKTile + 32 * kb_c;
        if (CAUSAL && kb0 > q0w + 31 + off) return;   // every key after every row's limit
        const bool mask = kb0 + 32 > p.Tk || (CAUSAL && kb0 + 31 > q0w + off);
        if constexpr (D == 128)
          keys32(kb0, st_c, kb_c, IC<2>{}, mask);
        else if (mask)
          keys32(kb0, st_c, kb_c, IC<1>{}, true);
        else
          keys32(kb0, st_c, kb_c, IC<0>{}, false);
      });
    }
  };
  if (ntiles > 0) issue(0, IC<0>{});
  for (int t = 0; t < ntiles; t += 2) {
    step(t, IC<0>{});
    if (t + 1 < ntiles) step(t + 1, IC<1>{});
  }

  if (my_q < p.Tq) {
    bf16* dqr = (bf16*)p.dq + ((size_t)bh * p.Tq + my_q) * D;
#pragma unroll
    for (int db = 0; db < ND; ++db) store_acc_row<D>(dqr, db, half, dq[db], p.scale);
  }
}

template <int D, bool CAUSAL>
hipError_t launch_bwd_t(const BwdParams& p, hipStream_t stream) {
  if (p.Tq > 0) {
    constexpr int RPB = kPrepThreads / (D / 8);
    const long long rows = (long long)p.B * p.Hq * p.Tqp;
    hipLaunchKernelGGL(bwd_prep_kernel<D>, dim3((unsigned)((rows + RPB - 1) / RPB)),
                       dim3(kPrepThreads), 0, stream, p);
    // 8 wavefronts (256 rows) per workgroup share each K/V tile; on grids
    // too small to fill the device twice over, 4 (128 rows) balance better.
    const long long heads = (long long)p.B * p.Hq;
    const long long n8 = (p.Tq + 255) / 256 * heads;
    if (n8 >= 2 * compute_units()) {
      hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL, 8>), dim3((unsigned)n8), dim3(512), 0, stream, p);
    } else {
      const long long n4 = (p.Tq + 127) / 128 * heads;
      hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL, 4>), dim3((unsigned)n4), dim3(256), 0, stream, p);
    }
  }
  if (p.Tk > 0) {
    const int nkb = (p.Tk + kKeysPerWg - 1) / kKeysPerWg;
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3((unsigned)nkb * p.B * p.Hkv * p.kparts),
                       dim3(kDkdvThreads), 0, stream, p);
    if (p.kparts > 1) {
      const size_t n8 = (size_t)p.B * p.Hkv * p.Tk * (D / 8);
      hipLaunchKernelGGL(bwd_dkdv_merge_kernel<D>, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0,
                         stream, p);
    }
  }
  return hipGetLastError();
}

}  // namespace

int bwd_key_parts(int B, int Hkv, int Tk, bool causal) {
  // A causal key block's work falls with its position, and with under two
  // workgroups per compute unit the first blocks set the kernel time.
  const long long wgs = (long long)B * Hkv * ((Tk + kKeysPerWg - 1) / kKeysPerWg);
  return causal && wgs < 2LL * compute_units() ? 2 : 1;
}

hipError_t launch_bwd(const BwdParams& p, int d, bool causal, hipStream_t stream) {
  if (d == 64) return causal ? launch_bwd_t<64, true>(p, stream) : launch_bwd_t<64, false>(p, stream);
  return causal ? launch_bwd_t<128, true>(p, stream) : launch_bwd_t<128, false>(p, stream);
}

}  // namespace fa
