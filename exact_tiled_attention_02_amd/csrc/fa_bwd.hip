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
//     K and V stay in registers and dK^T, dV^T in AGPR accumulators while
//     blocks of 32 query rows (Q, dO, L, D) of every query head of the group
//     stream through an LDS ring.  Per block a wavefront forms S = Q K^T and
//     dP = dO V^T (lane = key, registers = queries), P and dS on the VALU,
//     then dV^T += dO^T P and dK^T += Q^T dS with dO^T and Q^T read through
//     the transposing LDS read; the three steps of consecutive blocks are
//     software-pipelined (see the kernel).  Under the causal mask the query
//     rows that see none of the workgroup's keys are never visited.
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
// A workgroup owns 128 keys of one kv head, 32 per wavefront, with K and V
// rows in registers and dK^T, dV^T in AGPR accumulators (lane = key).  Its
// work is a sequence of 32-row query blocks -- every query head of the
// group, the rows that can see its keys -- and each block passes three
// steps, software-pipelined so that iteration k of the loop runs
//   phase 1: X(k)   S = Q K^T and dP = dO V^T of block k, with dS = P (dP - D)
//            of block k-1 and the bf16 packing of its P and dS on the VALU;
//   phase 2: Z(k-1) dV^T += dO^T P and dK^T += Q^T dS of block k-1, with
//            P = 2^(S c - L) of block k on the VALU,
// one or two VALU elements per matrix-core product, so that exponentials and
// conversions issue between independent products.  S and dP stay in AGPRs
// until the VALU reads them (dP alternates between two sets: dS of block k-1
// reads one while X(k) fills the other).  Rows of Q and dO, and the L and D
// values, stream through LDS rings of 5 stages; Z reads block k-1's rows with
// the transposing read.  Between the phases every wavefront waits for its
// copies of block k+1, the workgroup meets, and the copies of block k+3 are
// issued into the stage block k-2 used.  Iterations before the first block
// and after the last (pipeline fill and drain, and padding to an even count)
// compute with P = 0 on the data of a real block, so they add exactly zero.

// Copy 16 bytes per lane from a buffer resource (lane offset voff, range
// checked) or from global memory straight into LDS at lds + 16 * lane (lds
// the same for the whole wavefront).
__device__ __forceinline__ void buf_to_lds(__amdgpu_buffer_rsrc_t rsrc, uint32_t lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)(size_t)lds, 16, voff, 0, 0, 0);
}
__device__ __forceinline__ void glb_to_lds(const void* src, uint32_t lds) {
  __builtin_amdgcn_global_load_lds((glb_void_t*)src, (lds_void_t*)(size_t)lds, 16, 0, 0);
}

// acc += a * b on the bf16 matrix core, accumulator in AGPRs.
__device__ __forceinline__ void mfma_acc(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// acc = a * b on the bf16 matrix core, into AGPRs.
__device__ __forceinline__ void mfma_new(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=a"(acc) : "v"(a), "v"(b));
}

// One accumulator register read into a VGPR where it stands in the program.
__device__ __forceinline__ float acc_read(const float& a) {
  float v;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a));
  return v;
}

__device__ __forceinline__ void agpr_zero(f32x16& acc) {
  asm volatile("" : "=a"(acc) : "0"(f32x16{}));
}

// LDS read schedule of a dK/dV iteration.  Slot m (0 .. 2NS-1; the product
// of slot m is the X product m for m < NS, else the Z product m - NS) first
// issues the reads of operand m + LA -- X operands are one 16-byte read,
// Z operands two transposing reads, operands past the iteration's end are
// the next iteration's first ones -- then at slot NS/2 the 4 reads of the
// block's L and at slot NS + NS/2 the 4 reads of its D.  wait[m] is the
// lgkmcnt the product of slot m waits for: every read of its operand done,
// and at slot NS also L, at slot 0 also the previous iteration's D.
template <int NS, int LA>
struct DkdvSchedule {
  int wait[2 * NS];
  constexpr DkdvSchedule() : wait() {
    const int slr = NS / 2, sdr = NS + NS / 2;
    int last[4][2 * NS] = {};   // issue index of the last read of (iteration, operand)
    int issued[3][2 * NS] = {}; // reads issued through slot m's issues
    int lread[3] = {}, dread[3] = {};
    int n = 0;
    for (int it = 0; it < 3; ++it) {
      for (int m = 0; m < 2 * NS; ++m) {
        int f = m + LA, ti = it;
        if (f >= 2 * NS) {
          f -= 2 * NS;
          ti = it + 1;
        }
        n += f < NS ? 1 : 2;
        last[ti][f] = n - 1;
        if (m == slr) {
          n += 4;
          lread[it] = n - 1;
        }
        if (m == sdr) {
          n += 4;
          dread[it] = n - 1;
        }
        issued[it][m] = n;
      }
    }
    for (int m = 0; m < 2 * NS; ++m) {
      int w = issued[2][m] - 1 - last[2][m];
      if (m == NS && issued[2][m] - 1 - lread[2] < w) w = issued[2][m] - 1 - lread[2];
      if (m == 0 && issued[2][m] - 1 - dread[1] < w) w = issued[2][m] - 1 - dread[1];
      wait[m] = w;
    }
  }
};

template <int NS, int LA>
constexpr bool dkdv_schedule_ok() {
  constexpr DkdvSchedule<NS, LA> s{};
  for (int m = 0; m < 2 * NS; ++m)
    if (s.wait[m] < 0 || s.wait[m] > 15) return false;
  return true;
}

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(kDkdvThreads, 1) bwd_dkdv_kernel(const BwdParams p) {
  constexpr int NW = kDkdvThreads / 64;
  constexpr int NC = D / 16;                     // 16-deep steps over the head dim
  constexpr int ND = D / 32;                     // 32-wide head-dim blocks
  constexpr int NS = D / 8;                      // products per phase (2 NC = 4 ND)
  constexpr int EPS = 16 / NS;                   // P or dS elements per product
  constexpr int CPR = D / 8;                     // 16-byte chunks per row
  constexpr int RB = 32 * D * 2;                 // bytes of 32 rows of Q or dO
  constexpr int SBY = 2 * RB;                    // a stage: [Q | dO]
  constexpr int NST = 5;                         // stages per ring
  constexpr int LDR = NST * SBY;                 // L/D ring: stage = [L x32 | D x32] fp32
  constexpr int NCR = 32 * CPR / kDkdvThreads;   // row copies per thread and tensor
  constexpr int NV = 2 * NCR + 1;                // vector-memory instructions per iteration
  constexpr int LA = 4;                          // operands read ahead of their product
  constexpr int SLR = NS / 2;                    // slot that reads L of block k
  constexpr int SDR = NS + NS / 2;               // slot that reads D of block k
  static_assert(NCR >= 1, "tile too small for the workgroup");
  static_assert(dkdv_schedule_ok<NS, LA>(), "LDS read schedule exceeds the wait counter");
  constexpr DkdvSchedule<NS, LA> sched{};
  __shared__ __attribute__((aligned(16))) char lds[LDR + NST * 256];

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
  for (int i = 0; i < ND; ++i) {
    agpr_zero(dv[i]);
    agpr_zero(dk[i]);
  }

  // Blocks: rows qs + 32*i .. +31 of each of the g query heads, item
  // it = head * nblk + i.  Causal: row i sees key j iff j <= i + off, so rows
  // before k0 - off see none of these keys.
  const int off = p.causal_off;
  const int qs = CAUSAL ? max(0, k0 - off) / 32 * 32 : 0;
  const int nblk = qs < p.Tq ? (p.Tq - qs + 31) / 32 : 0;
  const int nit = p.g * nblk;
  const int i0 = (int)((long long)nit * part / p.kparts);
  const int i1 = (int)((long long)nit * (part + 1) / p.kparts);

  if (i1 > i0) {
    // Copy r of wavefront w fills LDS chunks [(r*NW + w)*64, +64) of a row
    // tile: chunk L is row L / CPR at position L % CPR, holding chunk
    // (L % CPR) ^ bswz(row) of that row.
    uint32_t csrc[NCR];
#pragma unroll
    for (int r = 0; r < NCR; ++r) {
      const int L = (r * NW + wave) * 64 + lane;
      const int row = L / CPR;
      csrc[r] = (uint32_t)(row * D + (((L % CPR) ^ bswz<D>(row)) << 3)) * 2u;
    }
    const int qbytes = p.Tq * D * 2;
    // Base of this wavefront's 1 KB of every tile in LDS, passed through an
    // empty statement once per iteration so that the compiler forms each
    // copy's destination there instead of holding them all in scalar
    // registers for the whole loop.
    uint32_t lb = lds_addr(lds) + wave * 1024;
    // A plane's base address in scalar registers (the compiler may hold
    // loop-invariant parts of it in vector registers, and a buffer descriptor
    // built from those would be treated as divergent).
    auto plane_ptr = [&](const void* base, size_t elems) __attribute__((always_inline)) {
      const uint64_t a = (uint64_t)(uintptr_t)((const bf16*)base + elems);
      const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
      const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
      return (void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
    };
    // Rows of Q and dO (rows past Tq read as zeros: the whole offset is in
    // the range-checked lane offset), and L and D (padded planes: always in
    // bounds; wavefronts 0, 1 copy L, 2, 3 copy D, 16 values each with 4
    // lanes) of the block at (plane, q0) into stage st.
    auto copy_block = [&](int plane, int q0, int st) __attribute__((always_inline)) {
      const __amdgpu_buffer_rsrc_t qr = __builtin_amdgcn_make_buffer_rsrc(
          plane_ptr(p.q, (size_t)plane * p.Tq * D), 0, qbytes, 0x00020000);
      const __amdgpu_buffer_rsrc_t gr = __builtin_amdgcn_make_buffer_rsrc(
          plane_ptr(p.dout, (size_t)plane * p.Tq * D), 0, qbytes, 0x00020000);
      const uint32_t base = (uint32_t)q0 * D * 2;
      const uint32_t sb = lb + (uint32_t)(st * SBY);
#pragma unroll
      for (int r = 0; r < NCR; ++r) {
        buf_to_lds(qr, sb + r * NW * 1024, csrc[r] + base);
        buf_to_lds(gr, sb + RB + r * NW * 1024, csrc[r] + base);
      }
      const float* src = (wave < 2 ? p.l2 : p.delta) + (size_t)plane * p.Tqp + q0 + 16 * (wave & 1) + 4 * lane;
      if (lane < 4) glb_to_lds(src, lb - wave * 1024 + LDR + st * 256 + 64 * wave);
    };

    // Walk over the blocks in sequence: item it = h * nblk + i runs from i0
    // to i1 - 1, and blocks outside [i0, i1) stand on the nearest end.
    struct Walk {
      int h, i;
    };
    const int plane0 = b * p.Hq + kvh * p.g;
    auto walk_start = [&]() __attribute__((always_inline)) {
      const int h = i0 / nblk;
      return Walk{h, i0 - h * nblk};
    };
    auto walk_to = [&](Walk& w, int j) __attribute__((always_inline)) {   // w is at block j - 1
      if (j > i0 && j < i1) {
        if (++w.i == nblk) {
          w.i = 0;
          ++w.h;
        }
      }
    };
    auto next_st = [](int s) __attribute__((always_inline)) { return s == NST - 1 ? 0 : s + 1; };

    // Per-lane LDS read bases at stage 0 (iterations add the stage).
    const TileReads<D> rd(lds_addr(lds), lane);
    const uint32_t la0 = lds_addr(lds) + LDR + 16 * half;   // L/D rows 8j + 4*half .. +3
    const float c = p.c;

    // Iterations k = kbeg .. i1 (an even count).
    const int niter = (i1 - i0 + 2) / 2 * 2;
    const int kbeg = i1 + 1 - niter;
    Walk cw = walk_start();   // copies: block kbeg - 1 first
    Walk mw = walk_start();   // masks: block kbeg first
    copy_block(plane0 + cw.h, qs + 32 * cw.i, NST - 1);
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      walk_to(cw, kbeg + j);
      copy_block(plane0 + cw.h, qs + 32 * cw.i, j);
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm<0>());
    asm volatile("s_barrier" ::: "memory");

    int st = 0;   // stage of block k
    uint32_t rk[NC];
#pragma unroll
    for (int s = 0; s < NC; ++s) rk[s] = rd.row[s];
    f32x16 sc, dp[2];
    agpr_zero(dp[1]);
    float pv[16];
    f32x4 lv[4], dl[4];
#pragma unroll
    for (int r = 0; r < 16; ++r) pv[r] = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) dl[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    bf16x8 pre[LA];
    // X operands of the first iteration, as the iteration before would have
    // read them.
    auto read_x = [&](const uint32_t (&r)[NC], auto f_c) __attribute__((always_inline)) {
      constexpr int F = decltype(f_c)::value;
      return lds_read_b128<(F % 2) * RB>(r[F / 2]);
    };
    static_for<0, LA>([&](auto f_c) { pre[f_c] = read_x(rk, f_c); });

    auto iteration = [&](const int k, auto par_c) __attribute__((always_inline)) {
      constexpr int P = decltype(par_c)::value;   // dP set written by X(k)
      const int stp = st == 0 ? NST - 1 : st - 1;  // stage of block k-1
      const int stn = next_st(st);                 // stage of block k+1
      uint32_t zk[2][ND], rn[NC];
#pragma unroll
      for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int db = 0; db < ND; ++db) zk[e][db] = rd.tr[e][db] + (uint32_t)(stp * SBY);
#pragma unroll
      for (int s = 0; s < NC; ++s) rn[s] = rd.row[s] + (uint32_t)(stn * SBY);
      const uint32_t la = la0 + (uint32_t)(st * 256);
      walk_to(mw, k);
      const int qy = qs + 32 * mw.i;
      const bool yvalid = k >= i0 && k < i1;
      const bool ymask = !yvalid || (CAUSAL && qy + off < kw + 31) || qy + 32 > p.Tq;

      bf16x8 cur[2 * NS];
      float dsv[16];
      uint32_t pw[8], sw[8];
      auto read_z = [&](auto f_c) __attribute__((always_inline)) {
        constexpr int G = decltype(f_c)::value - NS;
        constexpr int T = G / (2 * ND);   // 0: dO^T (dV), 1: Q^T (dK)
        constexpr int J = (G / ND) % 2;
        constexpr int DB = G % ND;
        constexpr int OFS = (T == 0 ? RB : 0) + J * 16 * D * 2;
        u32x2 v[2];
        v[0] = lds_read_tr<OFS>(zk[0][DB]);
        v[1] = lds_read_tr<OFS>(zk[1][DB]);
        return join_tr(v);
      };
      static_for<0, 2 * NS>([&](auto m_c) {
        constexpr int M = decltype(m_c)::value;
        constexpr int FA = M + LA;
        if constexpr (FA < NS)
          cur[FA] = read_x(rk, IC<FA>{});
        else if constexpr (FA < 2 * NS)
          cur[FA] = read_z(IC<FA>{});
        else
          pre[FA - 2 * NS] = read_x(rn, IC<FA - 2 * NS>{});
        if constexpr (M == SLR)
          static_for<0, 4>([&](auto j_c) { lv[j_c] = lds_read_f32x4<32 * j_c>(la); });
        if constexpr (M == SDR)
          static_for<0, 4>([&](auto j_c) { dl[j_c] = lds_read_f32x4<128 + 32 * j_c>(la); });
        lgkm_wait<sched.wait[M]>();
        if constexpr (M == 0) {
#pragma unroll
          for (int j = 0; j < 4; ++j) tie(dl[j]);
        }
        if constexpr (M == NS) {
#pragma unroll
          for (int j = 0; j < 4; ++j) tie(lv[j]);
        }
        bf16x8 a;
        if constexpr (M < LA)
          a = pre[M];
        else
          a = cur[M];
        if constexpr (M < NS) {
          // X(k): the S and dP chains alternate.
          constexpr int S = M / 2;
          if constexpr (M % 2 == 0) {
            if constexpr (S == 0)
              mfma_new(sc, a, kf[0]);
            else
              mfma_acc(sc, a, kf[S]);
          } else {
            if constexpr (S == 0)
              mfma_new(dp[P], a, vf[0]);
            else
              mfma_acc(dp[P], a, vf[S]);
          }
          // Block k-1: dS of EPS elements, and the bf16 packing of P (masked
          // at the end of the previous iteration) and of dS.
#pragma unroll
          for (int e = 0; e < EPS; ++e) {
            const int r = EPS * M + e;
            const float y = acc_read(dp[P ^ 1][r]);
            dsv[r] = pv[r] * (y - dl[r >> 2][r & 3]);
          }
          if constexpr ((EPS * M + EPS - 1) % 2 == 1) {
            constexpr int W = (EPS * M + EPS - 1) / 2;
            sw[W] = __builtin_bit_cast(uint32_t, to_bf16x2(dsv[2 * W], dsv[2 * W + 1]));
            tie(sw[W]);
          }
          if constexpr (M < 8) {
            pw[M] = __builtin_bit_cast(uint32_t, to_bf16x2(pv[2 * M], pv[2 * M + 1]));
            tie(pw[M]);
          }
          if constexpr (M == NS - 1) {
            // Every wavefront's copies of block k+1 have landed and nobody
            // reads the stage of block k-2 any more: refill it with block k+3.
            __builtin_amdgcn_s_waitcnt(vmcnt_imm<NV>());
            asm volatile("s_barrier" ::: "memory");
            asm volatile("" : "+s"(lb));
            walk_to(cw, k + 3);
            int st3 = next_st(stn);
            st3 = next_st(st3);
            copy_block(plane0 + cw.h, qs + 32 * cw.i, st3);
          }
        } else {
          // Z(k-1) with block k-1's P and dS, and P of EPS elements of block k.
          constexpr int G = M - NS;
          constexpr int T = G / (2 * ND);
          constexpr int J = (G / ND) % 2;
          constexpr int DB = G % ND;
          bf16x8 bop;
          const u32x4 wq = T == 0 ? u32x4{pw[4 * J], pw[4 * J + 1], pw[4 * J + 2], pw[4 * J + 3]}
                                  : u32x4{sw[4 * J], sw[4 * J + 1], sw[4 * J + 2], sw[4 * J + 3]};
          __builtin_memcpy(&bop, &wq, sizeof(wq));
          if constexpr (T == 0)
            mfma_acc(dv[DB], a, bop);
          else
            mfma_acc(dk[DB], a, bop);
#pragma unroll
          for (int e = 0; e < EPS; ++e) {
            const int r = EPS * G + e;
            const float x = acc_read(sc[r]);
            pv[r] = exp2_fast(fmaf(x, c, -lv[r >> 2][r & 3]));
            tie(pv[r]);
          }
        }
      });
      if (ymask) {
        // Row offsets 8*(r/4) + r%4 outside [lo, hi) are masked: rows past Tq
        // (or all, off this workgroup's blocks), and under the causal mask
        // rows before this lane's key.
        const int base = qy + 4 * half;
        const int lo = CAUSAL ? my_k - off - base : -64;
        const int hi = yvalid ? p.Tq - base : -64;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int o = 8 * (r >> 2) + (r & 3);
          pv[r] = (o >= lo && o < hi) ? pv[r] : 0.f;
        }
      }
#pragma unroll
      for (int s = 0; s < NC; ++s) rk[s] = rn[s];
      st = stn;
    };
    for (int k = kbeg; k < kbeg + niter; k += 2) {
      iteration(k, IC<0>{});
      iteration(k + 1, IC<1>{});
    }
    // Copies and reads issued for iterations that do not run.
    __builtin_amdgcn_s_waitcnt(vmcnt_imm<0>());
    lgkm_wait<0>();
  }

  // No accumulator is read within 24 wait states of its last product.
#pragma unroll
  for (int db = 0; db < ND; ++db) asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(dv[db]), "+a"(dk[db]));

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
