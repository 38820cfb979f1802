/*
 * fa.h -- exact tiled attention (FlashAttention forward and split-KV
 * flash-decoding) for AMD Instinct MI355X (gfx950): the C ABI.
 *
 * Sources cited (web pages; sections named as headed there):
 *   [FUSED07] "Модуль 07: Fused-операторы и FlashAttention" -- course
 *             LLM Inference Systems, hermes-agent.ru.
 *   [LESSON]  "FlashAttention: внимание без матрицы n×n" -- lesson 5.7.2,
 *             ai.flicky.cc.
 *   [NOTE]    "Atencja od strony jądra: FlashAttention, softmax online i
 *             połączona dekwantyzacja" -- trefon.com notes.
 *   [BOOK5]   "Глава 5. Операторы и среда выполнения" -- AI infra book,
 *             bojieli.github.io.
 *   [FA3QA]   "Как работает FlashAttention-3 математически?" -- aivaro.ru
 *             (the Hopper FlashAttention-3 design: FP8 operands with
 *             higher-precision accumulation, section 6).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every tensor pointer is a DEVICE pointer to a contiguous, row-major
 *    buffer owned by the caller.  Inputs are only read; outputs are fully
 *    overwritten.  The library never frees caller memory.
 *  - bf16 buffers hold IEEE bfloat16 bit patterns (2 bytes per element).
 *  - `stream` is a hipStream_t passed as void*; NULL means the default
 *    (null) stream.  Calls enqueue work and return without waiting for it
 *    ([BOOK5] section 5.1.3 "Stream, event и порядок завершения": launches
 *    are asynchronous and the caller synchronises before reading results).
 *    A fault inside a kernel therefore surfaces at the caller's next
 *    synchronisation, not in the return code.
 *  - Return value: FA_OK (0) or one of the fa_status codes below.  Argument
 *    checks happen before any HIP call, and a workspace is grown before the
 *    first kernel is launched: after FA_ERR_NULL, FA_ERR_SHAPE,
 *    FA_ERR_UNSUPPORTED, FA_ERR_ALLOC or FA_ERR_DEVICE nothing has been
 *    enqueued.  FA_ERR_LAUNCH from an entry point that launches several
 *    kernels (fa_decode and its 8-bit forms: a range kernel and a merge
 *    kernel; fa_bwd: up to four kernels) may leave the kernels launched
 *    before the rejected one enqueued; their results are then incomplete
 *    and the outputs must not be used.
 *  - Device addresses are not validated beyond non-NULL: passing buffers
 *    smaller than the stated shapes is undefined behaviour.
 *  - HIP graphs: fa_fwd, fa_fwd_f32, fa_fwd_fp8 and fa_decode_noalloc
 *    allocate nothing and enqueue only kernel launches (no memset, no copy),
 *    so a stream capture of them replays like the calls themselves; the
 *    graph keeps the pointers it was captured with and reads the inputs at
 *    each replay.  Make one eager fa_decode_noalloc call on the device
 *    before capturing it (its first call looks up the workspace's device
 *    address).  fa_decode, its 8-bit forms and fa_bwd may grow their
 *    workspace with stream-ordered allocation and are not meant for capture.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL = 1,         /* a required pointer is NULL                      */
  FA_ERR_SHAPE = 2,        /* negative size, Hq not a multiple of Hkv, ...    */
  FA_ERR_UNSUPPORTED = 3,  /* head dimension other than 64 or 128             */
  FA_ERR_ALLOC = 4,        /* a library workspace could not be allocated     */
  FA_ERR_LAUNCH = 5,       /* the HIP runtime rejected a kernel launch        */
  FA_ERR_DEVICE = 6,       /* no usable HIP device / runtime error            */
  FA_ERR_SCRATCH = 7       /* fa_decode_noalloc: workspace over the fixed size */
} fa_status;

/*
 * fa_fwd -- exact attention forward pass (prefill), bf16 in/out.
 *
 * Computes, for every batch b, query head hq, query row i:
 *     s_ij   = scale * <q[b,hq,i,:], k[b,kh,j,:]>,   kh = hq / (Hq / Hkv)
 *     o[b,hq,i,:] = sum_j softmax_j(s_ij) * v[b,kh,j,:]
 *     lse[b,hq,i] = log sum_j exp(s_ij)              (natural log)
 * over the keys j visible to row i:
 *     causal == 0   all j < Tk;
 *     causal == 1   j <= i (top-left alignment, the reference mask of
 *                   [FUSED07] section "FlashAttention-наив на numpy");
 *     causal == 2   j <= i + Tk - Tq (bottom-right alignment: the Tq queries
 *                   are the last Tq positions of a sequence whose first
 *                   Tk - Tq positions are already cached, i.e. chunked
 *                   prefill; Tq = 1 is the decode rule of [NOTE] section
 *                   "Prefill i dekodowanie to różne problemy").  With
 *                   Tq > Tk the first Tq - Tk rows see no key.
 * Rows that see no key get o = 0 and lse = -inf.  This is softmax(Q K^T * scale) V
 * computed tile by tile with the online softmax of [FUSED07] section
 * "Online softmax: вывод" and the forward pass of [LESSON] section
 * "Прямой проход FlashAttention"; neither the score matrix nor the
 * probabilities are written to memory.  Grouped-query attention follows
 * [NOTE] section "Prefill i dekodowanie to różne problemy" (g = Hq/Hkv query
 * heads share kv head hq / g); lse is the per-row log-sum-exp
 * L_i = m_i + log l_i of [LESSON] section "Обратный проход".
 *
 *   q   : [B, Hq,  Tq, d] bf16        k, v : [B, Hkv, Tk, d] bf16
 *   o   : [B, Hq,  Tq, d] bf16 (rounded to nearest even)
 *   lse : [B, Hq,  Tq] fp32, or NULL to skip it
 *   d   : 64 or 128.  Any finite scale is accepted (1/sqrt(d) is usual).
 *
 * Arithmetic: q.k products and p.v products on bf16 matrix cores with fp32
 * accumulation; the running max, sum and rescaling in fp32; the
 * probabilities are rounded to bf16 before the p.v product.
 * B == 0, Hq == 0 or Tq == 0 is a valid empty call.  Tk == 0 gives o = 0 and
 * lse = -inf.  Errors: FA_ERR_NULL (q, k, v or o NULL on a non-empty call),
 * FA_ERR_SHAPE (negative sizes, Hkv < 1, Hq % Hkv != 0, non-finite scale,
 * causal outside 0..2), FA_ERR_UNSUPPORTED (d not 64/128), FA_ERR_LAUNCH.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int Hq, int Hkv, int Tq, int Tk, int d, int causal, float scale,
           void* stream);

/*
 * fa_fwd_f32 -- the same operation and contract as fa_fwd with fp32 q, k, v
 * and o.  Products and accumulation are fp32 (fp32 matrix cores); the
 * probabilities stay fp32.
 */
int fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
               int B, int Hq, int Hkv, int Tq, int Tk, int d, int causal, float scale,
               void* stream);

/*
 * fa_fwd_fp8 -- fa_fwd over 8-bit inputs with block scales (the FP8 path of
 * [LESSON] section "FlashAttention-2, -3 и дальше" and [FA3QA] section 6:
 * E4M3 operands, higher-precision accumulation).
 *
 *   q      : [B, Hq,  Tq, d] uint8 E4M3 codes    qscale : [B, Hq, Tq] fp32
 *   k, v   : [B, Hkv, Tk, d] uint8 E4M3 codes    kscale, vscale : [B, Hkv] fp32
 *   o, lse : as fa_fwd (bf16, fp32)
 * The inputs stand for q[b,h,i,:] = qscale[b,h,i] * e4m3(q8[b,h,i,:]) (one
 * scale per query row, fixed by the whole row as in [BOOK5] section 5.4.3,
 * Example 5-7), k[b,h,j,:] = kscale[b,h] * e4m3(k8[b,h,j,:]) and v alike
 * (one scale per kv head).  Scales must be positive and finite.  Computes
 * exactly what fa_fwd computes for those inputs (same causal modes 0/1/2,
 * any finite scale), with this arithmetic: q.k products of the codes are
 * exact; the 8-bit matrix cores add each block of 64 of them with terms far
 * below the block's largest product partly dropped (on the device, a block
 * of one product of 448^2 and 63 of 1 summed to 448^2 + 56), and the blocks
 * in fp32; the online softmax is
 * fp32; each key tile's probabilities are scaled by a power of two that
 * puts the tile's largest in [224, 448) and rounded to E4M3 (relative error
 * at most 2^-4, absolute at most 2^-9/448 of the row's largest probability)
 * for the p.v product, which applies the power of two as the matrix
 * instruction's block scale and sums in fp32; the row sum uses the
 * unrounded probabilities; o is rounded to bf16.  Errors: as fa_fwd, and FA_ERR_NULL for a NULL scale
 * array on a non-empty call.
 */
int fa_fwd_fp8(const void* q, const void* k, const void* v, const float* qscale,
               const float* kscale, const float* vscale, void* o, float* lse, int B, int Hq,
               int Hkv, int Tq, int Tk, int d, int causal, float scale, void* stream);

/*
 * fa_bwd -- gradients of fa_fwd (training backward pass), bf16 in/out.
 *
 * Given the forward's inputs q, k, v, its output o and row log-sum-exp lse
 * (as fa_fwd wrote them, same causal flag and scale) and the gradient dout
 * of a loss with respect to o, computes the gradients with respect to q, k
 * and v by the recomputation of [LESSON] section "Обратный проход:
 * пересчитать дешевле, чем хранить": score tiles are computed again,
 * P_ij = exp(scale * q_i.k_j - lse_i) restores the probabilities without
 * normalising, and with D_i = dout_i . o_i
 *     dv_j = sum_i P_ij dout_i,          dP_ij = dout_i . v_j,
 *     dS_ij = P_ij (dP_ij - D_i),
 *     dq_i = scale * sum_j dS_ij k_j,    dk_j = scale * sum_i dS_ij q_i,
 * over the (i, j) pairs visible under the same mask as fa_fwd (causal 0, 1
 * or 2 as there).  With
 * grouped-query attention ([NOTE] section "Prefill i dekodowanie to różne
 * problemy") dk and dv of kv head kh sum the contributions of its g = Hq/Hkv
 * query heads.  Nothing of size Tq x Tk is stored.
 *
 *   q, o, dout, dq : [B, Hq,  Tq, d] bf16     lse : [B, Hq, Tq] fp32
 *   k, v, dk, dv   : [B, Hkv, Tk, d] bf16     d   : 64 or 128
 *
 * dq, dk and dv are fully overwritten (rounded to nearest even); keys that
 * no query sees get dk = dv = 0.  Arithmetic: bf16 matrix products with fp32
 * accumulation; P and dS are rounded to bf16 before the products that
 * consume them; D_i, the exponentials and the masking in fp32.  The result
 * is deterministic (no atomics; every output element is summed in a fixed
 * order).
 *
 * Workspace: D_i and lse_i * log2(e) per query row (2 * B * Hq * Tqp fp32,
 * Tqp = Tq rounded up to a multiple of 256) and, for causal calls with
 * fewer than two dK/dV workgroups (128 keys each) per compute unit, fp32
 * partial dK and dV of two halves of every key block's query work
 * (2 * 2 * B * Hkv * Tk * d fp32), summed in a fixed order by a merge
 * kernel.  It lives in the library-owned buffer of (device, stream) that
 * fa_decode also uses, grown on demand with stream-ordered allocation;
 * fa_release_workspace() frees it.
 * B == 0, Hq == 0 or Tq == Tk == 0 is a valid empty call.  Tq == 0 gives
 * dk = dv = 0 (q, o, lse, dout and dq may then be NULL); Tk == 0 gives
 * dq = 0 (k, v, dk and dv may then be NULL).  Errors: FA_ERR_NULL,
 * FA_ERR_SHAPE (negative sizes, Hkv < 1, Hq % Hkv != 0, non-finite scale,
 * causal outside 0..2, sizes whose workgroup counts overflow),
 * FA_ERR_UNSUPPORTED (d not 64/128),
 * FA_ERR_ALLOC, FA_ERR_DEVICE, FA_ERR_LAUNCH.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
           const void* dout, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Tq,
           int Tk, int d, int causal, float scale, void* stream);

/*
 * fa_decode -- single-query attention over a KV cache with split-KV
 * flash-decoding ([NOTE] section "Prefill i dekodowanie to różne problemy",
 * Flash-decoding paragraph).  The valid keys of every (sequence, kv head)
 * are laid end to end in one key space, which is cut into num_splits
 * contiguous ranges of equal length, one per workgroup, so every workgroup
 * streams the same number of cache bytes whatever the mix of sequence
 * lengths.  A range yields a partial (m, l, o) for the query-head group of
 * each kv head it touches, and a second kernel merges the partials of each
 * (sequence, query head) with the rescaling rule of [BOOK5] section 5.3.3
 * (Example 5-6).
 *
 *   q       : [B, Hq, d] bf16 (one query token per sequence)
 *   kcache  : [B, Hkv, Tk_max, d] bf16      vcache : same shape
 *   seqlens : [B] int32, DEVICE memory; key j of sequence b is visible iff
 *             j < seqlens[b].  Values are clamped to [0, Tk_max] on the
 *             device; slots at or beyond seqlens[b] are never read.
 *   o       : [B, Hq, d] bf16; a sequence with seqlens[b] == 0 gets o = 0.
 *   scale is fixed at 1/sqrt(d).
 *   num_splits: number of key ranges (workgroups).  0 lets the library use
 *             as many as the device keeps resident at once; a positive
 *             request is capped at 2^20.  The result does not depend on the
 *             split count beyond floating-point rounding, and for a fixed
 *             split count it is bitwise reproducible (the merge runs in a
 *             fixed order, [BOOK5] section 5.2.4 on split reductions and
 *             determinism).
 *
 * Workspace: the prefix sums of the sequence lengths ((B+1) int64) and the
 * partials ((num_splits + B*Hkv*(g/h)) * h * (d+2) fp32 values, h the query
 * heads one workgroup serves, g = Hq/Hkv) live in a buffer the library owns
 * per (device, stream), grown on demand with stream-ordered allocation on
 * `stream` and kept for reuse.  Concurrent calls on the same stream are
 * ordered by the stream; calls on different streams use different buffers.
 * fa_release_workspace() frees them.
 * Errors: FA_ERR_NULL, FA_ERR_SHAPE (negative sizes, Hq % Hkv != 0,
 * num_splits < 0), FA_ERR_UNSUPPORTED (d not 64/128), FA_ERR_ALLOC,
 * FA_ERR_LAUNCH, FA_ERR_DEVICE (num_splits == 0 and the current device
 * cannot be queried).
 */
int fa_decode(const void* q, const void* kcache, const void* vcache, const int* seqlens,
              void* o, int B, int Hq, int Hkv, int Tk_max, int d, int num_splits,
              void* stream);

/* Bytes of the fixed per-device workspace of fa_decode_noalloc. */
#define FA_DECODE_SCRATCH_BYTES (4u << 20)

/*
 * fa_decode_noalloc -- fa_decode for callers that cannot allocate device
 * memory: code being captured into a HIP graph, serving loops and harnesses
 * that forbid allocation.  Same arguments, operation, result (bitwise equal
 * to fa_decode with the same num_splits) and errors, but the workspace
 * (prefix sums and partials, sized as for fa_decode) is a fixed array of
 * FA_DECODE_SCRATCH_BYTES bytes inside the library, one per device, which
 * the device holds from the library's load until the process ends.  Nothing
 * is allocated or freed (no hipMalloc, hipFree or allocating library
 * routine); the first call on a device looks up the array's device address
 * once.  A call whose workspace would exceed the array returns
 * FA_ERR_SCRATCH with nothing enqueued (at d = 128 with four query heads
 * per workgroup a slot takes 2080 bytes, so about 2000 slots fit: e.g. the
 * 512 automatic key ranges plus up to about 1500 (sequence, kv-head group)
 * segments).  All calls on one device share the
 * array: calls that can overlap in time on one device (different streams,
 * several host threads) race and give wrong results; the caller orders
 * them.  fa_release_workspace() does not touch it.
 */
int fa_decode_noalloc(const void* q, const void* kcache, const void* vcache, const int* seqlens,
                      void* o, int B, int Hq, int Hkv, int Tk_max, int d, int num_splits,
                      void* stream);

/* The number of key ranges (workgroups) fa_decode uses for a request, after
 * the 0 = automatic choice (which needs a current HIP device) and the cap,
 * without launching anything.  Returns minus the status code on error. */
int fa_decode_workgroups(int B, int Hq, int Hkv, int Tk_max, int d, int num_splits);

/*
 * fa_decode_fp8 -- fa_decode over an 8-bit KV cache, dequantised inside the
 * kernel as each row is loaded ([NOTE] section "Prefill i dekodowanie to
 * różne problemy": decode streams the cache, so the bytes per cached key set
 * its speed, and a compressed cache is expanded in the attention kernel's
 * tile load rather than by a separate pass).
 *
 *   kcache, vcache : [B, Hkv, Tk_max, d] uint8 codes in the E4M3 format with
 *                    no infinities (OCP FP8 E4M3: bias 7, 3 mantissa bits,
 *                    largest finite 448, 0x7F/0xFF NaN)
 *   kscale, vscale : [B, Hkv, Tk_max] fp32, one scale per cached row
 * Row j of kv head h of sequence b stands for
 *     K[b,h,j,:] = kscale[b,h,j] * e4m3(kcache[b,h,j,:])   (V alike),
 * and the result is exact attention of the query over those rows, with the
 * same contract as fa_decode (q and o bf16, seqlens on the device, scale
 * 1/sqrt(d), num_splits, workspace, determinism, errors; FA_ERR_NULL also for
 * a NULL scale array when Tk_max > 0).  Arithmetic: codes widen exactly to
 * bf16; q.k with fp32 sums (on the bf16 matrix core at d = 128 with a group
 * of 4 or 8 query heads per kv head or a multiple of it, else as packed bf16
 * dot products), times the K row scale; the probability times the V row
 * scale is rounded to bf16 for the p.v product; the row sums use the
 * unscaled fp32 probabilities.
 */
int fa_decode_fp8(const void* q, const void* kcache, const void* vcache, const float* kscale,
                  const float* vscale, const int* seqlens, void* o, int B, int Hq, int Hkv,
                  int Tk_max, int d, int num_splits, void* stream);

/* fa_decode_workgroups for fa_decode_fp8. */
int fa_decode_fp8_workgroups(int B, int Hq, int Hkv, int Tk_max, int d, int num_splits);

/*
 * fa_decode_int8 -- fa_decode_fp8 with an int8 cache: the other common
 * low-bit KV format with one scale per cached row ([NOTE] section
 * "Prefill i dekodowanie to różne problemy").
 *
 *   kcache, vcache : [B, Hkv, Tk_max, d] int8 codes (two's complement, stored
 *                    as bytes)
 *   kscale, vscale : [B, Hkv, Tk_max] fp32, one scale per cached row
 * Row j of kv head h of sequence b stands for
 *     K[b,h,j,:] = kscale[b,h,j] * int8(kcache[b,h,j,:])   (V alike);
 * contract, errors and arithmetic as fa_decode_fp8 (every int8 value widens
 * exactly to bf16).
 */
int fa_decode_int8(const void* q, const void* kcache, const void* vcache, const float* kscale,
                   const float* vscale, const int* seqlens, void* o, int B, int Hq, int Hkv,
                   int Tk_max, int d, int num_splits, void* stream);

/* fa_decode_workgroups for fa_decode_int8. */
int fa_decode_int8_workgroups(int B, int Hq, int Hkv, int Tk_max, int d, int num_splits);

/*
 * fa_read_probe -- measurement utility, not part of the attention path:
 * reads `bytes` bytes of device memory at `src` exactly once with 16-byte
 * nontemporal loads (one 1 MiB chunk per workgroup, several loads in flight
 * per lane)
 * and XORs every 32-bit word into *sink (device memory, zeroed by the
 * caller), so that a caller can time the device's achievable read
 * bandwidth and report it beside fa_decode's, whose workload is a single
 * stream over the KV cache ([NOTE] "Prefill i dekodowanie to różne
 * problemy": decode runs at memory speed).  Enqueued on `stream`.
 * Errors: FA_ERR_SHAPE (bytes not a multiple of 16), FA_ERR_NULL,
 * FA_ERR_LAUNCH.  bytes == 0 is a no-op.
 */
int fa_read_probe(const void* src, size_t bytes, unsigned* sink, void* stream);

/* Static description of a status code (never NULL). */
const char* fa_strerror(int status);

/* Frees every decode workspace the library holds.  The caller must make sure
 * no fa_decode call is still executing on the device. */
void fa_release_workspace(void);

#ifdef __cplusplus
}
#endif
#endif /* FA_H_ */
