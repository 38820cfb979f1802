// Device-side building blocks shared by the attention kernels (gfx950).
//
// Vector types, the bf16 matrix-core tile operations and the small
// cross-lane helpers.  Everything here targets 64-lane wavefronts.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

// 2^x on the transcendental unit (v_exp_f32); 2^-inf = 0.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Streaming load: a nontemporal global load (the "nt" cache policy), for
// data that is read exactly once.  On gfx950 a contiguous 16-byte-per-lane
// stream of such loads reaches about 7 TB/s, against 6.0-6.4 TB/s for the
// same stream with the default policy.
template <typename T>
__device__ __forceinline__ T stream_load(const T* p) {
  return __builtin_nontemporal_load(p);
}

// Value of lane (lane ^ 32): the two halves of a wavefront trade values.
__device__ __forceinline__ float swap_halves(float x) {
  return __shfl_xor(x, 32, 64);
}

// D = A(32x16) * B(16x32) + C on the bf16 matrix core, fp32 accumulate.
// Lane l supplies A[l%32][8*(l/32) .. +8] and B[8*(l/32) .. +8][l%32]; the
// accumulator register r of lane l holds C[8*(r/4) + 4*(l/32) + r%4][l%32].
__device__ __forceinline__ f32x16 mma_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// D = A(32x2) * B(2x32) + C on the fp32 matrix core.  Lane l supplies
// A[l%32][l/32] and B[l/32][l%32]; accumulator layout as above.
__device__ __forceinline__ f32x16 mma_32x32x2_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Round two fp32 values to bf16 (nearest even) and pack them.
__device__ __forceinline__ bf16x2 to_bf16x2(float a, float b) {
  f32x2 x = {a, b};
  return __builtin_convertvector(x, bf16x2);
}

// Reinterpret a 32-bit word as two bf16 values.  Done through memcpy: a
// __builtin_bit_cast applied to an element of a vector inside an unrolled
// loop was observed to read element 0 every time (hipcc / clang 22).
__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t w) {
  bf16x2 r;
  __builtin_memcpy(&r, &w, sizeof(r));
  return r;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;
typedef __attribute__((address_space(3))) const char lds_char_t;

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(lds_char_t*)p;
}

// Copy 16 bytes per lane from a buffer resource (byte offset voff + soff)
// straight into LDS at lds_base + 16 * lane (lds_base must be the same for
// the whole wavefront).  A lane whose voff is at or past the resource's size
// reads zeros; the scalar soff is not part of that range check, so callers
// that rely on it keep soff = 0 and put every offset into voff.
__device__ __forceinline__ void copy16_buf_to_lds(__amdgpu_buffer_rsrc_t rsrc, void* lds_base,
                                                  uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)lds_base, 16, voff, soff, 0, 0);
}

// s_waitcnt immediate that waits for the vector-memory counter to drop to N
// and leaves the other counters unconstrained.
template <int N>
constexpr int vmcnt_imm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  return (N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8);
}

// Workgroup barrier of the tile loop.  __syncthreads() would also wait for
// every global->LDS copy still in flight (its release fence covers them),
// which would cap the copy lead at one tile; here each wavefront first waits
// for the copies it needs (vmcnt) and for its own LDS reads, then meets the
// others.  The memory clobber keeps the compiler from moving LDS accesses
// across it.
__device__ __forceinline__ void tile_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace fa
