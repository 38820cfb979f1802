// LDS access helpers shared by the tiled attention kernels (gfx950).
//
// The kernels copy tiles from HBM straight into LDS (global/buffer loads
// with an LDS destination).  The compiler treats such a copy as a write to
// all of LDS and, before any LDS read it emits itself, waits for every copy
// still in flight -- including copies into a different pipeline stage.  The
// operand reads below are therefore inline assembly: the kernel orders them
// with explicit lgkmcnt waits, and a read's result is usable only after such
// a wait has been tied to it (lds_wait_tie, or lgkm_wait followed by tie).
#pragma once
#include <type_traits>

#include "fa_device.h"

namespace fa {

template <int V>
using IC = std::integral_constant<int, V>;

// Calls f(IC<I>{}) for I = B .. E-1 (compile-time unrolled).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(IC<B>{});
    static_for<B + 1, E>(f);
  }
}

// Copy 16 bytes per lane from global memory straight into LDS at
// lds_base + 16 * lane (lds_base must be the same for the whole wavefront).
__device__ __forceinline__ void copy16_to_lds(const void* g, void* lds_base) {
  __builtin_amdgcn_global_load_lds((glb_void_t*)g, (lds_void_t*)lds_base, 16, 0, 0);
}

// Transposing LDS read (gfx950 ds_read_b64_tr_b16) at addr + OFF bytes:
// within each group of 16 lanes, output lane 4*q + e receives element e of
// the 8 bytes addressed by input lanes q, q + 4, q + 8, q + 12 (in that
// order).  So if input lane 4*j + q of the group addresses 4 consecutive
// bf16 values (columns 4q .. 4q+3) of row j of a row-major tile, output lane
// 4*q + e holds column 4q + e of rows 0..3: a column slice, ready to be a
// matrix-core operand whose lane index runs along the tile's columns.
template <int OFF>
__device__ __forceinline__ u32x2 lds_read_tr(uint32_t addr) {
  u32x2 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF));
  return r;
}

// Transposing 8-bit LDS read (gfx950 ds_read_b64_tr_b8) at addr + OFF bytes:
// within each group of 16 lanes, output lane 8*h + i receives byte i of the
// 8 bytes addressed by input lanes 2e + h, e = 0..7 (in that order).  So if
// input lane 2e + h addresses 8 consecutive bytes (columns c_h .. c_h + 7)
// of row r_e of a row-major byte tile, output lane 8*h + i holds column
// c_h + i of rows r_0 .. r_7.
template <int OFF>
__device__ __forceinline__ u32x2 lds_read_tr8(uint32_t addr) {
  u32x2 r;
  asm volatile("ds_read_b64_tr_b8 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF));
  return r;
}

// 16-byte LDS read at addr + OFF bytes.
template <int OFF>
__device__ __forceinline__ bf16x8 lds_read_b128(uint32_t addr) {
  bf16x8 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF));
  return r;
}

// 16-byte LDS read as four 32-bit words at addr + OFF bytes.
template <int OFF>
__device__ __forceinline__ u32x4 lds_read_u32x4(uint32_t addr) {
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF));
  return r;
}

// 16-byte LDS read of four fp32 values at addr + OFF bytes.
template <int OFF>
__device__ __forceinline__ f32x4 lds_read_f32x4(uint32_t addr) {
  f32x4 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF));
  return r;
}

// 16-byte LDS write of four fp32 values at addr + OFF bytes (inline assembly,
// so that the compiler does not first wait for the global->LDS copies in
// flight).  Complete once an lgkmcnt wait has covered it.
template <int OFF>
__device__ __forceinline__ void lds_write_f32x4(uint32_t addr, f32x4 v) {
  asm volatile("ds_write_b128 %0, %1 offset:%2" ::"v"(addr), "v"(v), "n"(OFF) : "memory");
}

// Wait until at most N LDS reads of this wavefront are outstanding, tied to
// the operand that needed the wait.
template <int N>
__device__ __forceinline__ void lds_wait_tie(bf16x8& v) {
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(v) : "n"(N));
}

// Wait until at most N LDS reads of this wavefront are outstanding (LDS
// reads complete in issue order).  Values whose reads were covered by the
// wait must then pass through tie() before their first use.
template <int N>
__device__ __forceinline__ void lgkm_wait() {
  static_assert(N >= 0 && N < 16, "lgkmcnt range");
  asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(N));
}

// Orders the uses of v after the preceding lgkm_wait(): an empty volatile
// statement that claims to modify v (volatile statements keep their order).
template <typename T>
__device__ __forceinline__ void tie(T& v) {
  asm volatile("" : "+v"(v));
}

}  // namespace fa
