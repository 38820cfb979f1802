// Read-bandwidth probe: streams a device buffer once with 16-byte loads so
// that the achievable HBM read rate of the device can be reported beside the
// decode kernel's (the published peak is not reachable by any kernel).  Not
// part of the attention path.
//
// One workgroup of 256 threads per 1 MiB chunk; each thread keeps 8
// nontemporal loads in flight (the fastest streaming pattern measured on
// gfx950 among grid sizes, unroll depths and cache policies) and folds the
// data into an XOR checksum, which the first lane of every workgroup
// combines into *sink with an atomic XOR, so the loads cannot be removed and
// the result is checkable.
#include <stdint.h>

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;
constexpr size_t kProbeChunk = (size_t)1 << 20;   // bytes per workgroup

__global__ void __launch_bounds__(kProbeThreads) read_probe_kernel(const u32x4* __restrict__ src,
                                                                  size_t n16, unsigned* sink) {
  constexpr size_t per = kProbeChunk / 16;
  const size_t lo = (size_t)blockIdx.x * per;
  const size_t hi = lo + per < n16 ? lo + per : n16;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (size_t i = lo + threadIdx.x; i < hi; i += (size_t)kProbeThreads * kProbeUnroll) {
    u32x4 r[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) {
      const size_t j = i + (size_t)u * kProbeThreads;
      r[u] = j < hi ? stream_load(src + j) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= r[u];
  }
  unsigned x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x ^= __shfl_xor(x, off, 64);
  if ((threadIdx.x & 63) == 0) atomicXor(sink, x);
}

}  // namespace

hipError_t launch_read_probe(const void* src, size_t bytes, unsigned* sink, hipStream_t stream) {
  const size_t n16 = bytes / 16;
  const size_t blocks = (bytes + kProbeChunk - 1) / kProbeChunk;
  hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)blocks), dim3(kProbeThreads), 0, stream,
                     (const u32x4*)src, n16, sink);
  return hipGetLastError();
}

}  // namespace fa
