// Streaming device copy: the measurement helper behind carve_stream_copy.  Every byte is
// read once and written once with 16-byte vector accesses and no reuse, so the rate it
// reaches is the device's achievable copy bandwidth, the second denominator next to the
// published HBM peak when a kernel's bytes are set against the memory roofline.
#include "carve_internal.h"

namespace carve {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;     // 16-byte vectors in flight per thread

// Grid-stride over tiles of kCopyThreads * kCopyUnroll vectors: all loads of a tile are
// issued before its stores, every access is coalesced across the wavefront, and the
// last tile is guarded element by element.
__global__ __launch_bounds__(kCopyThreads) void stream_copy_kernel(u32x4* __restrict__ dst,
                                                                   const u32x4* __restrict__ src, size_t n) {
  const size_t tile = (size_t)kCopyThreads * kCopyUnroll;
  for (size_t base = (size_t)blockIdx.x * tile; base < n; base += (size_t)gridDim.x * tile) {
    u32x4 r[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const size_t i = base + (size_t)u * kCopyThreads + threadIdx.x;
      if (i < n) r[u] = __builtin_nontemporal_load(src + i);
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const size_t i = base + (size_t)u * kCopyThreads + threadIdx.x;
      if (i < n) __builtin_nontemporal_store(r[u], dst + i);
    }
  }
}

hipError_t launch_stream_copy(void* dst, const void* src, size_t n16, int cus, hipStream_t st) {
  if (n16 == 0) return hipSuccess;
  const size_t tile = (size_t)kCopyThreads * kCopyUnroll;
  const size_t tiles = (n16 + tile - 1) / tile;
  const size_t cap = (size_t)(cus > 0 ? cus : 256) * 8;     // 8 workgroups per compute unit
  const unsigned grid = (unsigned)(tiles < cap ? tiles : cap);
  hipLaunchKernelGGL(stream_copy_kernel, dim3(grid), dim3(kCopyThreads), 0, st, (u32x4*)dst, (const u32x4*)src,
                     n16);
  return hipGetLastError();
}

}  // namespace carve
