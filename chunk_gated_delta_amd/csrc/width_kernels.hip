// Row resizing for calls whose key and value widths differ.  The state of the CARVE
// recurrence is d_v x d_k with independent widths (CARVE notes, section 1).  The chunk
// kernels are built for one width D on both axes, so such a call runs at D = max(d_k, d_v)
// on copies whose narrower axis is padded.  Padded key channels carry k = q = 0,
// log g = 0 and b = 1; padded value rows carry v = 0.  This file moves rows between
// the two widths: every row of w_in elements becomes a row of w_out elements, cut
// short or filled with a constant.
#include "carve_internal.h"

namespace carve {

// dst[r][c] = c < w_in ? src[r][c] : fill, for r < rows and c < w_out (element type E).
// Consecutive threads take consecutive destination elements, so stores are coalesced
// and loads are coalesced within each row.
template <typename E>
__global__ __launch_bounds__(256) void resize_rows_kernel(E* __restrict__ dst, const E* __restrict__ src,
                                                          size_t rows, size_t w_in, size_t w_out, E fill) {
  const size_t n = rows * w_out;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
    const size_t r = i / w_out, c = i - r * w_out;
    dst[i] = c < w_in ? src[r * w_in + c] : fill;
  }
}

hipError_t launch_resize_rows(void* dst, const void* src, size_t rows, size_t w_in, size_t w_out, int elem_bytes,
                              unsigned fill_bits, hipStream_t st) {
  const size_t n = rows * w_out;
  if (n == 0) return hipSuccess;
  const size_t blocks = (n + 255) / 256;
  const unsigned grid = (unsigned)(blocks < 8192 ? blocks : 8192);
  if (elem_bytes == 4) {
    hipLaunchKernelGGL(resize_rows_kernel<unsigned>, dim3(grid), dim3(256), 0, st, static_cast<unsigned*>(dst),
                       static_cast<const unsigned*>(src), rows, w_in, w_out, fill_bits);
  } else if (elem_bytes == 2) {
    hipLaunchKernelGGL(resize_rows_kernel<unsigned short>, dim3(grid), dim3(256), 0, st,
                       static_cast<unsigned short*>(dst), static_cast<const unsigned short*>(src), rows, w_in, w_out,
                       (unsigned short)(fill_bits & 0xffffu));
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace carve
