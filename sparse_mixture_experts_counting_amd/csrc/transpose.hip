// Batched matrix transpose: dst[b][c][r] = src[b][r][c].  Converts weights given row-major in the
// pages' shapes (d x d_ff, d_ff x d, d x E) into the column-major storage the layer takes; run once
// when weights are loaded, not per layer call.
#include "common.h"
#include "kernels.h"

namespace moe {

// A 64 x 64 tile per block through LDS (one padding element per row keeps the column reads
// conflict-free); 256 threads, 16 elements each.
template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(const T* __restrict__ src, int rows,
                                                        int cols, T* __restrict__ dst) {
  __shared__ T tile[64][65];
  const size_t plane = (size_t)rows * cols;
  const T* s = src + (size_t)blockIdx.z * plane;
  T* o = dst + (size_t)blockIdx.z * plane;
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = r0 + ty * 16 + i, c = c0 + tx;
    if (r < rows && c < cols) tile[ty * 16 + i][tx] = s[(size_t)r * cols + c];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int c = c0 + ty * 16 + i, r = r0 + tx;
    if (c < cols && r < rows) o[(size_t)c * rows + r] = tile[tx][ty * 16 + i];
  }
}

void launch_transpose(const void* src, int batch, int rows, int cols, int elem_bytes, void* dst,
                      hipStream_t s) {
  const dim3 grid((cols + 63) / 64, (rows + 63) / 64, batch);
  if (elem_bytes == 2)
    hipLaunchKernelGGL(transpose_kernel<uint16_t>, grid, dim3(256), 0, s, (const uint16_t*)src,
                       rows, cols, (uint16_t*)dst);
  else
    hipLaunchKernelGGL(transpose_kernel<uint32_t>, grid, dim3(256), 0, s, (const uint32_t*)src,
                       rows, cols, (uint32_t*)dst);
}

}  // namespace moe
