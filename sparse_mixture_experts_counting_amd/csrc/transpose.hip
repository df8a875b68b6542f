// Batched matrix transpose: dst[b][c][r] = src[b][r][c].  Converts weights given row-major in the
// pages' shapes (d x d_ff, d_ff x d, d x E) into the column-major storage the layer takes (once,
// when weights are loaded); the backward pass's bf16 transpose and row gather.
#include "common.h"
#include "gemm_common.h"
#include "kernels.h"

namespace moe {

// A 64 x 64 tile per block through LDS (one padding element per row keeps the column reads
// conflict-free); 256 threads, 16 elements each.  dst[b * dst_bstride + c * ldd + r].
template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(const T* __restrict__ src, int rows,
                                                        int cols, T* __restrict__ dst, int ldd,
                                                        long long dst_bstride) {
  __shared__ T tile[64][65];
  const T* s = src + (size_t)blockIdx.z * ((size_t)rows * cols);
  T* o = dst + (size_t)blockIdx.z * (size_t)dst_bstride;
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
    if (c < cols && r < rows) o[(size_t)c * ldd + r] = tile[tx][ty * 16 + i];
  }
}

void launch_transpose_ld(const void* src, int batch, int rows, int cols, int elem_bytes,
                         void* dst, int ldd, long long dst_bstride, hipStream_t s) {
  const dim3 grid((cols + 63) / 64, (rows + 63) / 64, batch);
  if (elem_bytes == 2)
    hipLaunchKernelGGL(transpose_kernel<uint16_t>, grid, dim3(256), 0, s, (const uint16_t*)src,
                       rows, cols, (uint16_t*)dst, ldd, dst_bstride);
  else
    hipLaunchKernelGGL(transpose_kernel<uint32_t>, grid, dim3(256), 0, s, (const uint32_t*)src,
                       rows, cols, (uint32_t*)dst, ldd, dst_bstride);
}

void launch_transpose(const void* src, int batch, int rows, int cols, int elem_bytes, void* dst,
                      hipStream_t s) {
  launch_transpose_ld(src, batch, rows, cols, elem_bytes, dst, rows, (long long)rows * cols, s);
}

// bf16 transpose of the backward pass (the weights, when the products cannot read them in place),
// 16 bytes per access: dst[b][c][r] = src[b][r][c] (rows, cols and ldd multiples of 8).  A block
// moves a 64 x 64 tile: each thread loads two 16-byte row chunks into a padded LDS tile (row pitch
// 72 elements), then gathers 8 rows of one column from LDS and stores them as one 16-byte chunk of
// a destination row.
__global__ __launch_bounds__(256) void transpose16_kernel(const uint16_t* __restrict__ src,
                                                          int rows, int cols,
                                                          uint16_t* __restrict__ dst, int ldd,
                                                          long long src_bstride,
                                                          long long dst_bstride) {
  constexpr int PITCH = 72;
  __shared__ __align__(16) uint16_t tile[64 * PITCH];
  const int p0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
  const uint16_t* s = src + (size_t)blockIdx.z * (size_t)src_bstride;
  uint16_t* o = dst + (size_t)blockIdx.z * (size_t)dst_bstride;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int q = threadIdx.x + 256 * i;
    const int rr = q >> 3, u = q & 7;
    const int r = p0 + rr, c = c0 + 8 * u;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (r < rows && c < cols) v = *reinterpret_cast<const u32x4*>(s + (size_t)r * cols + c);
    *reinterpret_cast<u32x4*>(&tile[rr * PITCH + 8 * u]) = v;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int q = threadIdx.x + 256 * i;
    const int cl = q >> 3, v = q & 7;
    const int c = c0 + cl, pc = p0 + 8 * v;
    if (c >= cols || pc >= rows) continue;
    u32x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = (uint32_t)tile[(8 * v + 2 * e) * PITCH + cl] |
             ((uint32_t)tile[(8 * v + 2 * e + 1) * PITCH + cl] << 16);
    *reinterpret_cast<u32x4*>(o + (size_t)c * ldd + pc) = w;
  }
}

void launch_transpose16(const void* src, int batch, int rows, int cols, void* dst, int ldd,
                        long long dst_bstride, hipStream_t s) {
  const dim3 grid((rows + 63) / 64, (cols + 63) / 64, batch);
  hipLaunchKernelGGL(transpose16_kernel, grid, dim3(256), 0, s, (const uint16_t*)src, rows, cols,
                     (uint16_t*)dst, ldd, (long long)rows * cols, dst_bstride);
}

// Expert-ordered copy of the token rows: dst[r] = src[gather[r] / gather_div] for the rows
// r < offsets[G] (16 bytes per access; cols a multiple of 8).  One block per row.
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint16_t* __restrict__ src,
                                                          int cols,
                                                          const int32_t* __restrict__ gather,
                                                          int gather_div,
                                                          const int32_t* __restrict__ offsets,
                                                          int G, uint16_t* __restrict__ dst) {
  const int r = blockIdx.x;
  if (r >= offsets[G]) return;
  const uint16_t* s = src + (size_t)(gather[r] / gather_div) * cols;
  uint16_t* o = dst + (size_t)r * cols;
  for (int c = 8 * threadIdx.x; c < cols; c += 8 * 256)
    *reinterpret_cast<u32x4*>(o + c) = *reinterpret_cast<const u32x4*>(s + c);
}

void launch_gather_rows(const void* src, int cols, const int32_t* gather, int gather_div,
                        const int32_t* offsets, int G, int rows_max, void* dst, hipStream_t s) {
  if (rows_max <= 0) return;
  hipLaunchKernelGGL(gather_rows_kernel, dim3(rows_max), dim3(256), 0, s, (const uint16_t*)src,
                     cols, gather, gather_div, offsets, G, (uint16_t*)dst);
}

}  // namespace moe
