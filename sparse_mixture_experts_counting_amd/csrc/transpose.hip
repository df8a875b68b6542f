// Batched matrix transpose: dst[b][c][r] = src[b][r][c].  Converts weights given row-major in the
// pages' shapes (d x d_ff, d_ff x d, d x E) into the column-major storage the layer takes (once,
// when weights are loaded), and lays out the transposed operands of the backward pass.
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

// Group-padded transpose of expert-ordered rows (bf16), the K-grouped operand layout:
// dst[c][kpad(offsets[g], g) + i] = src[row][c] for the i-th row of group g, where row =
// gather[r] / gather_div (or r) and r = offsets[g] + i; the up to 7 + 8 columns between groups are
// zero.  offsets == NULL is one group of `rows` rows at column 0 (columns up to the next multiple
// of 8 zero).  Columns past the last group's padding are not written.
__global__ __launch_bounds__(256) void transpose_grouped_kernel(
    const uint16_t* __restrict__ src, int src_rows, const int32_t* __restrict__ gather,
    int gather_div, const int32_t* __restrict__ offsets, int G, int rows, int cols,
    uint16_t* __restrict__ dst, int ldd) {
  __shared__ uint16_t tile[64][65];
  const int p0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  const int total = offsets ? offsets[G] : rows;
  const int pend = offsets ? kpad(total, G) : (rows + 7) & ~7;
#pragma unroll 4
  for (int i = 0; i < 16; ++i) {
    const int pc = p0 + ty * 16 + i, c = c0 + tx;
    int r = -1;
    if (pc < pend) {
      if (offsets) {                      // last group whose padded start is <= pc
        int lo = 0, hi = G - 1;
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (kpad(offsets[mid], mid) <= pc) lo = mid; else hi = mid - 1;
        }
        const int cand = offsets[lo] + (pc - kpad(offsets[lo], lo));
        r = cand < offsets[lo + 1] ? cand : -1;
      } else {
        r = pc < rows ? pc : -1;
      }
    }
    uint16_t v = 0;
    if (r >= 0 && c < cols) {
      const int row = gather ? gather[r] / gather_div : r;
      if (row >= 0 && row < src_rows) v = src[(size_t)row * cols + c];
    }
    tile[ty * 16 + i][tx] = v;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int c = c0 + ty * 16 + i, pc = p0 + tx;
    if (c < cols && pc < pend) dst[(size_t)c * ldd + pc] = tile[tx][ty * 16 + i];
  }
}

void launch_transpose_grouped(const void* src, int src_rows, const int32_t* gather,
                              int gather_div, const int32_t* offsets, int G, int rows_max,
                              int cols, void* dst, int ldd, hipStream_t s) {
  const dim3 grid((ldd + 63) / 64, (cols + 63) / 64);
  hipLaunchKernelGGL(transpose_grouped_kernel, grid, dim3(256), 0, s, (const uint16_t*)src,
                     src_rows, gather, gather_div, offsets, offsets ? G : 1, rows_max, cols,
                     (uint16_t*)dst, ldd);
}

}  // namespace moe
