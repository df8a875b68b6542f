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

// bf16 transposes of the backward pass, 16 bytes per access.  A block moves a 64 x 64 tile: the
// source rows of its 64 destination columns are resolved once into LDS, each thread loads two
// 16-byte row chunks into a padded LDS tile (row pitch 72 elements), then gathers 8 rows of one
// column from LDS and stores them as one 16-byte chunk of a destination row.
//   GROUPED = false: dst[b][c][r] = src[b][r][c] for r < rows (rows, cols and ldd multiples of 8).
//   GROUPED = true:  the group-padded layout of expert-ordered rows used by the K-grouped GEMM:
//     dst[c][kpad(offsets[g], g) + i] = src[row][c] for the i-th row of group g, where row =
//     gather[r] / gather_div (or r) and r = offsets[g] + i; the padding columns between groups are
//     zero.  offsets == NULL is one group of `rows` rows at column 0 (zero up to the next multiple
//     of 8).  Columns past the last group's padding are not written.
template <bool GROUPED>
__global__ __launch_bounds__(256) void transpose16_kernel(
    const uint16_t* __restrict__ src, int src_rows, int cols, const int32_t* __restrict__ gather,
    int gather_div, const int32_t* __restrict__ offsets, int G, int rows,
    uint16_t* __restrict__ dst, int ldd, long long src_bstride, long long dst_bstride) {
  constexpr int PITCH = 72;
  __shared__ __align__(16) uint16_t tile[64 * PITCH];
  __shared__ int s_row[64];
  const int p0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
  const uint16_t* s = src + (size_t)blockIdx.z * (size_t)src_bstride;
  uint16_t* o = dst + (size_t)blockIdx.z * (size_t)dst_bstride;
  int pend;
  if (GROUPED)
    pend = offsets ? kpad(offsets[G], G) : (rows + 7) & ~7;
  else
    pend = rows;
  if (threadIdx.x < 64) {
    const int pc = p0 + threadIdx.x;
    int r = -1;
    if (pc < pend) {
      if (GROUPED && offsets) {           // last group whose padded start is <= pc
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
      if (r >= 0 && GROUPED && gather) r = gather[r] / gather_div;
      if (r >= src_rows) r = -1;
    }
    s_row[threadIdx.x] = r;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int q = threadIdx.x + 256 * i;
    const int rr = q >> 3, u = q & 7;
    const int r = s_row[rr], c = c0 + 8 * u;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (r >= 0 && c < cols) v = *reinterpret_cast<const u32x4*>(s + (size_t)r * cols + c);
    *reinterpret_cast<u32x4*>(&tile[rr * PITCH + 8 * u]) = v;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int q = threadIdx.x + 256 * i;
    const int cl = q >> 3, v = q & 7;
    const int c = c0 + cl, pc = p0 + 8 * v;
    if (c >= cols || pc >= pend) continue;
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
  hipLaunchKernelGGL(transpose16_kernel<false>, grid, dim3(256), 0, s, (const uint16_t*)src, rows,
                     cols, nullptr, 1, nullptr, 1, rows, (uint16_t*)dst, ldd,
                     (long long)rows * cols, dst_bstride);
}

void launch_transpose_grouped(const void* src, int src_rows, const int32_t* gather,
                              int gather_div, const int32_t* offsets, int G, int rows_max,
                              int cols, void* dst, int ldd, hipStream_t s) {
  const dim3 grid((ldd + 63) / 64, (cols + 63) / 64);
  hipLaunchKernelGGL(transpose16_kernel<true>, grid, dim3(256), 0, s, (const uint16_t*)src,
                     src_rows, cols, gather, gather_div, offsets, offsets ? G : 1, rows_max,
                     (uint16_t*)dst, ldd, 0ll, 0ll);
}

}  // namespace moe
