// Measured ceilings of the chip, for the benchmark's report beside the published peaks: a loop of
// independent bf16 matrix instructions whose operands stay in registers (the most the matrix cores
// deliver on data that toggles like real operands), and a streaming copy (the most HBM delivers to
// a plain read-then-write kernel).  Neither is part of the layer.
#include "common.h"
#include "kernels.h"

#include <algorithm>

namespace moe {

// Eight waves per block; each wave keeps 8 independent 32 x 32 accumulators and issues
// v_mfma_f32_32x32x16_bf16 on two alternating operand sets loaded from `operands` (random bf16
// values), so consecutive instructions see different data.  Every accumulator is summed into
// `out` so that no instruction is dead.
__global__ __launch_bounds__(512) void peak_mfma_kernel(const uint16_t* __restrict__ operands,
                                                        int iters, float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  bf16x8 a[2], b[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    a[s] = *reinterpret_cast<const bf16x8*>(operands + (size_t)(2 * s) * 512 + lane * 8);
    b[s] = *reinterpret_cast<const bf16x8*>(operands + (size_t)(2 * s + 1) * 512 + lane * 8);
  }
  f32x16 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j & 1], b[j & 1], acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Each lane copies 8 16-byte units per iteration (all 8 loads issued before the stores, so 128
// bytes per lane are in flight), blocks striding over the buffer in 256 x 8-unit chunks; n16
// counts 16-byte units, and a tail shorter than one chunk is copied unit by unit.
__global__ __launch_bounds__(256) void peak_copy_kernel(const u32x4* __restrict__ src,
                                                        u32x4* __restrict__ dst, size_t n16) {
  constexpr int U = 8;
  const size_t chunk = 256 * U;
  const size_t full = n16 / chunk;
  for (size_t c = blockIdx.x; c < full; c += gridDim.x) {
    const size_t base = c * chunk + threadIdx.x;
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(src + base + (size_t)u * 256);
#pragma unroll
    for (int u = 0; u < U; ++u) __builtin_nontemporal_store(v[u], dst + base + (size_t)u * 256);
  }
  if (blockIdx.x == 0)
    for (size_t i = full * chunk + threadIdx.x; i < n16; i += 256) dst[i] = src[i];
}

void launch_peak_mfma(const void* operands, int blocks, int iters, float* out, hipStream_t s) {
  hipLaunchKernelGGL(peak_mfma_kernel, dim3(blocks), dim3(512), 0, s, (const uint16_t*)operands,
                     iters, out);
}

void launch_peak_copy(const void* src, void* dst, size_t bytes, hipStream_t s) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  const size_t n16 = bytes / 16;
  const size_t want = std::max<size_t>(n16 / (256 * 8), 1);
  const int grid = (int)std::min<size_t>(want, (size_t)cus * 8);
    hipLaunchKernelGGL(peak_copy_kernel, dim3(grid), dim3(256), 0, s, (const u32x4*)src,
                       (u32x4*)dst, n16);
}

}  // namespace moe
