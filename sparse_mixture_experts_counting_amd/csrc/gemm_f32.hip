// fp32 grouped GEMM on the vector ALUs (the fp32 layer dtype; small shapes).  Same grouped-GEMM
// contract and epilogues as the bf16 matrix-core kernel: C[r, n] = sum_k A[src(r), k] B_g[n, k]
// (weights [N][K], the [out][in] layout of a linear layer), with the SwiGLU epilogue
// silu(x.w1) * (x.w3) fused for the expert up projection.  K must be a multiple of 4.
#include "common.h"
#include "gemm_common.h"
#include "kernels.h"

namespace moe {

template <int NMAT, int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const GemmParams p) {
  constexpr int BM = 64, BN = 64, BK = 16;
  __shared__ float As[BK][BM + 4];
  __shared__ float Bs[NMAT][BK][BN + 4];
  const int NT = (p.N + BN - 1) / BN;
  TileCoord tc;
  if (!find_tile<BM>(p, NT, blockIdx.x, tc)) return;
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int n_base = tc.n_tile * BN;
  const int K = p.K, N = p.N;
  const float* A = (const float*)p.A;
  const float* Bm[2] = {(const float*)p.B0 + (size_t)tc.g * p.b_gstride,
                        NMAT == 2 ? (const float*)p.B1 + (size_t)tc.g * p.b_gstride : nullptr};

  // A loader: row tid/4, 4 consecutive k.
  const int a_row = tid >> 2, a_k = (tid & 3) * 4;
  const int grow = tc.row0 + a_row;
  const bool a_ok = grow < tc.row_end;
  int src = grow;
  if (a_ok && p.gather) src = p.gather[grow] / p.gather_div;
  const float* a_ptr = A + (size_t)(a_ok ? src : 0) * K;
  // B loader: weight row (output column) tid/4, 4 consecutive k.
  const int b_n = tid >> 2, b_k = (tid & 3) * 4;
  const bool b_ok = n_base + b_n < N;

  float acc[NMAT][4][4];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[m][i][j] = 0.f;

  for (int k0 = 0; k0 < K; k0 += BK) {
    f32x4 av = {0.f, 0.f, 0.f, 0.f};
    if (a_ok && k0 + a_k < K) av = *reinterpret_cast<const f32x4*>(a_ptr + k0 + a_k);
#pragma unroll
    for (int q = 0; q < 4; ++q) As[a_k + q][a_row] = av[q];
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
      f32x4 bv = {0.f, 0.f, 0.f, 0.f};
      if (b_ok && k0 + b_k < K)
        bv = *reinterpret_cast<const f32x4*>(Bm[m] + (size_t)(n_base + b_n) * K + k0 + b_k);
#pragma unroll
      for (int q = 0; q < 4; ++q) Bs[m][b_k + q][b_n] = bv[q];
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; ++kk) {
      float a[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int m = 0; m < NMAT; ++m) {
        float b[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) b[j] = Bs[m][kk][tx * 4 + j];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[m][i][j] = fmaf(a[i], b[j], acc[m][i][j]);
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = tc.row0 + ty * 4 + i;
    if (row >= tc.row_end) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n_base + tx * 4 + j;
      if (col >= N) continue;
      float v;
      if constexpr (EPI == EPI_SWIGLU) {
        const float g = acc[0][i][j];
        v = g / (1.0f + expf(-g)) * acc[NMAT - 1][i][j];
      } else if constexpr (EPI == EPI_STORE) {
        v = acc[0][i][j];
      } else {
        v = acc[0][i][j] + (p.bias ? p.bias[col] : 0.f);
      }
      ((float*)p.C)[(size_t)row * p.ldc + col] = v;
    }
  }
}

hipError_t launch_gemm_f32(const GemmParams& p, int rows_max, int epi, hipStream_t s) {
  const int NT = (p.N + 63) / 64;
  const int grid = tiles_upper_bound(rows_max, p.G, p.offsets != nullptr, 64, NT);
  if (grid <= 0) return hipSuccess;
  if (epi == EPI_SWIGLU)
    hipLaunchKernelGGL((gemm_f32_kernel<2, EPI_SWIGLU>), dim3(grid), dim3(256), 0, s, p);
  else if (epi == EPI_STORE)
    hipLaunchKernelGGL((gemm_f32_kernel<1, EPI_STORE>), dim3(grid), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((gemm_f32_kernel<1, EPI_STORE_F32_BIAS>), dim3(grid), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace moe
