// bf16 grouped GEMM on the CDNA4 matrix cores (v_mfma_f32_32x32x16_bf16, fp32 accumulate).
//
// Used for the expert FFN (the page "Mixture of experts (MoE)" (tirogla), How it works step 4: one
// grouped GEMM over the experts' contiguous batches) and for the router product when E is large.
//
// Tiling: a 256-thread block (4 waves, WGM x WGN) computes a BM x BN tile of C (for NMAT = 2 two
// B matrices share the tile: w1 and w3 of the SwiGLU expert, and the epilogue forms
// silu(x.w1) * (x.w3) in registers, so the gate and up products never leave the chip).  K is walked
// in steps of 64 through LDS:
//   A (activation rows, K contiguous) is gathered row by row (token of each assignment) with
//     16-byte loads and stored as [BM][64+8] bf16;
//   B (weights [K][N], N contiguous) is loaded as 8x8 bf16 blocks (eight 16-byte rows), transposed
//     in registers and stored K-contiguous as [BN][64+8], so both MFMA operands are read from LDS
//     with one 16-byte read per lane.
// The next K step is fetched into registers while the current one is multiplied.
#include "common.h"
#include "gemm_common.h"
#include "kernels.h"

namespace moe {

static constexpr int kBK = 64;
static constexpr int kLDK = kBK + 8;  // padded LDS row (144 bytes): conflict-free 16-byte reads

// Transpose an 8x8 block of bf16: in[r] holds row r (8 values along n); out[n] gets column n
// (8 values along r).
__device__ __forceinline__ void transpose8x8(const u32x4 (&in)[8], u32x4 (&out)[8]) {
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    const int w = n >> 1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t lo = in[2 * j][w];
      const uint32_t hi = in[2 * j + 1][w];
      out[n][j] = (n & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
    }
  }
}

template <int BM, int BN, int NMAT, int WGM, int WGN, int EPI>
__global__ __launch_bounds__(256, 1) void gemm_bf16_kernel(const GemmParams p) {
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int A_CHUNKS = BM * (kBK / 8) / 256;             // 16-byte A chunks per thread
  constexpr int B_BLOCKS = NMAT * (kBK / 8) * (BN / 8) / 256;  // 8x8 B blocks per thread
  static_assert(WGM * WGN == 4, "4 waves");
  static_assert(A_CHUNKS >= 1 && B_BLOCKS >= 1, "tile too small for 256 threads");
  static_assert(BM * (kBK / 8) % 256 == 0 && NMAT * (kBK / 8) * (BN / 8) % 256 == 0, "tiling");

  extern __shared__ __align__(16) uint16_t smem[];
  uint16_t* As = smem;
  uint16_t* Bs = smem + BM * kLDK;

  const int NT = (p.N + BN - 1) / BN;
  TileCoord tc;
  if (!find_tile<BM>(p, NT, blockIdx.x, tc)) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm0 = (wave % WGM) * WM;
  const int wn0 = (wave / WGM) * WN;
  const int n_base = tc.n_tile * BN;
  const int K = p.K, N = p.N;

  const uint16_t* Ab = (const uint16_t*)p.A;
  const uint16_t* B0 = (const uint16_t*)p.B0 + (size_t)tc.g * p.b_gstride;
  const uint16_t* B1 = NMAT == 2 ? (const uint16_t*)p.B1 + (size_t)tc.g * p.b_gstride : nullptr;

  // A rows handled by this thread (fixed for the whole K loop).
  const uint16_t* a_src[A_CHUNKS];
  int a_kc[A_CHUNKS];
  bool a_ok[A_CHUNKS];
#pragma unroll
  for (int i = 0; i < A_CHUNKS; ++i) {
    const int c = tid + 256 * i;
    const int row = c >> 3;
    a_kc[i] = (c & 7) * 8;
    const int grow = tc.row0 + row;
    a_ok[i] = grow < tc.row_end;
    int src = grow;
    if (a_ok[i] && p.gather) src = p.gather[grow] / p.gather_div;
    a_src[i] = Ab + (size_t)(a_ok[i] ? src : 0) * K;
  }
  // B blocks handled by this thread.
  const uint16_t* b_src[B_BLOCKS];
  int b_kb[B_BLOCKS], b_lds[B_BLOCKS];
  bool b_ok[B_BLOCKS];
#pragma unroll
  for (int i = 0; i < B_BLOCKS; ++i) {
    const int b = tid + 256 * i;
    const int mat = b / (8 * (BN / 8));
    const int rem = b % (8 * (BN / 8));
    const int kb = rem & 7, nb = rem >> 3;
    const int col = n_base + nb * 8;
    b_ok[i] = col < N;
    b_kb[i] = kb * 8;
    b_src[i] = (mat == 0 ? B0 : B1) + (b_ok[i] ? col : 0);
    b_lds[i] = (mat * BN + nb * 8) * kLDK + kb * 8;
  }

  u32x4 a_reg[A_CHUNKS];
  u32x4 b_reg[B_BLOCKS][8];
  const u32x4 zero = {0u, 0u, 0u, 0u};

  auto load_tile = [&](int k0) {
#pragma unroll
    for (int i = 0; i < A_CHUNKS; ++i) {
      const int k = k0 + a_kc[i];
      a_reg[i] = (a_ok[i] && k < K) ? *reinterpret_cast<const u32x4*>(a_src[i] + k) : zero;
    }
#pragma unroll
    for (int i = 0; i < B_BLOCKS; ++i) {
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int k = k0 + b_kb[i] + r;
        b_reg[i][r] = (b_ok[i] && k < K)
                          ? *reinterpret_cast<const u32x4*>(b_src[i] + (size_t)k * N)
                          : zero;
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < A_CHUNKS; ++i) {
      const int c = tid + 256 * i;
      *reinterpret_cast<u32x4*>(As + (c >> 3) * kLDK + a_kc[i]) = a_reg[i];
    }
#pragma unroll
    for (int i = 0; i < B_BLOCKS; ++i) {
      u32x4 t[8];
      transpose8x8(b_reg[i], t);
#pragma unroll
      for (int n = 0; n < 8; ++n) *reinterpret_cast<u32x4*>(Bs + b_lds[i] + n * kLDK) = t[n];
    }
  };

  f32x16 acc[NMAT][TM][TN];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[m][i][j][r] = 0.f;

  const int KT = (K + kBK - 1) / kBK;
  load_tile(0);
  store_tile();
  __syncthreads();
  const int lrow = lane & 31;
  const int lk = (lane >> 5) * 8;
  for (int kt = 0; kt < KT; ++kt) {
    if (kt + 1 < KT) load_tile((kt + 1) * kBK);
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      bf16x8 af[TM];
      bf16x8 bfr[NMAT][TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(As + (wm0 + i * 32 + lrow) * kLDK + ks * 16 + lk);
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          bfr[m][j] = *reinterpret_cast<const bf16x8*>(
              Bs + (m * BN + wn0 + j * 32 + lrow) * kLDK + ks * 16 + lk);
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[m][i][j] =
                __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[m][j], acc[m][i][j], 0, 0, 0);
    }
    __syncthreads();
    if (kt + 1 < KT) {
      store_tile();
      __syncthreads();
    }
  }

  // Epilogue.  Accumulator register r of a 32x32 tile holds row 8*(r/4) + 4*(lane/32) + r%4 and
  // column lane%32.
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = n_base + wn0 + j * 32 + (lane & 31);
      if (col >= N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = tc.row0 + wm0 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row >= tc.row_end) continue;
        if constexpr (EPI == EPI_SWIGLU) {
          const float g = acc[0][i][j][r];
          const float u = acc[NMAT - 1][i][j][r];
          const float h = g / (1.0f + expf(-g)) * u;
          ((uint16_t*)p.C)[(size_t)row * p.ldc + col] = f32_to_bf16(h);
        } else if constexpr (EPI == EPI_STORE) {
          ((uint16_t*)p.C)[(size_t)row * p.ldc + col] = f32_to_bf16(acc[0][i][j][r]);
        } else {
          ((float*)p.C)[(size_t)row * p.ldc + col] =
              acc[0][i][j][r] + (p.bias ? p.bias[col] : 0.f);
        }
      }
    }
  }
}

template <int BM, int BN, int NMAT, int WGM, int WGN, int EPI>
static hipError_t launch_gemm_bf16_t(const GemmParams& p, int rows_max, hipStream_t s) {
  auto kern = gemm_bf16_kernel<BM, BN, NMAT, WGM, WGN, EPI>;
  const size_t lds = (size_t)(BM + NMAT * BN) * kLDK * sizeof(uint16_t);
  static bool attr_set = false;  // the attribute is per function; setting it twice is harmless
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int NT = (p.N + BN - 1) / BN;
  const int grid = tiles_upper_bound(rows_max, p.G, p.offsets != nullptr, BM, NT);
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(256), lds, s, p);
  return hipGetLastError();
}

hipError_t launch_gemm_bf16(const GemmParams& p, int rows_max, int epi, hipStream_t s) {
  switch (epi) {
    case EPI_SWIGLU:
      return launch_gemm_bf16_t<256, 128, 2, 2, 2, EPI_SWIGLU>(p, rows_max, s);
    case EPI_STORE:
      return launch_gemm_bf16_t<256, 256, 1, 2, 2, EPI_STORE>(p, rows_max, s);
    default:
      return launch_gemm_bf16_t<64, 256, 1, 2, 2, EPI_STORE_F32_BIAS>(p, rows_max, s);
  }
}

}  // namespace moe
