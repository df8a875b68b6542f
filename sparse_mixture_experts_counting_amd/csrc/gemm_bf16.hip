// bf16 grouped GEMM on the CDNA4 matrix cores (v_mfma_f32_32x32x16_bf16, fp32 accumulate).
//
// Used for the expert FFN (the page "Mixture of experts (MoE)" (tirogla), How it works step 4: one
// grouped GEMM over the experts' contiguous batches) and for the router product when E is large.
//
// Tiling: a 256-thread block (4 waves, WGM x WGN) computes a BM x BN tile of C (for NMAT = 2 two
// B matrices share the tile: w1 and w3 of the SwiGLU expert, and the epilogue forms
// silu(x.w1) * (x.w3) in registers, so the gate and up products never leave the chip).  K is walked
// in steps of 64 through a double-buffered LDS:
//   A (activation rows, K contiguous) is gathered row by row (token of each assignment) with
//     16-byte loads and stored as [BM][64+8] bf16;
//   B (weights [K][N], N contiguous) is loaded as 8x8 bf16 blocks (eight 16-byte rows), transposed
//     in registers and stored K-contiguous as [BN][64+8], so both MFMA operands are read from LDS
//     with one 16-byte read per lane.
// Pipeline, one barrier per K step: at the top of step kt the registers hold tile kt+1 (loaded one
// step earlier); they are written to the idle LDS buffer, the loads of tile kt+2 are issued, and the
// MFMAs run on tile kt from the other buffer.
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

template <int BM, int BN, int NMAT>
constexpr size_t gemm_stage_elems() {
  return (size_t)(BM + NMAT * BN) * kLDK;
}

template <int BM, int BN, int NMAT, int WGM, int WGN, int EPI, bool KFULL>
__global__ __launch_bounds__(256, 1) void gemm_bf16_kernel(const GemmParams p) {
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int A_CHUNKS = BM * (kBK / 8) / 256;             // 16-byte A chunks per thread
  constexpr int B_BLOCKS = NMAT * (kBK / 8) * (BN / 8) / 256;  // 8x8 B blocks per thread
  constexpr int STAGE = (int)gemm_stage_elems<BM, BN, NMAT>();
  static_assert(WGM * WGN == 4, "4 waves");
  static_assert(BN % 64 == 0, "the B matrix of a wave's blocks must be uniform");
  static_assert(A_CHUNKS >= 1 && B_BLOCKS >= 1, "tile too small for 256 threads");
  static_assert(BM * (kBK / 8) % 256 == 0 && NMAT * (kBK / 8) * (BN / 8) % 256 == 0, "tiling");

  extern __shared__ __align__(16) uint16_t smem[];

  const int NT = (p.N + BN - 1) / BN;
  TileCoord tc;
  if (!find_tile<BM>(p, NT, blockIdx.x, tc)) return;
  tc.g = __builtin_amdgcn_readfirstlane(tc.g);
  tc.row0 = __builtin_amdgcn_readfirstlane(tc.row0);
  tc.row_end = __builtin_amdgcn_readfirstlane(tc.row_end);
  tc.n_tile = __builtin_amdgcn_readfirstlane(tc.n_tile);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm0 = (wave % WGM) * WM;
  const int wn0 = (wave / WGM) * WN;
  const int n_base = tc.n_tile * BN;
  const int K = p.K, N = p.N;

  // Buffer descriptors: 32-bit offsets, and loads past the end of a matrix return zeros.
  const __amdgpu_buffer_rsrc_t rA =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.A, (short)0, p.a_rows * K * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t rB0 = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const uint16_t*)p.B0 + (size_t)tc.g * p.b_gstride), (short)0, K * N * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t rB1 =
      NMAT == 2 ? __builtin_amdgcn_make_buffer_rsrc(
                      (void*)((const uint16_t*)p.B1 + (size_t)tc.g * p.b_gstride), (short)0,
                      K * N * 2, 0x00020000)
                : rB0;

  // A rows handled by this thread (fixed for the whole K loop).  Rows past the group's end load a
  // valid row of the group instead; they only feed accumulator rows that are never stored.
  uint32_t a_off[A_CHUNKS];
  int a_kc[A_CHUNKS];
#pragma unroll
  for (int i = 0; i < A_CHUNKS; ++i) {
    const int c = tid + 256 * i;
    const int row = c >> 3;
    a_kc[i] = (c & 7) * 8;
    const int grow = min(tc.row0 + row, tc.row_end - 1);
    const int src = p.gather ? p.gather[grow] / p.gather_div : grow;
    a_off[i] = (uint32_t)(src * K + a_kc[i]) * 2u;
  }
  // B blocks handled by this thread: rows kb*8..kb*8+7 of the K step, columns col..col+7.
  // Columns past N read the next row's values (or zeros past the end); they only feed output
  // columns that are never stored.
  uint32_t b_off[B_BLOCKS];
  int b_kb[B_BLOCKS], b_lds[B_BLOCKS], b_mat[B_BLOCKS];
#pragma unroll
  for (int i = 0; i < B_BLOCKS; ++i) {
    // 8 * (BN / 8) = BN blocks per matrix; BN % 64 == 0 keeps the matrix index wave-uniform.
    const int mat = (wave * 64 + 256 * i) / BN;
    const int rem = (tid + 256 * i) % BN;
    const int kb = rem & 7, nb = rem >> 3;
    const int col = n_base + nb * 8;
    b_mat[i] = mat;
    b_kb[i] = kb * 8;
    b_off[i] = (uint32_t)(kb * 8 * N + col) * 2u;
    b_lds[i] = BM * kLDK + (mat * BN + nb * 8) * kLDK + kb * 8;
  }
  const uint32_t row_bytes = (uint32_t)N * 2u;

  u32x4 a_reg[A_CHUNKS];
  u32x4 b_reg[B_BLOCKS][8];
  const u32x4 zero = {0u, 0u, 0u, 0u};

  auto load_tile = [&](int k0) {
#pragma unroll
    for (int i = 0; i < A_CHUNKS; ++i) {
      if (KFULL || k0 + a_kc[i] < K)
        a_reg[i] = __builtin_amdgcn_raw_buffer_load_b128(rA, a_off[i] + (uint32_t)k0 * 2u, 0, 0);
      else
        a_reg[i] = zero;
    }
#pragma unroll
    for (int i = 0; i < B_BLOCKS; ++i) {
      const uint32_t base = b_off[i] + (uint32_t)k0 * row_bytes;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        if (KFULL || k0 + b_kb[i] + r < K)
          b_reg[i][r] = __builtin_amdgcn_raw_buffer_load_b128(b_mat[i] == 0 ? rB0 : rB1,
                                                              base + r * row_bytes, 0, 0);
        else
          b_reg[i][r] = zero;
      }
    }
  };
  auto store_tile = [&](uint16_t* buf) {
#pragma unroll
    for (int i = 0; i < A_CHUNKS; ++i) {
      const int c = tid + 256 * i;
      *reinterpret_cast<u32x4*>(buf + (c >> 3) * kLDK + a_kc[i]) = a_reg[i];
    }
#pragma unroll
    for (int i = 0; i < B_BLOCKS; ++i) {
      u32x4 t[8];
      transpose8x8(b_reg[i], t);
#pragma unroll
      for (int n = 0; n < 8; ++n) *reinterpret_cast<u32x4*>(buf + b_lds[i] + n * kLDK) = t[n];
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

  // Number of this wave's 32-row sub-tiles that hold at least one row of the group.
  const int rows_left = tc.row_end - (tc.row0 + wm0);
  const int tm_live = __builtin_amdgcn_readfirstlane(
      rows_left <= 0 ? 0 : (rows_left >= WM ? TM : (rows_left + 31) / 32));

  const int KT = (K + kBK - 1) / kBK;
  load_tile(0);
  store_tile(smem);
  if (KT > 1) load_tile(kBK);
  __syncthreads();
  const int lrow = lane & 31;
  const int lk = (lane >> 5) * 8;
  for (int kt = 0; kt < KT; ++kt) {
    const uint16_t* cur = smem + (kt & 1) * STAGE;
    if (kt + 1 < KT) {
      store_tile(smem + ((kt + 1) & 1) * STAGE);
      if (kt + 2 < KT) load_tile((kt + 2) * kBK);
    }
    const uint16_t* As = cur;
    const uint16_t* Bs = cur + BM * kLDK;
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
      for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[m][i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[m][j],
                                                                   acc[m][i][j], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  // Epilogue.  Accumulator register r of a 32x32 tile holds row 8*(r/4) + 4*(lane/32) + r%4 and
  // column lane%32.
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    if (i >= tm_live) continue;
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

template <int BM, int BN, int NMAT, int WGM, int WGN, int EPI, bool KFULL>
static hipError_t launch_gemm_bf16_k(const GemmParams& p, int rows_max, hipStream_t s) {
  auto kern = gemm_bf16_kernel<BM, BN, NMAT, WGM, WGN, EPI, KFULL>;
  const size_t lds = 2 * gemm_stage_elems<BM, BN, NMAT>() * sizeof(uint16_t);
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

template <int BM, int BN, int NMAT, int WGM, int WGN, int EPI>
static hipError_t launch_gemm_bf16_t(const GemmParams& p, int rows_max, hipStream_t s) {
  if (p.K % kBK == 0) return launch_gemm_bf16_k<BM, BN, NMAT, WGM, WGN, EPI, true>(p, rows_max, s);
  return launch_gemm_bf16_k<BM, BN, NMAT, WGM, WGN, EPI, false>(p, rows_max, s);
}

hipError_t launch_gemm_bf16(const GemmParams& p, int rows_max, int epi, hipStream_t s) {
  // K a multiple of 64: the direct-to-LDS kernel (gemm_bf16_lds.hip); else the general one below.
  const hipError_t e = launch_gemm_bf16_lds(p, rows_max, epi, s);
  if (e != hipErrorNotSupported) return e;
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
