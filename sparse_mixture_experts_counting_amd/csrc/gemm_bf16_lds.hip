// bf16 grouped GEMM, CDNA4 transposing-read variant (used when K is a multiple of BK).
//
// Same contract and epilogues as gemm_bf16.hip (expert up projection with the fused SwiGLU
// epilogue, down projection, router product).  Tiles move global -> registers -> LDS in 16-byte
// units; each wave "instruction slot" c owns 1 KB of LDS (lane l's unit at base + 16 l), and the
// choice of which global unit each lane fetches lays the tile out with an XOR swizzle instead of
// padding.  The B operand comes from:
//   - ds_read_b64_tr_b16 (gfx950): the transposing LDS read.  Inside each group of 16 lanes, lane 4a + c
//     receives element c of the 8-byte rows addressed by lanes a, a+4, a+8, a+12; pointing those
//     four lanes at four consecutive k-rows of the [K][N] weight tile gives every lane four
//     consecutive k of one column, i.e. the K-contiguous B operand of the matrix instruction,
//     read directly from the weights' own N-contiguous layout.
// A (activation rows, gathered through perm) is stored [BM][BK] with 16-byte units swizzled so that
// 16 consecutive rows of one unit hit 16 different bank groups (ds_read_b128); B is stored
// [BK][BN] per matrix with units swizzled by 4 * (k % 4) (conflict-free transposing reads).
// Pipeline: two LDS stages and two register sets: at step kt the registers holding step kt+1 are
// written to the idle LDS stage and refilled with step kt+3, so global loads have two steps to
// land.  One barrier per step, issued as a plain s_barrier after an LDS-only wait so that it does
// not drain the global loads in flight.  The operand reads of each 16-wide k slice are issued
// before the matrix instructions of the previous slice, across step boundaries too.
// (Loading straight into LDS with buffer_load ... lds would save the register round trip, but the
// compiler then has to assume every transposing read may alias a load in flight and waits for all
// of them before each read.)
#include "common.h"
#include "gemm_common.h"
#include "kernels.h"

#include <algorithm>
#include <type_traits>

namespace moe {

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) v4i16 lds_v4i16_t;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8_t;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4_t;

template <int BM, int BN, int NMAT, int BK>
constexpr int lds_stage_bytes() {
  return BM * BK * 2 + NMAT * BK * BN * 2;
}

// s_waitcnt immediate (gfx9 encoding): vector-memory count vm, LDS count lgkm, no export wait.
constexpr int waitcnt_imm(int vm, int lgkm) {
  return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | (lgkm << 8);
}

// Workgroup barrier without the memory fence of __syncthreads (which would wait for every load
// in flight); LDS ordering is provided by the explicit s_waitcnt before it.
__device__ __forceinline__ void barrier_no_fence() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

template <int BM, int BN, int NMAT, int BK, int STAGES, int MINB, int EPI>
__global__ __launch_bounds__(256, MINB) void gemm_bf16_lds_kernel(const GemmParams p) {
  constexpr int WM = BM / 2, WN = BN / 2;          // 2 x 2 waves
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int KS = BK / 16;                      // 16-wide k slices per step
  constexpr int A_BYTES = BM * BK * 2;
  constexpr int B_BYTES = BK * BN * 2;             // one matrix
  constexpr int STAGE = lds_stage_bytes<BM, BN, NMAT, BK>();
  constexpr int A_PER_WAVE = A_BYTES / 1024 / 4;   // 1 KB per wave instruction, 4 waves
  constexpr int B_CHUNKS = B_BYTES / 1024;         // per matrix
  constexpr int B_PER_WAVE = NMAT * B_CHUNKS / 4;
  constexpr int ROWB = BN * 2;                     // bytes per LDS row of B
  constexpr int UA = BK / 8;                       // 16-byte units per A row
  constexpr int R256 = 256 / (BK * 2);             // A rows per 256 bytes (one pass of the banks)
  static_assert(A_BYTES % 4096 == 0 && (NMAT * B_BYTES) % 4096 == 0, "whole KB per wave");
  static_assert(BN >= 128 && ROWB <= 1024 && 1024 % ROWB == 0, "B row swizzle needs 16 units");
  static_assert(BK == 32 || BK == 64, "BK");
  static_assert(STAGES == 2, "two LDS stages");

  extern __shared__ __align__(16) uint8_t smem[];

  const int NT = (p.N + BN - 1) / BN;
  TileCoord tc;
  // Split-K: consecutive blocks take the K chunks of one tile.
  const int kc = blockIdx.x % p.ksplit;
  if (!find_tile<BM>(p, NT, blockIdx.x / p.ksplit, tc)) return;
  tc.g = __builtin_amdgcn_readfirstlane(tc.g);
  tc.row0 = __builtin_amdgcn_readfirstlane(tc.row0);
  tc.row_end = __builtin_amdgcn_readfirstlane(tc.row_end);
  tc.n_tile = __builtin_amdgcn_readfirstlane(tc.n_tile);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm0 = (wave & 1) * WM;
  const int wn0 = (wave >> 1) * WN;
  const int n_base = tc.n_tile * BN;
  const int K = p.K, N = p.N;

  __amdgpu_buffer_rsrc_t rA =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.A, (short)0, p.a_rows * K * 2, 0x00020000);
  __amdgpu_buffer_rsrc_t rB0 = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const uint16_t*)p.B0 + (size_t)tc.g * p.b_gstride), (short)0, K * N * 2, 0x00020000);
  __amdgpu_buffer_rsrc_t rB1 =
      NMAT == 2 ? __builtin_amdgcn_make_buffer_rsrc(
                      (void*)((const uint16_t*)p.B1 + (size_t)tc.g * p.b_gstride), (short)0,
                      K * N * 2, 0x00020000)
                : rB0;

  // ---- global -> LDS load plan (fixed for the whole K loop) ----
  // ("Instruction" c below is a 1 KB slot of the stage: 64 lanes x 16 bytes.)
  // A: instruction c covers 1 KB = rows c*RPK .. c*RPK + RPK-1 (RPK = 1024 / (2 BK)); lane l
  // fills row m = c*RPK + l/UA, physical unit l%UA, which holds logical k-unit
  // (l%UA) ^ ((m / R256) % UA).  Rows past the group's end read a valid row (they only feed
  // accumulator rows that are never stored).
  uint32_t a_voff[A_PER_WAVE];
#pragma unroll
  for (int t = 0; t < A_PER_WAVE; ++t) {
    const int c = wave * A_PER_WAVE + t;
    const int m = c * (1024 / (2 * BK)) + lane / UA;
    const int u = (lane % UA) ^ ((m / R256) % UA);
    const int grow = min(tc.row0 + m, tc.row_end - 1);
    const int src = p.gather ? p.gather[grow] / p.gather_div : grow;
    a_voff[t] = (uint32_t)(src * K + 8 * u) * 2u;
  }
  // B: instruction c (of NMAT * B_CHUNKS) covers 1 KB of matrix c / B_CHUNKS: rows
  // k = cc * (1024 / ROWB) + (16 l) / ROWB, physical unit (16 l % ROWB) / 16 holding logical unit
  // pu ^ 4 (k % 4).  Columns past N are clamped to the last valid 8 (never stored).
  uint32_t b_voff[B_PER_WAVE];
#pragma unroll
  for (int t = 0; t < B_PER_WAVE; ++t) {
    const int c = wave * B_PER_WAVE + t;
    const int cc = c % B_CHUNKS;
    const int k = cc * (1024 / ROWB) + (lane * 16) / ROWB;
    const int pu = ((lane * 16) % ROWB) >> 4;
    const int u = pu ^ (4 * (k & 3));
    const int n = min(n_base + 8 * u, N - 8);
    b_voff[t] = (uint32_t)(k * N + n) * 2u;
  }

  // Global -> register loads of one K step into register set R, and register -> LDS stores.
  u32x4 a_reg[2][A_PER_WAVE];
  u32x4 b_reg[2][B_PER_WAVE];
  auto load_regs = [&](int R, int k0) {
#pragma unroll
    for (int t = 0; t < A_PER_WAVE; ++t)
      a_reg[R][t] = __builtin_amdgcn_raw_buffer_load_b128(rA, a_voff[t] + (uint32_t)k0 * 2u, 0, 0);
#pragma unroll
    for (int t = 0; t < B_PER_WAVE; ++t) {
      const int c = wave * B_PER_WAVE + t;
      const int mat = c / B_CHUNKS;
      b_reg[R][t] = __builtin_amdgcn_raw_buffer_load_b128(
          mat == 0 ? rB0 : rB1, b_voff[t] + (uint32_t)k0 * (uint32_t)N * 2u, 0, 0);
    }
  };
  auto store_regs = [&](int R, int stage_off) {
#pragma unroll
    for (int t = 0; t < A_PER_WAVE; ++t) {
      const int c = wave * A_PER_WAVE + t;
      *(lds_u32x4_t*)(smem + stage_off + c * 1024 + lane * 16) = a_reg[R][t];
    }
#pragma unroll
    for (int t = 0; t < B_PER_WAVE; ++t) {
      const int c = wave * B_PER_WAVE + t;
      const int mat = c / B_CHUNKS;
      const int cc = c % B_CHUNKS;
      *(lds_u32x4_t*)(smem + stage_off + A_BYTES + mat * B_BYTES + cc * 1024 + lane * 16) =
          b_reg[R][t];
    }
  };

  // ---- operand read plan ----
  const int l32 = lane & 31, h = lane >> 5;
  const int a_sw = (l32 / R256) % UA;                   // swizzle of this lane's A rows
  const int a_row_byte = (wm0 + l32) * (BK * 2);
  const int g16 = lane >> 4, s16 = lane & 15;
  const int qa = s16 >> 2, aa = s16 & 3;               // source row (k) and column quad
  const int kh = g16 >> 1, nh = g16 & 1;
  // Byte offset (inside a B matrix of a stage) of this lane's tr-read for sub-tile j, k slice 0:
  // row kh*8 + qa (and +4), column wn0 + 32 j + 16 nh + 4 aa.
  int b_rd[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int n = wn0 + 32 * j + 16 * nh + 4 * aa;
    const int r = kh * 8 + qa;
    b_rd[j] = r * ROWB + (((n >> 3) ^ (4 * qa)) << 4) + (n & 7) * 2;
  }

  f32x16 acc[NMAT][TM][TN];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[m][i][j][r] = 0.f;

  bf16x8 af[2][TM];
  bf16x8 bfr[2][NMAT][TN];
  auto read_frags = [&](int stage_off, int ks, int buf) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int unit = (2 * ks + h) ^ a_sw;
      af[buf][i] = *(const lds_bf16x8_t*)(smem + stage_off + a_row_byte + i * 32 * (BK * 2) +
                                          unit * 16);
    }
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int bo = stage_off + A_BYTES + m * B_BYTES + b_rd[j] + ks * 16 * ROWB;
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(smem + bo));
        const v4i16 hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(smem + bo + 4 * ROWB));
        const v8i16 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        bfr[buf][m][j] = __builtin_bit_cast(bf16x8, both);
      }
  };
  auto mfmas = [&](int buf) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[m][i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[buf][i], bfr[buf][m][j],
                                                                 acc[m][i][j], 0, 0, 0);
  };

  // The loop body is branch-free (branches inside it make the register allocator move the
  // accumulators between register files): prefetches past the last K step re-read the last step
  // (in bounds, never used), and KT is even so the two-step unroll is exact.
  const int Kc = K / p.ksplit;                        // this block's K chunk
  const int kbeg = kc * Kc;
  const int KT = Kc / BK;
  const int k_last = kbeg + (KT - 1) * BK;
  // Prologue: step 0 into LDS stage 0, steps 1 and 2 in the registers.
  load_regs(0, kbeg);
  load_regs(1, min(kbeg + BK, k_last));
  store_regs(0, 0);
  load_regs(0, min(kbeg + 2 * BK, k_last));
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
  barrier_no_fence();
  read_frags(0, 0, 0);
  // One K step; R = (kt + 1) & 1 is the register set written to LDS (a template constant, so the
  // register sets and LDS stages are addressed statically).
  auto step = [&](int kt, auto R) {
    constexpr int st = R() == 1 ? 0 : STAGE;       // kt even reads stage 0, odd reads stage 1
    constexpr int nx = R() == 1 ? STAGE : 0;
    // Step kt+1 (register set R) into the idle stage, then refill that set with step kt+3.
    store_regs(R(), nx);
    load_regs(R(), min(kbeg + (kt + 3) * BK, k_last));
#pragma unroll
    for (int ks = 0; ks < KS - 1; ++ks) {
      read_frags(st, ks + 1, (ks + 1) & 1);
      __builtin_amdgcn_sched_barrier(0);
      mfmas(ks & 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    // This wave's LDS stores of step kt+1 and reads of step kt are done; after the barrier every
    // wave's are.
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
    barrier_no_fence();
    read_frags(nx, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    mfmas((KS - 1) & 1);
    __builtin_amdgcn_sched_barrier(0);
  };
  for (int kt = 0; kt < KT; kt += 2) {
    step(kt, std::integral_constant<int, 1>());
    step(kt + 1, std::integral_constant<int, 0>());
  }

  // Epilogue.  Accumulator register r of a 32x32 tile holds row 8*(r/4) + 4*(lane/32) + r%4 and
  // column lane%32.
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = n_base + wn0 + j * 32 + l32;
      if (col >= N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = tc.row0 + wm0 + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        if (row >= tc.row_end) continue;
        if (p.ksplit > 1) {   // fp32 partial sums; splitk_finish_kernel applies the epilogue
#pragma unroll
          for (int m = 0; m < NMAT; ++m)
            p.part[((size_t)(kc * NMAT + m) * p.part_rows + row) * N + col] = acc[m][i][j][r];
        } else if constexpr (EPI == EPI_SWIGLU) {
          const float g = acc[0][i][j][r];
          const float u = acc[NMAT - 1][i][j][r];
          const float hv = g / (1.0f + expf(-g)) * u;
          ((uint16_t*)p.C)[(size_t)row * p.ldc + col] = f32_to_bf16(hv);
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

// Sum the K-chunk partials of every valid row in a fixed order and apply the epilogue.
// Rows past the valid count (offsets[G], or M for a single group) are untouched.
template <int NMAT, int EPI>
__global__ __launch_bounds__(256) void splitk_finish_kernel(const GemmParams p) {
  const int rows = p.offsets ? p.offsets[p.G] : p.M;
  const int nv = p.N / 8;                              // 8 columns per thread
  const size_t total = (size_t)rows * nv;
  for (size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x; idx < total;
       idx += (size_t)gridDim.x * 256) {
    const int row = (int)(idx / nv), c0 = (int)(idx % nv) * 8;
    float s[NMAT][8];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int q = 0; q < 8; ++q) s[m][q] = 0.f;
    for (int kc = 0; kc < p.ksplit; ++kc) {
#pragma unroll
      for (int m = 0; m < NMAT; ++m) {
        const f32x4* src = reinterpret_cast<const f32x4*>(
            p.part + ((size_t)(kc * NMAT + m) * p.part_rows + row) * p.N + c0);
        const f32x4 a = src[0], b = src[1];
        s[m][0] += a[0]; s[m][1] += a[1]; s[m][2] += a[2]; s[m][3] += a[3];
        s[m][4] += b[0]; s[m][5] += b[1]; s[m][6] += b[2]; s[m][7] += b[3];
      }
    }
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float v0, v1;
      if constexpr (EPI == EPI_SWIGLU) {
        const float g0 = s[0][2 * q], g1 = s[0][2 * q + 1];
        v0 = g0 / (1.0f + expf(-g0)) * s[NMAT - 1][2 * q];
        v1 = g1 / (1.0f + expf(-g1)) * s[NMAT - 1][2 * q + 1];
      } else {
        v0 = s[0][2 * q];
        v1 = s[0][2 * q + 1];
      }
      o[q] = pack_bf16x2(v0, v1);
    }
    *reinterpret_cast<u32x4*>((uint16_t*)p.C + (size_t)row * p.ldc + c0) = o;
  }
}

template <int BM, int BN, int NMAT, int BK, int STAGES, int MINB, int EPI>
static hipError_t launch_lds_t(const GemmParams& p, int rows_max, hipStream_t s) {
  auto kern = gemm_bf16_lds_kernel<BM, BN, NMAT, BK, STAGES, MINB, EPI>;
  const size_t lds = (size_t)STAGES * lds_stage_bytes<BM, BN, NMAT, BK>();
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int NT = (p.N + BN - 1) / BN;
  const int grid = tiles_upper_bound(rows_max, p.G, p.offsets != nullptr, BM, NT) * p.ksplit;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(256), lds, s, p);
  if (p.ksplit > 1) {
    const size_t items = (size_t)rows_max * (p.N / 8);
    const int fgrid = (int)std::min<size_t>((items + 255) / 256, 4096);
    hipLaunchKernelGGL((splitk_finish_kernel<NMAT, EPI>), dim3(fgrid), dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

// K chunks for the expert GEMMs: when the tile grid would leave CUs idle (few rows, e.g. decode),
// split K so that about 1024 blocks run, keeping every chunk a whole number of 64-deep steps.
static int splitk_factor(int rows_max, int G, bool grouped, int N, int K, int epi) {
  if (epi == EPI_STORE_F32_BIAS || K % 64 != 0) return 1;
  const int BM = 128, BN = (epi == EPI_SWIGLU) ? 128 : 256;
  const int mt = grouped ? std::min(G, rows_max) + rows_max / BM : (rows_max + BM - 1) / BM;
  const long long tiles = (long long)mt * ((N + BN - 1) / BN);
  int ks = 1;
  while (ks < 16 && tiles * ks * 2 <= 1024 && (K / 64) % (ks * 2) == 0) ks *= 2;
  return ks;
}

size_t gemm_bf16_partial_bytes(int rows_max, int G, bool grouped, int N, int K, int epi) {
  const int ks = splitk_factor(rows_max, G, grouped, N, K, epi);
  if (ks == 1) return 0;
  const int nmat = epi == EPI_SWIGLU ? 2 : 1;
  return (size_t)ks * nmat * rows_max * N * sizeof(float);
}

// Returns hipErrorNotSupported when the shape needs the general kernel (K not a multiple of 64:
// an even number of 32-deep steps).
hipError_t launch_gemm_bf16_lds(const GemmParams& p_in, int rows_max, int epi, hipStream_t s) {
  if (p_in.K % 64 != 0 || p_in.N < 8) return hipErrorNotSupported;
  GemmParams p = p_in;
  p.ksplit = splitk_factor(rows_max, p.G, p.offsets != nullptr, p.N, p.K, epi);
  p.part_rows = rows_max;
  if (p.ksplit > 1 && p.part == nullptr) p.ksplit = 1;   // no scratch given: no split
  switch (epi) {
    case EPI_SWIGLU:
      return launch_lds_t<128, 128, 2, 32, 2, 2, EPI_SWIGLU>(p, rows_max, s);
    case EPI_STORE:
      return launch_lds_t<128, 256, 1, 32, 2, 2, EPI_STORE>(p, rows_max, s);
    default:
      return launch_lds_t<128, 256, 1, 32, 2, 1, EPI_STORE_F32_BIAS>(p, rows_max, s);
  }
}

}  // namespace moe
