// Weight-only quantized grouped GEMM (experts stored in INT8 or INT4 with one fp32 scale per
// output channel, the quantization of the page "Mixture of Experts (MoE)" (starphix), Inference
// Optimization, Quantization, and of the vanos001 page, Quantized Experts):
//
//   C[r, n] = epilogue( s[g][n] * sum_k A[src(r), k] * q[g][n][k] )
//
// A is bf16 (gathered activation rows), q holds int8 values or two int4 values per byte (column 2j
// in the low nibble), s fp32.  The weights are streamed into LDS as stored (a half or a quarter of
// the bf16 bytes) and widened to bf16 after the LDS read; every |q| <= 127 is exact in bf16, so the
// matrix instruction (32x32x16 bf16, fp32 accumulate) forms exact products, and the scale is
// applied once per output in the epilogue (with K split, to the fp32 partials, whose sum
// splitk_finish_kernel takes in chunk order).  INT4 values enter as 136 + q (built from bit
// patterns) and the epilogue removes 136 times the activation row sums.
//
// Tiles: 32 activation rows x 128 weight rows per matrix, 4 waves (wave w owns weight rows
// 32 w .. 32 w + 31 of each matrix), made for decode-sized groups whose GEMMs are bound by the
// weight stream.  A stage holds K = 128 columns: every weight row contributes one 128-byte (INT8)
// or 64-byte (INT4) run per stage.  Direct-to-LDS buffer loads fill an NST-deep ring, one barrier per
// stage; units past the K range or rows past the group (or past N) are sent out of the buffer's
// range and read zeros.
#include "common.h"
#include "gemm_common.h"
#include "kernels.h"

#include <algorithm>
#include <atomic>
#include <climits>
#include <type_traits>

namespace moe {

typedef __attribute__((address_space(3))) void qlds_void_t;
typedef __attribute__((address_space(3))) bf16x8 qlds_bf16x8_t;
typedef uint32_t qu32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) qu32x2 qlds_u32x2_t;
typedef __attribute__((address_space(3))) uint32_t qlds_u32_t;

constexpr int kQBM = 32, kQBN = 128;

// A stage holds K = 128 columns: 128-byte (INT8) or 64-byte (INT4) runs of every weight row.
// INT8 double-buffers (two blocks per CU, 64 KB of weights in flight per CU), INT4 takes a
// 3-deep ring.
template <int BITS> constexpr int q_kb() { return 128; }                        // k per stage
template <int BITS> constexpr int q_nst() { return BITS == 8 ? 2 : 3; }
template <int BITS> constexpr int q_wb() { return q_kb<BITS>() * BITS / 8; }  // weight bytes per row
template <int NMAT, int BITS> constexpr int q_na() { return kQBM * q_kb<BITS>() * 2 / 1024; }
template <int NMAT, int BITS> constexpr int q_nb() { return NMAT * kQBN * q_wb<BITS>() / 1024; }
template <int NMAT, int BITS> constexpr int q_stage() {
  return (q_na<NMAT, BITS>() + q_nb<NMAT, BITS>()) * 1024;
}
template <int NMAT, int BITS> constexpr int q_lds() {
  return q_nst<BITS>() * q_stage<NMAT, BITS>();
}

// Swizzles of 16-byte units by row: 128-byte rows (8 units), 256-byte rows (16), 64-byte rows (4).
__device__ __forceinline__ int qswz8(int r) { return (r ^ ((r >> 3) & 3)) & 7; }
__device__ __forceinline__ int qswz16(int r) { return r & 15; }
__device__ __forceinline__ int qswz4(int r) { return ((r >> 2) ^ (r >> 1)) & 3; }

// Workgroup barrier without the memory fence of __syncthreads: the fence would also wait for the
// direct loads still in flight for later stages (each wave waits explicitly for the stage it needs).
__device__ __forceinline__ void q_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

template <int VM>
constexpr int q_wait() {                                  // s_waitcnt vmcnt(VM) lgkmcnt(0)
  static_assert(VM >= 0 && VM < 64, "vmcnt range");
  return (VM & 15) | ((VM >> 4) << 14) | (7 << 4);
}

// silu(g) = g / (1 + e^-g), the formula of the bf16 GEMM's epilogue.
__device__ __forceinline__ float silu_q(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * g));
}

// 8 int8 (two dwords) or 8 int4 (one dword) -> 8 bf16, exactly.
__device__ __forceinline__ bf16x8 widen8_i8(uint32_t lo, uint32_t hi) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[i] = (__bf16)(float)(int)(int8_t)(lo >> (8 * i));
    r[4 + i] = (__bf16)(float)(int)(int8_t)(hi >> (8 * i));
  }
  return r;
}
// 8 int4 (one dword) -> the bf16 values 136 + q, exactly, by bit patterns: with u = q + 8 in
// [0, 15] (the nibble with its top bit flipped), 0x4300 | u is the bf16 of 128 + u.  Ten
// instructions for 8 values (four bytes of the nibbles spread, then byte permutes that insert the
// 0x43 high bytes) instead of a sign extension and two conversions per value; the kernel subtracts
// 136 times the activation row sums in the epilogue.
__device__ __forceinline__ bf16x8 widen8_i4_biased(uint32_t w) {
  const uint32_t x = w ^ 0x88888888u;
  const uint32_t t = x & 0x0F0F0F0Fu;                  // u0 u2 u4 u6 (one per byte)
  const uint32_t s = (x >> 4) & 0x0F0F0F0Fu;           // u1 u3 u5 u7
  const uint32_t lo = __builtin_amdgcn_perm(s, t, 0x05010400u);   // u0 u1 u2 u3
  const uint32_t hi = __builtin_amdgcn_perm(s, t, 0x07030602u);   // u4 u5 u6 u7
  const uint32_t c = 0x43434343u;
  u32x4 d;
  d[0] = __builtin_amdgcn_perm(c, lo, 0x04010400u);    // (0x4300 | u0, 0x4300 | u1)
  d[1] = __builtin_amdgcn_perm(c, lo, 0x04030402u);
  d[2] = __builtin_amdgcn_perm(c, hi, 0x04010400u);
  d[3] = __builtin_amdgcn_perm(c, hi, 0x04030402u);
  return __builtin_bit_cast(bf16x8, d);
}

// NTB: the weight loads carry the non-temporal hint (bit 1 of the buffer loads' cache-policy
// operand), for launches that read every weight panel once (each group fits one tile of rows) in
// whole 128-byte lines (INT8): HBM serves such streamed reads about 10% faster.  (With 64-byte
// runs the hint costs the other half of each line a second fetch.)
template <int NMAT, int EPI, int BITS, bool NTB>
__global__ __launch_bounds__(256, 2) void gemm_q_kernel(const GemmParams p, const float* s0,
                                                        const float* s1) {
  constexpr int KB = q_kb<BITS>(), NST = q_nst<BITS>();
  constexpr int NA = q_na<NMAT, BITS>(), NB = q_nb<NMAT, BITS>(), NL = NA + NB;
  constexpr int DPW = NL / 4;
  constexpr int STAGE = q_stage<NMAT, BITS>();
  constexpr int RBA = KB * 2;                 // LDS bytes per activation row per stage
  constexpr int UPRA = RBA / 16, RPLA = 1024 / RBA;
  constexpr int KS = KB / 16;                 // 16-deep slices per stage
  static_assert(NL % 4 == 0, "loads split evenly over the waves");
  extern __shared__ __align__(16) uint8_t smem[];

  const int NT = (p.N + kQBN - 1) / kQBN;
  const TileScan ts = scan_tiles<kQBM>(p, NT);
  const int kc = blockIdx.x % p.ksplit;
  const int bid = blockIdx.x / p.ksplit;
  if (bid >= ts.total) return;
  TileCoord tc;
  tile_at<kQBM>(p, NT, ts, xcd_order(bid, ts.total), tc);
  tc.g = __builtin_amdgcn_readfirstlane(tc.g);
  tc.row0 = __builtin_amdgcn_readfirstlane(tc.row0);
  tc.row_end = __builtin_amdgcn_readfirstlane(tc.row_end);
  tc.n_tile = __builtin_amdgcn_readfirstlane(tc.n_tile);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int K = p.K, N = p.N;
  const int n_base = tc.n_tile * kQBN;
  const uint32_t krow_bytes = (uint32_t)K * BITS / 8;       // bytes of one weight row
  const uint32_t a_bytes = (uint32_t)p.a_rows * (uint32_t)K * 2u;
  const uint32_t b_bytes = (uint32_t)N * krow_bytes;
  const __amdgpu_buffer_rsrc_t rA =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.A, (short)0, a_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rB0 = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const uint8_t*)p.B0 + (size_t)tc.g * p.b_gstride), (short)0, b_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rB1 =
      NMAT == 2 ? __builtin_amdgcn_make_buffer_rsrc(
                      (void*)((const uint8_t*)p.B1 + (size_t)tc.g * p.b_gstride), (short)0,
                      b_bytes, 0x00020000)
                : rB0;

  const int Kc = K / p.ksplit;
  const int kbeg = kc * Kc, kend = kbeg + Kc;
  const int KT = Kc / KB;

  // Per load j of this wave: the byte offset at k = kbeg and the first k it must not reach.
  uint32_t voff[DPW];
  int kmax[DPW];
#pragma unroll
  for (int j = 0; j < DPW; ++j) {
    const int J = wave + 4 * j;
    if (J < NA) {
      const int row = J * RPLA + lane / UPRA;
      const int lu = (lane % UPRA) ^ (RBA == 128 ? qswz8(row) : qswz16(row));
      const int grow = tc.row0 + row;
      const bool live = grow < tc.row_end;
      const int src = live ? (p.gather ? p.gather[grow] / p.gather_div : grow) : 0;
      voff[j] = ((uint32_t)src * (uint32_t)K + (uint32_t)(kbeg + 8 * lu)) * 2u;
      kmax[j] = live ? kend - 8 * lu : INT_MIN;
    } else {
      constexpr int UPB = q_wb<BITS>() / 16;               // 16-byte units per weight row
      const int brow = (J - NA) * (64 / UPB) + lane / UPB;
      const int lu = (lane % UPB) ^ (UPB == 8 ? qswz8(brow) : qswz4(brow));
      const int n = n_base + (brow % kQBN);
      constexpr int KPU = 16 * 8 / BITS;                  // k per 16-byte unit
      voff[j] = (uint32_t)min(n, N - 1) * krow_bytes + (uint32_t)(kbeg * BITS / 8 + 16 * lu);
      kmax[j] = n < N ? kend - KPU * lu : INT_MIN;
    }
  }

  f32x16 acc[NMAT];
  // INT4: the weights enter as 136 + q; acc_s collects the activation row sums (the fragment
  // against ones), and the epilogue takes acc - 136 acc_s.
  f32x16 acc_s;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc_s[r] = 0.f;
  bf16x8 ones;
#pragma unroll
  for (int i = 0; i < 8; ++i) ones[i] = (__bf16)1.0f;
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[m][r] = 0.f;

  const int l32 = lane & 31, h = lane >> 5;
  const int a_row_off = l32 * RBA;
  const int swa = RBA == 128 ? qswz8(l32) : qswz16(l32);
  const int brow0 = wave * 32 + l32;                       // this lane's weight row in matrix 0

#define MOE_Q_ISSUE(SLOT, KT)                                                                 \
  do {                                                                                        \
    const int k0_ = kbeg + (KT) * KB;                                                         \
    const uint32_t a_k_ = (uint32_t)((KT) * KB) * 2u, b_k_ = (uint32_t)((KT) * KB * BITS / 8); \
    _Pragma("unroll") for (int j = 0; j < DPW; ++j) {                                         \
      const int J = wave + 4 * j;                                                             \
      const bool is_a = J < NA;                                                               \
      const bool second = NMAT == 2 && !is_a && (J - NA) >= NB / 2;                           \
      const uint32_t off_ =                                                                   \
          k0_ < kmax[j] ? voff[j] + (is_a ? a_k_ : b_k_) : (is_a ? a_bytes : b_bytes);        \
      qlds_void_t* const at_ = (qlds_void_t*)(smem + (SLOT) * STAGE + J * 1024);             \
      if (is_a)                                                                               \
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, at_, 16, (int)off_, 0, 0, 0);            \
      else                                                                                    \
        __builtin_amdgcn_raw_ptr_buffer_load_lds(second ? rB1 : rB0, at_, 16, (int)off_, 0, 0, \
                                                 NTB ? 2 : 0);                                \
    }                                                                                         \
  } while (0)
  // Operand reads of slice ks of a stage: the activation fragment (shared by both matrices) and
  // each matrix's 8 packed weights of this lane's row.
  typedef typename std::conditional<BITS == 8, qu32x2, uint32_t>::type wpack_t;
  auto read_a = [&](const uint8_t* sa, int ks) {
    return *(const qlds_bf16x8_t*)(sa + a_row_off + (((2 * ks + h) ^ swa) << 4));
  };
  auto read_w = [&](const uint8_t* sb, int m, int ks) {
    const int br = m * kQBN + brow0;
    if constexpr (BITS == 8)
      return *(const qlds_u32x2_t*)(sb + br * q_wb<BITS>() +
                                    ((ks ^ (q_wb<BITS>() == 128 ? qswz8(br) : qswz4(br))) << 4) +
                                    8 * h);
    else
      return *(const qlds_u32_t*)(sb + br * 64 + (((ks >> 1) ^ qswz4(br)) << 4) + 8 * (ks & 1) +
                                  4 * h);
  };
  auto widen = [&](wpack_t w) {
    if constexpr (BITS == 8)
      return widen8_i8(w[0], w[1]);
    else
      return widen8_i4_biased(w);
  };
#pragma unroll
  for (int s = 0; s < NST - 1; ++s) MOE_Q_ISSUE(s, s);
  __builtin_amdgcn_s_waitcnt(q_wait<DPW * (NST - 2)>());
  q_barrier();
  // Software pipeline: the reads of slice ks + 1 go out before slice ks is widened and multiplied;
  // the last slice of a stage is multiplied after the barrier, behind the next stage's first reads.
  bf16x8 a_c = read_a(smem, 0);
  wpack_t w_c[NMAT];
#pragma unroll
  for (int m = 0; m < NMAT; ++m) w_c[m] = read_w(smem + NA * 1024, m, 0);
  int st = 0;
  for (int kt = 0; kt < KT; ++kt) {
    MOE_Q_ISSUE(st == 0 ? NST - 1 : st - 1, kt + NST - 1);   // past the last step: zeros
    const uint8_t* sa = smem + st * STAGE;
    const uint8_t* sb = sa + NA * 1024;
#pragma unroll
    for (int ks = 0; ks < KS - 1; ++ks) {
      const bf16x8 a_n = read_a(sa, ks + 1);
      wpack_t w_n[NMAT];
#pragma unroll
      for (int m = 0; m < NMAT; ++m) w_n[m] = read_w(sb, m, ks + 1);
      __builtin_amdgcn_sched_barrier(0);   // keep the reads ahead of this slice's work
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
        acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_c, widen(w_c[m]), acc[m], 0, 0, 0);
      if constexpr (BITS == 4)
        acc_s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_c, ones, acc_s, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      a_c = a_n;
#pragma unroll
      for (int m = 0; m < NMAT; ++m) w_c[m] = w_n[m];
    }
    __builtin_amdgcn_s_waitcnt(q_wait<DPW * (NST - 2)>());
    q_barrier();
    st = st + 1 == NST ? 0 : st + 1;
    const uint8_t* na = smem + st * STAGE;
    const bf16x8 a_n = read_a(na, 0);
    wpack_t w_n[NMAT];
#pragma unroll
    for (int m = 0; m < NMAT; ++m) w_n[m] = read_w(na + NA * 1024, m, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
      acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_c, widen(w_c[m]), acc[m], 0, 0, 0);
    if constexpr (BITS == 4)
      acc_s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_c, ones, acc_s, 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    a_c = a_n;
#pragma unroll
    for (int m = 0; m < NMAT; ++m) w_c[m] = w_n[m];
  }
  __builtin_amdgcn_s_waitcnt(q_wait<0>());                   // no LDS write outlives the block
#undef MOE_Q_ISSUE

  // Register r: activation row 8 (r / 4) + 4 h + r % 4 of the tile, weight row l32 of the wave.
  const int col = n_base + wave * 32 + l32;
  if (col >= N) return;
  const float sc0 = s0[(size_t)tc.g * N + col];
  const float sc1 = NMAT == 2 ? s1[(size_t)tc.g * N + col] : 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = tc.row0 + 8 * (r >> 2) + 4 * h + (r & 3);
    if (row >= tc.row_end) continue;
    const float bias = BITS == 4 ? 136.0f * acc_s[r] : 0.f;
    const float v0 = (acc[0][r] - bias) * sc0;
    const float v1 = NMAT == 2 ? (acc[NMAT - 1][r] - bias) * sc1 : 0.f;
    if (p.ksplit > 1) {
      p.part[((size_t)(kc * NMAT) * p.part_rows + row) * N + col] = v0;
      if (NMAT == 2) p.part[((size_t)(kc * NMAT + 1) * p.part_rows + row) * N + col] = v1;
    } else if constexpr (EPI == EPI_SWIGLU) {
      ((uint16_t*)p.C)[(size_t)row * p.ldc + col] = f32_to_bf16(silu_q(v0) * v1);
    } else {
      ((uint16_t*)p.C)[(size_t)row * p.ldc + col] = f32_to_bf16(v0);
    }
  }
}

// K chunks: the fewest (power of two, chunks a whole number of stages) whose items keep the
// resident blocks at least 90% busy, up to 16.
static int q_split(long long tiles, int K, int KB, int slots) {
  int best = 1;
  double best_eff = 0.0;
  for (int ks = 1; ks <= 16; ks *= 2) {
    if (K % (ks * KB) != 0) break;
    const long long u = tiles * ks;
    const double eff = (double)u / ((double)((u + slots - 1) / slots) * slots);
    if (eff >= 0.9) return ks;
    if (eff > best_eff + 1e-9) {
      best_eff = eff;
      best = ks;
    }
  }
  return best;
}

static int q_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 256;
  return n > 0 ? n : 256;
}

int gemm_q_split(int rows_max, int G, bool grouped, int N, int K, int bits) {
  const int KB = bits == 8 ? q_kb<8>() : q_kb<4>();
  const long long NT = (N + kQBN - 1) / kQBN;
  const long long tiles = (long long)tiles_upper_bound(rows_max, G, grouped, kQBM, (int)NT);
  return q_split(tiles, K, KB, 2 * q_cus());
}

size_t gemm_q_partial_bytes(int rows_max, int G, bool grouped, int N, int K, int bits, int nmat) {
  const int ks = gemm_q_split(rows_max, G, grouped, N, K, bits);
  return ks > 1 ? (size_t)ks * nmat * rows_max * N * sizeof(float) : 0;
}

template <int NMAT, int EPI, int BITS, bool NTB>
static hipError_t launch_q_t(GemmParams p, int rows_max, const float* s0, const float* s1,
                             hipStream_t s) {
  auto kern = gemm_q_kernel<NMAT, EPI, BITS, NTB>;
  constexpr int lds = q_lds<NMAT, BITS>();
  static std::atomic<bool> attr_set[64];   // per device: the attribute is set on that device
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  if (!attr_set[dev].load(std::memory_order_acquire)) {
    // Setting it twice (two threads' first calls) is harmless.
    hipError_t e =
        hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    attr_set[dev].store(true, std::memory_order_release);
  }
  const bool grouped = p.offsets != nullptr;
  p.ksplit = p.part ? gemm_q_split(rows_max, p.G, grouped, p.N, p.K, BITS) : 1;
  p.part_rows = rows_max;
  const int NT = (p.N + kQBN - 1) / kQBN;
  const int tiles = tiles_upper_bound(rows_max, p.G, grouped, kQBM, NT);
  if (tiles <= 0) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3(tiles * p.ksplit), dim3(256), lds, s, p, s0, s1);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.ksplit > 1) launch_splitk_finish_bf16(p, rows_max, EPI, s);
  return hipGetLastError();
}

// Needs K a multiple of 128 and every operand under 2 GiB.
hipError_t launch_gemm_q(const GemmParams& p, int rows_max, int epi, int bits, const float* s0,
                         const float* s1, hipStream_t s) {
  if (p.K % 128 != 0 || p.N < 1 || p.N % 8 != 0 || (bits != 8 && bits != 4))
    return hipErrorNotSupported;
  if ((long long)p.a_rows * p.K * 2 >= (1ll << 31) ||
      (long long)p.N * p.K * bits / 8 >= (1ll << 31))
    return hipErrorNotSupported;
  // INT8 weights streamed once (the groups average at most one tile of rows): non-temporal.
  const bool grouped = p.offsets != nullptr;
  const bool nt8 = (grouped ? rows_max / std::max(p.G, 1) : rows_max) <= kQBM;
  if (epi == EPI_SWIGLU)
    return bits == 4    ? launch_q_t<2, EPI_SWIGLU, 4, false>(p, rows_max, s0, s1, s)
           : nt8        ? launch_q_t<2, EPI_SWIGLU, 8, true>(p, rows_max, s0, s1, s)
                        : launch_q_t<2, EPI_SWIGLU, 8, false>(p, rows_max, s0, s1, s);
  if (epi == EPI_STORE)
    return bits == 4    ? launch_q_t<1, EPI_STORE, 4, false>(p, rows_max, s0, s1, s)
           : nt8        ? launch_q_t<1, EPI_STORE, 8, true>(p, rows_max, s0, s1, s)
                        : launch_q_t<1, EPI_STORE, 8, false>(p, rows_max, s0, s1, s);
  return hipErrorNotSupported;
}

// Per-row symmetric quantization: s = max|w| / Q (fp32 division), q = rint(w / s) clamped to
// [-Q, Q]; a zero row gets s = 0, q = 0.  One block per row.
template <int BITS>
__global__ __launch_bounds__(256) void quantize_rows_kernel(const uint16_t* __restrict__ w,
                                                            int cols, uint8_t* __restrict__ q,
                                                            float* __restrict__ scale) {
  constexpr float Q = BITS == 8 ? 127.0f : 7.0f;
  __shared__ float red[4];
  const size_t row = blockIdx.x;
  const uint16_t* wr = w + row * cols;
  float amax = 0.f;
  for (int c = threadIdx.x; c < cols; c += 256) amax = fmaxf(amax, fabsf(bf16_to_f32(wr[c])));
  amax = wave_max(amax);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = amax / Q;
  if (threadIdx.x == 0) scale[row] = s;
  auto qv = [&](int c) -> int {
    if (!(s > 0.f)) return 0;
    const float v = rintf(bf16_to_f32(wr[c]) / s);
    return (int)fminf(fmaxf(v, -Q), Q);
  };
  if (BITS == 8) {
    for (int c = threadIdx.x; c < cols; c += 256) q[row * cols + c] = (uint8_t)(int8_t)qv(c);
  } else {
    const int half = cols / 2;
    for (int c = threadIdx.x; c < half; c += 256)
      q[row * half + c] = (uint8_t)((qv(2 * c) & 15) | ((qv(2 * c + 1) & 15) << 4));
  }
}

void launch_quantize_rows(const void* w, long long rows, int cols, int bits, void* q, float* scale,
                          hipStream_t s) {
  if (bits == 8)
    hipLaunchKernelGGL(quantize_rows_kernel<8>, dim3((unsigned)rows), dim3(256), 0, s,
                       (const uint16_t*)w, cols, (uint8_t*)q, scale);
  else
    hipLaunchKernelGGL(quantize_rows_kernel<4>, dim3((unsigned)rows), dim3(256), 0, s,
                       (const uint16_t*)w, cols, (uint8_t*)q, scale);
}

}  // namespace moe
