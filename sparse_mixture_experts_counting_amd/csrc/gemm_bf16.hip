// bf16 grouped GEMM on the CDNA4 matrix cores (v_mfma_f32_32x32x16_bf16, fp32 accumulate).
//
// Used for the expert FFN (the page "Mixture of experts (MoE)" (tirogla), How it works step 4: one
// grouped GEMM over the experts' contiguous batches), for the router product when E is large, and
// for the products of the backward pass.
// C[r, n] = sum_k A[src(r), k] * B_g[n, k]: in the forward both operands are K-contiguous
// (activation rows, and weights in the [out][in] layout of a linear layer), so both travel the
// same way.  The transposed modes read B (BT) or A and B (AT, the weight gradients) stored
// [K][N] / [K][M] instead.
//
// Tiling: a block of WGM x WGN waves computes a BM-row tile of C over BN columns (256 x 256 with
// 8 waves and one block per CU for large groups, 128 x 256 with 4 waves and two blocks per CU
// otherwise); for the SwiGLU up projection two weight matrices (w1 and w3) of 128 columns each
// share the tile and the epilogue forms silu(x.w1) * (x.w3) in registers, so the gate and up
// products never leave the chip.  K is walked in steps of BK = 64 (32 for the short decode tiles).
//
// LDS: every operand row holds the step's BK bf16 (BK / 8 16-byte units) with unit u of row r
// stored at u ^ swz(r); each operand read of the matrix instruction is one ds_read_b128 per lane
// and the swizzle puts 16 consecutive rows read at one unit in distinct banks.  Transposed
// operands are stored as K rows (unit u of row r at u ^ swzT(r)) and read with ds_read_b64_tr_b16.
//
// Pipeline: direct-to-LDS buffer loads (one wave-wide 16-byte load fills 1 KB of a stage) into a
// ring of stages, one barrier per step issued without the memory fence of __syncthreads (which
// would drain the loads in flight), the operand reads of the next 16-wide k slice issued before
// the matrix instructions of the current one, and the last slice of a step multiplied after the
// barrier.  256-row tiles split the ring: two A stages and three B stages, so a weight load has
// two steps to land.  (The fp32-output router product stages through two register sets instead.)
// Loads past the end of a block's K range, past a group's rows or past N are sent out of the
// buffer's range and read zeros.
//
// Split-K: when the tile grid would leave CUs idle (few rows per expert, e.g. decode), blocks also
// split K; each writes fp32 partials and splitk_finish_kernel sums them in a fixed order and
// applies the epilogue.  Otherwise the last partial round of tiles may be split over K and summed
// by tail_finish_kernel, also in a fixed order (results do not depend on either split).
#include "common.h"
#include "gemm_common.h"
#include "kernels.h"

#include <algorithm>
#include <atomic>
#include <climits>
#include <type_traits>

namespace moe {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4_t;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8_t;
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;
typedef __attribute__((address_space(3))) int lds_int_t;

// Transposed-B stages hold K rows of BN columns (2 BN bytes); unit u of row r is stored at
// u ^ swzT(r).  A transposing read takes 4 consecutive rows of 32 bytes at one unit pair; the
// swizzle sends those 4 rows (and the two column halves of a wave) to disjoint banks.
__device__ __forceinline__ int swzT(int r) { return 4 * (r & 3); }

// A raw buffer descriptor (base, stride 0, num_records bytes) held in scalar registers.
typedef uint32_t desc_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ desc_t make_desc(const void* base, uint32_t num_records) {
  const uint64_t a = (uint64_t)base;
  desc_t d;
  d[0] = __builtin_amdgcn_readfirstlane((uint32_t)a);
  d[1] = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xffffu);
  d[2] = __builtin_amdgcn_readfirstlane(num_records);
  d[3] = 0x00020000u;
  return d;
}

// One wave-wide 16-byte direct-to-LDS load (lane l to byte lds + 16 l), issued where the compiler
// does not see it: the transposing LDS reads would otherwise make it wait for every such load in
// flight (it cannot tell the stages apart) before each of them.  No register is written; the
// loads are waited for by the explicit vmcnt waits of the main loop.  The load reads M0, which
// needs one wait state after the scalar write (the compiler inserts it for its own loads).
template <bool NTL>
__device__ __forceinline__ void dma16(desc_t desc, uint32_t voff, uint32_t lds) {
  if constexpr (NTL)
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen nt lds"
                 :
                 : "v"(voff), "s"(desc), "s"(lds)
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(desc), "s"(lds)
                 : "memory", "m0");
}

// Physical 16-byte unit of logical unit u in LDS row r is u ^ swz(r).  Both forms depend on r % 32
// only, keep 16 consecutive rows read at one unit in distinct 4-bank groups (with 64 banks; and 8
// rows with 32 banks), and leave a row's units inside the row.
template <int BK>
__device__ __forceinline__ int swz(int r) {
  if constexpr (BK == 32)
    return ((r >> 2) ^ (r >> 1)) & 3;   // 64-byte rows: four units
  else
    return (r ^ ((r >> 3) & 3)) & 7;    // 128-byte rows: eight units
}

// Value of the other lane of an adjacent pair (lanes 2c and 2c + 1 swap: a DPP quad permute).
__device__ __forceinline__ float swap_pair(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
}

// silu(g) = g / (1 + e^-g) with the hardware base-2 exponential and reciprocal (about 1 ulp each;
// the result is rounded to bf16).  Saturates to g for large g and to -0 for very negative g.
__device__ __forceinline__ float silu(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * g));
}

template <int BM, int BN, int NMAT, int BK>
constexpr int stage_bytes() {
  return (BM + NMAT * BN) * BK * 2;
}

constexpr int kMaxLds = 160 * 1024;                 // LDS per CU (and per block) on gfx950

// With direct loads, a 2-stage ring and one block per CU, the B operand (the weights: the stream
// whose loads miss the caches) gets a third stage in the LDS the 2-stage ring leaves free, so its
// loads have two steps to land; A keeps the 2-stage ring.
template <int BM, int BN, int NMAT, int BK, int NST, int MINB>
constexpr int b_stages() {
  return (NST == 2 && MINB == 1 &&
          NST * BM * BK * 2 + (NST + 1) * NMAT * BN * BK * 2 <= kMaxLds)
             ? NST + 1
             : NST;
}

template <int BM, int BN, int NMAT, int BK, int NST, int MINB>
constexpr int lds_bytes() {
  return NST == 0 ? 2 * stage_bytes<BM, BN, NMAT, BK>()
                  : NST * BM * BK * 2 + b_stages<BM, BN, NMAT, BK, NST, MINB>() * NMAT * BN * BK * 2;
}

constexpr int waitcnt_lgkm0() {                    // s_waitcnt lgkmcnt(0), other counters free
  return 15 | (3 << 14) | (7 << 4) | (0 << 8);
}
template <int VM>
constexpr int waitcnt_vm_lgkm0() {                 // s_waitcnt vmcnt(VM) lgkmcnt(0)
  static_assert(VM >= 0 && VM < 64, "vmcnt range");
  return (VM & 15) | ((VM >> 4) << 14) | (7 << 4) | (0 << 8);
}

__device__ __forceinline__ void barrier_no_fence() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Splitting the last round of tiles.  With `slots` blocks resident at once, total tiles run in
// total / slots whole rounds and one partial round of `rem` tiles that would leave the rest of the
// GPU idle; those tiles are split into q K chunks (q a power of two up to 8 with rem * q <= slots,
// chunks a whole number of 64-deep steps), and tail_finish_kernel adds the chunks' fp32 partials in
// a fixed order.  q == 1 runs every tile whole.
struct TailPlan {
  int full;   // tiles run whole (a multiple of slots, or all of them)
  int rem;    // tiles split
  int q;      // K chunks per split tile
};

__device__ __forceinline__ TailPlan tail_plan(int total, int slots, int K) {
  TailPlan tp{total, 0, 1};
  if (slots <= 0 || K % 64 != 0) return tp;
  const int full = total / slots * slots, rem = total - full;
  int q = 1;
  while (q < 8 && rem * q * 2 <= slots && (K / 64) % (q * 2) == 0) q *= 2;
  if (rem == 0 || q == 1) return tp;
  tp.full = full;
  tp.rem = rem;
  tp.q = q;
  return tp;
}

// One output tile: the K loop over the block's range and the epilogue.  tc names the tile; kc /
// nsplit its K chunk when the tile is split (rtile >= 0: a split tile of the last round, written as
// tile-local partials); kg_beg / kg_len the reduction rows in the K-grouped mode.  Every thread of
// the block calls it with the same arguments.  NTB: the weight (B) loads carry the non-temporal
// hint (bit 1 of a buffer load's cache-policy operand), for launches that read every weight panel
// once (the decode-sized products, bound by the weight stream: HBM serves such reads about 10%
// faster); otherwise the default policy keeps panels that several row tiles share in the caches.
struct NoHook {
  __device__ void operator()() const {}
};

// `after_loop` runs in every wave once the K loop is done, before the epilogue.
template <int BM, int BN, int NMAT, int WGM, int WGN, int BK, int NST, int MINB, int EPI, bool TAIL,
          bool BT = false, bool AT = false, bool NTB = false, class Hook = NoHook>
__device__ __forceinline__ void gemm_tile(const GemmParams& p, TileCoord tc, int kc, int nsplit,
                                          int rtile, int kg_beg, int kg_len,
                                          Hook after_loop = Hook()) {
  constexpr int NTHR = 64 * WGM * WGN;
  constexpr int WM = BM / WGM, WN = BN / WGN;       // WGM x WGN waves
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int KS = BK / 16;                       // 16-wide k slices per step
  constexpr int RB = BK * 2;                        // LDS bytes per operand row per step
  constexpr int UPR = BK / 8;                       // 16-byte units per row per step
  constexpr int A_UNITS = BM * UPR / NTHR;          // units per thread per step
  constexpr int B_UNITS = NMAT * BN * UPR / NTHR;
  constexpr int ROWS_PER_LOAD = NTHR / UPR;         // operand rows covered by one load per thread
  // Register sets: with 32-deep steps a load is issued two steps ahead (two sets), with 64-deep
  // steps one step ahead (one set, the same number of registers).
  constexpr int NSETS = BK == 32 ? 2 : 1;
  constexpr int STAGE = stage_bytes<BM, BN, NMAT, BK>();
  constexpr int B_OFF = BM * RB;                    // B rows follow the A rows in a stage
  static_assert(BK == 32 || BK == 64, "K step");
  static_assert(A_UNITS * NTHR == BM * UPR && B_UNITS * NTHR == NMAT * BN * UPR, "even split");
  static_assert(BN % ROWS_PER_LOAD == 0, "a load stays inside one weight matrix");
  static_assert(TM * 32 == WM && TN * 32 == WN, "32 x 32 matrix-instruction tiles");
  // Direct-to-LDS loads (NST > 0 stages; NST == 0 stages through registers): one wave-wide
  // 16-byte load fills 1 KB of LDS (lane l at byte 16 l), i.e. DROWS rows of a stage; block b of a
  // stage is loaded by wave b % NW.
  constexpr bool DMA = NST > 0;
  constexpr int NW = WGM * WGN;
  constexpr int DROWS = 1024 / RB;
  constexpr int DPW = (BM + NMAT * BN) / (DROWS * NW);   // direct loads per wave per step
  constexpr int DPW_A = BM / (DROWS * NW);                // the first DPW_A of them are A rows
  // The 256-row tiles with split rings (K-contiguous operands): only the first half of the waves
  // (one per SIMD) issue the direct loads, twice as many each, so the other wave of every SIMD
  // never stalls behind the loads' address processing and keeps the matrix core busy.
  constexpr bool LSPLIT = DMA && NST == 2 && MINB == 1 && !BT && !AT &&
                          2 * BM * BK * 2 + 3 * NMAT * BN * BK * 2 <= kMaxLds;
  constexpr int NWL = LSPLIT ? NW / 2 : NW;               // waves that issue direct loads
  constexpr int DPWL = LSPLIT ? 2 * DPW : DPW;             // direct loads per loading wave
  constexpr int DPWL_A = LSPLIT ? 2 * DPW_A : DPW_A;
  static_assert(!DMA || (DPW_A * DROWS * NW == BM && DPW * DROWS * NW == BM + NMAT * BN &&
                         BN % (DROWS * NW) == 0), "direct loads split evenly");
  // Transposed B: a stage's B block is BK rows of RBT bytes; one direct load fills RPB rows.
  constexpr int RBT = BN * 2, UPB = RBT / 16, RPB = 1024 / RBT;
  static_assert(!BT || (DMA && NMAT == 1 && BN == 256 &&
                        (EPI == EPI_STORE || EPI == EPI_SWIGLU_BWD_SAVED || AT) &&
                        BK * RBT == BN * RB),
                "transposed B: direct loads, one 256-column matrix, bf16 output");
  // Transposed A (with transposed B: the weight gradients, both operands row-major activations
  // reduced over their rows): a stage's A block is BK rows of RAT bytes.
  constexpr int RAT = BM * 2, UPA = RAT / 16, RPA = 1024 / RAT;
  static_assert(!AT || (BT && BM == 256 && EPI == EPI_STORE_F32_BIAS), "transposed A");

  extern __shared__ __align__(16) uint8_t smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // N-fastest wave layout: waves w and w + 4, which share a SIMD, own different row slices, so a
  // tile whose valid rows end in its first half (a group's ragged last tile) keeps every SIMD's
  // matrix core busy with only one of its two waves.
  const int wm0 = (wave / WGN) * WM;
  const int wn0 = (wave % WGN) * WN;
  static_assert(WGM * WGN <= 4 || (WGN == 2 || WGN == 4), "row slices spread over the SIMDs");
  const int n_base = tc.n_tile * BN;
  const int K = p.K, N = p.N;

  // Buffer descriptors: 32-bit offsets, and loads at or past num_records return zeros.
  const int lda = p.lda ? p.lda : K, ldb = p.ldb ? p.ldb : K;
  const uint32_t a_bytes = (uint32_t)p.a_rows * (uint32_t)lda * 2u;
  // Transposed B: [K][N] with row stride ldb_t; each of the stacked matrices holds bt_k1 rows.
  const int ldb_t = p.ldb ? p.ldb : N;
  const uint32_t b_bytes =
      BT ? (uint32_t)(p.bt_k1 > 0 ? p.bt_k1 : K) * (uint32_t)ldb_t * 2u : (uint32_t)N * (uint32_t)ldb * 2u;
  const __amdgpu_buffer_rsrc_t rA =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.A, (short)0, a_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rB0 = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const uint16_t*)p.B0 + (size_t)tc.g * p.b_gstride), (short)0, b_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rB1 =
      (NMAT == 2 || BT) ? __builtin_amdgcn_make_buffer_rsrc(
                      (void*)((const uint16_t*)p.B1 + (size_t)tc.g * p.b_gstride), (short)0,
                      b_bytes, 0x00020000)
                : rB0;

  desc_t dA{}, dB0{}, dB1{};
  if constexpr (BT) {
    dA = make_desc(p.A, a_bytes);
    dB0 = make_desc((const uint16_t*)p.B0 + (size_t)tc.g * p.b_gstride, b_bytes);
    dB1 = make_desc(p.B1 ? (const uint16_t*)p.B1 + (size_t)tc.g * p.b_gstride : nullptr, b_bytes);
  }

  // Unit c = tid + NTHR i of an operand is row c / UPR, unit c % UPR (UPR consecutive lanes read
  // one row's step of K, 64 or 128 contiguous bytes).  A rows past the group's end and B rows past
  // N read a valid row instead; they only feed accumulators that are never stored.
  uint32_t a_voff[A_UNITS], b_voff[B_UNITS];
  int a_lds[A_UNITS], b_lds[B_UNITS];
  const int u = tid % UPR;
  // Source rows of the gathered operand rows: every index load is issued before any is used (a
  // load and its wait per row would serialise their latencies at the start of every tile).
  auto gather_rows = [&](auto NRc, auto row_of, int* src) {
    constexpr int NR = decltype(NRc)::value;
    if (p.gather) {
#pragma unroll
      for (int i = 0; i < NR; ++i) src[i] = p.gather[min(tc.row0 + row_of(i), tc.row_end - 1)];
#pragma unroll
      for (int i = 0; i < NR; ++i) src[i] = src[i] / p.gather_div;
    } else {
#pragma unroll
      for (int i = 0; i < NR; ++i) src[i] = min(tc.row0 + row_of(i), tc.row_end - 1);
    }
  };
  if constexpr (!DMA) {
    int src[A_UNITS];
    gather_rows(std::integral_constant<int, A_UNITS>(),
                [&](int i) { return tid / UPR + ROWS_PER_LOAD * i; }, src);
#pragma unroll
    for (int i = 0; i < A_UNITS; ++i) {
      const int row = tid / UPR + ROWS_PER_LOAD * i;
      a_voff[i] = ((uint32_t)src[i] * (uint32_t)lda + 8u * u) * 2u;
      a_lds[i] = row * RB + ((u ^ swz<BK>(row)) << 4);
    }
  }
#pragma unroll
  for (int i = 0; i < B_UNITS; ++i) {
    const int brow = tid / UPR + ROWS_PER_LOAD * i;   // row of the stage's B block
    const int n = min(n_base + brow % BN, N - 1);
    b_voff[i] = ((uint32_t)n * (uint32_t)ldb + 8u * u) * 2u;
    b_lds[i] = B_OFF + brow * RB + ((u ^ swz<BK>(brow)) << 4);
  }

  // Direct loads: lane l of the load for stage block b = wave + NW j covers stage row
  // DROWS b + l / UPR at physical unit l % UPR, so it fetches the logical unit stored there.
  uint32_t d_voff[DMA ? DPWL : 1];
  int d_kmax[DMA ? DPWL : 1];           // the load reads zeros for steps starting at k0 >= d_kmax
  if constexpr (DMA) {
    int dsrc[AT ? 1 : DPWL_A];
    if constexpr (!AT)
      gather_rows(std::integral_constant<int, DPWL_A>(),
                  [&](int j) { return (wave + NWL * j) * DROWS + lane / UPR; }, dsrc);
#pragma unroll
    for (int j = 0; j < DPWL; ++j) {
      const int srow = (wave + NWL * j) * DROWS + lane / UPR;
      const int uu = (lane % UPR) ^ swz<BK>(srow);
      d_kmax[j] = 0;   // set below, once the K range is known
      if (j < DPWL_A) {
        if constexpr (AT) {   // row kr of the stage's A block (a K row), columns m
          const int kr = (wave + NW * j) * RPA + lane / UPA;
          const int ua = (lane % UPA) ^ swzT(kr);
          const int m = min(tc.row0 + 8 * ua, tc.row_end - 8);
          d_voff[j] = ((uint32_t)kr * (uint32_t)lda + (uint32_t)m) * 2u;
        } else {
          d_voff[j] = ((uint32_t)dsrc[j] * (uint32_t)lda + 8u * uu) * 2u;
        }
      } else if constexpr (BT) {
        // Row kr of the stage's B block (a K row), physical unit lane % UPB.
        const int kr = (wave + NW * (j - DPW_A)) * RPB + lane / UPB;
        const int ub = (lane % UPB) ^ swzT(kr);
        const int n = min(n_base + 8 * ub, N - 8);
        d_voff[j] = ((uint32_t)kr * (uint32_t)ldb_t + (uint32_t)n) * 2u;
      } else {
        const int n = min(n_base + (srow - BM) % BN, N - 1);
        d_voff[j] = ((uint32_t)n * (uint32_t)ldb + 8u * uu) * 2u;
      }
    }
  }

  // Uniform across the block (the compiler cannot always prove it through the tile scan).
  const int Kc = __builtin_amdgcn_readfirstlane(p.kgrouped ? kg_len : K / nsplit);
  const int kbeg = __builtin_amdgcn_readfirstlane(p.kgrouped ? kg_beg : kc * Kc);
  const int kend = kbeg + Kc;
  const int KT = (Kc + BK - 1) / BK;
  const int k_last = kbeg + (KT - 1) * BK;
  if constexpr (DMA) {
#pragma unroll
    for (int j = 0; j < DPWL; ++j) {
      const int srow = (wave + NWL * j) * DROWS + lane / UPR;
      // Rows past the group's end (A) or past N (B) feed only results that are never stored:
      // they read zeros without touching memory.
      const bool live = j < DPWL_A ? tc.row0 + srow < tc.row_end : n_base + (srow - BM) % BN < N;
      d_kmax[j] = live ? kend - 8 * ((lane % UPR) ^ swz<BK>(srow)) : INT_MIN;
      if constexpr (BT) {
        if (j >= DPW_A) {   // a K row: live while k0 + kr < kend and its 8 columns lie below N
          const int kr = (wave + NW * (j - DPW_A)) * RPB + lane / UPB;
          const int ub = (lane % UPB) ^ swzT(kr);
          d_kmax[j] = n_base + 8 * ub < N ? kend - kr : INT_MIN;
        }
      }
      if constexpr (AT) {
        if (j < DPW_A) {    // likewise for A: its 8 columns below the row count M
          const int kr = (wave + NW * j) * RPA + lane / UPA;
          const int ua = (lane % UPA) ^ swzT(kr);
          d_kmax[j] = tc.row0 + 8 * ua < tc.row_end ? kend - kr : INT_MIN;
        }
      }
    }
  }

  u32x4 a_reg[DMA ? 1 : NSETS][DMA ? 1 : A_UNITS];
  u32x4 b_reg[DMA ? 1 : NSETS][DMA ? 1 : B_UNITS];
  auto load_regs = [&](int set, int k0) {
    if constexpr (!TAIL) k0 = min(k0, k_last);
    const uint32_t koff = (uint32_t)k0 * 2u;
    const bool in_range = !TAIL || (k0 + 8 * u < kend);
#pragma unroll
    for (int i = 0; i < A_UNITS; ++i)
      a_reg[set][i] =
          __builtin_amdgcn_raw_buffer_load_b128(rA, in_range ? a_voff[i] + koff : a_bytes, 0, 0);
#pragma unroll
    for (int i = 0; i < B_UNITS; ++i) {
      const bool second = NMAT == 2 && (ROWS_PER_LOAD * i) / BN == 1;   // static per i
      b_reg[set][i] = __builtin_amdgcn_raw_buffer_load_b128(
          second ? rB1 : rB0, in_range ? b_voff[i] + koff : b_bytes, 0, NTB ? 2 : 0);
    }
  };
  // Direct loads of the step starting at k0 into the stage at stage_off.  Units at or past the end
  // of this block's K range (a ragged K, or a step past the last one) are sent out of the buffer's
  // range: they read zeros and touch no memory.
  // Loads j in [J0, J1) (A blocks first, then B): an A block goes to a_off + its offset in a
  // stage, a B block to b_off + its offset (b_off is the B stage's address minus B_OFF).  With
  // LSPLIT only the loading waves call it.
  auto issue_dma_range = [&](int a_off, int b_off, int k0, auto J0, auto J1) {
    const uint32_t koff = (uint32_t)k0 * 2u;
#pragma unroll
    for (int j = decltype(J0)::value; j < decltype(J1)::value; ++j) {
      const bool is_a = j < DPWL_A;
      bool second = NMAT == 2 && !is_a && ((j - DPWL_A) * DROWS * NWL) / BN == 1;
      uint32_t step_off = koff;
      if constexpr (BT) {
        if (!is_a) {   // K rows: k0 moves along rows; past bt_k1 they come from B1
          second = p.bt_k1 > 0 && k0 >= p.bt_k1;
          step_off = (uint32_t)(second ? k0 - p.bt_k1 : k0) * (uint32_t)ldb_t * 2u;
        }
      }
      if constexpr (AT) {
        if (is_a) step_off = (uint32_t)k0 * (uint32_t)lda * 2u;
      }
      const uint32_t voff = k0 < d_kmax[j] ? d_voff[j] + step_off : (is_a ? a_bytes : b_bytes);
      if constexpr (BT) {
        const uint32_t lds_at = (uint32_t)(size_t)(lds_void_t*)(smem + (is_a ? a_off : b_off) +
                                                                (wave + NWL * j) * 1024);
        if (is_a)
          dma16<false>(dA, voff, lds_at);
        else
          dma16<NTB>(second ? dB1 : dB0, voff, lds_at);
      } else {
        lds_void_t* const lds_at =
            (lds_void_t*)(smem + (is_a ? a_off : b_off) + (wave + NWL * j) * 1024);
        // (The router product streams its activations: with at most 256 experts, one column
        // tile, every x element is read once; non-temporal.)
        if (is_a)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, lds_at, 16, (int)voff, 0, 0,
                                                   (EPI == EPI_STORE_F32_BIAS && !AT) ? 2 : 0);
        else
          __builtin_amdgcn_raw_ptr_buffer_load_lds(second ? rB1 : rB0, lds_at, 16, (int)voff, 0, 0,
                                                   NTB ? 2 : 0);
      }
    }
  };
  auto issue_dma = [&](int stage_off, int k0) {
    issue_dma_range(stage_off, stage_off, k0, std::integral_constant<int, 0>(),
                    std::integral_constant<int, DPW>());
  };
  auto store_regs = [&](int set, int stage_off) {
#pragma unroll
    for (int i = 0; i < A_UNITS; ++i)
      *(lds_u32x4_t*)(smem + stage_off + a_lds[i]) = a_reg[set][i];
#pragma unroll
    for (int i = 0; i < B_UNITS; ++i)
      *(lds_u32x4_t*)(smem + stage_off + b_lds[i]) = b_reg[set][i];
  };

  // Operand reads: lane l takes row (or weight row) l % 32 of a 32-row block and k 8 (l / 32) .. +7
  // of the 16-wide slice ks, i.e. logical unit 2 ks + l / 32, stored at unit (l / 32 ^ swz) ^ 2 ks.
  // Block bases are multiples of 32 rows, so the swizzle depends on l % 32 only.
  const int l32 = lane & 31, h = lane >> 5;
  const int su = (h ^ swz<BK>(l32)) << 4;
  int a_rd[KS], b_rd[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    a_rd[ks] = (wm0 + l32) * RB + (su ^ (ks << 5));
    b_rd[ks] = B_OFF + (wn0 + l32) * RB + (su ^ (ks << 5));
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
  // Transposed B: lane l needs column l % 32 and K 8 (l / 32) .. +7 of a 32-column block.  Two
  // transposing reads (rows r .. r+3, then r+4 .. r+7) each give a lane 4 K values of one column:
  // in a group of 16 lanes, lane 4 q + a names row r + q and columns 4 a .. 4 a + 3, and lane s of
  // the group receives column s of the 4 rows.
  int bt_rd[BT ? TN : 1];
  if constexpr (BT) {
    const int g16 = lane >> 4, s16 = lane & 15, qa = s16 >> 2, aa = s16 & 3;
    const int kh = g16 >> 1, nh = g16 & 1;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int n = wn0 + 32 * j + 16 * nh + 4 * aa;
      const int r = 8 * kh + qa;
      bt_rd[j] = B_OFF + r * RBT + (((n >> 3) ^ swzT(r)) << 4) + (n & 7) * 2;
    }
  }
  int at_rd[AT ? TM : 1];
  if constexpr (AT) {   // the same lane pattern over the A block's rows and M columns
    const int g16 = lane >> 4, s16 = lane & 15, qa = s16 >> 2, aa = s16 & 3;
    const int kh = g16 >> 1, nh = g16 & 1;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int m = wm0 + 32 * i + 16 * nh + 4 * aa;
      const int r = 8 * kh + qa;
      at_rd[i] = r * RAT + (((m >> 3) ^ swzT(r)) << 4) + (m & 7) * 2;
    }
  }
  auto read_frags2 = [&](int a_off, int b_off, int ks, int buf) {
    if constexpr (AT) {
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const uint8_t* ap = smem + a_off + at_rd[i] + ks * 16 * RAT;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)ap);
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(ap + 4 * RAT));
        const i16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        af[buf][i] = __builtin_bit_cast(bf16x8, both);
      }
    } else {
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[buf][i] = *(const lds_bf16x8_t*)(smem + a_off + a_rd[ks] + i * 32 * RB);
    }
    if constexpr (BT) {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const uint8_t* bp = smem + b_off + bt_rd[j] + ks * 16 * RBT;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)bp);
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(bp + 4 * RBT));
        const i16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        bfr[buf][0][j] = __builtin_bit_cast(bf16x8, both);
      }
    } else {
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          bfr[buf][m][j] =
              *(const lds_bf16x8_t*)(smem + b_off + b_rd[ks] + (m * BN + j * 32) * RB);
    }
  };
  auto read_frags = [&](int stage_off, int ks, int buf) { read_frags2(stage_off, stage_off, ks, buf); };
  // The slice's LDS reads spread over its matrix instructions, ceil(reads / matrix instructions)
  // after each (one for K-contiguous operands, two for the transposing reads of the weight
  // gradients), rather than in one burst ahead of them.
  constexpr int NRD = (AT ? 2 * TM : TM) + (BT ? 2 * TN : NMAT * TN);
  constexpr int NMF = TM * NMAT * TN;
  auto interleave = [&]() {
    constexpr int R = (NRD + NMF - 1) / NMF;
    constexpr int P = NRD / R;
#pragma unroll
    for (int q = 0; q < P; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
    }
    if constexpr (NRD - P * R > 0) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, NRD - P * R, 0);
    }
    constexpr int USED = P + (NRD - P * R > 0 ? 1 : 0);
    if constexpr (NMF > USED) __builtin_amdgcn_sched_group_barrier(0x008, NMF - USED, 0);
  };
  // As interleave(), with NV direct loads placed too, one after each of the first NV matrix
  // instructions, so that a wave's load issue never holds back a run of its matrix instructions.
  auto interleave_v = [&](auto NVc) {
    constexpr int NV = decltype(NVc)::value;
    constexpr int R = (NRD + NMF - 1) / NMF;
#pragma unroll
    for (int q = 0; q < NMF; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
#pragma unroll
      for (int r = 0; r < R; ++r)
        if (q * R + r < NRD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      if (q < NV) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
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

  // A wave whose row slice lies wholly past the group's end only takes its share of the loads and
  // the barriers (the loop is instantiated twice, so that neither copy branches inside).
  const bool active = tc.row0 + wm0 < tc.row_end;
  if constexpr (DMA) {
    // NST-stage ring: the loads of step kt+NST-1 go into the stage that step kt-1 used, so a load
    // has NST-1 steps to land; the barrier that ends step kt waits only for step kt+1's loads.
    constexpr int NSB = b_stages<BM, BN, NMAT, BK, NST, MINB>();
    constexpr int A_BYTES = BM * RB, B_BYTES = NMAT * BN * RB;
    // Split rings: A stage s at s * A_BYTES, B stage s at NST * A_BYTES + s * B_BYTES.  In step kt
    // the loads of A(kt + 1) go out before those of B(kt + 2), so waiting until only the latter
    // are in flight (vmcnt counts in issue order) leaves A(kt + 1) and B(kt + 1) landed.
    auto run_split = [&](auto MATH, auto LOADER) {
      constexpr bool math = decltype(MATH)::value;
      constexpr bool loader = decltype(LOADER)::value;
      constexpr int DPW_B = DPWL - DPWL_A;
      auto dma_range = [&](int a_off, int b_off, int k0, auto J0, auto J1) {
        if constexpr (loader) issue_dma_range(a_off, b_off, k0, J0, J1);
      };
      const std::integral_constant<int, 0> j0;
      const std::integral_constant<int, DPWL_A> ja;
      const std::integral_constant<int, DPWL> j1;
      auto b_at = [&](int sb) { return NST * A_BYTES + sb * B_BYTES - B_OFF; };
      // Part Q (of the KS - 1 slices before the barrier) of step kt's loads, in issue order: the
      // A(kt + 1) blocks, then the B(kt + 2) blocks, cut into equal runs.
      auto dma_part = [&](auto Q, int kt, int na, int fb) {
        constexpr int q = decltype(Q)::value;
        constexpr int lo = DPWL * q / (KS - 1), hi = DPWL * (q + 1) / (KS - 1);
        constexpr int alo = lo < DPWL_A ? lo : DPWL_A, ahi = hi < DPWL_A ? hi : DPWL_A;
        constexpr int blo = lo > DPWL_A ? lo : DPWL_A, bhi = hi > DPWL_A ? hi : DPWL_A;
        dma_range(na * A_BYTES, 0, kbeg + (kt + 1) * BK, std::integral_constant<int, alo>(),
                  std::integral_constant<int, ahi>());
        dma_range(0, b_at(fb), kbeg + (kt + 2) * BK, std::integral_constant<int, blo>(),
                  std::integral_constant<int, bhi>());
        return std::integral_constant<int, loader ? hi - lo : 0>();
      };
      dma_range(0, 0, kbeg, j0, ja);
      dma_range(0, b_at(0), kbeg, ja, j1);
      dma_range(0, b_at(1), kbeg + BK, ja, j1);
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0<DPW_B>());
      barrier_no_fence();
      if constexpr (math) read_frags2(0, b_at(0), 0, 0);
      int sa = 0, sb = 0;                           // stages of step kt
      for (int kt = 0; kt < KT; ++kt) {
        const int na = sa ^ 1;
        const int nb = sb + 1 == NSB ? 0 : sb + 1;
        const int fb = sb == 0 ? NSB - 1 : sb - 1;  // stage of step kt + 2
        // K-contiguous operands: the step's loads spread over the slices (the transposing tiles of
        // the backward products, whose loads are inline assembly, issue them all first: measured
        // faster there).
        constexpr bool spread = !BT && !AT;
        if constexpr (math) {
          if constexpr (!spread) {
            dma_range(na * A_BYTES, 0, kbeg + (kt + 1) * BK, j0, ja);
            dma_range(0, b_at(fb), kbeg + (kt + 2) * BK, ja, j1);
          }
          // Slice ks: a part of the step's loads, the reads of slice ks + 1 and the matrix
          // instructions of slice ks, interleaved.
          auto slice = [&](auto KSc) {
            constexpr int ks = decltype(KSc)::value;
            if constexpr (spread) {
              const auto nv = dma_part(KSc, kt, na, fb);
              read_frags2(sa * A_BYTES, b_at(sb), ks + 1, (ks + 1) & 1);
              mfmas(ks & 1);
              interleave_v(nv);
            } else {
              read_frags2(sa * A_BYTES, b_at(sb), ks + 1, (ks + 1) & 1);
              mfmas(ks & 1);
              interleave();
            }
            __builtin_amdgcn_sched_barrier(0);
          };
          static_assert(KS == 4, "64-deep steps: three slices before the barrier");
          slice(std::integral_constant<int, 0>());
          slice(std::integral_constant<int, 1>());
          slice(std::integral_constant<int, 2>());
        } else {
          dma_range(na * A_BYTES, 0, kbeg + (kt + 1) * BK, j0, ja);
          dma_range(0, b_at(fb), kbeg + (kt + 2) * BK, ja, j1);
        }
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0<DPW_B>());
        barrier_no_fence();
        if constexpr (math) {
          read_frags2(na * A_BYTES, b_at(nb), 0, 0);
          mfmas((KS - 1) & 1);
          interleave();
          __builtin_amdgcn_sched_barrier(0);
        }
        sa = na;
        sb = nb;
      }
      // The last step's loads (past the end of K: zeros) land before the block may exit.
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0<0>());
    };
    auto run = [&](auto MATH) {
      constexpr bool math = decltype(MATH)::value;
#pragma unroll
      for (int s = 0; s < NST - 1; ++s) issue_dma(s * STAGE, kbeg + s * BK);
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0<DPW * (NST - 2)>());
      barrier_no_fence();
      if constexpr (math) read_frags(0, 0, 0);
      int st = 0;                                   // stage of step kt
      for (int kt = 0; kt < KT; ++kt) {
        const int nx = st + 1 == NST ? 0 : st + 1;
        const int fr = st == 0 ? NST - 1 : st - 1;
        issue_dma(fr * STAGE, kbeg + (kt + NST - 1) * BK);
        if constexpr (math) {
#pragma unroll
          for (int ks = 0; ks < KS - 1; ++ks) {
            read_frags(st * STAGE, ks + 1, (ks + 1) & 1);
            mfmas(ks & 1);
            interleave();
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0<DPW * (NST - 2)>());
        barrier_no_fence();
        if constexpr (math) {
          read_frags(nx * STAGE, 0, 0);
          mfmas((KS - 1) & 1);
          interleave();
          __builtin_amdgcn_sched_barrier(0);
        }
        st = nx;
      }
      // The loads of the steps past the end (zeros) land in LDS before the block may exit or
      // take another tile.
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0<0>());
    };
    if constexpr (NSB > NST) {
      static_assert(NST == 2, "split rings take a 2-stage A ring");
      // (LSPLIT: the other waves issue no loads; each kind runs its own copy of the loop.)
      const bool loader = !LSPLIT || wave < NWL;
      if (active) {
        if (loader)
          run_split(std::true_type(), std::true_type());
        else
          run_split(std::true_type(), std::false_type());
      } else {
        if (loader)
          run_split(std::false_type(), std::true_type());
        else
          run_split(std::false_type(), std::false_type());
      }
    } else {
      if (active)
        run(std::true_type());
      else
        run(std::false_type());
    }
  } else {
    auto run = [&](auto MATH) {
      constexpr bool math = decltype(MATH)::value;
      load_regs(0, kbeg);
      if constexpr (NSETS == 2) load_regs(1, kbeg + BK);
      store_regs(0, 0);
      load_regs(0, kbeg + NSETS * BK);
      __builtin_amdgcn_s_waitcnt(waitcnt_lgkm0());
      barrier_no_fence();
      if constexpr (math) read_frags(0, 0, 0);
      // One K step; S is true when kt is even (reads stage 0, fills stage 1).
      auto step = [&](int kt, auto S) {
        constexpr int st = decltype(S)::value ? 0 : STAGE;
        constexpr int nx = decltype(S)::value ? STAGE : 0;
        constexpr int set = (NSETS == 2 && decltype(S)::value) ? 1 : 0;
        store_regs(set, nx);                              // step kt+1 into the idle stage
        load_regs(set, kbeg + (kt + 1 + NSETS) * BK);     // and a later step into its registers
        if constexpr (math) {
#pragma unroll
          for (int ks = 0; ks < KS - 1; ++ks) {
            read_frags(st, ks + 1, (ks + 1) & 1);
            mfmas(ks & 1);
            interleave();
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        __builtin_amdgcn_s_waitcnt(waitcnt_lgkm0());
        barrier_no_fence();
        if constexpr (math) {
          read_frags(nx, 0, 0);
          mfmas((KS - 1) & 1);
          interleave();
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      // An odd step count runs one extra step; then K is ragged (TAIL) and it reads zeros.
      for (int kt = 0; kt < KT; kt += 2) {
        step(kt, std::true_type());
        step(kt + 1, std::false_type());
      }
    };
    if (active)
      run(std::true_type());
    else
      run(std::false_type());
  }
  after_loop();
  if (!active) return;

  // Epilogue.  Accumulator register r of a 32x32 tile holds row 8 (r / 4) + 4 (lane / 32) + r % 4
  // and column lane % 32.
  const bool partial = p.ksplit > 1 || rtile >= 0;
  void* const Cg = p.kgrouped ? (void*)((char*)p.C + (size_t)tc.g * p.c_gstride *
                                                         (EPI == EPI_STORE_F32_BIAS ? 4 : 2))
                              : p.C;
  if constexpr (EPI == EPI_SWIGLU_BWD) {   // never split (the launcher passes no workspace)
    if (N % 2 == 0 && p.ldc % 2 == 0) {
      // Two columns per lane as in the bf16 store below: after the pair exchange the even lane
      // holds row a and the odd lane row b of columns (2c, 2c+1); dh is read and h, da, db are
      // written 4 bytes at a time.
      // The 8 loads of dh of a 32 x 32 block are issued before its stores (one round trip).
      const bool odd = lane & 1;
#pragma unroll
      for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int col0 = n_base + wn0 + j * 32 + (l32 & ~1);
          uint32_t dhws[8];
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const int rr = odd ? 2 * q + 1 : 2 * q;
            const int row = tc.row0 + wm0 + i * 32 + 8 * (rr >> 2) + 4 * h + (rr & 3);
            dhws[q] = 0;
            if (row < tc.row_end && col0 < N)
              dhws[q] = *(const uint32_t*)((const uint16_t*)p.D + (size_t)row * N + col0);
          }
#pragma unroll
          for (int r = 0; r < 16; r += 2) {
            const float ga = swap_pair(odd ? acc[0][i][j][r] : acc[0][i][j][r + 1]);
            const float gb = swap_pair(odd ? acc[NMAT - 1][i][j][r] : acc[NMAT - 1][i][j][r + 1]);
            const int rr = odd ? r + 1 : r;
            const int row = tc.row0 + wm0 + i * 32 + 8 * (rr >> 2) + 4 * h + (rr & 3);
            if (row >= tc.row_end || col0 >= N) continue;
            float a[2], b[2];
            a[0] = odd ? ga : acc[0][i][j][r];
            a[1] = odd ? acc[0][i][j][r + 1] : ga;
            b[0] = odd ? gb : acc[NMAT - 1][i][j][r];
            b[1] = odd ? acc[NMAT - 1][i][j][r + 1] : gb;
            const size_t o = (size_t)row * N + col0;
            const uint32_t dhw = dhws[r >> 1];
            float hv[2], da[2], db[2];
#pragma unroll
            for (int q = 0; q < 2; ++q) {
              const float dh = q ? bf16_hi(dhw) : bf16_lo(dhw);
              const float sg =
                  __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * a[q]));
              const float sa = a[q] * sg;
              hv[q] = sa * b[q];
              da[q] = dh * b[q] * (sg * (1.0f + a[q] * (1.0f - sg)));
              db[q] = dh * sa;
            }
            *(uint32_t*)((uint16_t*)p.H + o) = pack_bf16x2(hv[0], hv[1]);
            uint16_t* dab = (uint16_t*)p.C + (size_t)row * p.ldc + col0;
            *(uint32_t*)dab = pack_bf16x2(da[0], da[1]);
            *(uint32_t*)(dab + N) = pack_bf16x2(db[0], db[1]);
          }
        }
      }
      return;
    }
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
          const float a = acc[0][i][j][r], b = acc[NMAT - 1][i][j][r];
          const size_t o = (size_t)row * N + col;
          const float dh = bf16_to_f32(((const uint16_t*)p.D)[o]);
          const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * a));
          const float sa = a * sg;
          ((uint16_t*)p.H)[o] = f32_to_bf16(sa * b);
          uint16_t* dab = (uint16_t*)p.C + (size_t)row * p.ldc + col;
          dab[0] = f32_to_bf16(dh * b * (sg * (1.0f + a * (1.0f - sg))));
          dab[N] = f32_to_bf16(dh * sa);
        }
      }
    }
    return;
  }
  if constexpr (EPI == EPI_SWIGLU_BWD_SAVED) {   // never split (the launcher passes no workspace)
    // The accumulator is dh; a and b come from the forward pass's saved bf16 values.  Per 32 x 32
    // block all 16 loads of a and b are issued before any store, so that one memory round trip
    // (not one per row pair: the stores may alias the loads) covers the block.
    if (N % 2 == 0 && p.ldc % 2 == 0 && p.ldd % 2 == 0) {
      const bool odd = lane & 1;
#pragma unroll
      for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int col0 = n_base + wn0 + j * 32 + (l32 & ~1);
          float dh[8][2];
          uint32_t aw[8], bw[8];
          int rows[8];
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const int r = 2 * q;
            const float g = swap_pair(odd ? acc[0][i][j][r] : acc[0][i][j][r + 1]);
            const int rr = odd ? r + 1 : r;
            rows[q] = tc.row0 + wm0 + i * 32 + 8 * (rr >> 2) + 4 * h + (rr & 3);
            dh[q][0] = odd ? g : acc[0][i][j][r];
            dh[q][1] = odd ? acc[0][i][j][r + 1] : g;
            aw[q] = bw[q] = 0;
            if (rows[q] < tc.row_end && col0 < N) {
              const uint16_t* ab = (const uint16_t*)p.D + (size_t)rows[q] * p.ldd + col0;
              aw[q] = *(const uint32_t*)ab;
              bw[q] = *(const uint32_t*)(ab + N);
            }
          }
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            if (rows[q] >= tc.row_end || col0 >= N) continue;
            float da[2], db[2];
#pragma unroll
            for (int c = 0; c < 2; ++c) {
              const float a = c ? bf16_hi(aw[q]) : bf16_lo(aw[q]);
              const float b = c ? bf16_hi(bw[q]) : bf16_lo(bw[q]);
              const float sg =
                  __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * a));
              da[c] = dh[q][c] * b * (sg * (1.0f + a * (1.0f - sg)));
              db[c] = dh[q][c] * (a * sg);
            }
            uint16_t* dab = (uint16_t*)p.C + (size_t)rows[q] * p.ldc + col0;
            *(uint32_t*)dab = pack_bf16x2(da[0], da[1]);
            *(uint32_t*)(dab + N) = pack_bf16x2(db[0], db[1]);
          }
        }
      }
      return;
    }
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
          const float dh = acc[0][i][j][r];
          const uint16_t* ab = (const uint16_t*)p.D + (size_t)row * p.ldd + col;
          const float a = bf16_to_f32(ab[0]), b = bf16_to_f32(ab[N]);
          const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * a));
          uint16_t* dab = (uint16_t*)p.C + (size_t)row * p.ldc + col;
          dab[0] = f32_to_bf16(dh * b * (sg * (1.0f + a * (1.0f - sg))));
          dab[N] = f32_to_bf16(dh * (a * sg));
        }
      }
    }
    return;
  }
  if (EPI == EPI_STORE_F32_BIAS && rtile < 0 && N % 4 == 0 && p.ldc % 4 == 0) {
    // fp32 output, four columns per 16-byte store: the four lanes of a quad hold one column each
    // of four consecutive rows; two DPP exchanges (lane ^ 1, then lane ^ 2) transpose that 4 x 4
    // block, so lane 4c + s holds row s of columns 4c .. 4c + 3.  The stores are non-temporal:
    // the output (the weight gradients, 4 bytes per weight) is not read again by this kernel and
    // would otherwise push the operand tiles out of the caches.  A K-split product writes its
    // chunk's partial sums the same way (no bias, cached stores) into its slice of the scratch.
    const bool kpart = !AT && p.ksplit > 1;   // (the weight gradients never split)
    float* const Cout = kpart ? p.part + (size_t)kc * p.part_rows * N : (float*)Cg;
    const int ldo = kpart ? N : p.ldc;
    const float* const bias = kpart ? nullptr : p.bias;
    const int s4 = lane & 3;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int col0 = n_base + wn0 + j * 32 + (l32 & ~3);
        f32x4 bias4 = {0.f, 0.f, 0.f, 0.f};
        if (bias && col0 < N) bias4 = *(const f32x4*)(bias + col0);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float a[4], b[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) a[t] = acc[0][i][j][4 * q + t];
          // Exchange across lane ^ 1: swap bit 0 of the lane with bit 0 of the slot.
          const bool o1 = s4 & 1;
          const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(
                                __builtin_bit_cast(int, o1 ? a[0] : a[1]), 0xB1, 0xF, 0xF, false));
          const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(
                                __builtin_bit_cast(int, o1 ? a[2] : a[3]), 0xB1, 0xF, 0xF, false));
          b[0] = o1 ? r0 : a[0];
          b[1] = o1 ? a[1] : r0;
          b[2] = o1 ? r1 : a[2];
          b[3] = o1 ? a[3] : r1;
          // Exchange across lane ^ 2: swap bit 1 of the lane with bit 1 of the slot.
          const bool o2 = s4 & 2;
          const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(
                                __builtin_bit_cast(int, o2 ? b[0] : b[2]), 0x4E, 0xF, 0xF, false));
          const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(
                                __builtin_bit_cast(int, o2 ? b[1] : b[3]), 0x4E, 0xF, 0xF, false));
          f32x4 w;
          w[0] = (o2 ? r2 : b[0]) + bias4[0];
          w[1] = (o2 ? r3 : b[1]) + bias4[1];
          w[2] = (o2 ? b[2] : r2) + bias4[2];
          w[3] = (o2 ? b[3] : r3) + bias4[3];
          const int row = tc.row0 + wm0 + i * 32 + 8 * q + 4 * h + s4;
          if (row < tc.row_end && col0 < N) {
            f32x4* dst = (f32x4*)(Cout + (size_t)row * ldo + col0);
            if (kpart)   // read back soon by the finishing kernel: keep it in the caches
              *dst = w;
            else
              __builtin_nontemporal_store(w, dst);
          }
        }
      }
    }
    return;
  }
  if (EPI != EPI_STORE_F32_BIAS && !partial && N % 2 == 0 && p.ldc % 2 == 0) {
    // bf16 output, two columns per 4-byte store: lanes 2c and 2c+1 swap one value of each pair of
    // rows (a DPP quad permute), so the even lane holds row a and the odd lane row b of columns
    // (2c, 2c+1).
    const bool odd = lane & 1;
    // A wave whose whole WM x WN block lies inside the output (no addend, no saved a and b) stores
    // through a buffer descriptor based at its block: the lane's row pair and column go into one
    // 32-bit offset computed once, and each register's row step into a wave-uniform offset, so the
    // stores need no per-store address arithmetic or bounds checks.
    if constexpr (EPI == EPI_SWIGLU || EPI == EPI_STORE) {
      const bool whole = __builtin_amdgcn_readfirstlane(
          (int)(tc.row0 + wm0 + WM <= tc.row_end && n_base + wn0 + WN <= N && !p.D));
      if (whole) {
        const int ldc2 = __builtin_amdgcn_readfirstlane(p.ldc * 2);   // row stride in bytes
        const int row_base = __builtin_amdgcn_readfirstlane(tc.row0 + wm0);
        const __amdgpu_buffer_rsrc_t rC = __builtin_amdgcn_make_buffer_rsrc(
            (void*)((char*)Cg + (size_t)row_base * ldc2 + (size_t)(n_base + wn0) * 2), (short)0,
            0x7fffffff, 0x00020000);
        const int voff = (4 * h + (odd ? 1 : 0)) * ldc2 + (l32 & ~1) * 2;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            float v[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              if constexpr (epi_swiglu(EPI))
                v[r] = silu(acc[0][i][j][r]) * acc[NMAT - 1][i][j][r];
              else
                v[r] = acc[0][i][j][r];
            }
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
              const float send = odd ? v[r] : v[r + 1];
              const float got = __builtin_bit_cast(
                  float,
                  __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, send), 0xB1, 0xF, 0xF, false));
              const float lo = odd ? got : v[r], hi = odd ? v[r + 1] : got;
              // Row i * 32 + 8 (r / 4) + (r % 4) of the block (plus the lane's 4 h + odd), columns
              // j * 32 + the lane's pair.
              const int soff = (i * 32 + 8 * (r >> 2) + (r & 3)) * ldc2 + j * 64;
              __builtin_amdgcn_raw_buffer_store_b32(pack_bf16x2(lo, hi), rC, voff, soff, 0);
            }
          }
        }
        return;
      }
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int col0 = n_base + wn0 + j * 32 + (l32 & ~1);
        float v[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          if constexpr (epi_swiglu(EPI))
            v[r] = silu(acc[0][i][j][r]) * acc[NMAT - 1][i][j][r];
          else
            v[r] = acc[0][i][j][r];
        }
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float send = odd ? v[r] : v[r + 1];
          const float got = __builtin_bit_cast(
              float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, send), 0xB1, 0xF, 0xF, false));
          const int rr = odd ? r + 1 : r;
          const int row = tc.row0 + wm0 + i * 32 + 8 * (rr >> 2) + 4 * h + (rr & 3);
          if constexpr (EPI == EPI_SWIGLU_SAVE) {   // a and b beside h, exchanged the same way
            const float ga = swap_pair(odd ? acc[0][i][j][r] : acc[0][i][j][r + 1]);
            const float gb = swap_pair(odd ? acc[NMAT - 1][i][j][r] : acc[NMAT - 1][i][j][r + 1]);
            if (row < tc.row_end && col0 < N) {
              uint16_t* dst = (uint16_t*)Cg + (size_t)row * p.ldc + col0;
              *(uint32_t*)(dst + N) = odd ? pack_bf16x2(ga, acc[0][i][j][r + 1])
                                          : pack_bf16x2(acc[0][i][j][r], ga);
              *(uint32_t*)(dst + 2 * N) = odd ? pack_bf16x2(gb, acc[NMAT - 1][i][j][r + 1])
                                              : pack_bf16x2(acc[NMAT - 1][i][j][r], gb);
            }
          }
          if (row < tc.row_end && col0 < N) {
            float lo = odd ? got : v[r], hi = odd ? v[r + 1] : got;
            if (EPI == EPI_STORE && p.D) {   // the addend, rounded with the sum
              const uint32_t add =
                  *(const uint32_t*)((const uint16_t*)p.D + (size_t)row * p.ldd + col0);
              lo += __builtin_bit_cast(float, add << 16);
              hi += __builtin_bit_cast(float, add & 0xffff0000u);
            }
            *(uint32_t*)((uint16_t*)Cg + (size_t)row * p.ldc + col0) = pack_bf16x2(lo, hi);
          }
        }
      }
    }
    return;
  }
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
        } else if (rtile >= 0) {   // tile-local fp32 partials; tail_finish_kernel sums them
#pragma unroll
          for (int m = 0; m < NMAT; ++m)
            p.part[(((size_t)rtile * nsplit + kc) * NMAT + m) * (BM * BN) + (row - tc.row0) * BN +
                   (col - n_base)] = acc[m][i][j][r];
        } else if constexpr (epi_swiglu(EPI)) {
          const float g = acc[0][i][j][r];
          const float v = acc[NMAT - 1][i][j][r];
          uint16_t* dst = (uint16_t*)Cg + (size_t)row * p.ldc + col;
          dst[0] = f32_to_bf16(silu(g) * v);
          if constexpr (EPI == EPI_SWIGLU_SAVE) {
            dst[N] = f32_to_bf16(g);
            dst[2 * N] = f32_to_bf16(v);
          }
        } else if constexpr (EPI == EPI_STORE) {
          const float add =
              p.D ? bf16_to_f32(((const uint16_t*)p.D)[(size_t)row * p.ldd + col]) : 0.f;
          ((uint16_t*)Cg)[(size_t)row * p.ldc + col] = f32_to_bf16(acc[0][i][j][r] + add);
        } else {
          ((float*)Cg)[(size_t)row * p.ldc + col] =
              acc[0][i][j][r] + (p.bias ? p.bias[col] : 0.f);
        }
      }
    }
  }
}

// The grouped GEMM kernel: each block finds its tile (K-grouped, every tile split over K, or whole
// rounds with the last partial round split) and computes it.
template <int BM, int BN, int NMAT, int WGM, int WGN, int BK, int NST, int MINB, int EPI, bool TAIL,
          bool BT = false, bool AT = false, bool NTB = false>
__global__ __launch_bounds__(64 * WGM * WGN, MINB) void gemm_bf16_kernel(const GemmParams p) {
  const int NT = (p.N + BN - 1) / BN;
  TileCoord tc;
  int kc = 0, nsplit = p.ksplit, rtile = -1;
  int kg_beg = 0, kg_len = 0;               // K-grouped mode: this group's reduction columns
  if (p.kgrouped) {
    // Tiles group-major; inside a group, bands of 4 m-tiles walked n-tile by n-tile, so 32
    // consecutive tiles form a 4 x 8 block that reads 4 A and 8 B tiles.  Blocks are dealt to the
    // 8 XCDs in turn (block b on XCD b % 8); in each whole round of p.slots blocks, XCD x takes
    // chunk 8 r + x of p.slots / 8 consecutive tiles, so the CUs sharing an L2 share operand
    // tiles, while consecutive chunks (a group's work, which grows with its row count) still go
    // to different XCDs.  The last partial round takes tiles in index order.
    const int MT = (p.M + BM - 1) / BM;
    const int per = MT * NT;
    const int total = p.G * per;
    int t = blockIdx.x;
    if (t >= total) return;
    const int round = p.slots >= 8 ? p.slots : 8, chunk = round / 8;
    if (t < total / round * round) {
      const int x = t & 7, k = t >> 3;
      t = ((k / chunk) * 8 + x) * chunk + k % chunk;
    }
    tc.g = t / per;
    const int local = t - tc.g * per;
    constexpr int GM = 4;
    const int band = local / (GM * NT);
    const int m_first = band * GM;
    const int gm = min(MT - m_first, GM);
    const int in = local - band * GM * NT;
    tc.row0 = (m_first + in % gm) * BM;
    tc.row_end = p.M;
    tc.n_tile = in / gm;
    const int o0 = p.offsets[tc.g];
    kg_beg = __builtin_amdgcn_readfirstlane(o0);
    kg_len = __builtin_amdgcn_readfirstlane(p.offsets[tc.g + 1] - o0);
  } else if (p.ksplit > 1) {                // every tile split over K
    const TileScan ts = scan_tiles<BM>(p, NT);
    kc = blockIdx.x % p.ksplit;
    const int bid = blockIdx.x / p.ksplit;
    if (bid >= ts.total) return;
    tile_at<BM>(p, NT, ts, xcd_order(bid, ts.total), tc);
  } else {                                  // whole rounds as is, the last partial round split
    const TileScan ts = scan_tiles<BM>(p, NT);
    const TailPlan tp = tail_plan(ts.total, p.slots, p.K);
    if ((int)blockIdx.x < tp.full) {
      tile_at<BM>(p, NT, ts, xcd_order(blockIdx.x, tp.full), tc);
    } else {
      const int w = blockIdx.x - tp.full;
      rtile = w / tp.q;
      kc = w % tp.q;
      nsplit = tp.q;
      if (rtile >= tp.rem) return;
      tile_at<BM>(p, NT, ts, tp.full + rtile, tc);
    }
  }
  tc.g = __builtin_amdgcn_readfirstlane(tc.g);
  tc.row0 = __builtin_amdgcn_readfirstlane(tc.row0);
  tc.row_end = __builtin_amdgcn_readfirstlane(tc.row_end);
  tc.n_tile = __builtin_amdgcn_readfirstlane(tc.n_tile);

  gemm_tile<BM, BN, NMAT, WGM, WGN, BK, NST, MINB, EPI, TAIL, BT, AT, NTB>(p, tc, kc, nsplit,
                                                                          rtile, kg_beg, kg_len);
}

// ---------------------------------------------------------------------------------------------
// Block-sparse dropless tiling of a grouped product whose group sizes are skewed (many experts with
// a few rows beside a few with thousands: the fine-grained, Zipf-routed layer).  The tiles form a
// block-sparse map over (expert, row block, column block), built on the device from `offsets`:
//   - a group with at least one whole 256-row block ("big") gets, for every column tile, its whole
//     256-row tiles followed by one tile for its remainder rows, so the remainder reuses the
//     column tile's weight panel from L2 instead of streaming the expert's weights a second time;
//   - a group with fewer than 256 rows ("small") gets one tile per column tile.
// Inside a big group, row tiles go in bands (below) so that an XCD's chunk of a round shares
// both its activation and its weight panels in L2.
// A tile of at most 64 rows runs as a thin tile (64 x BN, 8 waves in 2 x 4, a 4-stage ring: 96 KB of
// weights in flight per CU, for the weight-streaming tiles whose speed is set by bytes in flight);
// any other tile as the tall 256-row tile of the matrix-bound path.  Both kinds are one launch: the
// small groups' tiles are spread evenly through the big groups' tiles (tile t of the merged order is
// small when floor((t + 1) S / (S + B)) > floor(t S / (S + B)), S small and B big tiles), so every
// CU alternates between matrix-bound and weight-streaming work and HBM streams the small experts'
// weights while the matrix cores work.  Blocks are dealt to the XCDs by rounds (each
// XCD takes one chunk of every round of resident blocks), so every XCD gets the same mix of tall,
// thin and remainder tiles.  No K split: every tile sums its full K range.
// ---------------------------------------------------------------------------------------------
constexpr int kBsTall = 256;   // rows of a tall tile
constexpr int kBsThin = 64;    // rows of a thin tile (tiles of at most this many rows run thin)

struct BsScan {
  int big, small;              // tiles of each sequence in all groups
  int g0, g1;                  // this lane's groups [g0, g1)
  int big_mine, big_incl;      // tiles of the big sequence in this lane's groups, and inclusive
  int small_mine, small_incl;  // likewise for the small sequence
};

__device__ __forceinline__ BsScan bs_scan(const GemmParams& p, int NT) {
  BsScan s;
  const int lane = __lane_id();
  const int per = (p.G + 63) >> 6;
  s.g0 = min(p.G, lane * per);
  s.g1 = min(p.G, s.g0 + per);
  int big = 0, small = 0;
  for (int g = s.g0; g < s.g1; ++g) {
    const int n = p.offsets[g + 1] - p.offsets[g];
    if (n >= kBsTall)
      big += (n / kBsTall + (n % kBsTall != 0)) * NT;
    else if (n > 0)
      small += NT;
  }
  int bi = big, si = small;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int ub = __shfl_up(bi, o, 64), us = __shfl_up(si, o, 64);
    if (lane >= o) {
      bi += ub;
      si += us;
    }
  }
  s.big_mine = big;
  s.big_incl = bi;
  s.small_mine = small;
  s.small_incl = si;
  s.big = __shfl(bi, 63, 64);
  s.small = __shfl(si, 63, 64);
  return s;
}

// Whether the small groups' tiles follow all of the big groups' (bs_tile_at): a 256-row bf16
// panel of K columns over 2 MB.
__host__ __device__ constexpr bool bs_small_last(int K) { return K > 4096; }

// Tile t of the merged order of the block-sparse map -> coordinates (s from bs_scan).
__device__ __forceinline__ void bs_tile_at(const GemmParams& p, int NT, const BsScan& s, int t,
                                           TileCoord& tc) {
  const int total = s.big + s.small;
  // Small groups' tiles spread evenly through the big groups' (so that their weight streams run
  // beside matrix-bound tiles), unless a tall tile's operand panels (256 rows x K) are larger than
  // half an XCD's L2: then the big groups' tiles go first, in near lock step, so that the tiles of
  // a chunk still share their panels in L2, and the small groups' streams follow.
  int small_before, is_small;
  if (bs_small_last(p.K)) {
    is_small = t >= s.big;
    small_before = is_small ? t - s.big : 0;
  } else {
    const long long S = s.small, TT = total;
    small_before = (int)((long long)t * S / TT);
    is_small = (int)((long long)(t + 1) * S / TT) > small_before;
  }
  const int idx = is_small ? small_before : t - small_before;
  const int incl = is_small ? s.small_incl : s.big_incl;
  const int mine = is_small ? s.small_mine : s.big_mine;
  const int lane = __lane_id();
  const uint64_t own = __ballot(idx >= incl - mine && idx < incl);
  const int owner = __ffsll((long long)own) - 1;
  int g_found = 0, base = 0;
  if (lane == owner) {
    base = incl - mine;
    for (int g = s.g0; g < s.g1; ++g) {
      const int n = p.offsets[g + 1] - p.offsets[g];
      const int c = is_small ? (n > 0 && n < kBsTall ? NT : 0)
                             : (n >= kBsTall ? (n / kBsTall + (n % kBsTall != 0)) * NT : 0);
      if (idx < base + c) {
        g_found = g;
        break;
      }
      base += c;
    }
  }
  g_found = __shfl(g_found, owner, 64);
  base = __shfl(base, owner, 64);
  const int rs = p.offsets[g_found], re = p.offsets[g_found + 1];
  const int local = idx - base;
  tc.g = g_found;
  if (is_small) {                      // one tile per column tile
    tc.row0 = rs;
    tc.row_end = re;
    tc.n_tile = local;
  } else {
    // A group's row tiles (whole 256-row tiles, then the remainder) in bands of GM, each band
    // walked column tile by column tile: 32 consecutive tiles (one XCD's chunk of a round) then
    // read GM activation panels and 32 / GM weight panels.  A group of at most 8 row tiles is
    // one band (its remainder stays beside the whole tiles that share its weight panel); larger
    // groups take bands of 4 (a 4 x 8 block: 12 panels instead of up to 33).
    const int n = re - rs;
    const int per_n = n / kBsTall + (n % kBsTall != 0);
    const int GM = per_n <= 8 ? per_n : 4;
    const int band = local / (GM * NT);
    const int m_first = band * GM;
    const int gm = min(per_n - m_first, GM);
    const int in = local - band * GM * NT;
    tc.n_tile = in / gm;
    tc.row0 = rs + (m_first + in % gm) * kBsTall;
    tc.row_end = min(tc.row0 + kBsTall, re);
  }
}

// Tile `bid` (block order) of the block-sparse map -> coordinates; false past the last tile.
__device__ __forceinline__ bool bs_tile(const GemmParams& p, int NT, int bid, TileCoord& tc) {
  const BsScan s = bs_scan(p, NT);
  const int total = s.big + s.small;
  if (bid >= total) return false;
  bs_tile_at(p, NT, s, xcd_round_order(bid, total, p.slots), tc);
  return true;
}

// Ticket j of XCD x -> tile of the merged order, or -1 past XCD x's share.  The same tiles the
// hardware's round-robin dealing of blocks (block b on XCD b % 8) gives XCD x under
// xcd_round_order: in each whole round of `round` tiles its chunk of round / 8 consecutive tiles,
// then every eighth tile of the last partial round.
__device__ __forceinline__ int bs_ticket_tile(int x, int j, int total, int round) {
  const int chunk = round >> 3;
  const int whole = round >= 8 ? total / round : 0;
  if (j < whole * chunk) return (j / chunk) * round + x * chunk + j % chunk;
  const int t = whole * round + x + 8 * (j - whole * chunk);
  return t < total ? t : -1;
}

// Tile shapes of the block-sparse launch per epilogue: two weight matrices of 128 columns each
// (SwiGLU forward, SwiGLU backward), else one of 256; the tall tile's wave layout is that of the
// ordinary launch (4 x 2, or 2 x 4 for weights read transposed).
constexpr int bs_nmat(int epi) { return epi_swiglu(epi) || epi == EPI_SWIGLU_BWD ? 2 : 1; }
constexpr int bs_bn(int epi) { return bs_nmat(epi) == 2 ? 128 : 256; }

template <int EPI, bool BT, class Hook = NoHook>
__device__ __forceinline__ void bs_run_tile(const GemmParams& p, TileCoord tc,
                                            Hook after_loop = Hook()) {
  constexpr int NMAT = bs_nmat(EPI);
  constexpr int BN = bs_bn(EPI);                     // columns per matrix, both tile kinds
  tc.g = __builtin_amdgcn_readfirstlane(tc.g);
  tc.row0 = __builtin_amdgcn_readfirstlane(tc.row0);
  tc.row_end = __builtin_amdgcn_readfirstlane(tc.row_end);
  tc.n_tile = __builtin_amdgcn_readfirstlane(tc.n_tile);
  if (tc.row_end - tc.row0 <= kBsThin) {
    // A thin tile that starts its group is the whole of a small group, the only reader of its
    // weight panel (non-temporal weight loads); else it is a big group's remainder, which shares
    // the panel with the group's whole tiles.
    if (tc.row0 == p.offsets[tc.g])
      gemm_tile<kBsThin, BN, NMAT, 2, 4, 64, 4, 1, EPI, false, BT, false, true>(
          p, tc, 0, 1, -1, 0, 0, after_loop);
    else
      gemm_tile<kBsThin, BN, NMAT, 2, 4, 64, 4, 1, EPI, false, BT, false, false>(
          p, tc, 0, 1, -1, 0, 0, after_loop);
  } else
    gemm_tile<kBsTall, BN, NMAT, BT ? 2 : 4, BT ? 4 : 2, 64, 2, 1, EPI, false, BT, false, false>(
        p, tc, 0, 1, -1, 0, 0, after_loop);
}

// One block per tile: the hardware deals the blocks to the CUs.
template <int EPI, bool BT>
__global__ __launch_bounds__(512, 1) void gemm_bs_kernel(const GemmParams p) {
  const int NT = (p.N + bs_bn(EPI) - 1) / bs_bn(EPI);
  TileCoord tc;
  if (!bs_tile(p, NT, blockIdx.x, tc)) return;
  bs_run_tile<EPI, BT>(p, tc);
}

// One block per CU taking tiles from counters.  The hardware hands a CU the next block of its
// dealing order only when that block's turn comes, so with tiles of unequal length (thin and
// tall) CUs wait between blocks; here each block takes the next tile of its XCD's share as soon
// as it is done (the same tiles per XCD, so the L2 sharing is unchanged), then helps the other
// XCDs once its own share is gone.  The map scan runs once per block.  Every block ends when all
// eight counters are past their shares, so the grid always drains.
template <int EPI, bool BT>
__global__ __launch_bounds__(512, 1) void gemm_bs_persistent_kernel(const GemmParams p) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int NT = (p.N + bs_bn(EPI) - 1) / bs_bn(EPI);
  const BsScan s = bs_scan(p, NT);
  const int total = __builtin_amdgcn_readfirstlane(s.big + s.small);
  // HW_REG_XCC_ID: the XCD this block runs on.
  const int x0 = (int)(__builtin_amdgcn_s_getreg(20 | (31 << 11)) & 7);
  const bool wave0 = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) == 0;
  int tried = 0;   // wave 0: XCD shares found empty so far
  // Wave 0 takes the next tile (-1 when every share is gone); its lane 0 does the atomics, and
  // every value stays wave-uniform.
  auto take = [&]() {
    int t = -1;
    while (tried < 8) {
      const int x = (x0 + tried) & 7;
      int j = 0;
      if (__lane_id() == 0) j = atomicAdd(p.tickets + x, 1);
      t = bs_ticket_tile(x, __builtin_amdgcn_readfirstlane(j), total, p.slots);
      if (t >= 0) break;
      ++tried;
    }
    return t;
  };
  int next = wave0 ? take() : -1;
  for (;;) {
    if (threadIdx.x == 0) {
      *(lds_int_t*)smem = next;   // an LDS store (a generic one would also count as a memory op)
      __builtin_amdgcn_s_waitcnt(waitcnt_lgkm0());
    }
    // Bare barriers: they order the LDS only.  (A fenced barrier would also wait for the
    // previous tile's output stores, which may drain while the next tile starts.)
    barrier_no_fence();
    const int t = __builtin_amdgcn_readfirstlane(*(lds_int_t*)smem);
    barrier_no_fence();   // read by every wave before the tile's loads overwrite it
    if (t < 0) break;
    TileCoord tc;
    bs_tile_at(p, NT, s, t, tc);
    // The next tile is taken once the K loop is done, before this tile's output stores (whose
    // completion a later wait on the atomic's result would otherwise include).
    bs_run_tile<EPI, BT>(p, tc, [&]() {
      if (wave0) next = take();
    });
    // Every wave has waited for its LDS reads and its direct loads at the end of the K loop.
    barrier_no_fence();
  }
}

__global__ void zero_tickets_kernel(int* tickets) {
  if (threadIdx.x < 8) tickets[threadIdx.x] = 0;
}

// Sum the K-chunk partials of every valid row in a fixed order and apply the epilogue.
// Rows past the valid count (offsets[G], or M for a single group) are untouched.
template <int NMAT, int EPI>
__global__ __launch_bounds__(256) void splitk_finish_kernel(const GemmParams p) {
  const int rows = p.offsets ? p.offsets[p.G] : p.M;
  const int nv = p.N / 8;                              // 8 columns per thread
  const size_t total = (size_t)rows * nv;
  // fp32 output rows (and the bias) on 16-byte boundaries: vector stores.
  const bool vec_out = EPI == EPI_STORE_F32_BIAS && p.ldc % 4 == 0 &&
                       ((uintptr_t)p.C & 15) == 0 && ((uintptr_t)p.bias & 15) == 0;
  for (size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x; idx < total;
       idx += (size_t)gridDim.x * 256) {
    const int row = (int)(idx / nv), c0 = (int)(idx % nv) * 8;
    float s[NMAT][8];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int q = 0; q < 8; ++q) s[m][q] = 0.f;
    // Chunks in groups of four: the group's loads are all issued before any of them is added, and
    // the additions keep chunk order (the same sums as one chunk at a time).
    constexpr int KG = 4;
    for (int kc0 = 0; kc0 < p.ksplit; kc0 += KG) {
      f32x4 a[KG][NMAT], b[KG][NMAT];
#pragma unroll
      for (int j = 0; j < KG; ++j)
#pragma unroll
        for (int m = 0; m < NMAT; ++m) {
          if (kc0 + j < p.ksplit) {
            const f32x4* src = reinterpret_cast<const f32x4*>(
                p.part + ((size_t)((kc0 + j) * NMAT + m) * p.part_rows + row) * p.N + c0);
            a[j][m] = src[0];
            b[j][m] = src[1];
          }
        }
#pragma unroll
      for (int j = 0; j < KG; ++j)
#pragma unroll
        for (int m = 0; m < NMAT; ++m) {
          if (kc0 + j < p.ksplit) {
            s[m][0] += a[j][m][0]; s[m][1] += a[j][m][1];
            s[m][2] += a[j][m][2]; s[m][3] += a[j][m][3];
            s[m][4] += b[j][m][0]; s[m][5] += b[j][m][1];
            s[m][6] += b[j][m][2]; s[m][7] += b[j][m][3];
          }
        }
    }
    if constexpr (EPI == EPI_STORE_F32_BIAS) {   // the router's fp32 logits (+ bias)
      float* dst = (float*)p.C + (size_t)row * p.ldc + c0;
      if (vec_out) {   // two 16-byte stores (and bias loads)
        f32x4 b0 = {0.f, 0.f, 0.f, 0.f}, b1 = b0;
        if (p.bias) {
          b0 = *reinterpret_cast<const f32x4*>(p.bias + c0);
          b1 = *reinterpret_cast<const f32x4*>(p.bias + c0 + 4);
        }
        f32x4 o0, o1;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          o0[q] = s[0][q] + b0[q];
          o1[q] = s[0][4 + q] + b1[q];
        }
        *reinterpret_cast<f32x4*>(dst) = o0;
        *reinterpret_cast<f32x4*>(dst + 4) = o1;
      } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) dst[q] = s[0][q] + (p.bias ? p.bias[c0 + q] : 0.f);
      }
      continue;
    }
    u32x4 o, oa, ob;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float v0, v1;
      if constexpr (epi_swiglu(EPI)) {
        const float g0 = s[0][2 * q], g1 = s[0][2 * q + 1];
        v0 = silu(g0) * s[NMAT - 1][2 * q];
        v1 = silu(g1) * s[NMAT - 1][2 * q + 1];
        oa[q] = pack_bf16x2(g0, g1);
        ob[q] = pack_bf16x2(s[NMAT - 1][2 * q], s[NMAT - 1][2 * q + 1]);
      } else {
        v0 = s[0][2 * q];
        v1 = s[0][2 * q + 1];
      }
      o[q] = pack_bf16x2(v0, v1);
    }
    uint16_t* dst = (uint16_t*)p.C + (size_t)row * p.ldc + c0;
    *reinterpret_cast<u32x4*>(dst) = o;
    if constexpr (EPI == EPI_SWIGLU_SAVE) {
      *reinterpret_cast<u32x4*>(dst + p.N) = oa;
      *reinterpret_cast<u32x4*>(dst + 2 * p.N) = ob;
    }
  }
}

// Blocks kFinishSplit r .. +kFinishSplit-1 finish split tile r of the last round, a slice of rows
// each: they sum the q chunks' partials in chunk order and apply the epilogue (8 columns per item).
static constexpr int kFinishSplit = 8;

template <int BM, int BN, int NMAT, int EPI>
__global__ __launch_bounds__(256) void tail_finish_kernel(const GemmParams p) {
  const int NT = (p.N + BN - 1) / BN;
  const TileScan ts = scan_tiles<BM>(p, NT);
  const TailPlan tp = tail_plan(ts.total, p.slots, p.K);
  const int r = blockIdx.x / kFinishSplit, slice = blockIdx.x % kFinishSplit;
  if (r >= tp.rem) return;
  TileCoord tc;
  tile_at<BM>(p, NT, ts, tp.full + r, tc);
  const int n_base = tc.n_tile * BN;
  const float* base = p.part + (size_t)r * tp.q * NMAT * (BM * BN);
  constexpr int ITEMS = BM * BN / 8 / kFinishSplit;
  for (int e = slice * ITEMS + threadIdx.x; e < (slice + 1) * ITEMS; e += 256) {
    const int lr = e / (BN / 8), lc = (e % (BN / 8)) * 8;
    const int row = tc.row0 + lr, col = n_base + lc;
    if (row >= tc.row_end || col >= p.N) continue;
    float s[NMAT][8];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int c = 0; c < 8; ++c) s[m][c] = 0.f;
    for (int kc = 0; kc < tp.q; ++kc) {
#pragma unroll
      for (int m = 0; m < NMAT; ++m) {
        const f32x4* src = reinterpret_cast<const f32x4*>(
            base + (size_t)(kc * NMAT + m) * (BM * BN) + lr * BN + lc);
        const f32x4 a = src[0], b = src[1];
        s[m][0] += a[0]; s[m][1] += a[1]; s[m][2] += a[2]; s[m][3] += a[3];
        s[m][4] += b[0]; s[m][5] += b[1]; s[m][6] += b[2]; s[m][7] += b[3];
      }
    }
    u32x4 o, oa, ob;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float v0, v1;
      if constexpr (epi_swiglu(EPI)) {
        const float g0 = s[0][2 * c], g1 = s[0][2 * c + 1];
        v0 = silu(g0) * s[NMAT - 1][2 * c];
        v1 = silu(g1) * s[NMAT - 1][2 * c + 1];
        oa[c] = pack_bf16x2(g0, g1);
        ob[c] = pack_bf16x2(s[NMAT - 1][2 * c], s[NMAT - 1][2 * c + 1]);
      } else {
        v0 = s[0][2 * c];
        v1 = s[0][2 * c + 1];
      }
      o[c] = pack_bf16x2(v0, v1);
    }
    uint16_t* dst = (uint16_t*)p.C + (size_t)row * p.ldc + col;
    *reinterpret_cast<u32x4*>(dst) = o;
    if constexpr (EPI == EPI_SWIGLU_SAVE) {
      *reinterpret_cast<u32x4*>(dst + p.N) = oa;
      *reinterpret_cast<u32x4*>(dst + 2 * p.N) = ob;
    }
  }
}

// Compute units of the current device, cached per device (0 when unknown).  Written at most once
// per device with the same value, so concurrent first calls are harmless; atomics keep the reads
// well defined.
static int device_cus() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int c = cus[dev].load(std::memory_order_relaxed);
  if (c == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) n = 0;
    c = n > 0 ? n : -1;
    cus[dev].store(c, std::memory_order_relaxed);
  }
  return c > 0 ? c : 0;
}

template <int BM, int BN, int NMAT, int WGM, int WGN, int BK, int NST, int MINB, int EPI, bool TAIL,
          bool BT = false, bool AT = false, bool NTB = false>
static hipError_t launch_t(const GemmParams& p, int rows_max, hipStream_t s) {
  auto kern = gemm_bf16_kernel<BM, BN, NMAT, WGM, WGN, BK, NST, MINB, EPI, TAIL, BT, AT, NTB>;
  const size_t lds = (size_t)lds_bytes<BM, BN, NMAT, BK, NST, MINB>();
  static std::atomic<bool> attr_set[64];   // per device: the attribute is set on that device
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  if (!attr_set[dev].load(std::memory_order_acquire)) {
    // Setting it twice (two threads' first calls) is harmless.
    hipError_t e = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set[dev].store(true, std::memory_order_release);
  }
  GemmParams q = p;
  // The last partial round of tiles is split over K when the epilogue allows it (bf16 output, 8
  // columns per finishing item) and the caller gave scratch for the partials.
  const bool tail = p.ksplit == 1 && p.part != nullptr && EPI != EPI_STORE_F32_BIAS &&
                    EPI != EPI_SWIGLU_BWD && EPI != EPI_SWIGLU_BWD_SAVED && !p.kgrouped &&
                    p.N % 8 == 0 && p.K % 64 == 0;
  q.slots = tail ? device_cus() * MINB : 0;
  if (p.kgrouped) q.slots = device_cus() / 8 * 8 * MINB;   // blocks per round (tile order only)
  const int NT = (p.N + BN - 1) / BN;
  const int tiles = p.kgrouped ? p.G * ((p.M + BM - 1) / BM) * NT
                               : tiles_upper_bound(rows_max, p.G, p.offsets != nullptr, BM, NT);
  const int grid = tiles * p.ksplit + (p.kgrouped ? 0 : q.slots);
  if (tiles <= 0) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * WGM * WGN), lds, s, q);
  if (q.slots > 0 && !p.kgrouped) {
    if constexpr (EPI != EPI_STORE_F32_BIAS && EPI != EPI_SWIGLU_BWD &&
                  EPI != EPI_SWIGLU_BWD_SAVED)
      hipLaunchKernelGGL((tail_finish_kernel<BM, BN, NMAT, EPI>), dim3(q.slots * kFinishSplit),
                         dim3(256), 0, s, q);
  }
  return hipGetLastError();
}

// The block-sparse launch (every bf16-output epilogue, weights K-contiguous or transposed).
size_t gemm_bf16_partial_bytes(int rows_max, int G, bool grouped, int N, int K, int epi);

template <int EPI, bool BT>
static hipError_t launch_bs_t(const GemmParams& p, int rows_max, hipStream_t s) {
  static_assert(lds_bytes<kBsThin, bs_bn(EPI), bs_nmat(EPI), 64, 4, 1>() == kMaxLds &&
                    lds_bytes<kBsTall, bs_bn(EPI), bs_nmat(EPI), 64, 2, 1>() == kMaxLds,
                "both tile kinds fill the LDS the launch asks for");
  const int NT = (p.N + bs_bn(EPI) - 1) / bs_bn(EPI);
  // Every group yields at most floor(n_g / 256) + 1 tiles per column tile.
  const int tiles = tiles_upper_bound(rows_max, p.G, true, kBsTall, NT);
  if (tiles <= 0) return hipSuccess;
  // One block per CU taking tiles from counters when there can be more than two rounds of tiles
  // (with fewer, a block has at most a tile or two and the counters only add their latency) and
  // the caller's split-K scratch (which this launch does not otherwise use) can hold them; else
  // one block per tile.  (The SwiGLU-backward epilogues never get scratch: they run on whole sums
  // only.)
  constexpr bool can_persist = EPI == EPI_SWIGLU || EPI == EPI_SWIGLU_SAVE || EPI == EPI_STORE;
  const int round = device_cus() / 8 * 8;
  const bool persistent = can_persist && p.part != nullptr && round >= 8 && tiles > 2 * round &&
                          gemm_bf16_partial_bytes(rows_max, p.G, true, p.N, p.K, EPI) >= 64;
  void (*kern)(GemmParams) = gemm_bs_kernel<EPI, BT>;
  if constexpr (can_persist) {
    if (persistent) kern = gemm_bs_persistent_kernel<EPI, BT>;
  }
  static std::atomic<bool> attr_set[64][2];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  if (!attr_set[dev][persistent].load(std::memory_order_acquire)) {
    hipError_t e = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLds);
    if (e != hipSuccess) return e;
    attr_set[dev][persistent].store(true, std::memory_order_release);
  }
  GemmParams q = p;
  q.ksplit = 1;
  q.slots = round;   // one block per CU: the blocks of one round
  if (persistent) {
    q.tickets = (int*)p.part;
    hipLaunchKernelGGL(zero_tickets_kernel, dim3(1), dim3(64), 0, s, q.tickets);
    hipLaunchKernelGGL(kern, dim3(std::min(tiles, q.slots)), dim3(512), kMaxLds, s, q);
  } else {
    q.tickets = nullptr;
    hipLaunchKernelGGL(kern, dim3(tiles), dim3(512), kMaxLds, s, q);
  }
  return hipGetLastError();
}

static hipError_t launch_bs(const GemmParams& p, int rows_max, int epi, hipStream_t s) {
  switch (epi) {
    case EPI_SWIGLU: return launch_bs_t<EPI_SWIGLU, false>(p, rows_max, s);
    case EPI_SWIGLU_SAVE: return launch_bs_t<EPI_SWIGLU_SAVE, false>(p, rows_max, s);
    case EPI_SWIGLU_BWD: return launch_bs_t<EPI_SWIGLU_BWD, false>(p, rows_max, s);
    case EPI_STORE:
      return p.bt ? launch_bs_t<EPI_STORE, true>(p, rows_max, s)
                  : launch_bs_t<EPI_STORE, false>(p, rows_max, s);
    case EPI_SWIGLU_BWD_SAVED:
      return p.bt ? launch_bs_t<EPI_SWIGLU_BWD_SAVED, true>(p, rows_max, s)
                  : launch_bs_t<EPI_SWIGLU_BWD_SAVED, false>(p, rows_max, s);
    default: return hipErrorNotSupported;
  }
}

template <int BM, int BN, int NMAT, int WGM, int WGN, int BK, int NST, int MINB, int EPI,
          bool BT = false, bool NTB = false>
static hipError_t launch_tail_or_not(const GemmParams& p, int rows_max, hipStream_t s) {
  // The direct-load path handles any K range; the register path needs an even step count.
  const bool even_steps = NST > 0 || (p.K / p.ksplit) % (2 * BK) == 0;
  return even_steps
             ? launch_t<BM, BN, NMAT, WGM, WGN, BK, NST, MINB, EPI, false, BT, false, NTB>(p, rows_max, s)
             : launch_t<BM, BN, NMAT, WGM, WGN, BK, NST, MINB, EPI, true, BT, false, NTB>(p, rows_max, s);
}

static void launch_splitk_finish(const GemmParams& p, int rows_max, int epi, hipStream_t s) {
  const size_t items = (size_t)rows_max * (p.N / 8);
  const int fgrid = (int)std::min<size_t>((items + 255) / 256, 4096);
  if (fgrid <= 0) return;
  if (epi == EPI_SWIGLU)
    hipLaunchKernelGGL((splitk_finish_kernel<2, EPI_SWIGLU>), dim3(fgrid), dim3(256), 0, s, p);
  else if (epi == EPI_SWIGLU_SAVE)
    hipLaunchKernelGGL((splitk_finish_kernel<2, EPI_SWIGLU_SAVE>), dim3(fgrid), dim3(256), 0, s,
                       p);
  else if (epi == EPI_STORE_F32_BIAS)
    hipLaunchKernelGGL((splitk_finish_kernel<1, EPI_STORE_F32_BIAS>), dim3(fgrid), dim3(256), 0, s,
                       p);
  else
    hipLaunchKernelGGL((splitk_finish_kernel<1, EPI_STORE>), dim3(fgrid), dim3(256), 0, s, p);
}

void launch_splitk_finish_bf16(const GemmParams& p, int rows_max, int epi, hipStream_t s) {
  launch_splitk_finish(p, rows_max, epi, s);
}

// 256-row tiles (8 waves, one block per CU) when the groups are large enough to fill them: they
// load a third fewer operand bytes per flop than 128-row tiles.  Smaller groups (fine-grained
// experts, decode) keep 128-row tiles so that ragged group ends waste less.
static bool use_big_tiles(int rows_max, int G, bool grouped, int epi) {
  if (epi == EPI_STORE_F32_BIAS) return false;
  return rows_max >= 256 * (grouped ? std::max(G, 1) : 1);
}

// K chunks for the expert GEMMs when the tiles alone would fill less than two rounds of the
// resident blocks (few rows per expert, e.g. decode).  Compute-bound shapes take the smallest
// power-of-two split (chunks a
// whole number of 64-deep steps) whose work items fill at least one round with the rounds at
// least 90% busy on average, else the split that keeps them busiest (or, when no split fills a
// round, the largest).
static int splitk_factor(int rows_max, int G, bool grouped, int N, int K, int epi) {
  if (epi == EPI_STORE_F32_BIAS) {
    // The router product (one dense group, fp32 logits): 256 x 256 tiles, one block per CU.  A
    // few thousand tokens give too few tiles to cover the GPU, so K is split into the smallest
    // power-of-two number of chunks (whole 64-deep steps, at most 8) whose blocks fill one round.
    if (grouped || K % 64 != 0 || N % 8 != 0) return 1;
    const long long tiles = (long long)((rows_max + 255) / 256) * ((N + 255) / 256);
    const int cus = device_cus();
    const long long slots = 1ll * (cus > 0 ? cus : 256);
    int ks = 1;
    while (ks < 8 && tiles * ks < slots && (K / 64) % (ks * 2) == 0) ks *= 2;
    return ks;
  }
  if (K % 64 != 0 || N % 8 != 0) return 1;
  if (use_big_tiles(rows_max, G, grouped, epi)) return 1;
  const int BM = 128, BN = epi_swiglu(epi) ? 128 : 256;
  const int mt = grouped ? std::min(G, rows_max) + rows_max / BM : (rows_max + BM - 1) / BM;
  const long long tiles = (long long)mt * ((N + BN - 1) / BN);
  const int cus = device_cus();
  // Two work items per CU: the transposed-weight short tiles run two blocks per CU, the others
  // one block per CU over two rounds (measured no slower on the weight stream than one round).
  const long long slots = 2ll * (cus > 0 ? cus : 256);
  if (tiles >= 2 * slots) return 1;
  // Fewer rows than a tile per group: weight streaming, bound by HBM; one round of one block per
  // CU keeps HBM busy, so split only as far as that round needs (fewer partial sums to add, and
  // each block's stream long enough to hide its ring's fill: measured 6% faster on the decode down
  // projection than splitting for two blocks per CU).
  if ((grouped ? rows_max / std::max(G, 1) : rows_max) < BM) {
    const long long round1 = cus > 0 ? cus : 256;
    int ks = 1;
    while (ks < 16 && tiles * ks < round1 && (K / 64) % (ks * 2) == 0) ks *= 2;
    return ks;
  }
  auto busy = [&](long long items) {                    // mean occupancy of the rounds
    const long long rounds = (items + slots - 1) / slots;
    return (double)items / (double)(rounds * slots);
  };
  int best = 1, largest = 1;
  double best_busy = tiles >= slots ? busy(tiles) : 0.0;
  for (int ks = 1; ks <= 16 && (K / 64) % ks == 0; ks *= 2) {
    const long long items = tiles * ks;
    largest = ks;
    if (items < slots) continue;
    if (busy(items) >= 0.9) return ks;
    if (busy(items) > best_busy + 0.02) {
      best = ks;
      best_busy = busy(items);
    }
  }
  return best_busy > 0.0 ? best : largest;   // no split fills a round: split the most
}

// Scratch for the fp32 partial sums: every tile split (few rows), or the split tiles of the last
// round (at most one round of blocks, each a BM x BN tile of NMAT partials; 256 KB per CU for
// every tile configuration used here).
size_t gemm_bf16_partial_bytes(int rows_max, int G, bool grouped, int N, int K, int epi) {
  if (epi == EPI_STORE_F32_BIAS) {
    const int ks = splitk_factor(rows_max, G, grouped, N, K, epi);
    return ks > 1 ? (size_t)ks * rows_max * N * sizeof(float) : 0;
  }
  const int nmat = epi_swiglu(epi) ? 2 : 1;
  const int ks = splitk_factor(rows_max, G, grouped, N, K, epi);
  if (ks > 1) return (size_t)ks * nmat * rows_max * N * sizeof(float);
  if (N % 8 != 0 || K % 64 != 0) return 0;
  const bool big = use_big_tiles(rows_max, G, grouped, epi);
  const int BM = big ? 256 : 128, BN = epi_swiglu(epi) ? 128 : 256, minb = big ? 1 : 2;
  return (size_t)device_cus() * minb * nmat * BM * BN * sizeof(float);
}

// The tile configuration of each epilogue: 256-row tiles (8 waves, one block per CU) or 128-row
// tiles (4 waves, two blocks per CU).
// `per_group`: rows per group on average.  With fewer rows than a short tile, the short tiles read
// every weight panel once, so the forward products load their weights with the non-temporal hint;
// with at most 64 rows they take 64-row tiles (8 waves in 2 x 4, a 4-stage ring: 96 KB of weights
// in flight per CU instead of 64 KB, the decode-sized products being bound by the weight stream).
static hipError_t launch_cfg(const GemmParams& p, int rows_max, int epi, bool big, int per_group,
                             hipStream_t s) {
  const bool streams = !big && per_group < 128;
  const bool thin = streams && per_group <= 64;
  switch (epi) {
    case EPI_SWIGLU:   // short tiles: 64-deep steps (128-byte runs per weight row), one block per CU
      if (big) return launch_tail_or_not<256, 128, 2, 4, 2, 64, 2, 1, EPI_SWIGLU>(p, rows_max, s);
      if (thin)
        return launch_tail_or_not<64, 128, 2, 2, 4, 64, 4, 1, EPI_SWIGLU, false, true>(p, rows_max, s);
      return streams
                 ? launch_tail_or_not<128, 128, 2, 2, 2, 64, 3, 1, EPI_SWIGLU, false, true>(p, rows_max,
                                                                                          s)
                 : launch_tail_or_not<128, 128, 2, 2, 2, 64, 3, 1, EPI_SWIGLU>(p, rows_max, s);
    case EPI_SWIGLU_SAVE:   // the same tiles, storing a and b beside h
      return big ? launch_tail_or_not<256, 128, 2, 4, 2, 64, 2, 1, EPI_SWIGLU_SAVE>(p, rows_max, s)
                 : launch_tail_or_not<128, 128, 2, 2, 2, 64, 3, 1, EPI_SWIGLU_SAVE>(p, rows_max, s);
    case EPI_STORE:   // short tiles: 64-deep steps (128-byte runs per weight row), one block per CU
      if (p.bt)
        return big ? launch_tail_or_not<256, 256, 1, 2, 4, 64, 2, 1, EPI_STORE, true>(p, rows_max, s)
                   : launch_tail_or_not<128, 256, 1, 2, 2, 32, 3, 2, EPI_STORE, true>(p, rows_max, s);
      if (big) return launch_tail_or_not<256, 256, 1, 4, 2, 64, 2, 1, EPI_STORE>(p, rows_max, s);
      if (thin)
        return launch_tail_or_not<64, 256, 1, 2, 4, 64, 4, 1, EPI_STORE, false, true>(p, rows_max, s);
      return streams
                 ? launch_tail_or_not<128, 256, 1, 2, 2, 64, 3, 1, EPI_STORE, false, true>(p, rows_max,
                                                                                         s)
                 : launch_tail_or_not<128, 256, 1, 2, 2, 64, 3, 1, EPI_STORE>(p, rows_max, s);
    case EPI_SWIGLU_BWD:
      return big ? launch_tail_or_not<256, 128, 2, 4, 2, 64, 2, 1, EPI_SWIGLU_BWD>(p, rows_max, s)
                 : launch_tail_or_not<128, 128, 2, 2, 2, 32, 3, 2, EPI_SWIGLU_BWD>(p, rows_max, s);
    case EPI_SWIGLU_BWD_SAVED:   // the dh product's tiles (transposed B as stored, or K-contiguous)
      if (p.bt)
        return big ? launch_tail_or_not<256, 256, 1, 2, 4, 64, 2, 1, EPI_SWIGLU_BWD_SAVED, true>(
                         p, rows_max, s)
                   : launch_tail_or_not<128, 256, 1, 2, 2, 32, 3, 2, EPI_SWIGLU_BWD_SAVED, true>(
                         p, rows_max, s);
      return big ? launch_tail_or_not<256, 256, 1, 4, 2, 64, 2, 1, EPI_SWIGLU_BWD_SAVED>(p, rows_max,
                                                                                      s)
                 : launch_tail_or_not<128, 256, 1, 2, 2, 32, 3, 2, EPI_SWIGLU_BWD_SAVED>(p, rows_max,
                                                                                      s);
    default:   // the router product: the 256 x 256 direct-load tiles, one block per CU
      return launch_tail_or_not<256, 256, 1, 4, 2, 64, 2, 1, EPI_STORE_F32_BIAS>(p, rows_max, s);
  }
}

// Needs K (and the row strides) a multiple of 8 (16-byte rows) and every operand under 2 GiB
// (32-bit buffer offsets).
hipError_t launch_gemm_bf16(const GemmParams& p_in, int rows_max, int epi, hipStream_t s) {
  const int lda = p_in.lda ? p_in.lda : p_in.K;
  const int ldb = p_in.ldb ? p_in.ldb : (p_in.bt ? p_in.N : p_in.K);
  // (With transposed A and B, K counts rows of both: any count.)
  if ((!p_in.at && p_in.K % 8 != 0) || lda % 8 != 0 || ldb % 8 != 0 || p_in.N < 1 ||
      p_in.K < (p_in.at ? 1 : 8))
    return hipErrorNotSupported;
  const long long b_rows = p_in.bt ? (p_in.bt_k1 > 0 ? p_in.bt_k1 : p_in.K) : p_in.N;
  if ((long long)p_in.a_rows * lda * 2 >= (1ll << 31) || b_rows * ldb * 2 >= (1ll << 31))
    return hipErrorNotSupported;
  if (p_in.at && !(p_in.bt && p_in.kgrouped)) return hipErrorNotSupported;
  if (p_in.bt && p_in.kgrouped) {
    // Weight gradients from row-major operands: A [K][M], B [K][N], M and N multiples of 8.
    if (!p_in.at || epi != EPI_STORE_F32_BIAS || p_in.N % 8 != 0 || p_in.M % 8 != 0 ||
        ldb < p_in.N || lda < p_in.M || p_in.bt_k1 != 0)
      return hipErrorNotSupported;
  } else if (p_in.bt) {
    // Transposed B: bf16 output, N a multiple of 8, the stacked matrices split on a 64-deep step.
    if ((epi != EPI_STORE && epi != EPI_SWIGLU_BWD_SAVED) || p_in.N % 8 != 0 || ldb < p_in.N ||
        (p_in.bt_k1 > 0 && (p_in.bt_k1 % 64 != 0 || p_in.bt_k1 >= p_in.K)))
      return hipErrorNotSupported;
  }
  GemmParams p = p_in;
  const bool grouped = p.offsets != nullptr;
  if (p.kgrouped) {             // weight gradients: fp32 out, 256 x 256 tiles, no split
    if (!grouped || epi != EPI_STORE_F32_BIAS || p.gather || !p.at) return hipErrorNotSupported;
    p.ksplit = 1;
    p.part = nullptr;
    return launch_t<256, 256, 1, 4, 2, 64, 2, 1, EPI_STORE_F32_BIAS, false, true, true>(p, 0, s);
  }
  // These epilogues run on whole sums only.
  if (epi == EPI_SWIGLU_BWD || epi == EPI_SWIGLU_BWD_SAVED) p.part = nullptr;
  if (epi == EPI_STORE && p.D) {   // the addend: one group, no split
    if (grouped) return hipErrorNotSupported;
    p.part = nullptr;
  }
  if (epi == EPI_SWIGLU_BWD_SAVED && (!p.D || p.ldd < 2 * p.N)) return hipErrorInvalidValue;
  if (epi == EPI_SWIGLU_SAVE && p.ldc < 3 * p.N) return hipErrorInvalidValue;
  p.ksplit = splitk_factor(rows_max, p.G, grouped, p.N, p.K, epi);
  p.part_rows = rows_max;
  if (p.ksplit > 1 && p.part == nullptr) p.ksplit = 1;   // no scratch given: no split
  const bool big = use_big_tiles(rows_max, p.G, grouped, epi);
  hipError_t e;
  const bool skewed = big && grouped && p.ksplit == 1 && epi != EPI_STORE_F32_BIAS &&
                     (long long)rows_max < 512ll * p.G;
  if (big && grouped && p.ksplit == 1 && epi != EPI_STORE_F32_BIAS &&
      (skewed || epi_swiglu(epi))) {
    // One block-sparse launch of tall and thin tiles: every product of skewed groups (a few
    // hundred rows per group on average), and the SwiGLU up projection whenever the groups fill
    // 256-row tiles (its few-row remainders run as thin tiles).  Evenly filled groups give the
    // other products too few tiles, whose last round the K-split tiling balances.
    e = launch_bs(p, rows_max, epi, s);
  } else {
    e = launch_cfg(p, rows_max, epi, big, grouped ? rows_max / std::max(p.G, 1) : rows_max, s);
  }
  if (e != hipSuccess) return e;
  if (p.ksplit > 1) launch_splitk_finish(p, rows_max, epi, s);
  return hipGetLastError();
}

}  // namespace moe
