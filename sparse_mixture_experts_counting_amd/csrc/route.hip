// Router product (few experts), gating + top-k, and the deterministic reduction of the loss
// partials.  The method is the Score and Select steps of the page "Mixture of experts (MoE)"
// (tirogla), How it works steps 1-2 and its Code `route`; gating modes as listed there.
#include "common.h"
#include "kernels.h"

#include <math.h>

namespace moe {

// ---------------------------------------------------------------------------------------------
// Router product for E <= 16 experts: logits[t, e] = sum_j x[t, j] w_r[e, j] (+ bias[e]), W_r in
// the [E][d] layout of a linear layer.  Memory bound on x.  A block of 4 waves takes TPB = 64 / EP
// tokens (EP = E rounded up to a power of two, at least 4; or 64 for one token per block when the
// batch is small), so that its TPB x EP (token, expert) sums are one per lane; the waves split d in four, and lanes stride over 8-wide slices of their
// quarter (16-byte loads of x and of every W_r row; d is a multiple of 8).  Each lane's 64 partial
// sums are reduced across the wave by a butterfly that halves the values a lane carries at every
// step (63 lane exchanges in all), leaving lane l with the total of sum l; the four waves' totals
// are added in a fixed order.
// ---------------------------------------------------------------------------------------------
template <int E>
constexpr int pow2_at_least() {      // at least 4, so that a block takes at most 16 tokens
  return E <= 4 ? 4 : E <= 8 ? 8 : 16;
}

template <typename TIn>
__device__ __forceinline__ void load8(const TIn* p, float* f) {
  if constexpr (sizeof(TIn) == 2) {
    unpack8(*reinterpret_cast<const u32x4*>(p), f);
  } else {
    const f32x4 a = reinterpret_cast<const f32x4*>(p)[0], b = reinterpret_cast<const f32x4*>(p)[1];
    f[0] = a[0]; f[1] = a[1]; f[2] = a[2]; f[3] = a[3];
    f[4] = b[0]; f[5] = b[1]; f[6] = b[2]; f[7] = b[3];
  }
}

template <typename TIn, int E, int EP>
__global__ __launch_bounds__(256) void router_small_e_kernel(const TIn* __restrict__ x,
                                                             const TIn* __restrict__ w_r,
                                                             const float* __restrict__ bias, int T,
                                                             int d, float* __restrict__ logits) {
  static_assert(EP >= E && EP <= 64 && (EP & (EP - 1)) == 0, "expert slots per token");
  constexpr int TPB = 64 / EP;
  __shared__ float part[4][64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * TPB;
  float v[64];                                   // v[i * EP + e]: token t0 + i, expert e
#pragma unroll
  for (int q = 0; q < 64; ++q) v[q] = 0.f;

  const int nchunk = d >> 3;
  const int per = (nchunk + 3) >> 2;
  const int c_end = min(nchunk, (wave + 1) * per);
  for (int c = wave * per + lane; c < c_end; c += 64) {
    float w[E][8];
#pragma unroll
    for (int e = 0; e < E; ++e) load8(w_r + (size_t)e * d + c * 8, w[e]);
#pragma unroll
    for (int i = 0; i < TPB; ++i) {
      const int t = t0 + i;
      if (t < T) {
        float xv[8];
        load8(x + (size_t)t * d + c * 8, xv);
#pragma unroll
        for (int kk = 0; kk < 8; ++kk)
#pragma unroll
          for (int e = 0; e < E; ++e) v[i * EP + e] = fmaf(xv[kk], w[e][kk], v[i * EP + e]);
      }
    }
  }
  // Butterfly: at offset o a lane keeps the half of its 2 o values selected by bit o of its lane
  // id and adds the partner's copy of that half.
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const bool upper = lane & o;
#pragma unroll
    for (int q = 0; q < o; ++q) {
      const float send = upper ? v[q] : v[o + q];
      const float keep = upper ? v[o + q] : v[q];
      v[q] = keep + __shfl_xor(send, o, 64);
    }
  }
  part[wave][lane] = v[0];
  __syncthreads();
  if (wave == 0) {
    const float sum = ((part[0][lane] + part[1][lane]) + part[2][lane]) + part[3][lane];
    const int t = t0 + lane / EP, e = lane % EP;
    if (t < T && e < E) logits[(size_t)t * E + e] = sum + (bias ? bias[e] : 0.f);
  }
}

// A few hundred tokens or fewer: one token per block (64 expert slots, most of them idle), so
// that the blocks spread over many CUs; otherwise TPB tokens per block as above.
template <typename TIn, int E>
static void launch_router_small_e_t(const void* x, const void* w_r, const float* bias, int T,
                                    int d, float* logits, hipStream_t s) {
  constexpr int EP = pow2_at_least<E>();
  constexpr int TPB = 64 / EP;
  if (T < 1024) {
    hipLaunchKernelGGL((router_small_e_kernel<TIn, E, 64>), dim3(T), dim3(256), 0, s,
                       (const TIn*)x, (const TIn*)w_r, bias, T, d, logits);
    return;
  }
  const int blocks = (T + TPB - 1) / TPB;
  hipLaunchKernelGGL((router_small_e_kernel<TIn, E, EP>), dim3(blocks), dim3(256), 0, s,
                     (const TIn*)x, (const TIn*)w_r, bias, T, d, logits);
}

template <typename TIn>
static void launch_router_small_e_d(const void* x, const void* w_r, const float* bias, int T,
                                    int d, int E, float* logits, hipStream_t s) {
  switch (E) {
#define MOE_CASE(n) \
  case n: launch_router_small_e_t<TIn, n>(x, w_r, bias, T, d, logits, s); break;
    MOE_CASE(1) MOE_CASE(2) MOE_CASE(3) MOE_CASE(4) MOE_CASE(5) MOE_CASE(6) MOE_CASE(7)
    MOE_CASE(8) MOE_CASE(9) MOE_CASE(10) MOE_CASE(11) MOE_CASE(12) MOE_CASE(13) MOE_CASE(14)
    MOE_CASE(15) MOE_CASE(16)
#undef MOE_CASE
    default: break;
  }
}

// The same product on the matrix cores for batches of at least 1024 bf16 tokens with d a multiple of
// 2048: a block of 16 waves takes 16 tokens; wave w reduces over its sixteenth of d with
// v_mfma_f32_32x32x16_bf16 (A: the 16 token rows, padded to 32; B: the E expert rows of W_r,
// padded to 32), every lane loading 16-byte pieces that cover 256 contiguous bytes of a row per
// batch of eight instructions; the waves' fp32 partial sums are added in wave order through
// LDS.  The products of bf16 values are exact in the fp32 accumulators, so the logits lie within
// the same rounding bound as the vector form's.  Memory bound on x, which every lane streams
// with the non-temporal hint (read once).
constexpr int kRouterMfmaTok = 16, kRouterMfmaWaves = 16, kRouterMfmaU = 8;

template <int E>
__global__ __launch_bounds__(1024) void router_mfma_kernel(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ w_r,
                                                          const float* __restrict__ bias, int T,
                                                          int d, float* __restrict__ logits) {
  __shared__ float part[kRouterMfmaWaves][kRouterMfmaTok][E];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const int t0 = blockIdx.x * kRouterMfmaTok;
  const int kw = d / kRouterMfmaWaves;               // this wave's K range: [wave kw, +kw)
  const bool row_ok = l32 < kRouterMfmaTok && t0 + l32 < T;
  const bool col_ok = l32 < E;
  const u32x4* xr = reinterpret_cast<const u32x4*>(
      x + (size_t)(row_ok ? t0 + l32 : 0) * d + (size_t)wave * kw + 8 * h);
  const u32x4* wr = reinterpret_cast<const u32x4*>(
      w_r + (size_t)(col_ok ? l32 : 0) * d + (size_t)wave * kw + 8 * h);
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  for (int k = 0; k < kw; k += 16 * kRouterMfmaU) {
    u32x4 a[kRouterMfmaU], b[kRouterMfmaU];
#pragma unroll
    for (int u = 0; u < kRouterMfmaU; ++u) {
      a[u] = row_ok ? __builtin_nontemporal_load(xr + (k + 16 * u) / 8) : zero;
      b[u] = col_ok ? wr[(k + 16 * u) / 8] : zero;
    }
#pragma unroll
    for (int u = 0; u < kRouterMfmaU; ++u)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[u]),
                                                    __builtin_bit_cast(bf16x8, b[u]), acc, 0, 0,
                                                    0);
  }
  // Register r holds token row 8 (r / 4) + 4 h + r % 4 and expert column l32.
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = 8 * (r >> 2) + 4 * h + (r & 3);
    if (row < kRouterMfmaTok && col_ok) part[wave][row][l32] = acc[r];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kRouterMfmaTok * E; i += 1024) {
    const int row = i / E, e = i % E, t = t0 + row;
    if (t >= T) continue;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < kRouterMfmaWaves; ++w) v += part[w][row][e];
    logits[(size_t)t * E + e] = v + (bias ? bias[e] : 0.f);
  }
}

template <int E>
static void launch_router_mfma_t(const void* x, const void* w_r, const float* bias, int T, int d,
                                 float* logits, hipStream_t s) {
  const int blocks = (T + kRouterMfmaTok - 1) / kRouterMfmaTok;
  hipLaunchKernelGGL((router_mfma_kernel<E>), dim3(blocks), dim3(1024), 0, s, (const uint16_t*)x,
                     (const uint16_t*)w_r, bias, T, d, logits);
}

void launch_router_small_e(const void* x, const void* w_r, const float* bias, int T, int d, int E,
                           bool bf16, float* logits, hipStream_t s) {
  if (bf16 && T >= 1024 && d % (kRouterMfmaWaves * 16 * kRouterMfmaU) == 0) {
    switch (E) {
#define MOE_CASE(n) \
  case n: launch_router_mfma_t<n>(x, w_r, bias, T, d, logits, s); return;
      MOE_CASE(1) MOE_CASE(2) MOE_CASE(3) MOE_CASE(4) MOE_CASE(5) MOE_CASE(6) MOE_CASE(7)
      MOE_CASE(8) MOE_CASE(9) MOE_CASE(10) MOE_CASE(11) MOE_CASE(12) MOE_CASE(13) MOE_CASE(14)
      MOE_CASE(15) MOE_CASE(16)
#undef MOE_CASE
      default: break;
    }
  }
  if (bf16)
    launch_router_small_e_d<uint16_t>(x, w_r, bias, T, d, E, logits, s);
  else
    launch_router_small_e_d<float>(x, w_r, bias, T, d, E, logits, s);
}

// Router product for any E (E > 16 and not a multiple of 8): one thread per (token, expert), the
// token row staged in LDS in slices.  Plain and slow; the wide-E shapes of interest take the
// matrix-core path instead.
template <typename TIn>
__global__ __launch_bounds__(256) void router_generic_kernel(const TIn* __restrict__ x,
                                                             const TIn* __restrict__ w_r,
                                                             const float* __restrict__ bias, int T,
                                                             int d, int E,
                                                             float* __restrict__ logits) {
  __shared__ float xs[1024];
  const int t = blockIdx.x;
  const int e = blockIdx.y * 256 + threadIdx.x;
  float acc = 0.f;
  for (int j0 = 0; j0 < d; j0 += 1024) {
    const int n = min(1024, d - j0);
    __syncthreads();
    for (int j = threadIdx.x; j < n; j += 256) {
      if constexpr (sizeof(TIn) == 2)
        xs[j] = bf16_to_f32(x[(size_t)t * d + j0 + j]);
      else
        xs[j] = x[(size_t)t * d + j0 + j];
    }
    __syncthreads();
    if (e < E) {
      for (int j = 0; j < n; ++j) {
        float w;
        if constexpr (sizeof(TIn) == 2)
          w = bf16_to_f32(w_r[(size_t)e * d + j0 + j]);
        else
          w = w_r[(size_t)e * d + j0 + j];
        acc = fmaf(xs[j], w, acc);
      }
    }
  }
  if (e < E) logits[(size_t)t * E + e] = acc + (bias ? bias[e] : 0.f);
}

void launch_router_generic(const void* x, const void* w_r, const float* bias, int T, int d, int E,
                           bool bf16, float* logits, hipStream_t s) {
  dim3 grid(T, (E + 255) / 256);
  if (bf16)
    hipLaunchKernelGGL(router_generic_kernel<uint16_t>, grid, dim3(256), 0, s, (const uint16_t*)x,
                       (const uint16_t*)w_r, bias, T, d, E, logits);
  else
    hipLaunchKernelGGL(router_generic_kernel<float>, grid, dim3(256), 0, s, (const float*)x,
                       (const float*)w_r, bias, T, d, E, logits);
}

// ---------------------------------------------------------------------------------------------
// Gating + top-k.  One wave per token row; lane l holds experts l, l+64, ... (EPL of them).
// Selection ranks on an integer key built from the float32 score so that -0.0 == +0.0 and equal
// scores go to the lower expert index: key = (order-preserving bits of the score) << 32 | ~e.  The
// score is the logit, or logit + select_bias[e] (one float32 add) for aux-loss-free balancing; the
// gates, P and the z-loss always use the logit.
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ uint32_t ordered_bits(float v) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;  // -0.0 -> +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float from_ordered_bits(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o ^ 0x80000000u) : ~o);
}

// Lane l's logits of one row (experts l, l + 64, ...), every load issued before any is used (lanes
// past E read expert E - 1; gate_row masks them).
template <int EPL>
__device__ __forceinline__ void load_row(const float* row, int E, float (&v)[EPL]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    v[i] = row[e < E ? e : E - 1];
  }
}

// Gating, top-k and the loss terms of one row t, by one wave.  `v` holds the lane's logits of the
// row as load_row reads them; acc_p[i] (expert lane + 64 i) and acc_l accumulate the row's softmax
// probabilities and squared logsumexp.
// `sb` holds the lane's selection biases (as load_row reads them) when `biased`.
template <int EPL>
__device__ __forceinline__ void gate_row(float (&v)[EPL], bool biased, const float (&sb)[EPL],
                                         int t, int E, int k, int mode,
                                         int32_t* __restrict__ topk_idx,
                                         float* __restrict__ topk_gate, float* acc_p,
                                         float& acc_l) {
  const int lane = threadIdx.x & 63;
  uint32_t key[EPL];   // order-preserving bits of the score
  uint32_t live = 0;   // bit i: expert lane + 64 i exists and is not selected yet
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    if (e < E) {
      key[i] = ordered_bits(biased ? v[i] + sb[i] : v[i]);
      live |= 1u << i;
    } else {
      v[i] = -INFINITY;
      key[i] = 0u;
    }
  }
  // Full-row softmax (for P_e) and logsumexp (for the z-loss).
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < EPL; ++i) m = fmaxf(m, v[i]);
  m = wave_max_dpp(m);
  float ex[EPL];
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    ex[i] = (lane + 64 * i < E) ? expf(v[i] - m) : 0.f;
    s += ex[i];
  }
  s = wave_sum_dpp(s);
  const float inv_s = 1.0f / s;
#pragma unroll
  for (int i = 0; i < EPL; ++i) acc_p[i] += ex[i] * inv_s;
  const float lse = m + logf(s);
  acc_l += lse * lse;

  // Top-k by repeated wave arg-max: the largest live score, then among the live experts holding
  // it the lowest index (the first nonzero ballot over i, its lowest lane), which leaves the
  // selection.  v0 is the largest selected logit (the first one selected when there is no
  // selection bias), the shift that keeps the gates finite.
  int my_e = 0;
  float my_v = -INFINITY;
  for (int j = 0; j < k; ++j) {
    uint32_t best = 0u;
#pragma unroll
    for (int i = 0; i < EPL; ++i) best = max(best, ((live >> i) & 1u) ? key[i] : 0u);
    best = wave_max_u32_dpp(best);
    int e_j = -1;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const uint64_t b = __ballot(((live >> i) & 1u) && key[i] == best);
      if (e_j < 0 && b != 0ull) e_j = 64 * i + (int)__builtin_ctzll(b);
    }
    if (lane == (e_j & 63)) live &= ~(1u << (e_j >> 6));
    float v_j = from_ordered_bits(best);
    if (biased) {   // the score is biased: take the logit from the lane that holds it
      float own = v[0];
#pragma unroll
      for (int i = 1; i < EPL; ++i)
        if ((e_j >> 6) == i) own = v[i];
      v_j = readlane_f32(own, e_j & 63);
    }
    if (lane == j) {
      my_e = e_j;
      my_v = v_j;
    }
  }
  const float v0 = wave_max_dpp(my_v);
  float w = 0.f;
  if (lane < k) {
    if (mode == 0)
      w = expf(my_v - v0);
    else if (mode == 1)
      w = expf(my_v - m) * inv_s;
    else
      w = expf(log_sigmoid(my_v) - log_sigmoid(v0));
  }
  float g = w;
  if (mode != 1) g = w / wave_sum_dpp(w);
  if (lane < k) {
    topk_idx[(size_t)t * k + lane] = my_e;
    topk_gate[(size_t)t * k + lane] = g;
  }
}

// kGateWaves waves per block, a wave per row at a time; the waves' P and lse partials are added in
// wave order, one partial per block.
static constexpr int kGateWaves = 16;

template <int EPL>
__global__ __launch_bounds__(64 * kGateWaves) void gate_topk_kernel(
    const float* __restrict__ logits, const float* __restrict__ select_bias, int T, int E, int k,
    int mode, int rows_per_block, int32_t* __restrict__ topk_idx, float* __restrict__ topk_gate,
    float* __restrict__ part_p, float* __restrict__ part_l) {
  __shared__ float red_p[kGateWaves][64 * EPL];
  __shared__ float red_l[kGateWaves];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int row0 = blockIdx.x * rows_per_block;
  const int row1 = min(T, row0 + rows_per_block);

  float acc_p[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) acc_p[i] = 0.f;
  float acc_l = 0.f;
  // The selection biases are the same for every row; the next row's logits are loaded while this
  // row is gated.
  float sb[EPL] = {}, nxt[EPL];
  const bool biased = select_bias != nullptr;
  if (biased) load_row<EPL>(select_bias, E, sb);
  int t = row0 + wave;
  if (t < row1) load_row<EPL>(logits + (size_t)t * E, E, nxt);
  for (; t < row1; t += kGateWaves) {
    float v[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) v[i] = nxt[i];
    if (t + kGateWaves < row1) load_row<EPL>(logits + (size_t)(t + kGateWaves) * E, E, nxt);
    gate_row<EPL>(v, biased, sb, t, E, k, mode, topk_idx, topk_gate, acc_p, acc_l);
  }

  if (part_p) {
#pragma unroll
    for (int i = 0; i < EPL; ++i) red_p[wave][lane + 64 * i] = acc_p[i];
    if (lane == 0) red_l[wave] = acc_l;
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += 64 * kGateWaves) {
      float v = red_p[0][e];
#pragma unroll
      for (int w = 1; w < kGateWaves; ++w) v += red_p[w][e];
      part_p[(size_t)blockIdx.x * E + e] = v;
    }
    if (threadIdx.x == 0) {
      float v = red_l[0];
#pragma unroll
      for (int w = 1; w < kGateWaves; ++w) v += red_l[w];
      part_l[blockIdx.x] = v;
    }
  }
}

// Sum the per-block partials in a fixed order: one wave per expert (lanes stride over the blocks,
// then a fixed butterfly), the lse partials by the extra wave E.  Deterministic.
__global__ __launch_bounds__(256) void route_finalize_kernel(const float* __restrict__ part_p,
                                                             const float* __restrict__ part_l,
                                                             int nblk, int E,
                                                             float* __restrict__ prob_sum,
                                                             float* __restrict__ lse_sq_sum) {
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item > E) return;
  float s = 0.f;
  if (item < E) {
    if (!prob_sum) return;
    for (int b = lane; b < nblk; b += 64) s += part_p[(size_t)b * E + item];
    s = wave_sum(s);
    if (lane == 0) prob_sum[item] = s;
  } else {
    if (!lse_sq_sum) return;
    for (int b = lane; b < nblk; b += 64) s += part_l[b];
    s = wave_sum(s);
    if (lane == 0) lse_sq_sum[0] = s;
  }
}

int gate_rows_per_block(int T) {
  // One row per wave up to 4096 rows (each wave's rows are a chain of dependent reductions), two
  // from 8192 rows (fewer partials for the finalizing pass to add).
  return T >= 8192 ? 2 * kGateWaves : kGateWaves;
}

void launch_gate_topk(const float* logits, const float* select_bias, int T, int E, int k, int mode,
                      int32_t* topk_idx, float* topk_gate, float* part_p, float* part_l,
                      float* prob_sum, float* lse_sq_sum, hipStream_t s) {
  const int rpb = gate_rows_per_block(T);
  const int nblk = (T + rpb - 1) / rpb;
  float* pp = (prob_sum || lse_sq_sum) ? part_p : nullptr;
  const int epl = (E + 63) / 64;
#define MOE_GATE(n)                                                                          \
  hipLaunchKernelGGL((gate_topk_kernel<n>), dim3(nblk), dim3(64 * kGateWaves), 0, s, logits,     \
                     select_bias, T, E, k, mode, rpb, topk_idx, topk_gate, pp, part_l)
  if (epl <= 1) MOE_GATE(1);
  else if (epl <= 2) MOE_GATE(2);
  else if (epl <= 4) MOE_GATE(4);
  else if (epl <= 8) MOE_GATE(8);
  else MOE_GATE(16);
#undef MOE_GATE
  if (pp)
    hipLaunchKernelGGL(route_finalize_kernel, dim3((E + 1 + 3) / 4), dim3(256), 0, s, part_p,
                       part_l, nblk, E, prob_sum, lse_sq_sum);
}

size_t route_workspace_bytes(int T, int E) {
  const int rpb = gate_rows_per_block(T);
  const size_t nblk = (size_t)(T + rpb - 1) / rpb;
  return nblk * E * sizeof(float) + nblk * sizeof(float) + 256;
}

}  // namespace moe
