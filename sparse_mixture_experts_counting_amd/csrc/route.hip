// Router product (few experts), gating + top-k, and the deterministic reduction of the loss
// partials.  The method is the Score and Select steps of the page "Mixture of experts (MoE)"
// (tirogla), How it works steps 1-2 and its Code `route`; gating modes as listed there.
#include "common.h"
#include "kernels.h"

#include <math.h>

namespace moe {

// ---------------------------------------------------------------------------------------------
// Router product for E <= 16 experts: logits[t, e] = sum_j x[t, j] w_r[e, j] (+ bias[e]), W_r in
// the [E][d] layout of a linear layer.  Memory bound on x; one wave handles TPW tokens, lanes
// stride over 8-wide slices of d, and each lane reads the matching 8 values of every W_r row
// (16-byte aligned: d is a multiple of 8).
// ---------------------------------------------------------------------------------------------
template <typename TIn, int E, int TPW>
__global__ __launch_bounds__(256) void router_small_e_kernel(const TIn* __restrict__ x,
                                                             const TIn* __restrict__ w_r,
                                                             const float* __restrict__ bias, int T,
                                                             int d, float* __restrict__ logits) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int t0 = (blockIdx.x * 4 + wave) * TPW;
  if (t0 >= T) return;
  float acc[TPW][E];
#pragma unroll
  for (int i = 0; i < TPW; ++i)
#pragma unroll
    for (int e = 0; e < E; ++e) acc[i][e] = 0.f;

  const int nchunk = d >> 3;
  for (int c = lane; c < nchunk; c += 64) {
    float w[E][8];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if constexpr (sizeof(TIn) == 2) {
        unpack8(*reinterpret_cast<const u32x4*>(w_r + (size_t)e * d + c * 8), w[e]);
      } else {
        const f32x4* src = reinterpret_cast<const f32x4*>(w_r + (size_t)e * d + c * 8);
        const f32x4 a = src[0], b = src[1];
        w[e][0] = a[0]; w[e][1] = a[1]; w[e][2] = a[2]; w[e][3] = a[3];
        w[e][4] = b[0]; w[e][5] = b[1]; w[e][6] = b[2]; w[e][7] = b[3];
      }
    }
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int t = t0 + i;
      if (t < T) {
        float xv[8];
        if constexpr (sizeof(TIn) == 2) {
          u32x4 q = *reinterpret_cast<const u32x4*>(x + (size_t)t * d + c * 8);
          unpack8(q, xv);
        } else {
          const f32x4* p = reinterpret_cast<const f32x4*>(x + (size_t)t * d + c * 8);
          f32x4 a = p[0], b = p[1];
          xv[0] = a[0]; xv[1] = a[1]; xv[2] = a[2]; xv[3] = a[3];
          xv[4] = b[0]; xv[5] = b[1]; xv[6] = b[2]; xv[7] = b[3];
        }
#pragma unroll
        for (int kk = 0; kk < 8; ++kk)
#pragma unroll
          for (int e = 0; e < E; ++e) acc[i][e] = fmaf(xv[kk], w[e][kk], acc[i][e]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < TPW; ++i)
#pragma unroll
    for (int e = 0; e < E; ++e) acc[i][e] = wave_sum(acc[i][e]);
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int t = t0 + i;
      if (t < T) {
#pragma unroll
        for (int e = 0; e < E; ++e) logits[(size_t)t * E + e] = acc[i][e] + (bias ? bias[e] : 0.f);
      }
    }
  }
}

template <typename TIn, int E>
static void launch_router_small_e_t(const void* x, const void* w_r, const float* bias, int T,
                                    int d, float* logits, hipStream_t s) {
  constexpr int TPW = 4;
  const int blocks = (T + 4 * TPW - 1) / (4 * TPW);
  hipLaunchKernelGGL((router_small_e_kernel<TIn, E, TPW>), dim3(blocks), dim3(256), 0, s,
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

void launch_router_small_e(const void* x, const void* w_r, const float* bias, int T, int d, int E,
                           bool bf16, float* logits, hipStream_t s) {
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
// Selection ranks on an integer key built from the float32 logit so that -0.0 == +0.0 and equal
// logits go to the lower expert index: key = (order-preserving bits of the logit) << 32 | ~e.
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ uint32_t ordered_bits(float v) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;  // -0.0 -> +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float from_ordered_bits(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o ^ 0x80000000u) : ~o);
}
// log(sigmoid(v)) = min(v, 0) - log1p(exp(-|v|)), finite for every finite v.
__device__ __forceinline__ float log_sigmoid(float v) {
  return fminf(v, 0.f) - log1pf(expf(-fabsf(v)));
}

template <int EPL>
__global__ __launch_bounds__(256) void gate_topk_kernel(const float* __restrict__ logits, int T,
                                                        int E, int k, int mode, int rows_per_block,
                                                        int32_t* __restrict__ topk_idx,
                                                        float* __restrict__ topk_gate,
                                                        float* __restrict__ part_p,
                                                        float* __restrict__ part_l) {
  __shared__ float red_p[4][1024];
  __shared__ float red_l[4];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int row0 = blockIdx.x * rows_per_block;
  const int row1 = min(T, row0 + rows_per_block);

  float acc_p[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) acc_p[i] = 0.f;
  float acc_l = 0.f;

  for (int t = row0 + wave; t < row1; t += 4) {
    const float* row = logits + (size_t)t * E;
    float v[EPL];
    uint64_t key[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = lane + 64 * i;
      if (e < E) {
        v[i] = row[e];
        key[i] = ((uint64_t)ordered_bits(v[i]) << 32) | (uint32_t)(~e);
      } else {
        v[i] = -INFINITY;
        key[i] = 0ull;
      }
    }
    // Full-row softmax (for P_e) and logsumexp (for the z-loss).
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < EPL; ++i) m = fmaxf(m, v[i]);
    m = wave_max(m);
    float ex[EPL];
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      ex[i] = (lane + 64 * i < E) ? expf(v[i] - m) : 0.f;
      s += ex[i];
    }
    s = wave_sum(s);
    const float inv_s = 1.0f / s;
#pragma unroll
    for (int i = 0; i < EPL; ++i) acc_p[i] += ex[i] * inv_s;
    const float lse = m + logf(s);
    acc_l += lse * lse;

    // Top-k by repeated wave arg-max over the keys.
    int my_e = 0;
    float my_v = 0.f;
    float v0 = 0.f;
    for (int j = 0; j < k; ++j) {
      uint64_t best = key[0];
#pragma unroll
      for (int i = 1; i < EPL; ++i) best = key[i] > best ? key[i] : best;
      best = wave_max_u64(best);
      const int e_j = (int)(~(uint32_t)best);
      const float v_j = from_ordered_bits((uint32_t)(best >> 32));
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (lane + 64 * i == e_j) key[i] = 0ull;
      if (j == 0) v0 = v_j;
      if (lane == j) {
        my_e = e_j;
        my_v = v_j;
      }
    }
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
    if (mode != 1) g = w / wave_sum(w);
    if (lane < k) {
      topk_idx[(size_t)t * k + lane] = my_e;
      topk_gate[(size_t)t * k + lane] = g;
    }
  }

  if (part_p) {
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = lane + 64 * i;
      if (e < E) red_p[wave][e] = acc_p[i];
    }
    if (lane == 0) red_l[wave] = acc_l;
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += 256)
      part_p[(size_t)blockIdx.x * E + e] = ((red_p[0][e] + red_p[1][e]) + red_p[2][e]) + red_p[3][e];
    if (threadIdx.x == 0) part_l[blockIdx.x] = ((red_l[0] + red_l[1]) + red_l[2]) + red_l[3];
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
  // Enough blocks to cover the chip for large T, few partials for small T.
  if (T >= 8192) return 32;
  if (T >= 1024) return 16;
  return 8;
}

void launch_gate_topk(const float* logits, int T, int E, int k, int mode, int32_t* topk_idx,
                      float* topk_gate, float* part_p, float* part_l, float* prob_sum,
                      float* lse_sq_sum, hipStream_t s) {
  const int rpb = gate_rows_per_block(T);
  const int nblk = (T + rpb - 1) / rpb;
  float* pp = (prob_sum || lse_sq_sum) ? part_p : nullptr;
  const int epl = (E + 63) / 64;
#define MOE_GATE(n)                                                                          \
  hipLaunchKernelGGL((gate_topk_kernel<n>), dim3(nblk), dim3(256), 0, s, logits, T, E, k, mode, \
                     rpb, topk_idx, topk_gate, pp, part_l)
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
