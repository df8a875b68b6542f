// Expert Choice routing: each expert takes the C tokens with the largest router probability (the
// page "Mixture of Experts (MoE)" (starphix), Router Variants; the chipfoundry glossary entry on
// MoE, Routing Strategies and Variants: experts select their top tokens, so every expert gets the
// same load).
//   ec_scores: p[t, e] = softmax over experts of logits row t (fp32).
//   ec_select: per expert, the exact C-th largest score by a 4-pass MSB radix select over the
//              order-preserving integer image of the scores, then a block-wide compaction in token
//              order that keeps every score above it and the lowest-index tokens among the equal
//              ones; rows of an expert are listed in increasing token order.
#include "common.h"
#include "kernels.h"

namespace moe {

// One wave per row.
__global__ __launch_bounds__(256) void ec_scores_kernel(const float* __restrict__ logits, int T,
                                                        int E, float* __restrict__ scores) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int lane = threadIdx.x & 63;
  const float* L = logits + (size_t)t * E;
  float m = -INFINITY;
  for (int e = lane; e < E; e += 64) m = fmaxf(m, L[e]);
  m = wave_max(m);
  float s = 0.f;
  for (int e = lane; e < E; e += 64) s += expf(L[e] - m);
  s = wave_sum(s);
  const float inv = 1.0f / s;
  for (int e = lane; e < E; e += 64) scores[(size_t)t * E + e] = expf(L[e] - m) * inv;
}

// Order-preserving image of a float as an unsigned integer (larger float, larger integer).
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t b = __float_as_uint(f == 0.0f ? 0.0f : f);   // -0 ranks as +0
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

constexpr int kEcThreads = 1024;

// Exclusive block-wide prefix sum of a 0/1 flag; returns this thread's prefix and the block total.
__device__ __forceinline__ int block_excl_scan(bool flag, int* s_wave, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t bal = __ballot(flag);
  const int in_wave = __popcll(bal & lanemask_lt());
  if (lane == 0) s_wave[wave] = __popcll(bal);
  __syncthreads();
  int before = 0, sum = 0;
  for (int w = 0; w < kEcThreads / 64; ++w) {
    const int c = s_wave[w];
    if (w < wave) before += c;
    sum += c;
  }
  __syncthreads();
  total = sum;
  return before + in_wave;
}

__global__ __launch_bounds__(kEcThreads) void ec_select_kernel(const float* __restrict__ S, int T,
                                                               int E, int C,
                                                               int32_t* __restrict__ offsets,
                                                               int32_t* __restrict__ perm,
                                                               float* __restrict__ gate,
                                                               int32_t* __restrict__ slot) {
  __shared__ int hist[256];
  __shared__ int s_wave[kEcThreads / 64];
  __shared__ uint32_t s_prefix;
  __shared__ int s_need;
  const int e = blockIdx.x;
  const int c = min(C, T);
  if (threadIdx.x == 0) {
    offsets[e] = e * c;
    if (e == E - 1) offsets[E] = E * c;
  }
  uint32_t thr = 0;                        // C-th largest key
  int need = 0;                            // keys equal to thr to take, lowest token index first
  if (c < T) {
    uint32_t prefix = 0, mask = 0;
    int remaining = c;
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      for (int i = threadIdx.x; i < 256; i += kEcThreads) hist[i] = 0;
      __syncthreads();
      for (int t = threadIdx.x; t < T; t += kEcThreads) {
        const uint32_t k = order_key(S[(size_t)t * E + e]);
        if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & 255], 1);
      }
      __syncthreads();
      if (threadIdx.x == 0) {
        int cum = 0, b = 255;
        for (; b > 0; --b) {
          if (cum + hist[b] >= remaining) break;
          cum += hist[b];
        }
        s_prefix = prefix | ((uint32_t)b << shift);
        s_need = remaining - cum;
      }
      __syncthreads();
      prefix = s_prefix;
      remaining = s_need;
      mask |= 255u << shift;
      __syncthreads();
    }
    thr = prefix;
    need = remaining;
  }
  int ties_before = 0, sel_before = 0;
  for (int base = 0; base < T; base += kEcThreads) {
    const int t = base + threadIdx.x;
    float v = 0.f;
    uint32_t k = 0;
    if (t < T) {
      v = S[(size_t)t * E + e];
      k = order_key(v);
    }
    const bool live = t < T;
    const bool gt = live && (c >= T || k > thr);
    const bool eq = live && c < T && k == thr;
    int n_eq;
    const int eq_rank = ties_before + block_excl_scan(eq, s_wave, n_eq);
    const bool sel = gt || (eq && eq_rank < need);
    int n_sel;
    const int pos = sel_before + block_excl_scan(sel, s_wave, n_sel);
    if (live) {
      const int r = e * c + pos;
      slot[(size_t)t * E + e] = sel ? r : -1;
      if (sel) {
        perm[r] = t;
        gate[r] = v;
      }
    }
    ties_before += n_eq;
    sel_before += n_sel;
  }
}

void launch_expert_choice(const float* logits, int T, int E, int C, bool scores_in, float* scores,
                          int32_t* offsets, int32_t* perm, float* gate, int32_t* slot,
                          hipStream_t s) {
  if (!scores_in)
    hipLaunchKernelGGL(ec_scores_kernel, dim3((T + 3) / 4), dim3(256), 0, s, logits, T, E, scores);
  hipLaunchKernelGGL(ec_select_kernel, dim3(E), dim3(kEcThreads), 0, s, scores, T, E, C, offsets,
                     perm, gate, slot);
}

}  // namespace moe
