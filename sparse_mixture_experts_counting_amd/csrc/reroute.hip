// Overflow rerouting: assignments past an expert's capacity go to the token's next-best expert
// instead of being dropped (the chipfoundry glossary entry on MoE, Architecture Components,
// Expert Capacity; "DL S077 - Mixture of Experts (MoE) Intuition" (dineshblog), section 3.2: or
// routed to their second choice).  Two rounds: round 1 is the ordinary capacity dispatch; in round 2
// the j-th overflowed slot of a token proposes the token's expert of rank k + j, and the proposals
// take the room the experts have left, in assignment order.
//   reroute_propose: per token, the proposals (ranks k.. by repeated arg-max in the order of the
//                    forward selection) and the gates of the final selection;
//   reroute_place:   per expert, which proposals fit (block-wide scan in assignment order);
//   reroute_offsets: kept rows per expert -> offsets;
//   reroute_scatter: per assignment, its row in the merged layout (round-1 rows of an expert first,
//                    then its round-2 rows, each in assignment order).
#include "common.h"
#include "kernels.h"

namespace moe {

// Ranking key of the forward selection: larger score first, -0 equal to +0, ties to the lower
// expert index (the caller breaks ties on the index).
__device__ __forceinline__ uint32_t rank_key(float f) {
  const uint32_t b = __float_as_uint(f == 0.0f ? 0.0f : f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// One wave per token; lane l holds experts l, l + 64, ... (E <= 1024).
__global__ __launch_bounds__(256) void reroute_propose_kernel(
    const float* __restrict__ logits, const float* __restrict__ select_bias,
    const int32_t* __restrict__ topk_idx, const float* __restrict__ topk_gate,
    const int32_t* __restrict__ inv, int T, int E, int k, int mode, int32_t* __restrict__ idx2,
    float* __restrict__ gate2, int32_t* __restrict__ proposal, int32_t* __restrict__ r2rank) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int lane = threadIdx.x & 63;
  const float* L = logits + (size_t)t * E;
  int n_over = 0;
  for (int s = 0; s < k; ++s) {
    const int a = t * k + s;
    const int e = topk_idx[a];
    if (inv[a] < 0 && e >= 0 && e < E) ++n_over;
  }
  if (n_over == 0) {
    for (int s = lane; s < k; s += 64) {
      const int a = t * k + s;
      idx2[a] = topk_idx[a];
      gate2[a] = topk_gate[a];
      proposal[a] = -1;
      r2rank[a] = -1;
    }
    return;
  }
  constexpr int PER = 16;                           // experts per lane (E <= 1024)
  uint32_t key[PER];
  bool taken[PER];
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int e = lane + 64 * q;
    taken[q] = e >= E;
    key[q] = 0;
    if (e < E) key[q] = rank_key(select_bias ? L[e] + select_bias[e] : L[e]);
  }
  // Ranks 0 .. k + n_over - 1; rank k + j goes to the j-th overflowed slot.
  int j = 0;
  const int ranks = min(E, k + n_over);
  for (int r = 0; r < ranks; ++r) {
    uint64_t best = 0;                               // (key << 32) | (E - 1 - e): max wins
#pragma unroll
    for (int q = 0; q < PER; ++q)
      if (!taken[q]) {
        const uint64_t c = ((uint64_t)key[q] << 32) | (uint32_t)(E - 1 - (lane + 64 * q));
        best = c > best ? c : best;
      }
    best = wave_max_u64(best);
    const int e = E - 1 - (int)(uint32_t)best;
#pragma unroll
    for (int q = 0; q < PER; ++q)
      if (lane + 64 * q == e) taken[q] = true;
    if (r >= k) {                                    // the j-th overflowed slot of the token
      int seen = 0;
      for (int s = 0; s < k; ++s) {
        const int a = t * k + s;
        const int e0 = topk_idx[a];
        if (inv[a] < 0 && e0 >= 0 && e0 < E) {
          if (seen == j && lane == 0) proposal[a] = e;
          ++seen;
        }
      }
      ++j;
    }
  }
  // Final selection: lane 0 walks the slots (an overflowed slot takes its proposal), and slot s's
  // expert goes to lane s.
  int my_e = 0, jj = 0;
  for (int s = 0; s < k; ++s) {
    int e = 0;
    if (lane == 0) {
      const int a = t * k + s;
      const int e0 = topk_idx[a];
      e = e0;
      if (inv[a] < 0 && e0 >= 0 && e0 < E) {
        if (k + jj < E) {
          e = proposal[a];
        } else {
          proposal[a] = -1;
        }
        ++jj;
      } else {
        proposal[a] = -1;
      }
      idx2[a] = e;
      r2rank[a] = -1;
    }
    e = __shfl(e, 0, 64);
    if (lane == s) my_e = e;
  }
  // The gates of the final selection, with the numerics of moe_route's gating: softmax over the
  // selected and the renormalised sigmoids are shifted by the largest selected logit v0 (in
  // log-sigmoid form for the latter), so they stay finite however far the selected logits lie
  // below the row maximum or below zero; softmax over all E uses the row maximum and its sum.
  const float my_v = lane < k ? L[my_e] : -INFINITY;
  float g;
  if (mode == 1) {
    float m = -INFINITY;
    for (int e = lane; e < E; e += 64) m = fmaxf(m, L[e]);
    m = wave_max(m);
    float zall = 0.f;
    for (int e = lane; e < E; e += 64) zall += expf(L[e] - m);
    zall = wave_sum(zall);
    g = expf(my_v - m) * (1.0f / zall);
  } else {
    const float v0 = wave_max(my_v);
    float w = 0.f;
    if (lane < k) w = mode == 0 ? expf(my_v - v0) : expf(log_sigmoid(my_v) - log_sigmoid(v0));
    g = w / wave_sum(w);
  }
  if (lane < k) gate2[t * k + lane] = g;
}

constexpr int kRrThreads = 1024;

__device__ __forceinline__ int rr_block_excl_scan(bool flag, int* s_wave, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t bal = __ballot(flag);
  const int in_wave = __popcll(bal & lanemask_lt());
  if (lane == 0) s_wave[wave] = __popcll(bal);
  __syncthreads();
  int before = 0, sum = 0;
  for (int w = 0; w < kRrThreads / 64; ++w) {
    const int c = s_wave[w];
    if (w < wave) before += c;
    sum += c;
  }
  __syncthreads();
  total = sum;
  return before + in_wave;
}

// One block per expert: the proposals for it, in assignment order, take its remaining room.
__global__ __launch_bounds__(kRrThreads) void reroute_place_kernel(
    const int32_t* __restrict__ proposal, const int32_t* __restrict__ offsets1, int A, int C,
    int32_t* __restrict__ r2rank, int32_t* __restrict__ kept2) {
  __shared__ int s_wave[kRrThreads / 64];
  const int e = blockIdx.x;
  const int room = max(0, C - (offsets1[e + 1] - offsets1[e]));
  int before = 0;
  for (int base = 0; base < A; base += kRrThreads) {
    const int a = base + threadIdx.x;
    const bool mine = a < A && proposal[a] == e;
    int n;
    const int rank = before + rr_block_excl_scan(mine, s_wave, n);
    if (mine && rank < room) r2rank[a] = rank;
    before += n;
  }
  if (threadIdx.x == 0) kept2[e] = min(before, room);
}

// Single block: offsets2 = exclusive prefix sum of round-1 + round-2 rows; n_dropped.
__global__ __launch_bounds__(kRrThreads) void reroute_offsets_kernel(
    const int32_t* __restrict__ offsets1, const int32_t* __restrict__ kept2, int E, int A,
    int32_t* __restrict__ offsets2, int32_t* __restrict__ n_dropped) {
  __shared__ int s_val[kRrThreads];
  __shared__ int s_carry;
  if (threadIdx.x == 0) s_carry = 0;
  __syncthreads();
  for (int base = 0; base < E; base += kRrThreads) {
    const int e = base + threadIdx.x;
    const int v = e < E ? (offsets1[e + 1] - offsets1[e]) + kept2[e] : 0;
    s_val[threadIdx.x] = v;
    __syncthreads();
    for (int o = 1; o < kRrThreads; o <<= 1) {     // inclusive Hillis-Steele scan
      const int add = threadIdx.x >= o ? s_val[threadIdx.x - o] : 0;
      __syncthreads();
      s_val[threadIdx.x] += add;
      __syncthreads();
    }
    const int carry = s_carry;
    if (e < E) offsets2[e] = carry + s_val[threadIdx.x] - v;
    __syncthreads();
    if (threadIdx.x == kRrThreads - 1) s_carry = carry + s_val[kRrThreads - 1];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    offsets2[E] = s_carry;
    n_dropped[0] = A - s_carry;
  }
}

__global__ __launch_bounds__(256) void reroute_scatter_kernel(
    const int32_t* __restrict__ topk_idx, const int32_t* __restrict__ inv1,
    const int32_t* __restrict__ offsets1, const int32_t* __restrict__ proposal,
    const int32_t* __restrict__ r2rank, const int32_t* __restrict__ offsets2, int A, int E,
    int32_t* __restrict__ perm2, int32_t* __restrict__ inv2) {
  const int a = blockIdx.x * 256 + threadIdx.x;
  if (a >= A) return;
  int row = -1;
  const int e1 = topk_idx[a];
  if (inv1[a] >= 0 && e1 >= 0 && e1 < E) {
    row = offsets2[e1] + (inv1[a] - offsets1[e1]);
  } else if (r2rank[a] >= 0) {
    const int e2 = proposal[a];
    row = offsets2[e2] + (offsets1[e2 + 1] - offsets1[e2]) + r2rank[a];
  }
  inv2[a] = row;
  if (row >= 0) perm2[row] = a;
}

size_t reroute_workspace_bytes(int A, int E) { return ((size_t)2 * A + E) * sizeof(int32_t); }

void launch_reroute(const float* logits, const float* select_bias, const int32_t* topk_idx,
                    const float* topk_gate, const int32_t* offsets1, const int32_t* inv1, int T,
                    int E, int k, int capacity, int mode, int32_t* idx2, float* gate2,
                    int32_t* offsets2, int32_t* perm2, int32_t* inv2, int32_t* n_dropped,
                    int32_t* ws, hipStream_t s) {
  const int A = T * k;
  int32_t* proposal = ws;
  int32_t* r2rank = ws + A;
  int32_t* kept2 = ws + 2 * A;
  const int C = capacity > 0 ? capacity : A;
  hipLaunchKernelGGL(reroute_propose_kernel, dim3((T + 3) / 4), dim3(256), 0, s, logits,
                     select_bias, topk_idx, topk_gate, inv1, T, E, k, mode, idx2, gate2, proposal,
                     r2rank);
  hipLaunchKernelGGL(reroute_place_kernel, dim3(E), dim3(kRrThreads), 0, s, proposal, offsets1, A,
                     C, r2rank, kept2);
  hipLaunchKernelGGL(reroute_offsets_kernel, dim3(1), dim3(kRrThreads), 0, s, offsets1, kept2, E,
                     A, offsets2, n_dropped);
  hipLaunchKernelGGL(reroute_scatter_kernel, dim3((A + 255) / 256), dim3(256), 0, s, topk_idx,
                     inv1, offsets1, proposal, r2rank, offsets2, A, E, perm2, inv2);
}

}  // namespace moe
