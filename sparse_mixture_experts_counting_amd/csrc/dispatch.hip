// Dispatch: a stable counting sort of the T*k assignments by expert with capacity C, overflow
// dropped in assignment order (the page "Mixture of experts (MoE)" (tirogla), How it works step 3
// and Code `dispatch`).
//
// Three passes over fixed chunks of CHUNK assignments:
//   1. per-chunk histogram (LDS atomics; order does not matter for counts) -> hist[e][chunk]
//   2. one block: per expert, exclusive scan over chunks (stream position of each chunk's first
//      assignment to e), counts, kept = min(counts, C), offsets = exclusive scan of kept
//   3. per chunk: stable rank of every assignment among the chunk's earlier assignments to the
//      same expert (wave ballots + a wave-ordered LDS running count), then the global rank decides
//      kept / dropped and the kept ones are scattered to perm / inv.
// Everything is integer arithmetic in a fixed order, so the result is bitwise deterministic.
#include "common.h"
#include "kernels.h"

namespace moe {

static constexpr int kChunk = 2048;   // assignments per block
static constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void dispatch_hist_kernel(const int32_t* __restrict__ idx,
                                                                 int A, int E, int nchunk,
                                                                 int32_t* __restrict__ hist) {
  __shared__ int32_t h[1024];
  for (int e = threadIdx.x; e < E; e += kThreads) h[e] = 0;
  __syncthreads();
  const int a0 = blockIdx.x * kChunk;
  const int a1 = min(A, a0 + kChunk);
  for (int a = a0 + threadIdx.x; a < a1; a += kThreads) {
    const int e = idx[a];
    if (e >= 0 && e < E) atomicAdd(&h[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kThreads) hist[(size_t)e * nchunk + blockIdx.x] = h[e];
}

// One block of 1024 threads; thread e owns expert e.
__global__ __launch_bounds__(1024) void dispatch_scan_kernel(int32_t* __restrict__ hist, int E,
                                                             int nchunk, int A, int capacity,
                                                             int32_t* __restrict__ counts,
                                                             int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ n_dropped) {
  __shared__ int32_t sc[1024];
  const int e = threadIdx.x;
  int kept = 0;
  if (e < E) {
    int32_t* h = hist + (size_t)e * nchunk;
    int run = 0;
    for (int c = 0; c < nchunk; ++c) {
      const int v = h[c];
      h[c] = run;  // position of chunk c's first assignment to e in e's stream
      run += v;
    }
    counts[e] = run;
    kept = (capacity > 0 && run > capacity) ? capacity : run;
  }
  sc[e] = kept;
  __syncthreads();
  // Inclusive Hillis-Steele scan over 1024 entries.
  for (int o = 1; o < 1024; o <<= 1) {
    const int v = (e >= o) ? sc[e - o] : 0;
    __syncthreads();
    sc[e] += v;
    __syncthreads();
  }
  if (e < E) offsets[e] = sc[e] - kept;
  if (e == 0) {
    offsets[E] = sc[1023];
    n_dropped[0] = A - sc[1023];
  }
}

__global__ __launch_bounds__(kThreads) void dispatch_scatter_kernel(
    const int32_t* __restrict__ idx, int A, int E, int nbits, int nchunk, int capacity,
    const int32_t* __restrict__ base /* [E][nchunk] */, const int32_t* __restrict__ offsets,
    int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
  __shared__ int32_t run[1024];
  for (int e = threadIdx.x; e < E; e += kThreads) run[e] = 0;
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int a0 = blockIdx.x * kChunk;
  const int a1 = min(A, a0 + kChunk);
  for (int r0 = a0; r0 < a1; r0 += kThreads) {
    const int a = r0 + threadIdx.x;
    int e = -1;
    if (a < a1) {
      e = idx[a];
      if (e < 0 || e >= E) {
        inv[a] = -1;
        e = -1;
      }
    }
    const bool valid = e >= 0;
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = valid && ((e >> b) & 1);
      const uint64_t m = __ballot(bit);
      peers &= bit ? m : ~m;
    }
    const int below = __popcll(peers & lanemask_lt());
    const int total = __popcll(peers);
    int rank = 0;
    for (int w = 0; w < kThreads / 64; ++w) {
      if (wave == w && valid) {
        const int b = run[e];
        rank = b + below;
        if (below == 0) run[e] = b + total;
      }
      __syncthreads();
    }
    if (valid) {
      const int g = base[(size_t)e * nchunk + blockIdx.x] + rank;
      if (capacity <= 0 || g < capacity) {
        const int pos = offsets[e] + g;
        perm[pos] = a;
        inv[a] = pos;
      } else {
        inv[a] = -1;
      }
    }
  }
}

size_t dispatch_workspace_bytes(int A, int E) {
  const size_t nchunk = (size_t)(A + kChunk - 1) / kChunk;
  return nchunk * E * sizeof(int32_t) + 256;
}

void launch_dispatch(const int32_t* topk_idx, int A, int E, int capacity, int32_t* counts,
                     int32_t* offsets, int32_t* perm, int32_t* inv, int32_t* n_dropped,
                     int32_t* hist, hipStream_t s) {
  const int nchunk = (A + kChunk - 1) / kChunk;
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  hipLaunchKernelGGL(dispatch_hist_kernel, dim3(nchunk), dim3(kThreads), 0, s, topk_idx, A, E,
                     nchunk, hist);
  hipLaunchKernelGGL(dispatch_scan_kernel, dim3(1), dim3(1024), 0, s, hist, E, nchunk, A, capacity,
                     counts, offsets, n_dropped);
  hipLaunchKernelGGL(dispatch_scatter_kernel, dim3(nchunk), dim3(kThreads), 0, s, topk_idx, A, E,
                     nbits, nchunk, capacity, hist, offsets, perm, inv);
}

}  // namespace moe
