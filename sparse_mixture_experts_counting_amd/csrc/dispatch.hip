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

#include <mutex>

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
    // Chunks in groups of eight: the group's counts are loaded before any is replaced.
    constexpr int G8 = 8;
    for (int c0 = 0; c0 < nchunk; c0 += G8) {
      int v[G8];
#pragma unroll
      for (int j = 0; j < G8; ++j) v[j] = c0 + j < nchunk ? h[c0 + j] : 0;
#pragma unroll
      for (int j = 0; j < G8; ++j) {
        if (c0 + j < nchunk) h[c0 + j] = run;  // position of the chunk's first assignment to e
        run += v[j];
      }
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

// The three passes in one block of 1024 threads for at most one chunk of assignments (A <= 2048,
// decode-sized batches), where the launches, not the work, would set the time: the histogram and
// the scan as above with a single chunk (its first assignment to e is e's first), then the
// stable scatter by the first four waves exactly as dispatch_scatter_kernel ranks them (the other
// waves only take part in the barriers).  The same integers as the three-kernel path.
__global__ __launch_bounds__(1024) void dispatch_one_chunk_kernel(
    const int32_t* __restrict__ idx, int A, int E, int nbits, int capacity,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
    int32_t* __restrict__ inv, int32_t* __restrict__ n_dropped) {
  __shared__ int32_t h[1024];
  __shared__ int32_t sc[1024];
  __shared__ int32_t run[1024];
  const int tid = threadIdx.x;
  h[tid] = 0;
  run[tid] = 0;
  __syncthreads();
  for (int a = tid; a < A; a += 1024) {
    const int e = idx[a];
    if (e >= 0 && e < E) atomicAdd(&h[e], 1);
  }
  __syncthreads();
  int kept = 0;
  if (tid < E) {
    counts[tid] = h[tid];
    kept = (capacity > 0 && h[tid] > capacity) ? capacity : h[tid];
  }
  sc[tid] = kept;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int v = (tid >= o) ? sc[tid - o] : 0;
    __syncthreads();
    sc[tid] += v;
    __syncthreads();
  }
  const int off = sc[tid] - kept;   // exclusive prefix of kept at expert tid
  if (tid < E) offsets[tid] = off;
  if (tid == 0) {
    offsets[E] = sc[1023];
    n_dropped[0] = A - sc[1023];
  }
  __syncthreads();
  h[tid] = off;                     // h now holds each expert's first row
  __syncthreads();
  const bool scatter = tid < kThreads;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  for (int r0 = 0; r0 < A; r0 += kThreads) {
    const int a = r0 + tid;
    int e = -1;
    if (scatter && a < A) {
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
      if (capacity <= 0 || rank < capacity) {
        const int pos = h[e] + rank;
        perm[pos] = a;
        inv[a] = pos;
      } else {
        inv[a] = -1;
      }
    }
  }
}

// Up to kBlockA assignments (a prefill-sized batch) in one block of 16 waves, no workspace: wave w
// ranks the assignments of its contiguous segment (64 at a time, in order) among the segment's
// earlier ones to the same expert, counting per expert in its own LDS row; one thread per expert
// then turns the 16 rows into exclusive prefixes over the waves (so an assignment's rank in its
// expert's stream is its wave's prefix plus its rank in the segment), the counts, kept and
// offsets follow as in dispatch_scan_kernel, and every assignment is placed.  The same integers
// as the chunked path, in one launch instead of three.
static constexpr int kBlockA = 16384, kBlockWaves = 16, kBlockPer = kBlockA / (64 * kBlockWaves);

__global__ __launch_bounds__(1024) void dispatch_block_kernel(
    const int32_t* __restrict__ idx, int A, int E, int nbits, int capacity,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
    int32_t* __restrict__ inv, int32_t* __restrict__ n_dropped) {
  __shared__ int32_t cnt[kBlockWaves][1024];   // per wave, then the waves' exclusive prefixes
  __shared__ int32_t sc[1024];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < kBlockWaves * 1024; e += 1024) (&cnt[0][0])[e] = 0;
  __syncthreads();
  // The wave's segment: whole 64-assignment windows, in assignment order.
  const int per_wave = ((A + 63) / 64 + kBlockWaves - 1) / kBlockWaves;   // windows per wave
  const int a_beg = wave * per_wave * 64;
  int my_e[kBlockPer], my_rank[kBlockPer];
#pragma unroll
  for (int i = 0; i < kBlockPer; ++i) {
    my_e[i] = -1;
    my_rank[i] = 0;
    if (i >= per_wave) continue;                 // uniform over the wave
    const int a = a_beg + i * 64 + lane;
    int e = -1;
    if (a < A) {
      e = idx[a];
      if (e < 0 || e >= E) e = -1;
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
    if (valid) {
      const int run = cnt[wave][e];              // every lane reads before the leader writes
      my_rank[i] = run + below;
      if (below == 0) cnt[wave][e] = run + total;
    }
    my_e[i] = e;
  }
  __syncthreads();
  int kept = 0;
  if (tid < E) {
    int run = 0;
    for (int w = 0; w < kBlockWaves; ++w) {
      const int v = cnt[w][tid];
      cnt[w][tid] = run;
      run += v;
    }
    counts[tid] = run;
    kept = (capacity > 0 && run > capacity) ? capacity : run;
  }
  sc[tid] = kept;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int v = (tid >= o) ? sc[tid - o] : 0;
    __syncthreads();
    sc[tid] += v;
    __syncthreads();
  }
  if (tid < E) offsets[tid] = sc[tid] - kept;
  if (tid == 0) {
    offsets[E] = sc[1023];
    n_dropped[0] = A - sc[1023];
  }
  __syncthreads();
  if (tid < E) sc[tid] -= kept;                  // each expert's first row
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kBlockPer; ++i) {
    if (i >= per_wave) continue;
    const int a = a_beg + i * 64 + lane;
    if (a >= A) continue;
    const int e = my_e[i];
    if (e < 0) {
      inv[a] = -1;
      continue;
    }
    const int g = cnt[wave][e] + my_rank[i];
    if (capacity <= 0 || g < capacity) {
      const int pos = sc[e] + g;
      perm[pos] = a;
      inv[a] = pos;
    } else {
      inv[a] = -1;
    }
  }
}

size_t dispatch_workspace_bytes(int A, int E) {
  const size_t nchunk = (size_t)(A + kChunk - 1) / kChunk;
  return nchunk * E * sizeof(int32_t) + 256;
}

// Scratch of the entry point that allocates nothing (moe_dispatch_noalloc): the per-chunk
// histogram lives in this fixed device array instead of a caller's workspace.  Every call on one
// GPU uses that GPU's copy, so calls that overlap on a GPU race; the histogram pass overwrites
// every entry a call reads, so nothing needs clearing between calls.
static constexpr size_t kDispatchScratchBytes = 1u << 20;
static __device__ __align__(256) int32_t scratch[kDispatchScratchBytes / sizeof(int32_t)];

size_t dispatch_scratch_bytes() { return kDispatchScratchBytes; }

// Device address of this GPU's scratch, looked up on the first call on each device (with that
// device current) and kept.  In host code `scratch` names a host-side stand-in, never the device
// memory; only the address looked up here may be handed to kernels.  Returns nullptr when the
// lookup fails (the next call tries again).
int32_t* dispatch_scratch() {
  static std::mutex mu;
  static int32_t* ptr[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess) ptr[dev] = (int32_t*)p;
  }
  return ptr[dev];
}

void launch_dispatch(const int32_t* topk_idx, int A, int E, int capacity, int32_t* counts,
                     int32_t* offsets, int32_t* perm, int32_t* inv, int32_t* n_dropped,
                     int32_t* hist, hipStream_t s) {
  const int nchunk = (A + kChunk - 1) / kChunk;
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  if (nchunk == 1) {
    hipLaunchKernelGGL(dispatch_one_chunk_kernel, dim3(1), dim3(1024), 0, s, topk_idx, A, E,
                       nbits, capacity, counts, offsets, perm, inv, n_dropped);
    return;
  }
  if (A <= kBlockA) {
    hipLaunchKernelGGL(dispatch_block_kernel, dim3(1), dim3(1024), 0, s, topk_idx, A, E, nbits,
                       capacity, counts, offsets, perm, inv, n_dropped);
    return;
  }
  hipLaunchKernelGGL(dispatch_hist_kernel, dim3(nchunk), dim3(kThreads), 0, s, topk_idx, A, E,
                     nchunk, hist);
  hipLaunchKernelGGL(dispatch_scan_kernel, dim3(1), dim3(1024), 0, s, hist, E, nchunk, A, capacity,
                     counts, offsets, n_dropped);
  hipLaunchKernelGGL(dispatch_scatter_kernel, dim3(nchunk), dim3(kThreads), 0, s, topk_idx, A, E,
                     nbits, nchunk, capacity, hist, offsets, perm, inv);
}

}  // namespace moe
