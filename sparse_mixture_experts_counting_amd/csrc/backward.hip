// Backward pass of the layer: the non-GEMM steps.  The objective is J = <dy, y> + L_aux + z (a task
// loss whose gradient with respect to y is dy, plus the load-balancing and z losses of the page
// "Mixture of experts (MoE)" (tirogla), How it works step 6, which also states that the routed
// fraction f carries no gradient while the mean probability P does).
//   combine_backward: d_out[r] = gate[t,s] * dy[t] for the kept row r of assignment t*k+s, and
//                     d_gate[t,s] = <dy[t], out[r]> (0 for a dropped assignment);
//   gate_backward:    d_logits from d_gate through the gating function, plus the L_aux and z terms;
//   router_wgrad:     dW_r[e][j] = sum_t d_logits[t][e] x[t][j] (fp32 partials over token chunks,
//                     added in chunk order);
//   router_xgrad:     dx[t][j] = sum_e d_logits[t][e] W_r[e][j] (+ an added input).
#include "common.h"
#include "kernels.h"

#include <algorithm>

namespace moe {

// One block per token; 16-byte column chunks per thread; one pass over the token's slots.
__global__ __launch_bounds__(256) void combine_backward_kernel(
    const uint16_t* __restrict__ dy, const uint16_t* __restrict__ out,
    const int32_t* __restrict__ inv, const float* __restrict__ gate, int T, int d, int k,
    uint16_t* __restrict__ d_out, float* __restrict__ d_gate) {
  __shared__ float red[32][8];
  const int t = blockIdx.x;
  const int nchunk = d / 8;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, nw = blockDim.x >> 6;
  for (int s = 0; s < k; ++s) {
    const int r = inv[(size_t)t * k + s];
    if (r < 0) {                          // uniform over the block
      if (threadIdx.x == 0) d_gate[(size_t)t * k + s] = 0.f;
      continue;
    }
    const float g = gate[(size_t)t * k + s];
    float dot = 0.f;
    for (int c = threadIdx.x; c < nchunk; c += blockDim.x) {
      float a[8], b[8];
      unpack8(*reinterpret_cast<const u32x4*>(dy + (size_t)t * d + c * 8), a);
      unpack8(*reinterpret_cast<const u32x4*>(out + (size_t)r * d + c * 8), b);
      u32x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        o[i] = pack_bf16x2(g * a[2 * i], g * a[2 * i + 1]);
        dot = fmaf(a[2 * i], b[2 * i], dot);
        dot = fmaf(a[2 * i + 1], b[2 * i + 1], dot);
      }
      *reinterpret_cast<u32x4*>(d_out + (size_t)r * d + c * 8) = o;
    }
    dot = wave_sum(dot);
    if (lane == 0) red[s & 31][wave] = dot;
    __syncthreads();
    if (threadIdx.x == 0) {
      float v = 0.f;
      for (int w = 0; w < nw; ++w) v += red[s & 31][w];
      d_gate[(size_t)t * k + s] = v;
    }
    __syncthreads();
  }
}

void launch_combine_backward(const void* dy, const void* out, const int32_t* inv,
                             const float* gate, int T, int d, int k, void* d_out, float* d_gate,
                             hipStream_t s) {
  int threads = 64;
  while (threads < 256 && threads * 8 < d) threads *= 2;
  hipLaunchKernelGGL(combine_backward_kernel, dim3(T), dim3(threads), 0, s, (const uint16_t*)dy,
                     (const uint16_t*)out, inv, gate, T, d, k, (uint16_t*)d_out, d_gate);
}

// One wave per token row; lane j handles experts j, j + 64, ...  Per row, with p the full softmax
// and lse its log-normaliser (recomputed from the fp32 logits):
//   gates  SOFTMAX_TOPK: dL[e_s] += g_s (dg_s - sum g dg)
//          SOFTMAX_ALL:  dL[j]   += p_j (dp_j - sum p dp), dp = dg on the selected experts
//          SIGMOID_TOPK: dL[e_s] += sig'(L) (dg_s - sum g dg) / sum sig(L_sel)
//   L_aux: dL[j] += p_j (c_j - sum_e p_e c_e), c_e = alpha E f_e / T, f_e = counts_e / (T k)
//   z:     dL[j] += 2 beta lse p_j / T
// g_s are the forward gates (topk_gate).
__global__ __launch_bounds__(256) void gate_backward_kernel(
    const float* __restrict__ logits, const int32_t* __restrict__ topk_idx,
    const float* __restrict__ topk_gate, const float* __restrict__ d_gate,
    const int32_t* __restrict__ counts, int T, int E, int k, int mode, float alpha, float beta,
    float* __restrict__ d_logits) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int lane = threadIdx.x & 63;
  const float* L = logits + (size_t)t * E;
  float m = -INFINITY;
  for (int e = lane; e < E; e += 64) m = fmaxf(m, L[e]);
  m = wave_max(m);
  float z = 0.f;
  for (int e = lane; e < E; e += 64) z += __expf(L[e] - m);
  z = wave_sum(z);
  const float lse = m + __logf(z);
  const float cscale = alpha * (float)E / ((float)T * (float)k * (float)T);
  float pc = 0.f;                         // sum_e p_e c_e
  if (counts)
    for (int e = lane; e < E; e += 64) pc += __expf(L[e] - lse) * cscale * (float)counts[e];
  pc = wave_sum(pc);
  // sum over the selected of g dg (softmax-topk, sigmoid) or p dg (softmax-all)
  float sgd = 0.f, ssig = 0.f;
  for (int s = 0; s < k; ++s) {
    const int e = topk_idx[(size_t)t * k + s];
    const float dg = d_gate[(size_t)t * k + s];
    if (mode == 1)
      sgd += __expf(L[e] - lse) * dg;
    else
      sgd += topk_gate[(size_t)t * k + s] * dg;
    if (mode == 2) ssig += 1.0f / (1.0f + __expf(-L[e]));
  }
  const float zc = 2.0f * beta * lse / (float)T;
  for (int e = lane; e < E; e += 64) {
    const float p = __expf(L[e] - lse);
    const float c = counts ? cscale * (float)counts[e] : 0.f;
    float v = p * (c - pc) + zc * p;
    for (int s = 0; s < k; ++s) {
      if (topk_idx[(size_t)t * k + s] != e) continue;
      const float dg = d_gate[(size_t)t * k + s];
      if (mode == 0) {
        v += topk_gate[(size_t)t * k + s] * (dg - sgd);
      } else if (mode == 1) {
        v += p * dg;
      } else {
        const float sg = 1.0f / (1.0f + __expf(-L[e]));
        v += sg * (1.0f - sg) * (dg - sgd) / ssig;
      }
    }
    if (mode == 1) v -= p * sgd;
    d_logits[(size_t)t * E + e] = v;
  }
}

void launch_gate_backward(const float* logits, const int32_t* topk_idx, const float* topk_gate,
                          const float* d_gate, const int32_t* counts, int T, int E, int k, int mode,
                          float alpha, float beta, float* d_logits, hipStream_t s) {
  hipLaunchKernelGGL(gate_backward_kernel, dim3((T + 3) / 4), dim3(256), 0, s, logits, topk_idx,
                     topk_gate, d_gate, counts, T, E, k, mode, alpha, beta, d_logits);
}

// dW_r partials: block (j-tile of 256 columns, e-tile of 32 experts, token chunk); thread j keeps
// 32 fp32 sums over its chunk's tokens, reading d_logits of the chunk from LDS.
constexpr int kWgradE = 32, kWgradTok = 64;

template <bool BF16>
__global__ __launch_bounds__(256) void router_wgrad_kernel(const void* __restrict__ x,
                                                           const float* __restrict__ dL, int T,
                                                           int d, int E, int chunk,
                                                           float* __restrict__ part) {
  __shared__ float sd[kWgradTok][kWgradE];
  const int j = blockIdx.x * 256 + threadIdx.x;
  const int e0 = blockIdx.y * kWgradE;
  const int t_beg = blockIdx.z * chunk, t_end = min(T, t_beg + chunk);
  float acc[kWgradE];
#pragma unroll
  for (int i = 0; i < kWgradE; ++i) acc[i] = 0.f;
  for (int t0 = t_beg; t0 < t_end; t0 += kWgradTok) {
    __syncthreads();
    for (int q = threadIdx.x; q < kWgradTok * kWgradE; q += 256) {
      const int tt = q / kWgradE, ee = q % kWgradE;
      const int t = t0 + tt, e = e0 + ee;
      sd[tt][ee] = (t < t_end && e < E) ? dL[(size_t)t * E + e] : 0.f;
    }
    __syncthreads();
    if (j < d) {
      const int nt = min(kWgradTok, t_end - t0);
      for (int tt = 0; tt < nt; ++tt) {
        const size_t o = (size_t)(t0 + tt) * d + j;
        const float xv = BF16 ? bf16_to_f32(((const uint16_t*)x)[o]) : ((const float*)x)[o];
#pragma unroll
        for (int i = 0; i < kWgradE; ++i) acc[i] = fmaf(sd[tt][i], xv, acc[i]);
      }
    }
  }
  if (j < d) {
#pragma unroll
    for (int i = 0; i < kWgradE; ++i)
      if (e0 + i < E) part[((size_t)blockIdx.z * E + e0 + i) * d + j] = acc[i];
  }
}

__global__ __launch_bounds__(256) void sum_chunks_kernel(const float* __restrict__ part, int n,
                                                         int nchunk, float* __restrict__ out) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < (size_t)n;
       i += (size_t)gridDim.x * 256) {
    float v = 0.f;
    for (int c = 0; c < nchunk; ++c) v += part[(size_t)c * n + i];
    out[i] = v;
  }
}

int router_wgrad_chunks(int T) {
  int chunk = kWgradTok;
  while ((T + chunk - 1) / chunk > 16) chunk *= 2;
  return (T + chunk - 1) / chunk;
}

void launch_router_wgrad(const void* x, bool bf16, const float* dL, int T, int d, int E,
                         float* part, float* dw, hipStream_t s) {
  const int nchunk = router_wgrad_chunks(T);
  const int chunk = (T + nchunk - 1) / nchunk;
  const dim3 grid((d + 255) / 256, (E + kWgradE - 1) / kWgradE, nchunk);
  if (bf16)
    hipLaunchKernelGGL(router_wgrad_kernel<true>, grid, dim3(256), 0, s, x, dL, T, d, E, chunk,
                       part);
  else
    hipLaunchKernelGGL(router_wgrad_kernel<false>, grid, dim3(256), 0, s, x, dL, T, d, E, chunk,
                       part);
  const int n = E * d;
  hipLaunchKernelGGL(sum_chunks_kernel, dim3(std::min((n + 255) / 256, 4096)), dim3(256), 0, s,
                     part, n, nchunk, dw);
}

// dx = d_logits W_r (+ add): block (j-tile of 256 columns, 32 tokens); d_logits rows of the
// tokens staged in LDS 256 experts at a time, expert-major (the 32 tokens' values of one expert
// contiguous, read as eight 16-byte broadcasts per 32 FMAs; rows padded to 36 floats against bank
// conflicts of the staging writes); fp32 sums in expert order, rounded once.
template <bool BF16>
__global__ __launch_bounds__(256) void router_xgrad_kernel(const float* __restrict__ dL,
                                                           const void* __restrict__ w_r, int T,
                                                           int d, int E,
                                                           const void* __restrict__ add,
                                                           void* __restrict__ dx) {
  constexpr int TT = 32, EC = 256, TP = TT + 4;
  __shared__ __align__(16) float sd[EC][TP];
  const int j = blockIdx.x * 256 + threadIdx.x;
  const int t0 = blockIdx.y * TT;
  float acc[TT];
#pragma unroll
  for (int i = 0; i < TT; ++i) acc[i] = 0.f;
  for (int e0 = 0; e0 < E; e0 += EC) {
    __syncthreads();
    for (int q = threadIdx.x; q < TT * EC; q += 256) {
      const int tt = q / EC, ee = q % EC;
      sd[ee][tt] = (t0 + tt < T && e0 + ee < E) ? dL[(size_t)(t0 + tt) * E + e0 + ee] : 0.f;
    }
    __syncthreads();
    if (j < d) {
      const int ne = min(EC, E - e0);
      for (int ee = 0; ee < ne; ++ee) {
        const size_t o = (size_t)(e0 + ee) * d + j;
        const float w = BF16 ? bf16_to_f32(((const uint16_t*)w_r)[o]) : ((const float*)w_r)[o];
        const f32x4* col = reinterpret_cast<const f32x4*>(sd[ee]);
#pragma unroll
        for (int i4 = 0; i4 < TT / 4; ++i4) {
          const f32x4 v = col[i4];
          acc[4 * i4 + 0] = fmaf(v[0], w, acc[4 * i4 + 0]);
          acc[4 * i4 + 1] = fmaf(v[1], w, acc[4 * i4 + 1]);
          acc[4 * i4 + 2] = fmaf(v[2], w, acc[4 * i4 + 2]);
          acc[4 * i4 + 3] = fmaf(v[3], w, acc[4 * i4 + 3]);
        }
      }
    }
  }
  if (j >= d) return;
#pragma unroll
  for (int i = 0; i < TT; ++i) {
    const int t = t0 + i;
    if (t >= T) break;
    const size_t o = (size_t)t * d + j;
    float v = acc[i];
    if (add) v += BF16 ? bf16_to_f32(((const uint16_t*)add)[o]) : ((const float*)add)[o];
    if (BF16)
      ((uint16_t*)dx)[o] = f32_to_bf16(v);
    else
      ((float*)dx)[o] = v;
  }
}

void launch_router_xgrad(const float* dL, const void* w_r, bool bf16, int T, int d, int E,
                         const void* add, void* dx, hipStream_t s) {
  const dim3 grid((d + 255) / 256, (T + 31) / 32);
  if (bf16)
    hipLaunchKernelGGL(router_xgrad_kernel<true>, grid, dim3(256), 0, s, dL, w_r, T, d, E, add,
                       dx);
  else
    hipLaunchKernelGGL(router_xgrad_kernel<false>, grid, dim3(256), 0, s, dL, w_r, T, d, E, add,
                       dx);
}

// Matrix-core form of the two router products (bf16 activations and weights, E a multiple of 64).
// d_logits (fp32) enters as three bf16 terms, hi = bf16(v), mid = bf16(v - hi),
// lo = bf16(v - hi - mid) (round to nearest even; each difference is exact in fp32), whose sum
// is v to within 2^-24 |v|; the products of bf16 terms with bf16 x or w_r are exact in the fp32
// accumulators.  Row t of `terms` holds [hi | mid | lo], 3E values.  Block 0 also writes the
// token-chunk boundaries of the weight-gradient product: offs[g] = min(g * chunk, T), g <= G.
__global__ __launch_bounds__(256) void split_terms_kernel(const float* __restrict__ dL, int T,
                                                          int E, uint16_t* __restrict__ terms,
                                                          int32_t* __restrict__ offs, int G,
                                                          int chunk) {
  if (blockIdx.x == 0)
    for (int g = threadIdx.x; g <= G; g += 256) offs[g] = (int)min((long long)g * chunk, (long long)T);
  const size_t n = (size_t)T * E;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
    const size_t t = i / E, e = i % E;
    const float v = dL[i];
    const uint16_t hi = f32_to_bf16(v);
    const float r1 = v - bf16_to_f32(hi);
    const uint16_t mid = f32_to_bf16(r1);
    const uint16_t lo = f32_to_bf16(r1 - bf16_to_f32(mid));
    uint16_t* row = terms + t * 3 * E;
    row[e] = hi;
    row[E + e] = mid;
    row[2 * E + e] = lo;
  }
}

// dW[e][j] = sum over chunks g in order of (part[g][e][j] + part[g][E + e][j]) + part[g][2E + e][j]
// (the hi, mid and lo terms' products of chunk g).
__global__ __launch_bounds__(256) void sum_terms_kernel(const float* __restrict__ part, int G,
                                                        int E, int d, float* __restrict__ dw) {
  const size_t n = (size_t)E * d, per = 3 * n;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
    float v = 0.f;
    for (int g = 0; g < G; ++g) {
      const float* q = part + (size_t)g * per + i;
      v += (q[0] + q[n]) + q[2 * n];
    }
    dw[i] = v;
  }
}

void launch_split_terms(const float* dL, int T, int E, void* terms, int32_t* offs, int G,
                        int chunk, hipStream_t s) {
  const size_t n = (size_t)T * E;
  const int grid = (int)std::min<size_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(split_terms_kernel, dim3(grid), dim3(256), 0, s, dL, T, E, (uint16_t*)terms,
                     offs, G, chunk);
}

void launch_sum_terms(const float* part, int G, int E, int d, float* dw, hipStream_t s) {
  const size_t n = (size_t)E * d;
  const int grid = (int)std::min<size_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(sum_terms_kernel, dim3(grid), dim3(256), 0, s, part, G, E, d, dw);
}

__global__ void dense_offsets_kernel(int32_t* o, int T) {
  if (threadIdx.x == 0) {
    o[0] = 0;
    o[1] = T;
  }
}

void launch_dense_offsets(int32_t* o, int T, hipStream_t s) {
  hipLaunchKernelGGL(dense_offsets_kernel, dim3(1), dim3(64), 0, s, o, T);
}

}  // namespace moe
