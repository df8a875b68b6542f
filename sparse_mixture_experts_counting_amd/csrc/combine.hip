// Combine and loss reduction.
//   combine: y[t] = sum_s gate[t,s] * out[inv[t*k+s]] (+ shared[t]); the page "Mixture of experts
//            (MoE)" (tirogla), How it works step 5 and Code `combine`.
//   losses:  aux = alpha * E * sum_e (counts_e / (T*k)) * (prob_sum_e / T); z = beta * lse2 / T;
//            the same page, How it works step 6 and Code `aux_loss`, `z_loss`.
#include "common.h"
#include "kernels.h"

#include <type_traits>

namespace moe {

// One block per token row; each thread owns 16-byte column chunks.  k is at most kCombineMaxK (the
// expert-choice layout passes one slot per expert).  Gathers the token's k expert
// rows through inv, sums in fp32 in slot order and writes y once.
template <bool BF16>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ expert_out,
                                                      const int32_t* __restrict__ inv,
                                                      const float* __restrict__ gate, int T, int d,
                                                      int k, const void* __restrict__ shared_out,
                                                      void* __restrict__ y) {
  __shared__ int32_t s_pos[kCombineMaxK];
  __shared__ float s_g[kCombineMaxK];
  __shared__ int s_n;
  const int t = blockIdx.x;
  for (int i = threadIdx.x; i < k; i += blockDim.x) {
    s_pos[i] = inv[(size_t)t * k + i];
    s_g[i] = gate ? gate[(size_t)t * k + i] : 1.0f;
  }
  __syncthreads();
  // The first wave packs the kept slots to the front, in slot order (a dropped or empty slot
  // adds nothing; the Expert Choice layout has one slot per expert, most of them empty).  Each
  // 64-slot window is read by all lanes before any lane writes, and no write lands past its slot.
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int base = 0;
    for (int s0 = 0; s0 < k; s0 += 64) {
      const int sl = s0 + lane;
      const int pos = sl < k ? s_pos[sl] : -1;
      const float g = sl < k ? s_g[sl] : 0.f;
      const bool ok = pos >= 0;
      const uint64_t m = __ballot(ok);
      if (ok) {
        const int at = base + __popcll(m & lanemask_lt());
        s_pos[at] = pos;
        s_g[at] = g;
      }
      base += __popcll(m);
    }
    if (lane == 0) s_n = base;
  }
  __syncthreads();
  const int nk = s_n;                 // kept slots, packed
  constexpr int VEC = BF16 ? 8 : 4;  // elements per 16-byte chunk
  const int nchunk = d / VEC;
  // Slots in groups of eight: a group's row loads are all issued before any of them is added,
  // and the sums keep slot order.
  constexpr int KG = 8;
  typedef typename std::conditional<BF16, u32x4, f32x4>::type chunk_t;
  for (int c = threadIdx.x; c < nchunk; c += blockDim.x) {
    float acc[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) acc[i] = 0.f;
    for (int s0 = 0; s0 < nk; s0 += KG) {
      chunk_t raw[KG];
#pragma unroll
      for (int j = 0; j < KG; ++j) {
        const int pos = s0 + j < nk ? s_pos[s0 + j] : -1;
        if (pos >= 0)   // every expert row is read once: non-temporal loads
          raw[j] = __builtin_nontemporal_load(reinterpret_cast<const chunk_t*>(
              (const char*)expert_out + ((size_t)pos * d + (size_t)c * VEC) * (BF16 ? 2 : 4)));
      }
#pragma unroll
      for (int j = 0; j < KG; ++j) {
        if (s0 + j >= nk) continue;
        const float g = s_g[s0 + j];
        float v[VEC];
        if constexpr (BF16) {
          unpack8(raw[j], v);
        } else {
          v[0] = raw[j][0]; v[1] = raw[j][1]; v[2] = raw[j][2]; v[3] = raw[j][3];
        }
#pragma unroll
        for (int i = 0; i < VEC; ++i) acc[i] = fmaf(g, v[i], acc[i]);
      }
    }
    if (shared_out) {
      float v[VEC];
      if constexpr (BF16) {
        unpack8(*reinterpret_cast<const u32x4*>((const uint16_t*)shared_out + (size_t)t * d + c * 8), v);
      } else {
        const f32x4 q = *reinterpret_cast<const f32x4*>((const float*)shared_out + (size_t)t * d + c * 4);
        v[0] = q[0]; v[1] = q[1]; v[2] = q[2]; v[3] = q[3];
      }
#pragma unroll
      for (int i = 0; i < VEC; ++i) acc[i] += v[i];
    }
    if constexpr (BF16) {
      u32x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(acc[2 * i], acc[2 * i + 1]);
      *reinterpret_cast<u32x4*>((uint16_t*)y + (size_t)t * d + c * 8) = o;
    } else {
      f32x4 o = {acc[0], acc[1], acc[2], acc[3]};
      *reinterpret_cast<f32x4*>((float*)y + (size_t)t * d + c * 4) = o;
    }
  }
}

void launch_combine(const void* expert_out, const int32_t* inv, const float* gate, int T, int d,
                    int k, bool bf16, const void* shared_out, void* y, hipStream_t s) {
  const int vec = bf16 ? 8 : 4;
  int threads = 64;
  while (threads < 256 && threads * vec < d) threads *= 2;
  if (bf16)
    hipLaunchKernelGGL(combine_kernel<true>, dim3(T), dim3(threads), 0, s, expert_out, inv, gate, T,
                       d, k, shared_out, y);
  else
    hipLaunchKernelGGL(combine_kernel<false>, dim3(T), dim3(threads), 0, s, expert_out, inv, gate,
                       T, d, k, shared_out, y);
}

// One block; fixed-order fp64 reduction over the experts so the result is deterministic.
__global__ __launch_bounds__(256) void aux_loss_kernel(const int32_t* __restrict__ counts,
                                                       const float* __restrict__ prob_sum,
                                                       const float* __restrict__ lse_sq_sum, int T,
                                                       int E, int k, float alpha, float beta,
                                                       float* __restrict__ aux,
                                                       float* __restrict__ z) {
  __shared__ double part[256];
  double s = 0.0;
  for (int e = threadIdx.x; e < E; e += 256) s += (double)counts[e] * (double)prob_sum[e];
  part[threadIdx.x] = s;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) part[threadIdx.x] += part[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double TT = (double)T;
    aux[0] = (float)((double)alpha * (double)E * part[0] / ((double)k * TT * TT));
    z[0] = (float)((double)beta * (double)lse_sq_sum[0] / TT);
  }
}

void launch_aux_loss(const int32_t* counts, const float* prob_sum, const float* lse_sq_sum, int T,
                     int E, int k, float alpha, float beta, float* aux, float* z, hipStream_t s) {
  hipLaunchKernelGGL(aux_loss_kernel, dim3(1), dim3(256), 0, s, counts, prob_sum, lse_sq_sum, T, E,
                     k, alpha, beta, aux, z);
}

// Aux-loss-free balancing step: b_e += rate * sign(T*k - E*counts_e) (integer comparison of the
// load with the mean load T*k/E; one float32 add).  The tirogla page, Implementation notes; the
// DL S077 page, 8.2.
__global__ __launch_bounds__(256) void update_select_bias_kernel(const int32_t* __restrict__ counts,
                                                                 int T, int E, int k, float rate,
                                                                 float* __restrict__ bias) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= E) return;
  const long long diff = (long long)T * k - (long long)E * counts[e];
  const float sgn = diff > 0 ? 1.0f : (diff < 0 ? -1.0f : 0.0f);
  bias[e] = bias[e] + rate * sgn;
}

void launch_update_select_bias(const int32_t* counts, int T, int E, int k, float rate,
                               float* select_bias, hipStream_t s) {
  hipLaunchKernelGGL(update_select_bias_kernel, dim3((E + 255) / 256), dim3(256), 0, s, counts, T,
                     E, k, rate, select_bias);
}

}  // namespace moe
