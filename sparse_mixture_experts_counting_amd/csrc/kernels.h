// Host-side launchers of the libmoe kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

struct GemmParams;

// route.hip
void launch_router_small_e(const void* x, const void* w_r, const float* bias, int T, int d, int E,
                           bool bf16, float* logits, hipStream_t s);
void launch_gate_topk(const float* logits, const float* select_bias, int T, int E, int k, int mode,
                      int32_t* topk_idx, float* topk_gate, float* part_p, float* part_l,
                      float* prob_sum, float* lse_sq_sum, hipStream_t s);
size_t route_workspace_bytes(int T, int E);

int gate_rows_per_block(int T);

// dispatch.hip
size_t dispatch_workspace_bytes(int A, int E);
void launch_dispatch(const int32_t* topk_idx, int A, int E, int capacity, int32_t* counts,
                     int32_t* offsets, int32_t* perm, int32_t* inv, int32_t* n_dropped,
                     int32_t* hist, hipStream_t s);
size_t dispatch_scratch_bytes();
int32_t* dispatch_scratch();

// gemm_bf16.hip / gemm_f32.hip
hipError_t launch_gemm_bf16(const GemmParams& p, int rows_max, int epi, hipStream_t s);
size_t gemm_bf16_partial_bytes(int rows_max, int G, bool grouped, int N, int K, int epi);
hipError_t launch_gemm_f32(const GemmParams& p, int rows_max, int epi, hipStream_t s);
void launch_splitk_finish_bf16(const GemmParams& p, int rows_max, int epi, hipStream_t s);

// gemm_q.hip (weight-only INT8 / INT4 experts)
int gemm_q_split(int rows_max, int G, bool grouped, int N, int K, int bits);
size_t gemm_q_partial_bytes(int rows_max, int G, bool grouped, int N, int K, int bits, int nmat);
hipError_t launch_gemm_q(const GemmParams& p, int rows_max, int epi, int bits, const float* s0,
                         const float* s1, hipStream_t s);
void launch_quantize_rows(const void* w, long long rows, int cols, int bits, void* q, float* scale,
                          hipStream_t s);

// combine.hip
constexpr int kCombineMaxK = 1024;
void launch_combine(const void* expert_out, const int32_t* inv, const float* gate, int T, int d,
                    int k, bool bf16, const void* shared_out, void* y, hipStream_t s);
void launch_update_select_bias(const int32_t* counts, int T, int E, int k, float rate,
                                float* select_bias, hipStream_t s);
void launch_aux_loss(const int32_t* counts, const float* prob_sum, const float* lse_sq_sum, int T,
                     int E, int k, float alpha, float beta, float* aux, float* z, hipStream_t s);

// transpose.hip
void launch_transpose(const void* src, int batch, int rows, int cols, int elem_bytes, void* dst,
                      hipStream_t s);
void launch_transpose_ld(const void* src, int batch, int rows, int cols, int elem_bytes,
                         void* dst, int ldd, long long dst_bstride, hipStream_t s);
void launch_transpose16(const void* src, int batch, int rows, int cols, void* dst, int ldd,
                        long long dst_bstride, hipStream_t s);
void launch_gather_rows(const void* src, int cols, const int32_t* gather, int gather_div,
                        const int32_t* offsets, int G, int rows_max, void* dst, hipStream_t s);

// backward.hip
void launch_combine_backward(const void* dy, const void* out, const int32_t* inv,
                             const float* gate, int T, int d, int k, void* d_out, float* d_gate,
                             hipStream_t s);
void launch_gate_backward(const float* logits, const int32_t* topk_idx, const float* topk_gate,
                          const float* d_gate, const int32_t* counts, int T, int E, int k, int mode,
                          float alpha, float beta, float* d_logits, hipStream_t s);
int router_wgrad_chunks(int T);
void launch_router_wgrad(const void* x, bool bf16, const float* dL, int T, int d, int E,
                         float* part, float* dw, hipStream_t s);
void launch_router_xgrad(const float* dL, const void* w_r, bool bf16, int T, int d, int E,
                         const void* add, void* dx, hipStream_t s);
void launch_dense_offsets(int32_t* o, int T, hipStream_t s);
// Matrix-core router backward: d_logits as three bf16 terms [T][3E] (and the token-chunk offsets
// [G+1] of the weight-gradient product), and the fixed-order sum of its per-chunk, per-term
// partials [G][3E][d] into dW [E][d].
void launch_split_terms(const float* dL, int T, int E, void* terms, int32_t* offs, int G,
                        int chunk, hipStream_t s);
void launch_sum_terms(const float* part, int G, int E, int d, float* dw, hipStream_t s);

// reroute.hip
size_t reroute_workspace_bytes(int A, int E);
void launch_reroute(const float* logits, const float* select_bias, const int32_t* topk_idx,
                    const float* topk_gate, const int32_t* offsets1, const int32_t* inv1, int T,
                    int E, int k, int capacity, int mode, int32_t* idx2, float* gate2,
                    int32_t* offsets2, int32_t* perm2, int32_t* inv2, int32_t* n_dropped,
                    int32_t* ws, hipStream_t s);

// expert_choice.hip
void launch_expert_choice(const float* logits, int T, int E, int C, bool scores_in, float* scores,
                          int32_t* offsets, int32_t* perm, float* gate, int32_t* slot,
                          hipStream_t s);

// peak.hip (measurement only)
void launch_peak_mfma(const void* operands, int blocks, int iters, float* out, hipStream_t s);
void launch_peak_copy(const void* src, void* dst, size_t bytes, hipStream_t s);

}  // namespace moe
