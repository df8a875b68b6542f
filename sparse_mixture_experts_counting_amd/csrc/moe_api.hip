// The libmoe C ABI (declared in include/moe.h): argument checks, workspace carving and kernel
// launches.  Host code only; every call enqueues on the caller's stream and returns.
#include "moe.h"

#include <hip/hip_runtime.h>

#include "gemm_common.h"
#include "kernels.h"

namespace moe {
void launch_router_generic(const void* x, const void* w_r, const float* bias, int T, int d, int E,
                           bool bf16, float* logits, hipStream_t s);
}

namespace {

constexpr int kMaxE = 1024;
constexpr int kMaxK = 32;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
size_t align_up(size_t v) { return (v + 255) & ~(size_t)255; }
size_t elem_bytes(moe_dtype dt) { return dt == MOE_BF16 ? 2 : 4; }
bool dtype_ok(moe_dtype dt) { return dt == MOE_F32 || dt == MOE_BF16; }
bool fits_i32(long long v) { return v >= 0 && v <= 0x7fffffffLL; }

moe_status launched(hipError_t e = hipSuccess) {
  if (e != hipSuccess) return MOE_ERR_DEVICE;
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_DEVICE;
}

// Split-K scratch of the two expert GEMMs (bf16 matrix-core path only; they run one after the
// other, so one region serves both).
size_t ffn_partial_bytes(int rows, bool grouped, int G, int d, int d_ff, moe_dtype dt) {
  if (dt != MOE_BF16) return 0;
  const size_t up = moe::gemm_bf16_partial_bytes(rows, G, grouped, d_ff, d, moe::EPI_SWIGLU);
  const size_t dn = moe::gemm_bf16_partial_bytes(rows, G, grouped, d, d_ff, moe::EPI_STORE);
  return align_up(up > dn ? up : dn);
}

size_t h_bytes(int rows, int d_ff, moe_dtype dt) {
  return align_up((size_t)rows * d_ff * elem_bytes(dt));
}

// moe_expert_ffn workspace: h, then the split-K scratch.
size_t ffn_workspace_bytes(int rows, bool grouped, int G, int d, int d_ff, moe_dtype dt) {
  return h_bytes(rows, d_ff, dt) + ffn_partial_bytes(rows, grouped, G, d, d_ff, dt);
}

}  // namespace

extern "C" {

const char* moe_status_str(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_ARG: return "MOE_ERR_ARG: invalid argument";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: shape or mode not supported";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace too small";
    case MOE_ERR_DEVICE: return "MOE_ERR_DEVICE: kernel launch failed";
  }
  return "unknown moe_status";
}

size_t moe_workspace_bytes(int T, int d, int d_ff, int E, int k, moe_dtype dt) {
  if (T < 1 || E < 1 || k < 1 || d_ff < 1 || d < 1) return 0;
  size_t r = align_up(moe::route_workspace_bytes(T, E));
  size_t q = align_up(moe::dispatch_workspace_bytes(T * k, E));
  size_t f = ffn_workspace_bytes(T * k, true, E, d, d_ff, dt);
  const size_t fs = ffn_workspace_bytes(T, false, 1, d, d_ff, dt);   // shared / dense expert
  f = f > fs ? f : fs;
  size_t m = r > q ? r : q;
  return m > f ? m : f;
}

moe_status moe_route(const void* x, const void* w_r, const float* logit_bias,
                     const float* select_bias, int T, int d, int E, int k, moe_dtype dt,
                     moe_gating gating, unsigned flags, float* logits, int32_t* topk_idx,
                     float* topk_gate, float* prob_sum, float* lse_sq_sum, void* workspace,
                     size_t ws_bytes, void* stream) {
  const bool logits_in = (flags & MOE_ROUTE_LOGITS_IN) != 0;
  if (T < 1 || E < 1 || k < 1 || k > E) return MOE_ERR_ARG;
  if (flags & ~MOE_ROUTE_LOGITS_IN) return MOE_ERR_ARG;
  if (!logits || !topk_idx || !topk_gate) return MOE_ERR_ARG;
  if (!dtype_ok(dt) || gating < MOE_GATE_SOFTMAX_TOPK || gating > MOE_GATE_SIGMOID_TOPK)
    return MOE_ERR_ARG;
  if (logits_in && logit_bias) return MOE_ERR_ARG;
  if (!logits_in) {
    if (!x || !w_r || d < 1) return MOE_ERR_ARG;
    if (!aligned16(x) || !aligned16(w_r)) return MOE_ERR_ARG;
  }
  if (E > kMaxE || k > kMaxK) return MOE_ERR_UNSUPPORTED;
  if (!logits_in && (d % 8) != 0) return MOE_ERR_UNSUPPORTED;
  if (!fits_i32((long long)T * E) || !fits_i32((long long)T * k) ||
      (!logits_in && !fits_i32((long long)T * d)))
    return MOE_ERR_UNSUPPORTED;
  const bool want_partials = prob_sum || lse_sq_sum;
  if (want_partials) {
    if (!workspace) return MOE_ERR_ARG;
    if (ws_bytes < moe::route_workspace_bytes(T, E)) return MOE_ERR_WORKSPACE;
  }
  hipStream_t s = (hipStream_t)stream;
  const bool bf16 = dt == MOE_BF16;
  if (!logits_in) {
    if (E <= 16) {
      moe::launch_router_small_e(x, w_r, logit_bias, T, d, E, bf16, logits, s);
    } else if (E % 8 == 0) {
      moe::GemmParams p{};
      p.A = x;
      p.a_rows = T;
      p.M = T;
      p.N = E;
      p.K = d;
      p.B0 = w_r;
      p.C = logits;
      p.ldc = E;
      p.bias = logit_bias;
      p.gather_div = 1;
      hipError_t e = bf16 ? moe::launch_gemm_bf16(p, T, moe::EPI_STORE_F32_BIAS, s)
                          : moe::launch_gemm_f32(p, T, moe::EPI_STORE_F32_BIAS, s);
      if (e != hipSuccess) return MOE_ERR_DEVICE;
    } else {
      moe::launch_router_generic(x, w_r, logit_bias, T, d, E, bf16, logits, s);
    }
  }
  float* part_p = nullptr;
  float* part_l = nullptr;
  if (want_partials) {
    const int rpb = moe::gate_rows_per_block(T);
    const size_t nblk = (size_t)(T + rpb - 1) / rpb;
    part_p = (float*)workspace;
    part_l = part_p + nblk * E;
  }
  moe::launch_gate_topk(logits, select_bias, T, E, k, (int)gating, topk_idx, topk_gate, part_p,
                        part_l, prob_sum, lse_sq_sum, s);
  return launched();
}

moe_status moe_dispatch(const int32_t* topk_idx, int T, int E, int k, int capacity,
                        int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv,
                        int32_t* n_dropped, void* workspace, size_t ws_bytes, void* stream) {
  if (T < 1 || E < 1 || k < 1 || k > E) return MOE_ERR_ARG;
  if (!topk_idx || !counts || !offsets || !perm || !inv || !n_dropped || !workspace)
    return MOE_ERR_ARG;
  if (E > kMaxE || k > kMaxK) return MOE_ERR_UNSUPPORTED;
  if (!fits_i32((long long)T * k)) return MOE_ERR_UNSUPPORTED;
  if (ws_bytes < moe::dispatch_workspace_bytes(T * k, E)) return MOE_ERR_WORKSPACE;
  moe::launch_dispatch(topk_idx, T * k, E, capacity, counts, offsets, perm, inv, n_dropped,
                       (int32_t*)workspace, (hipStream_t)stream);
  return launched();
}

static moe_status check_ffn_args(const void* x, const void* wa, const void* wb, const void* out,
                                 bool grouped, const int32_t* offsets, int T, int d, int d_ff,
                                 int E, int k, moe_dtype dt) {
  if (T < 1 || d < 1 || d_ff < 1 || E < 1 || k < 1) return MOE_ERR_ARG;
  if (!x || !wa || !wb || !out || !dtype_ok(dt)) return MOE_ERR_ARG;
  if (grouped && (!offsets || k > E)) return MOE_ERR_ARG;
  if (!grouped && E != 1) return MOE_ERR_ARG;
  if (!aligned16(x) || !aligned16(wa) || !aligned16(wb) || !aligned16(out)) return MOE_ERR_ARG;
  if (E > kMaxE || k > kMaxK) return MOE_ERR_UNSUPPORTED;
  if ((d % 8) != 0 || (d_ff % 8) != 0) return MOE_ERR_UNSUPPORTED;
  const long long rows_max = grouped ? (long long)T * k : T;
  if (!fits_i32((long long)T * k) || !fits_i32(rows_max * d) || !fits_i32(rows_max * d_ff) ||
      !fits_i32((long long)T * d))
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

static hipError_t run_up(const void* x, const int32_t* perm, const int32_t* offsets, int T, int d,
                         int d_ff, int E, int k, const void* w1, const void* w3, bool bf16, void* h,
                         void* part, hipStream_t s) {
  moe::GemmParams up{};
  up.A = x;
  up.a_rows = T;
  up.gather = perm;
  up.gather_div = k;
  up.offsets = perm ? offsets : nullptr;
  up.G = perm ? E : 1;
  up.M = T;
  up.N = d_ff;
  up.K = d;
  up.B0 = w1;
  up.B1 = w3;
  up.b_gstride = (long long)d * d_ff;
  up.C = h;
  up.ldc = d_ff;
  up.part = (float*)part;
  const int rows_max = perm ? T * k : T;
  return bf16 ? moe::launch_gemm_bf16(up, rows_max, moe::EPI_SWIGLU, s)
              : moe::launch_gemm_f32(up, rows_max, moe::EPI_SWIGLU, s);
}

static hipError_t run_down(const void* h, const int32_t* offsets, int T, int d, int d_ff, int E,
                           int k, const void* w2, bool bf16, void* out, void* part, hipStream_t s) {
  moe::GemmParams dn{};
  dn.A = h;
  dn.a_rows = offsets ? T * k : T;
  dn.gather_div = 1;
  dn.offsets = offsets;
  dn.G = offsets ? E : 1;
  dn.M = T;
  dn.N = d;
  dn.K = d_ff;
  dn.B0 = w2;
  dn.b_gstride = (long long)d_ff * d;
  dn.C = out;
  dn.ldc = d;
  dn.part = (float*)part;
  const int rows_max = offsets ? T * k : T;
  return bf16 ? moe::launch_gemm_bf16(dn, rows_max, moe::EPI_STORE, s)
              : moe::launch_gemm_f32(dn, rows_max, moe::EPI_STORE, s);
}

moe_status moe_expert_ffn(const void* x, const int32_t* perm, const int32_t* offsets, int T, int d,
                          int d_ff, int E, int k, const void* w1, const void* w3, const void* w2,
                          moe_dtype dt, void* out, void* workspace, size_t ws_bytes,
                          void* stream) {
  moe_status st = check_ffn_args(x, w1, w3, out, perm != nullptr, offsets, T, d, d_ff, E, k, dt);
  if (st != MOE_OK) return st;
  if (!w2 || !aligned16(w2) || !workspace || !aligned16(workspace)) return MOE_ERR_ARG;
  const int rows_max = perm ? T * k : T;
  const bool grouped = perm != nullptr;
  if (ws_bytes < ffn_workspace_bytes(rows_max, grouped, E, d, d_ff, dt)) return MOE_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  const bool bf16 = dt == MOE_BF16;
  void* part = (char*)workspace + h_bytes(rows_max, d_ff, dt);
  hipError_t e = run_up(x, perm, offsets, T, d, d_ff, E, k, w1, w3, bf16, workspace, part, s);
  if (e != hipSuccess) return MOE_ERR_DEVICE;
  e = run_down(workspace, perm ? offsets : nullptr, T, d, d_ff, E, k, w2, bf16, out, part, s);
  if (e != hipSuccess) return MOE_ERR_DEVICE;
  return launched();
}

moe_status moe_expert_up(const void* x, const int32_t* perm, const int32_t* offsets, int T, int d,
                         int d_ff, int E, int k, const void* w1, const void* w3, moe_dtype dt,
                         void* h, void* workspace, size_t ws_bytes, void* stream) {
  moe_status st = check_ffn_args(x, w1, w3, h, perm != nullptr, offsets, T, d, d_ff, E, k, dt);
  if (st != MOE_OK) return st;
  const int rows_max = perm ? T * k : T;
  const size_t need = ffn_partial_bytes(rows_max, perm != nullptr, E, d, d_ff, dt);
  if (workspace && !aligned16(workspace)) return MOE_ERR_ARG;
  if (workspace && ws_bytes < need) return MOE_ERR_WORKSPACE;
  hipError_t e = run_up(x, perm, offsets, T, d, d_ff, E, k, w1, w3, dt == MOE_BF16, h,
                        need ? workspace : nullptr, (hipStream_t)stream);
  return e != hipSuccess ? MOE_ERR_DEVICE : launched();
}

moe_status moe_expert_down(const void* h, const int32_t* offsets, int T, int d, int d_ff, int E,
                           int k, const void* w2, moe_dtype dt, void* out, void* workspace,
                           size_t ws_bytes, void* stream) {
  moe_status st = check_ffn_args(h, w2, w2, out, offsets != nullptr, offsets, T, d, d_ff, E, k, dt);
  if (st != MOE_OK) return st;
  const int rows_max = offsets ? T * k : T;
  const size_t need = ffn_partial_bytes(rows_max, offsets != nullptr, E, d, d_ff, dt);
  if (workspace && !aligned16(workspace)) return MOE_ERR_ARG;
  if (workspace && ws_bytes < need) return MOE_ERR_WORKSPACE;
  hipError_t e = run_down(h, offsets, T, d, d_ff, E, k, w2, dt == MOE_BF16, out,
                          need ? workspace : nullptr, (hipStream_t)stream);
  return e != hipSuccess ? MOE_ERR_DEVICE : launched();
}

moe_status moe_combine(const void* expert_out, const int32_t* inv, const float* topk_gate, int T,
                       int d, int k, moe_dtype dt, const void* shared_out, void* y, void* stream) {
  if (T < 1 || d < 1 || k < 1) return MOE_ERR_ARG;
  if (!expert_out || !inv || !topk_gate || !y || !dtype_ok(dt)) return MOE_ERR_ARG;
  if (!aligned16(expert_out) || !aligned16(y) || (shared_out && !aligned16(shared_out)))
    return MOE_ERR_ARG;
  if (k > kMaxK) return MOE_ERR_UNSUPPORTED;
  if ((d % 8) != 0) return MOE_ERR_UNSUPPORTED;
  if (!fits_i32((long long)T * k) || !fits_i32((long long)T * k * (long long)d))
    return MOE_ERR_UNSUPPORTED;
  moe::launch_combine(expert_out, inv, topk_gate, T, d, k, dt == MOE_BF16, shared_out, y,
                      (hipStream_t)stream);
  return launched();
}

moe_status moe_update_select_bias(const int32_t* counts, int T, int E, int k, float rate,
                                  float* select_bias, void* stream) {
  if (T < 1 || E < 1 || k < 1 || !counts || !select_bias) return MOE_ERR_ARG;
  if (E > kMaxE || k > kMaxK) return MOE_ERR_UNSUPPORTED;
  moe::launch_update_select_bias(counts, T, E, k, rate, select_bias, (hipStream_t)stream);
  return launched();
}

moe_status moe_aux_loss(const int32_t* counts, const float* prob_sum, const float* lse_sq_sum,
                        int T, int E, int k, float alpha, float beta, float* aux, float* z,
                        void* stream) {
  if (T < 1 || E < 1 || k < 1) return MOE_ERR_ARG;
  if (!counts || !prob_sum || !lse_sq_sum || !aux || !z) return MOE_ERR_ARG;
  if (E > kMaxE) return MOE_ERR_UNSUPPORTED;
  moe::launch_aux_loss(counts, prob_sum, lse_sq_sum, T, E, k, alpha, beta, aux, z,
                       (hipStream_t)stream);
  return launched();
}

moe_status moe_transpose(const void* src, int batch, int rows, int cols, moe_dtype dt, void* dst,
                         void* stream) {
  if (!src || !dst || batch < 1 || rows < 1 || cols < 1 || !dtype_ok(dt)) return MOE_ERR_ARG;
  if ((rows + 63) / 64 > 65535 || batch > 65535) return MOE_ERR_UNSUPPORTED;
  const long long elems = (long long)batch * rows * cols;
  if (elems / batch / rows != cols) return MOE_ERR_UNSUPPORTED;
  moe::launch_transpose(src, batch, rows, cols, (int)elem_bytes(dt), dst, (hipStream_t)stream);
  return launched();
}

}  // extern "C"
