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

// Split-K scratch of the router's matrix-core product (E > 16, bf16), placed after the gating
// partials in moe_route's workspace.
size_t router_partial_bytes(int T, int d, int E, moe_dtype dt) {
  if (dt != MOE_BF16 || E <= 16 || E % 8 != 0 || d % 8 != 0) return 0;
  return align_up(moe::gemm_bf16_partial_bytes(T, 1, false, E, d, moe::EPI_STORE_F32_BIAS));
}

size_t h_bytes(int rows, int d_ff, moe_dtype dt) {
  return align_up((size_t)rows * d_ff * elem_bytes(dt));
}

// moe_expert_ffn workspace: h, then the split-K scratch.
size_t ffn_workspace_bytes(int rows, bool grouped, int G, int d, int d_ff, moe_dtype dt) {
  return h_bytes(rows, d_ff, dt) + ffn_partial_bytes(rows, grouped, G, d, d_ff, dt);
}

// The input-gradient products read the weights as stored (the GEMM's transposed-B mode) when
// d_ff is a multiple of 64, so that the stacked w1 / w3 of dx split on a 64-deep step; otherwise
// they read transposed copies made in the workspace.
bool bwd_weights_in_place(int d_ff) { return d_ff % 64 == 0; }

// moe_expert_backward workspace (bf16): the transposed weights (only without in-place weights),
// the row-major intermediates, the expert-ordered copy of the token rows (grouped only), two ints
// of dense offsets and the split-K scratch of the input-gradient products, in this order.
struct BwdLayout {
  size_t w2t, w13t, dh, h, dab, xg, offs, part, total;
};
BwdLayout bwd_layout(int rows, bool grouped, int G, int d, int d_ff) {
  BwdLayout L;
  size_t o = 0;
  auto take = [&](size_t bytes) { const size_t at = o; o += align_up(bytes); return at; };
  const bool in_place = bwd_weights_in_place(d_ff);
  L.w2t = take(in_place ? 0 : (size_t)G * d_ff * d * 2);
  L.w13t = take(in_place ? 0 : (size_t)G * d * 2 * d_ff * 2);
  L.dh = take((size_t)rows * d_ff * 2);
  L.h = take((size_t)rows * d_ff * 2);
  L.dab = take((size_t)rows * 2 * d_ff * 2);
  L.xg = take(grouped ? (size_t)rows * d * 2 : 0);
  L.offs = take(16);
  const size_t p1 = moe::gemm_bf16_partial_bytes(rows, G, grouped, d_ff, d, moe::EPI_STORE);
  const size_t p2 = moe::gemm_bf16_partial_bytes(rows, G, grouped, d, 2 * d_ff, moe::EPI_STORE);
  L.part = take(p1 > p2 ? p1 : p2);
  L.total = o;
  return L;
}

// The router products run on the matrix cores for bf16 operands with E a multiple of 64 (the
// stacked-K weight reads split on a 64-deep step) while every operand stays under 2 GiB (32-bit
// buffer offsets); otherwise on the vector units.
bool route_bwd_mfma(int T, int d, int E, moe_dtype dt) {
  const long long two_gib = 1ll << 31;
  return dt == MOE_BF16 && E % 64 == 0 && (long long)T * 3 * E * 2 < two_gib &&
         (long long)T * d * 2 < two_gib &&
         (long long)E * d * 2 < two_gib;
}

// Token chunks of the matrix-core weight-gradient product: enough 256 x 256 tiles for a round of
// the CUs (3E x d outputs per chunk), at most 16.
int route_bwd_chunks(int T, int d, int E) {
  const long long tiles = (long long)((3 * E + 255) / 256) * ((d + 255) / 256);
  int G = (int)std::min<long long>(16, std::max<long long>(1, (256 + tiles - 1) / tiles));
  return std::max(1, std::min(G, T));
}

struct RouteBwdLayout {
  size_t terms, offs, part, total;
};

RouteBwdLayout route_bwd_layout(int T, int d, int E) {
  RouteBwdLayout L{};
  const int G = route_bwd_chunks(T, d, E);
  L.terms = 0;
  L.offs = align_up((size_t)T * 3 * E * sizeof(uint16_t));
  L.part = L.offs + align_up((size_t)(G + 1) * sizeof(int32_t));
  L.total = L.part + align_up((size_t)G * 3 * E * d * sizeof(float));
  return L;
}

size_t route_bwd_bytes(int T, int d, int E) {
  const size_t valu = align_up((size_t)moe::router_wgrad_chunks(T) * E * d * sizeof(float));
  const size_t mfma = route_bwd_layout(T, d, E).total;
  return valu > mfma ? valu : mfma;
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
    default: break;
  }
  return "unknown moe_status";
}

size_t moe_workspace_bytes(int T, int d, int d_ff, int E, int k, moe_dtype dt) {
  if (T < 1 || E < 1 || k < 1 || d_ff < 1 || d < 1) return 0;
  size_t r = align_up(moe::route_workspace_bytes(T, E)) + router_partial_bytes(T, d, E, dt);
  size_t q = align_up(moe::dispatch_workspace_bytes(T * k, E));
  const size_t rr = align_up(moe::reroute_workspace_bytes(T * k, E));
  q = q > rr ? q : rr;
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
  if (workspace && !aligned16(workspace)) return MOE_ERR_ARG;
  hipStream_t s = (hipStream_t)stream;
  const bool bf16 = dt == MOE_BF16;
  if (!logits_in) {
    if (E <= 16) {
      moe::launch_router_small_e(x, w_r, logit_bias, T, d, E, bf16, logits, s);
    } else if (E % 8 == 0) {
      // The matrix-core product splits K over the workspace past the gating partials when the
      // workspace holds them (few tokens: too few tiles to cover the GPU); otherwise it runs
      // unsplit.  Either way the fp32 sums are within the same rounding bound.
      const size_t at = align_up(moe::route_workspace_bytes(T, E));
      const size_t need = router_partial_bytes(T, d, E, dt);
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
      if (need && workspace && ws_bytes >= at + need) p.part = (float*)((char*)workspace + at);
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

moe_status moe_dispatch_noalloc(const int32_t* topk_idx, int T, int E, int k, int capacity,
                                int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv,
                                int32_t* n_dropped, void* stream) {
  if (T < 1 || E < 1 || k < 1 || k > E) return MOE_ERR_ARG;
  if (!topk_idx || !counts || !offsets || !perm || !inv || !n_dropped) return MOE_ERR_ARG;
  if (E > kMaxE || k > kMaxK) return MOE_ERR_UNSUPPORTED;
  if (!fits_i32((long long)T * k)) return MOE_ERR_UNSUPPORTED;
  if (moe::dispatch_workspace_bytes(T * k, E) > moe::dispatch_scratch_bytes())
    return MOE_ERR_UNSUPPORTED;
  int32_t* hist = moe::dispatch_scratch();
  if (!hist) return MOE_ERR_DEVICE;
  moe::launch_dispatch(topk_idx, T * k, E, capacity, counts, offsets, perm, inv, n_dropped, hist,
                       (hipStream_t)stream);
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

// Rows r of expert e are [offsets[e], offsets[e+1]); row r reads x row perm[r] / gather_div; at most
// rows_max rows (perm == NULL: one dense group of T rows).
static hipError_t run_up_rows(const void* x, const int32_t* perm, int gather_div,
                              const int32_t* offsets, int T, int d, int d_ff, int E, int rows_max,
                              const void* w1, const void* w3, bool bf16, void* h, void* part,
                              hipStream_t s) {
  moe::GemmParams up{};
  up.A = x;
  up.a_rows = T;
  up.gather = perm;
  up.gather_div = gather_div;
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
  return bf16 ? moe::launch_gemm_bf16(up, rows_max, moe::EPI_SWIGLU, s)
              : moe::launch_gemm_f32(up, rows_max, moe::EPI_SWIGLU, s);
}

static hipError_t run_up(const void* x, const int32_t* perm, const int32_t* offsets, int T, int d,
                         int d_ff, int E, int k, const void* w1, const void* w3, bool bf16, void* h,
                         void* part, hipStream_t s) {
  return run_up_rows(x, perm, k, offsets, T, d, d_ff, E, perm ? T * k : T, w1, w3, bf16, h, part,
                     s);
}

static hipError_t run_down_rows(const void* h, const int32_t* offsets, int T, int d, int d_ff,
                                int E, int rows_max, const void* w2, bool bf16, void* out,
                                void* part, hipStream_t s, int lda = 0) {
  moe::GemmParams dn{};
  dn.A = h;
  dn.lda = lda;
  dn.a_rows = rows_max;
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
  return bf16 ? moe::launch_gemm_bf16(dn, rows_max, moe::EPI_STORE, s)
              : moe::launch_gemm_f32(dn, rows_max, moe::EPI_STORE, s);
}

static hipError_t run_down(const void* h, const int32_t* offsets, int T, int d, int d_ff, int E,
                           int k, const void* w2, bool bf16, void* out, void* part, hipStream_t s) {
  return run_down_rows(h, offsets, T, d, d_ff, E, offsets ? T * k : T, w2, bf16, out, part, s);
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

moe_status moe_expert_ffn_save(const void* x, const int32_t* perm, const int32_t* offsets, int T,
                               int d, int d_ff, int E, int k, const void* w1, const void* w3,
                               const void* w2, moe_dtype dt, void* out, void* saved,
                               void* workspace, size_t ws_bytes, void* stream) {
  moe_status st = check_ffn_args(x, w1, w3, out, perm != nullptr, offsets, T, d, d_ff, E, k, dt);
  if (st != MOE_OK) return st;
  if (!w2 || !aligned16(w2) || !saved || !aligned16(saved)) return MOE_ERR_ARG;
  if (dt != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  const int rows_max = perm ? T * k : T;
  const bool grouped = perm != nullptr;
  if (!fits_i32((long long)rows_max * 6 * d_ff)) return MOE_ERR_UNSUPPORTED;   // bytes of saved
  const size_t need = ffn_partial_bytes(rows_max, grouped, E, d, d_ff, dt);
  if (need && (!workspace || !aligned16(workspace))) return MOE_ERR_ARG;
  if (ws_bytes < need) return MOE_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  void* part = need ? workspace : nullptr;
  moe::GemmParams up{};   // h | a | b per row of saved
  up.A = x;
  up.a_rows = T;
  up.gather = perm;
  up.gather_div = k;
  up.offsets = grouped ? offsets : nullptr;
  up.G = grouped ? E : 1;
  up.M = T;
  up.N = d_ff;
  up.K = d;
  up.B0 = w1;
  up.B1 = w3;
  up.b_gstride = (long long)d * d_ff;
  up.C = saved;
  up.ldc = 3 * d_ff;
  up.part = (float*)part;
  if (moe::launch_gemm_bf16(up, rows_max, moe::EPI_SWIGLU_SAVE, s) != hipSuccess)
    return MOE_ERR_DEVICE;
  if (run_down_rows(saved, grouped ? offsets : nullptr, T, d, d_ff, E, rows_max, w2, true, out,
                    part, s, 3 * d_ff) != hipSuccess)
    return MOE_ERR_DEVICE;
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
  if (!expert_out || !inv || !y || !dtype_ok(dt)) return MOE_ERR_ARG;
  if (!aligned16(expert_out) || !aligned16(y) || (shared_out && !aligned16(shared_out)))
    return MOE_ERR_ARG;
  if (k > moe::kCombineMaxK) return MOE_ERR_UNSUPPORTED;
  if ((d % 8) != 0) return MOE_ERR_UNSUPPORTED;
  // inv is indexed in 32 bits; row offsets into expert_out and y are 64-bit in the kernel
  if (!fits_i32((long long)T * k) || !fits_i32((long long)T * d)) return MOE_ERR_UNSUPPORTED;
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

size_t moe_gathered_workspace_bytes(int rows_max, int d, int d_ff, int E, moe_dtype dt) {
  if (rows_max < 1 || d < 1 || d_ff < 1 || E < 1) return 0;
  return ffn_workspace_bytes(rows_max, true, E, d, d_ff, dt);
}

moe_status moe_expert_ffn_gathered(const void* x, const int32_t* rows, const int32_t* offsets,
                                   int T, int d, int d_ff, int E, int rows_max, const void* w1,
                                   const void* w3, const void* w2, moe_dtype dt, void* out,
                                   void* workspace, size_t ws_bytes, void* stream) {
  if (T < 1 || d < 1 || d_ff < 1 || E < 1 || rows_max < 1) return MOE_ERR_ARG;
  if (!x || !rows || !offsets || !w1 || !w3 || !w2 || !out || !workspace || !dtype_ok(dt))
    return MOE_ERR_ARG;
  if (!aligned16(x) || !aligned16(w1) || !aligned16(w3) || !aligned16(w2) || !aligned16(out) ||
      !aligned16(workspace))
    return MOE_ERR_ARG;
  if (E > kMaxE) return MOE_ERR_UNSUPPORTED;
  if ((d % 8) != 0 || (d_ff % 8) != 0) return MOE_ERR_UNSUPPORTED;
  if (!fits_i32((long long)rows_max * d) || !fits_i32((long long)rows_max * d_ff) ||
      !fits_i32((long long)T * d))
    return MOE_ERR_UNSUPPORTED;
  if (ws_bytes < ffn_workspace_bytes(rows_max, true, E, d, d_ff, dt)) return MOE_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  const bool bf16 = dt == MOE_BF16;
  void* part = (char*)workspace + h_bytes(rows_max, d_ff, dt);
  hipError_t e = run_up_rows(x, rows, 1, offsets, T, d, d_ff, E, rows_max, w1, w3, bf16,
                             workspace, part, s);
  if (e != hipSuccess) return MOE_ERR_DEVICE;
  e = run_down_rows(workspace, offsets, T, d, d_ff, E, rows_max, w2, bf16, out, part, s);
  if (e != hipSuccess) return MOE_ERR_DEVICE;
  return launched();
}

size_t q_workspace_bytes(int rows, bool grouped, int G, int d, int d_ff, int bits) {
  const size_t up = moe::gemm_q_partial_bytes(rows, G, grouped, d_ff, d, bits, 2);
  const size_t dn = moe::gemm_q_partial_bytes(rows, G, grouped, d, d_ff, bits, 1);
  return align_up((size_t)rows * d_ff * 2) + align_up(up > dn ? up : dn);
}

size_t moe_q_workspace_bytes(int T, int d, int d_ff, int E, int k, int bits) {
  if (T < 1 || d < 1 || d_ff < 1 || E < 1 || k < 1 || (bits != 8 && bits != 4)) return 0;
  const size_t a = q_workspace_bytes(T * k, true, E, d, d_ff, bits);
  const size_t b = q_workspace_bytes(T, false, 1, d, d_ff, bits);
  return a > b ? a : b;
}

moe_status moe_quantize_weights(const void* w, int batch, int rows, int cols, moe_dtype dt,
                                int bits, void* q, float* scale, void* stream) {
  if (!w || !q || !scale || batch < 1 || rows < 1 || cols < 1) return MOE_ERR_ARG;
  if (bits != 8 && bits != 4) return MOE_ERR_ARG;
  if (dt != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (bits == 4 && cols % 2 != 0) return MOE_ERR_UNSUPPORTED;
  const long long nrows = (long long)batch * rows;
  if (nrows > 0x7fffffffLL || nrows * cols / rows / batch != cols) return MOE_ERR_UNSUPPORTED;
  moe::launch_quantize_rows(w, nrows, cols, bits, q, scale, (hipStream_t)stream);
  return launched();
}

moe_status moe_expert_ffn_q(const void* x, const int32_t* perm, const int32_t* offsets, int T,
                            int d, int d_ff, int E, int k, int bits, const void* q1,
                            const float* s1, const void* q3, const float* s3, const void* q2,
                            const float* s2, moe_dtype dt, void* out, void* workspace,
                            size_t ws_bytes, void* stream) {
  const bool grouped = perm != nullptr;
  moe_status st = check_ffn_args(x, q1, q3, out, grouped, offsets, T, d, d_ff, E, k, dt);
  if (st != MOE_OK) return st;
  if (!q2 || !s1 || !s3 || !s2 || !workspace || !aligned16(q2) || !aligned16(workspace))
    return MOE_ERR_ARG;
  if (bits != 8 && bits != 4) return MOE_ERR_ARG;
  if (dt != MOE_BF16 || d % 128 != 0 || d_ff % 128 != 0) return MOE_ERR_UNSUPPORTED;
  const int G = grouped ? E : 1;
  const int rows = grouped ? T * k : T;
  if (ws_bytes < q_workspace_bytes(rows, grouped, G, d, d_ff, bits)) return MOE_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  void* h = workspace;
  float* part = (float*)((char*)workspace + align_up((size_t)rows * d_ff * 2));
  moe::GemmParams up{};
  up.A = x; up.a_rows = T; up.gather = perm; up.gather_div = k;
  up.offsets = grouped ? offsets : nullptr; up.G = G; up.M = T;
  up.N = d_ff; up.K = d; up.B0 = q1; up.B1 = q3;
  up.b_gstride = (long long)d_ff * d * bits / 8;
  up.C = h; up.ldc = d_ff; up.part = part;
  if (moe::launch_gemm_q(up, rows, moe::EPI_SWIGLU, bits, s1, s3, s) != hipSuccess)
    return MOE_ERR_DEVICE;
  moe::GemmParams dn{};
  dn.A = h; dn.a_rows = rows; dn.gather_div = 1;
  dn.offsets = grouped ? offsets : nullptr; dn.G = G; dn.M = T;
  dn.N = d; dn.K = d_ff; dn.B0 = q2;
  dn.b_gstride = (long long)d * d_ff * bits / 8;
  dn.C = out; dn.ldc = d; dn.part = part;
  if (moe::launch_gemm_q(dn, rows, moe::EPI_STORE, bits, s2, nullptr, s) != hipSuccess)
    return MOE_ERR_DEVICE;
  return launched();
}

moe_status moe_reroute(const float* logits, const float* select_bias, const int32_t* topk_idx,
                       const float* topk_gate, const int32_t* offsets, const int32_t* inv, int T,
                       int E, int k, int capacity, moe_gating gating, int32_t* topk_idx2,
                       float* topk_gate2, int32_t* offsets2, int32_t* perm2, int32_t* inv2,
                       int32_t* n_dropped2, void* workspace, size_t ws_bytes, void* stream) {
  if (T < 1 || E < 1 || k < 1 || k > E) return MOE_ERR_ARG;
  if (!logits || !topk_idx || !topk_gate || !offsets || !inv || !topk_idx2 || !topk_gate2 ||
      !offsets2 || !perm2 || !inv2 || !n_dropped2 || !workspace)
    return MOE_ERR_ARG;
  if (gating < MOE_GATE_SOFTMAX_TOPK || gating > MOE_GATE_SIGMOID_TOPK) return MOE_ERR_ARG;
  if (E > kMaxE || k > kMaxK) return MOE_ERR_UNSUPPORTED;
  if (!fits_i32((long long)T * E) || !fits_i32((long long)2 * T * k + E))
    return MOE_ERR_UNSUPPORTED;
  if (ws_bytes < moe::reroute_workspace_bytes(T * k, E)) return MOE_ERR_WORKSPACE;
  moe::launch_reroute(logits, select_bias, topk_idx, topk_gate, offsets, inv, T, E, k, capacity,
                      (int)gating, topk_idx2, topk_gate2, offsets2, perm2, inv2, n_dropped2,
                      (int32_t*)workspace, (hipStream_t)stream);
  return launched();
}

moe_status moe_expert_choice(const float* logits, int T, int E, int C, unsigned flags,
                             float* scores, int32_t* offsets, int32_t* perm, float* gate,
                             int32_t* slot, void* stream) {
  const bool scores_in = (flags & MOE_EC_SCORES_IN) != 0;
  if (T < 1 || E < 1 || C < 1 || (flags & ~MOE_EC_SCORES_IN)) return MOE_ERR_ARG;
  if (!scores || !offsets || !perm || !gate || !slot || (!scores_in && !logits))
    return MOE_ERR_ARG;
  if (E > kMaxE) return MOE_ERR_UNSUPPORTED;
  const long long c = C < T ? C : T;
  if (!fits_i32((long long)T * E) || !fits_i32(c * E)) return MOE_ERR_UNSUPPORTED;
  moe::launch_expert_choice(logits, T, E, C, scores_in, scores, offsets, perm, gate, slot,
                            (hipStream_t)stream);
  return launched();
}

size_t moe_backward_workspace_bytes(int T, int d, int d_ff, int E, int k, moe_dtype dt) {
  if (T < 1 || E < 1 || k < 1 || d_ff < 1 || d < 1 || dt != MOE_BF16) return 0;
  const size_t a = bwd_layout(T * k, true, E, d, d_ff).total;
  const size_t b = bwd_layout(T, false, 1, d, d_ff).total;   // shared / dense expert
  const size_t c = route_bwd_bytes(T, d, E);
  const size_t m = a > b ? a : b;
  return m > c ? m : c;
}

moe_status moe_combine_backward(const void* dy, const void* expert_out, const int32_t* inv,
                                const float* topk_gate, int T, int d, int k, moe_dtype dt,
                                void* d_out, float* d_gate, void* stream) {
  if (T < 1 || d < 1 || k < 1) return MOE_ERR_ARG;
  if (!dy || !expert_out || !inv || !topk_gate || !d_out || !d_gate || !dtype_ok(dt))
    return MOE_ERR_ARG;
  if (!aligned16(dy) || !aligned16(expert_out) || !aligned16(d_out)) return MOE_ERR_ARG;
  if (dt != MOE_BF16 || k > kMaxK || (d % 8) != 0) return MOE_ERR_UNSUPPORTED;
  if (!fits_i32((long long)T * k) || !fits_i32((long long)T * k * (long long)d))
    return MOE_ERR_UNSUPPORTED;
  moe::launch_combine_backward(dy, expert_out, inv, topk_gate, T, d, k, d_out, d_gate,
                               (hipStream_t)stream);
  return launched();
}

}  // extern "C"

// The expert backward chain; saved (or NULL) holds the forward's h | a | b rows
// (moe_expert_ffn_save), which replace the recomputation of a and b.
static moe_status expert_backward(const void* saved, const void* x, const int32_t* perm,
                                  const int32_t* offsets, int T, int d, int d_ff, int E, int k,
                                  const void* w1, const void* w3, const void* w2,
                                  const void* d_out, moe_dtype dt, void* dx_rows, float* dw1,
                                  float* dw3, float* dw2, void* workspace, size_t ws_bytes,
                                  void* stream) {
  const bool grouped = perm != nullptr;
  moe_status st = check_ffn_args(x, w1, w3, dx_rows, grouped, offsets, T, d, d_ff, E, k, dt);
  if (st != MOE_OK) return st;
  if (saved && !aligned16(saved)) return MOE_ERR_ARG;
  if (!w2 || !d_out || !dw1 || !dw3 || !dw2 || !workspace) return MOE_ERR_ARG;
  if (!aligned16(w2) || !aligned16(d_out) || !aligned16(dw1) || !aligned16(dw3) ||
      !aligned16(dw2) || !aligned16(workspace))
    return MOE_ERR_ARG;
  if (dt != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  const int G = grouped ? E : 1;
  const int rows = grouped ? T * k : T;
  // 32-bit element offsets inside one operand (the GEMMs offset each group's weights in 64 bits)
  if (!fits_i32((long long)rows * (saved ? 6 : 2) * d_ff) || !fits_i32((long long)rows * d) ||
      !fits_i32((long long)d * 2 * d_ff))
    return MOE_ERR_UNSUPPORTED;
  const BwdLayout L = bwd_layout(rows, grouped, G, d, d_ff);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  void *w2t = ws + L.w2t, *w13t = ws + L.w13t, *dh = ws + L.dh, *h = ws + L.h, *dab = ws + L.dab;
  void* xg = ws + L.xg;
  int32_t* offs = grouped ? (int32_t*)offsets : (int32_t*)(ws + L.offs);
  float* part = (float*)(ws + L.part);
  if (!grouped) moe::launch_dense_offsets(offs, T, s);

  const bool in_place = bwd_weights_in_place(d_ff);
  if (!in_place) {
    // Weights as the input-gradient products read them: w2T[e][n][i] = w2[e][i][n], and
    // w13T[e][i] = (w1[e][.][i], w3[e][.][i]) side by side (K = 2 d_ff).
    moe::launch_transpose16(w2, G, d, d_ff, w2t, d, (long long)d_ff * d, s);
    moe::launch_transpose16(w1, G, d_ff, d, w13t, 2 * d_ff, (long long)d * 2 * d_ff, s);
    moe::launch_transpose16(w3, G, d_ff, d, (uint16_t*)w13t + d_ff, 2 * d_ff,
                            (long long)d * 2 * d_ff, s);
  }
  hipError_t e;
  {   // dh = d_out w2 (rows of each expert); w2[e] is [d][d_ff], i.e. [K][N].  From saved
      // activations the epilogue turns dh into da, db at once.
    moe::GemmParams q{};
    q.A = d_out; q.a_rows = rows; q.gather_div = 1;
    q.offsets = grouped ? offsets : nullptr; q.G = G; q.M = T;
    q.N = d_ff; q.K = d; q.b_gstride = (long long)d_ff * d;
    if (in_place) {
      q.B0 = w2; q.bt = 1; q.ldb = d_ff;
    } else {
      q.B0 = w2t;
    }
    q.C = dh; q.ldc = d_ff; q.part = part;
    int epi = moe::EPI_STORE;
    if (saved) {
      q.C = dab; q.ldc = 2 * d_ff;
      q.D = (const uint16_t*)saved + d_ff; q.ldd = 3 * d_ff;
      epi = moe::EPI_SWIGLU_BWD_SAVED;
    }
    if ((e = moe::launch_gemm_bf16(q, rows, epi, s)) != hipSuccess) return MOE_ERR_DEVICE;
  }
  if (!saved) {   // a, b recomputed; h, da, db from dh
    moe::GemmParams q{};
    q.A = x; q.a_rows = T; q.gather = perm; q.gather_div = k;
    q.offsets = grouped ? offsets : nullptr; q.G = G; q.M = T;
    q.N = d_ff; q.K = d; q.B0 = w1; q.B1 = w3; q.b_gstride = (long long)d * d_ff;
    q.C = dab; q.ldc = 2 * d_ff; q.D = dh; q.H = h;
    if ((e = moe::launch_gemm_bf16(q, rows, moe::EPI_SWIGLU_BWD, s)) != hipSuccess)
      return MOE_ERR_DEVICE;
  }
  {   // dx_rows = da w1 + db w3: K = 2 d_ff over [da | db] and w1[e], w3[e] ([d_ff][d]) stacked
    moe::GemmParams q{};
    q.A = dab; q.a_rows = rows; q.gather_div = 1;
    q.offsets = grouped ? offsets : nullptr; q.G = G; q.M = T;
    q.N = d; q.K = 2 * d_ff;
    if (in_place) {
      q.B0 = w1; q.B1 = w3; q.bt = 1; q.bt_k1 = d_ff; q.ldb = d;
      q.b_gstride = (long long)d_ff * d;
    } else {
      q.B0 = w13t; q.b_gstride = (long long)d * 2 * d_ff;
    }
    q.C = dx_rows; q.ldc = d; q.part = part;
    if ((e = moe::launch_gemm_bf16(q, rows, moe::EPI_STORE, s)) != hipSuccess) return MOE_ERR_DEVICE;
  }
  // Weight gradients, reduced over each expert's rows of row-major operands (the GEMM reads both
  // transposed): dw2 = d_out^T h, dw1 = da^T x_e, dw3 = db^T x_e, with x_e the expert-ordered
  // token rows (gathered once; in dense mode x itself).
  const void* xe = x;
  if (grouped) {
    moe::launch_gather_rows(x, d, perm, k, offsets, G, rows, xg, s);
    xe = xg;
  }
  struct WG { const void* A; int M; int lda; const void* B; int N; int ldb; float* C; };
  const WG wg[3] = {{d_out, d, d, saved ? saved : h, d_ff, saved ? 3 * d_ff : d_ff, dw2},
                    {dab, d_ff, 2 * d_ff, xe, d, d, dw1},
                    {(const uint16_t*)dab + d_ff, d_ff, 2 * d_ff, xe, d, d, dw3}};
  for (const WG& w : wg) {
    moe::GemmParams q{};
    q.A = w.A; q.a_rows = rows; q.lda = w.lda; q.gather_div = 1;
    q.offsets = offs; q.G = G; q.M = w.M; q.N = w.N; q.K = rows;
    q.B0 = w.B; q.ldb = w.ldb; q.C = w.C; q.ldc = w.N;
    q.kgrouped = 1; q.at = 1; q.bt = 1; q.c_gstride = (long long)w.M * w.N;
    if ((e = moe::launch_gemm_bf16(q, rows, moe::EPI_STORE_F32_BIAS, s)) != hipSuccess)
      return MOE_ERR_DEVICE;
  }
  return launched();
}

extern "C" {

moe_status moe_expert_backward(const void* x, const int32_t* perm, const int32_t* offsets, int T,
                               int d, int d_ff, int E, int k, const void* w1, const void* w3,
                               const void* w2, const void* d_out, moe_dtype dt, void* dx_rows,
                               float* dw1, float* dw3, float* dw2, void* workspace,
                               size_t ws_bytes, void* stream) {
  return expert_backward(nullptr, x, perm, offsets, T, d, d_ff, E, k, w1, w3, w2, d_out, dt,
                         dx_rows, dw1, dw3, dw2, workspace, ws_bytes, stream);
}

moe_status moe_expert_backward_saved(const void* saved, const void* x, const int32_t* perm,
                                     const int32_t* offsets, int T, int d, int d_ff, int E, int k,
                                     const void* w1, const void* w3, const void* w2,
                                     const void* d_out, moe_dtype dt, void* dx_rows, float* dw1,
                                     float* dw3, float* dw2, void* workspace, size_t ws_bytes,
                                     void* stream) {
  if (!saved) return MOE_ERR_ARG;
  return expert_backward(saved, x, perm, offsets, T, d, d_ff, E, k, w1, w3, w2, d_out, dt,
                         dx_rows, dw1, dw3, dw2, workspace, ws_bytes, stream);
}

moe_status moe_route_backward(const void* x, const void* w_r, const float* logits,
                              const int32_t* topk_idx, const float* topk_gate,
                              const float* d_gate, const int32_t* counts, int T, int d, int E,
                              int k, moe_dtype dt, moe_gating gating, float alpha, float beta,
                              const void* dx_add, float* d_logits, float* dw_r, void* dx,
                              void* workspace, size_t ws_bytes, void* stream) {
  if (T < 1 || d < 1 || E < 1 || k < 1 || k > E) return MOE_ERR_ARG;
  if (!x || !w_r || !logits || !topk_idx || !topk_gate || !d_gate || !d_logits || !dw_r || !dx ||
      !workspace || !dtype_ok(dt))
    return MOE_ERR_ARG;
  if (gating < MOE_GATE_SOFTMAX_TOPK || gating > MOE_GATE_SIGMOID_TOPK) return MOE_ERR_ARG;
  if (!counts && alpha != 0.0f) return MOE_ERR_ARG;
  if (!aligned16(x) || !aligned16(w_r) || !aligned16(dx) || (dx_add && !aligned16(dx_add)))
    return MOE_ERR_ARG;
  if (E > kMaxE || k > kMaxK || (d % 8) != 0) return MOE_ERR_UNSUPPORTED;
  if (!fits_i32((long long)T * E) || !fits_i32((long long)T * d) ||
      !fits_i32((long long)E * d * 16))
    return MOE_ERR_UNSUPPORTED;
  if (ws_bytes < route_bwd_bytes(T, d, E)) return MOE_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  const bool bf16 = dt == MOE_BF16;
  moe::launch_gate_backward(logits, topk_idx, topk_gate, d_gate, alpha != 0.0f ? counts : nullptr,
                            T, E, k, (int)gating, alpha, beta, d_logits, s);
  if (!route_bwd_mfma(T, d, E, dt)) {
    moe::launch_router_wgrad(x, bf16, d_logits, T, d, E, (float*)workspace, dw_r, s);
    moe::launch_router_xgrad(d_logits, w_r, bf16, T, d, E, dx_add, dx, s);
    return launched();
  }
  // Matrix cores: d_logits as three bf16 terms (hi, mid, lo) of fp32 accuracy.
  const RouteBwdLayout L = route_bwd_layout(T, d, E);
  const int G = route_bwd_chunks(T, d, E);
  const int chunk = (T + G - 1) / G;
  char* ws = (char*)workspace;
  void* terms = ws + L.terms;
  int32_t* offs = (int32_t*)(ws + L.offs);
  float* part = (float*)(ws + L.part);
  moe::launch_split_terms(d_logits, T, E, terms, offs, G, chunk, s);
  hipError_t e;
  {   // dW_r partials: chunk g, term q -> rows q E .. q E + E - 1 of part[g] = terms^T x over the
      // chunk's tokens (both operands row-major, read transposed)
    moe::GemmParams q{};
    q.A = terms; q.a_rows = T; q.lda = 3 * E; q.gather_div = 1;
    q.offsets = offs; q.G = G; q.M = 3 * E; q.N = d; q.K = T;
    q.B0 = x; q.ldb = d; q.C = part; q.ldc = d;
    q.kgrouped = 1; q.at = 1; q.bt = 1; q.c_gstride = (long long)3 * E * d;
    if ((e = moe::launch_gemm_bf16(q, T, moe::EPI_STORE_F32_BIAS, s)) != hipSuccess)
      return MOE_ERR_DEVICE;
  }
  moe::launch_sum_terms(part, G, E, d, dw_r, s);
  {   // dx = [hi | mid] [w_r; w_r] (+ dx_add): K = 2E, w_r read as stored ([E][d], [K][N])
    moe::GemmParams q{};
    q.A = terms; q.a_rows = T; q.lda = 3 * E; q.gather_div = 1;
    q.M = T; q.N = d; q.K = 2 * E;
    q.B0 = w_r; q.B1 = w_r; q.bt = 1; q.bt_k1 = E; q.ldb = d;
    q.C = dx; q.ldc = d;
    q.D = dx_add; q.ldd = d;
    if ((e = moe::launch_gemm_bf16(q, T, moe::EPI_STORE, s)) != hipSuccess) return MOE_ERR_DEVICE;
  }
  return launched();
}

}  // extern "C"

extern "C" {

moe_status moe_peak_mfma(const void* operands, int blocks, int iters, float* out, void* stream) {
  if (!operands || !out || blocks < 1 || iters < 1) return MOE_ERR_ARG;
  if (!aligned16(operands)) return MOE_ERR_ARG;
  moe::launch_peak_mfma(operands, blocks, iters, out, (hipStream_t)stream);
  return launched();
}

moe_status moe_peak_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (!src || !dst || bytes < 16 || bytes % 16 != 0) return MOE_ERR_ARG;
  if (!aligned16(src) || !aligned16(dst)) return MOE_ERR_ARG;
  moe::launch_peak_copy(src, dst, bytes, (hipStream_t)stream);
  return launched();
}

}  // extern "C"
