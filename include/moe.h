/*
 * libmoe -- forward and backward passes of one top-k routed Mixture-of-Experts FFN layer on one
 * AMD MI355X (CDNA4, gfx950), as hand-written HIP kernels behind a plain C ABI.
 *
 * The method follows the page "Mixture of experts (MoE)" (tirogla.com/machine-learning/
 * mixture-of-experts.html), section "How it works": Score (router product and gating), Select
 * (top-k), Dispatch (counting sort by expert, at most C per expert), Compute (each expert's FFN on
 * its contiguous batch, as one grouped GEMM), Combine (gate-weighted sum, dropped assignments add
 * nothing) and Balance (load-balancing loss and router z-loss).  The expert is the SwiGLU MLP of
 * "DL S077 - Mixture of Experts (MoE) Intuition" (dineshblog.com), section 1.1.
 *
 * Conventions shared by every entry point
 *   - Every pointer is a DEVICE pointer (memory the caller allocated on the current HIP device),
 *     unless stated otherwise.  The caller owns every buffer, including the workspace; the
 *     library never allocates or frees device memory and never synchronises the host.  Buffers
 *     must stay valid until the work enqueued on `stream` has finished.  A workspace holds the
     call's scratch (partial sums, tile counters) while its work runs, so calls that may overlap
     (on different streams) need workspaces of their own.
 *   - `stream` is a hipStream_t passed as void*; NULL means the default stream.  Every call only
 *     enqueues work ordered on that stream and returns.  The library creates no streams or
 *     events of its own, so calls on different streams are independent and any call can be
 *     captured into a HIP graph.
 *   - Outputs are fully overwritten (no accumulate-into semantics) and must not alias inputs.
 *   - Integers are int32, row-major everywhere.  T tokens, d model width, E routed experts, k
 *     experts per token, d_ff expert width; assignment a = t*k + s for slot s of token t.
 *   - Errors are reported before anything is enqueued: MOE_ERR_ARG for a NULL required pointer or
 *     a size out of range (T < 1, d < 1, d_ff < 1, E < 1, k < 1, k > E), MOE_ERR_UNSUPPORTED for
 *     E > 1024, k > 32, or d / d_ff not a multiple of 8 (16-byte vector loads), MOE_ERR_WORKSPACE
 *     when ws_bytes is below what moe_workspace_bytes() returns.  MOE_ERR_DEVICE means a kernel
 *     launch failed (hipGetLastError after the launch).
 *   - Sizes are limited so that T*k*max(d, d_ff) fits in int32 element counts.
 */
#ifndef LIBMOE_MOE_H
#define LIBMOE_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Every enum below spans the whole int range (the two range enumerators are not values to pass),
 * so that any int a caller passes is a representable value that the checks can refuse: an
 * out-of-range value is MOE_ERR_ARG, never undefined behaviour in the library's C++ code. */
typedef enum {
  MOE_OK = 0,
  MOE_ERR_ARG = 1,
  MOE_ERR_UNSUPPORTED = 2,
  MOE_ERR_WORKSPACE = 3,
  MOE_ERR_DEVICE = 4,
  MOE_STATUS_RANGE_MIN_ = -0x7fffffff - 1,
  MOE_STATUS_RANGE_MAX_ = 0x7fffffff
} moe_status;

/* Element type of x, W_r, the expert weights, expert outputs and y.  Accumulation is always fp32
 * and router logits are always fp32 (the tirogla page, Implementation notes: compute the router in
 * fp32 because small logit differences decide routing). */
typedef enum {
  MOE_F32 = 0,
  MOE_BF16 = 1,
  MOE_DTYPE_RANGE_MIN_ = -0x7fffffff - 1,
  MOE_DTYPE_RANGE_MAX_ = 0x7fffffff
} moe_dtype;

/* Gating (the tirogla page, How it works, step 1). */
typedef enum {
  MOE_GATE_SOFTMAX_TOPK = 0, /* softmax over the k selected logits (Mixtral)                       */
  MOE_GATE_SOFTMAX_ALL = 1,  /* softmax over all E logits, keep the selected probabilities (Switch) */
  MOE_GATE_SIGMOID_TOPK = 2, /* sigmoid affinities renormalised over the k selected (DeepSeek-V3)   */
  MOE_GATING_RANGE_MIN_ = -0x7fffffff - 1,
  MOE_GATING_RANGE_MAX_ = 0x7fffffff
} moe_gating;

/* moe_route flag: skip the router product and read `logits` as an input. */
#define MOE_ROUTE_LOGITS_IN 0x1u

/* moe_expert_choice flag: `scores` is an input (the selection is taken on those values). */
#define MOE_EC_SCORES_IN 0x1u

/* Workspace bytes that cover every call below for this layer shape (max over the calls). */
size_t moe_workspace_bytes(int T, int d, int d_ff, int E, int k, moe_dtype dt);

/* Human-readable name of a status code (static string, host memory). */
const char* moe_status_str(moe_status s);

/*
 * moe_route -- Score and Select (the tirogla page, How it works steps 1-2, and its Code `route`;
 * the worked top-2 example of the dineshblog page, section 2).
 *
 *   logits[t,e] = sum_j x[t,j] * w_r[e,j] + logit_bias[e]      (fp32 accumulate)
 *   topk_idx[t,0..k)  the k largest scores of row t, in descending order; equal scores go to the
 *                     lower expert index first; -0.0 equals +0.0; -inf ranks last.  The score is
 *                     the logit, or logit + select_bias[e] (one fp32 add) when select_bias is
 *                     given: aux-loss-free balancing, which biases the selection only (the tirogla
 *                     page, Implementation notes; the dineshblog page, section 8.2).
 *   topk_gate[t,s]    from the logits, never the selection bias:
 *                     SOFTMAX_TOPK: exp(L_e - m) / sum_sel exp(L_s - m), m = row max
 *                     SOFTMAX_ALL:  exp(L_e - m) / sum_all exp(L_j - m)
 *                     SIGMOID_TOPK: sigmoid(L_e) / sum_sel sigmoid(L_s)
 *   prob_sum[e]       sum over tokens of the full-row softmax p[t,e] (the P_e numerator of the
 *                     load-balancing loss, in every gating mode)
 *   lse_sq_sum[0]     sum over tokens of logsumexp(row t)^2 (the z-loss numerator)
 *
 * x [T,d] row-major and w_r the d x E router matrix stored column-major (w_r[e*d + j] holds
 * element (j, e): the [out][in] weight of the bias-free linear layer that the dineshblog page,
 * section 1.2, declares as the router), both in dtype `dt`; logit_bias [E] fp32 or NULL (added to
 * the logits, so seen by selection, gates, P and z); select_bias [E] fp32 or NULL (selection
 * only); logits [T,E] fp32 (output, or input with MOE_ROUTE_LOGITS_IN, in which case x and w_r may
 * be NULL and logit_bias must be NULL); topk_idx [T,k] int32; topk_gate [T,k] fp32; prob_sum [E]
 * fp32; lse_sq_sum [1] fp32.
 * prob_sum and lse_sq_sum may be NULL.  Non-finite logits violate the precondition: routing is then
 * unspecified but memory-safe (indices stay in [0,E) and distinct within a row).
 * workspace (16-byte aligned, ws_bytes long) is required when prob_sum or lse_sq_sum is given (it
 * holds the per-block loss partials); it may be NULL otherwise.  When it is as large as
 * moe_workspace_bytes() for the layer, the matrix-core router product (bf16, E > 16) also splits
 * its reduction over d into fixed chunks there, summed in a fixed order (more blocks for a few
 * thousand tokens); a smaller workspace runs it unsplit.  The logits of both forms lie within the
 * same fp32 dot-product rounding bound; each form is bitwise deterministic.
 * Results are bitwise deterministic run to run.
 */
moe_status moe_route(const void* x, const void* w_r, const float* logit_bias,
                     const float* select_bias, int T, int d, int E, int k, moe_dtype dt,
                     moe_gating gating, unsigned flags, float* logits, int32_t* topk_idx,
                     float* topk_gate, float* prob_sum, float* lse_sq_sum, void* workspace,
                     size_t ws_bytes, void* stream);

/*
 * moe_dispatch -- Dispatch (the tirogla page, How it works step 3 and Code `dispatch`; capacity and
 * token dropping as in the dineshblog page, section 3.2).  A stable counting sort of the T*k
 * assignments by expert; each expert keeps its first `capacity` assignments in increasing
 * assignment order a = t*k + s, later ones are dropped.
 *
 *   counts[e]        assignments to e before capacity                      int32 [E]
 *   offsets[e]       exclusive prefix sum of kept_e = min(counts[e], C)     int32 [E+1]
 *   perm[r]          for offsets[e] <= r < offsets[e+1]: expert e's kept assignment ids in
 *                    increasing order; entries at r >= offsets[E] are unspecified  int32 [T*k]
 *   inv[a]           the r with perm[r] = a, or -1 when a was dropped       int32 [T*k]
 *   n_dropped[0]     T*k - offsets[E]                                       int32 [1]
 *
 * topk_idx [T,k] with entries in [0,E).  An out-of-range entry (checked on the device) is not counted
 * in counts, gets inv = -1 and is included in n_dropped.  capacity <= 0 means unlimited.
 * Deterministic.
 */
moe_status moe_dispatch(const int32_t* topk_idx, int T, int E, int k, int capacity,
                        int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv,
                        int32_t* n_dropped, void* workspace, size_t ws_bytes, void* stream);

/*
 * moe_dispatch_noalloc -- moe_dispatch for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the same kernels and
 * the same outputs, bit for bit, with the per-chunk histogram kept in a fixed 1 MiB device array
 * inside the library instead of a caller's workspace.  It allocates and frees nothing (the array
 * is part of the loaded library on every GPU it runs on, until the process ends); the first call
 * on a device looks up that device's copy.  Limit: ceil(T*k / 2048) * E * 4 + 256 bytes must not
 * exceed 1 MiB (about 522 k assignments at E = 1024, 2 M at E = 256), else MOE_ERR_UNSUPPORTED.
 * Every call on one GPU shares that GPU's array: calls that overlap in time on one GPU (two
 * streams, two threads) race and must be ordered by the caller.  Errors as moe_dispatch;
 * MOE_ERR_DEVICE also when the array's device address cannot be looked up.
 */
moe_status moe_dispatch_noalloc(const int32_t* topk_idx, int T, int E, int k, int capacity,
                                int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv,
                                int32_t* n_dropped, void* stream);

/*
 * moe_expert_ffn -- Compute (the tirogla page, How it works step 4: every expert runs its FFN on its
 * contiguous batch, as one grouped GEMM).  The expert is SwiGLU (the dineshblog page, section 1.1):
 *
 *   h[n]   = silu(sum_j x[t,j] w1[e][n][j]) * (sum_j x[t,j] w3[e][n][j])   silu(z) = z/(1+exp(-z))
 *   out[r][i] = sum_n h[n] w2[e][i][n]          for every row r in [offsets[e], offsets[e+1])
 *
 * where token t = perm[r] / k.  Rows are those of moe_dispatch: out is in perm order, and only rows
 * r < offsets[E] are written.  With perm == NULL the call is one dense group over the T tokens
 * (row r = token r; E must be 1 and offsets may be NULL): this is how a shared, always-on expert
 * runs (the starphix page, Expert Architectures: Shared + Specialized).
 *
 * x [T,d] row-major.  Expert e's matrices have the pages' shapes, w1 and w3 d x d_ff and w2
 * d_ff x d, each stored column-major: w1[(e*d_ff + n)*d + j] holds element (j, n) of w1_e, and
 * w2[(e*d + i)*d_ff + n] element (n, i) of w2_e.  That is the [out][in] weight layout of the
 * bias-free linear layers that the dineshblog page, section 1.1, declares, and it keeps both GEMM
 * operands contiguous along the reduced dimension.  out [T*k][d] (routed) or [T][d] (perm NULL);
 * all in dtype `dt`.  d and d_ff must be multiples of 8.  h is kept in the workspace in dtype `dt`
 * (bf16 layers round h to bf16 before the down projection; accumulation is fp32).  When the tiles
 * would leave the GPU under-filled, K is split over several blocks whose fp32 partial sums (also in
 * the workspace) are added in a fixed order, so results are bitwise deterministic run to run.
 */
moe_status moe_expert_ffn(const void* x, const int32_t* perm, const int32_t* offsets, int T, int d,
                          int d_ff, int E, int k, const void* w1, const void* w3, const void* w2,
                          moe_dtype dt, void* out, void* workspace, size_t ws_bytes, void* stream);

/*
 * moe_expert_up / moe_expert_down -- the two halves of moe_expert_ffn, for callers that keep h
 * themselves (to overlap the shared expert with the routed ones, or to time each half):
 *
 *   moe_expert_up:   h[r]   = silu(x_t . w1_e) * (x_t . w3_e)   h [rows][d_ff] in dtype `dt`
 *   moe_expert_down: out[r] = h[r] . w2_e                       out [rows][d]
 *
 * Same row convention as moe_expert_ffn (rows r < offsets[E], t = perm[r] / k); with perm == NULL
 * (up) or offsets == NULL (down) the call is one dense group over T rows and E must be 1.  h must
 * hold T*k rows (routed) or T rows (dense).  The workspace (sized by moe_workspace_bytes) holds
 * fp32 partial sums of K-split tiles: every tile when few rows leave the GPU under-filled
 * (decode-sized batches), else the tiles of a last, partial round of tiles.  Partials are added in
 * a fixed order, so results are bitwise deterministic run to run; a split changes only the order of
 * the fp32 sums.  Products of groups that fill 256-row tiles with more than two rounds of tiles
 * keep 8 tile counters there instead (one block per compute unit taking tiles; each tile is still
 * summed whole, in the same order).  The workspace may be NULL: the GEMMs then run unsplit and one
 * block per tile (equal up to the split's rounding order).  Same errors as moe_expert_ffn.
 */
moe_status moe_expert_up(const void* x, const int32_t* perm, const int32_t* offsets, int T, int d,
                         int d_ff, int E, int k, const void* w1, const void* w3, moe_dtype dt,
                         void* h, void* workspace, size_t ws_bytes, void* stream);
moe_status moe_expert_down(const void* h, const int32_t* offsets, int T, int d, int d_ff, int E,
                           int k, const void* w2, moe_dtype dt, void* out, void* workspace,
                           size_t ws_bytes, void* stream);

/*
 * moe_combine -- Combine (the tirogla page, How it works step 5 and Code `combine`):
 *
 *   y[t] = sum over s with inv[t*k+s] >= 0 of topk_gate[t,s] * expert_out[inv[t*k+s]]
 *          (+ shared_out[t] with weight 1 when shared_out is not NULL)
 *
 * Dropped assignments add nothing; the residual is not included (a token whose assignments were
 * all dropped gets y = 0, or its shared output).  Sums in fp32, rounds y once to dtype `dt`.
 * expert_out [T*k][d]; inv [T*k]; topk_gate [T,k] fp32, or NULL for weight 1 on every slot (the
 * backward pass adds each token's input-gradient rows this way); shared_out [T][d] or NULL;
 * y [T][d].  k may be up to 1024 here (the expert-choice layout passes k = E, inv = slot and
 * topk_gate = scores; see moe_expert_choice).
 */
moe_status moe_combine(const void* expert_out, const int32_t* inv, const float* topk_gate, int T,
                       int d, int k, moe_dtype dt, const void* shared_out, void* y, void* stream);

/*
 * moe_aux_loss -- Balance (the tirogla page, How it works step 6 and Code `aux_loss`, `z_loss`):
 *
 *   aux[0] = alpha * E * sum_e f_e * P_e,  f_e = counts[e] / (T*k),  P_e = prob_sum[e] / T
 *   z[0]   = beta * lse_sq_sum[0] / T
 *
 * counts from moe_dispatch (before capacity); prob_sum and lse_sq_sum from moe_route.  aux and z
 * are fp32 [1] each.  Equals alpha exactly in real arithmetic when either f or P is uniform.
 */
moe_status moe_aux_loss(const int32_t* counts, const float* prob_sum, const float* lse_sq_sum,
                        int T, int E, int k, float alpha, float beta, float* aux, float* z,
                        void* stream);

/*
 * moe_update_select_bias -- one aux-loss-free balancing step after a layer call (the tirogla page,
 * Implementation notes, where each bias moves after every step in the direction its expert's load
 * calls for; the dineshblog page, section 8.2, where it rises for experts that get too few tokens
 * and falls for those that get too many):
 *
 *   select_bias[e] += rate * sign(T*k - E*counts[e])      in place, fp32
 *
 * i.e. a fixed-size step towards the mean load T*k/E (counts from moe_dispatch, before capacity).
 * counts [E] int32, select_bias [E] fp32, device memory.
 */
moe_status moe_update_select_bias(const int32_t* counts, int T, int E, int k, float rate,
                                  float* select_bias, void* stream);

/*
 * moe_transpose -- weight layout conversion, outside the per-call path.  For b < batch:
 *
 *   dst[b][c][r] = src[b][r][c]      src [batch][rows][cols], dst [batch][cols][rows], dtype `dt`
 *
 * i.e. the column-major storage of a row-major rows x cols matrix.  Weights held row-major in the
 * pages' shapes (w1, w3: d x d_ff; w2: d_ff x d; W_r: d x E) become the arrays moe_route and
 * moe_expert_ffn take: call it once when the weights are loaded.  src and dst must not overlap.
 * Enqueues on `stream`; MOE_ERR_ARG for null pointers or non-positive sizes, MOE_ERR_UNSUPPORTED
 * when batch*rows*cols does not fit in 64-bit or a grid dimension exceeds 65535 blocks.
 */
moe_status moe_transpose(const void* src, int batch, int rows, int cols, moe_dtype dt, void* dst,
                         void* stream);

/*
 * moe_reroute -- overflow routed to the next-best expert instead of dropped (the chipfoundry
 * glossary entry on MoE, Architecture Components, Expert Capacity; the dineshblog page, section
 * 3.2: or routed to their second choice).  Runs after moe_route and moe_dispatch with capacity C
 * (its offsets and inv are round 1) and adds round 2: the j-th overflowed slot (slot order) of
 * token t proposes the token's expert of rank k + j in the ranking of moe_route (same scores,
 * select_bias included, same tie order); proposals take the room each expert has left after
 * round 1, in increasing assignment order; a proposal with no room, or a slot with no rank k + j
 * (k + j >= E), is dropped.
 *
 *   topk_idx2 [T,k]   topk_idx with each overflowed slot replaced by its proposal (kept or not)
 *   topk_gate2 [T,k]  the gating function over topk_idx2 (tokens with no overflow keep topk_gate)
 *   offsets2 [E+1], perm2 [T*k], inv2 [T*k], n_dropped2 [1]: the dispatch layout of the final
 *                     assignment, each expert's round-1 rows first, then its round-2 rows, each in
 *                     increasing assignment order (same conventions as moe_dispatch)
 *
 * logits [T,E] fp32 and select_bias [E] (or NULL) as given to moe_route; topk_idx, topk_gate from
 * moe_route; offsets, inv from moe_dispatch (capacity <= 0: nothing overflows and the outputs repeat
 * the inputs).  counts from moe_dispatch still feed moe_aux_loss (f counts the router's choices).
 * Workspace: (2 T k + E) int32 (covered by moe_workspace_bytes).  Deterministic.
 */
moe_status moe_reroute(const float* logits, const float* select_bias, const int32_t* topk_idx,
                       const float* topk_gate, const int32_t* offsets, const int32_t* inv, int T,
                       int E, int k, int capacity, moe_gating gating, int32_t* topk_idx2,
                       float* topk_gate2, int32_t* offsets2, int32_t* perm2, int32_t* inv2,
                       int32_t* n_dropped2, void* workspace, size_t ws_bytes, void* stream);

/*
 * moe_expert_choice -- Expert Choice routing (the starphix page, Router Variants: experts choose
 * tokens, with perfect load balance; the chipfoundry glossary entry on MoE, Routing Strategies and
 * Variants: experts select their top tokens instead of tokens selecting experts, no balancing
 * loss needed).  With p the router's softmax over experts and c = min(C, T):
 *
 *   scores[t,e]   = p[t,e] = exp(L[t,e] - m_t) / sum_j exp(L[t,j] - m_t)   fp32 [T,E] (output, or
 *                   input with MOE_EC_SCORES_IN, in which case logits may be NULL)
 *   expert e keeps the c tokens with the largest scores[.,e]; equal scores go to the lower token
 *   index (-0.0 equals +0.0); its rows are listed in increasing token order:
 *   offsets[e]    = e*c                                   int32 [E+1]
 *   perm[e*c + i] = the i-th kept token of expert e       int32 [E*c]
 *   gate[e*c + i] = scores[perm[e*c+i], e]                fp32 [E*c]
 *   slot[t*E + e] = the row of (t, e), or -1 when e did not keep t          int32 [T*E]
 *
 * logits [T,E] fp32 from moe_route (its top-k outputs are not used).  The layer then runs
 *   moe_expert_ffn_gathered(x, perm, offsets, ..., rows_max = E*c, ...) -> out [E*c][d]
 *   moe_combine(out, slot, scores, T, d, k = E, ...)   y[t] = sum over e keeping t of p[t,e] out[row]
 * (E <= 1024).  A token that no expert keeps gets y = 0 (or its shared output).  No workspace.
 * Deterministic: the selection is exact on the fp32 scores.
 */
moe_status moe_expert_choice(const float* logits, int T, int E, int C, unsigned flags,
                             float* scores, int32_t* offsets, int32_t* perm, float* gate,
                             int32_t* slot, void* stream);

/*
 * moe_expert_ffn_gathered -- moe_expert_ffn on explicit rows: row r of expert e
 * (offsets[e] <= r < offsets[e+1], offsets[E] <= rows_max) reads x row rows[r] (a token index in
 * [0, T)).  out [rows_max][d]; the workspace is moe_gathered_workspace_bytes(rows_max, ...).
 * Otherwise as moe_expert_ffn (weights, dtype, split-K determinism, errors).
 */
size_t moe_gathered_workspace_bytes(int rows_max, int d, int d_ff, int E, moe_dtype dt);
moe_status moe_expert_ffn_gathered(const void* x, const int32_t* rows, const int32_t* offsets,
                                   int T, int d, int d_ff, int E, int rows_max, const void* w1,
                                   const void* w3, const void* w2, moe_dtype dt, void* out,
                                   void* workspace, size_t ws_bytes, void* stream);

/*
 * Weight-only quantized experts (the starphix page, Inference Optimization, Quantization: experts
 * in INT8 or INT4 while the router stays 16-bit; the vanos001 page, Quantized Experts).  One fp32
 * scale per output channel (per row of a stored [out][in] weight matrix):
 *
 *   s[row] = max_c |w[row][c]| / Q,  Q = 127 (bits 8) or 7 (bits 4)        (fp32 division)
 *   q[row][c] = rint(w[row][c] / s[row]) clamped to [-Q, Q]; a zero row has s = 0, q = 0
 *
 * moe_quantize_weights converts bf16 weights [batch][rows][cols] (the storage moe_expert_ffn takes:
 * w1, w3 [E][d_ff][d], w2 [E][d][d_ff]) into q: int8 [batch][rows][cols] (bits 8) or bytes
 * [batch][rows][cols/2] holding columns 2j (low nibble) and 2j+1 (high nibble) as 4-bit two's
 * complement (bits 4; cols even), and scale fp32 [batch][rows].  Load time, not per call.
 *
 * moe_expert_ffn_q is moe_expert_ffn with the dequantized weights s * q: activations bf16, products
 * formed exactly from the integer weights, fp32 accumulation, the scale applied to each output;
 * h rounded to bf16 between the two GEMMs.  q1, q3 with s1, s3 [E][d_ff]; q2 with s2 [E][d].
 * bf16 layers only; d and d_ff must be multiples of 128.  Its kernels are made for decode-sized
 * groups (the weight stream bounds them; INT8 halves and INT4 quarters the streamed bytes).
 * Workspace: moe_q_workspace_bytes.  Deterministic (fixed-order split-K sums).
 */
size_t moe_q_workspace_bytes(int T, int d, int d_ff, int E, int k, int bits);
moe_status moe_quantize_weights(const void* w, int batch, int rows, int cols, moe_dtype dt,
                                int bits, void* q, float* scale, void* stream);
moe_status moe_expert_ffn_q(const void* x, const int32_t* perm, const int32_t* offsets, int T,
                            int d, int d_ff, int E, int k, int bits, const void* q1,
                            const float* s1, const void* q3, const float* s3, const void* q2,
                            const float* s2, moe_dtype dt, void* out, void* workspace,
                            size_t ws_bytes, void* stream);

/*
 * Backward pass.  The objective is J = <dy, y> + aux + z: a task loss whose gradient with respect
 * to y is dy [T][d], plus the two router losses of moe_aux_loss (the tirogla page, How it works
 * step 6: f_e is a count and carries no gradient, P_e and the logsumexp do; the vanos001 page,
 * Load Balancing Loss, adds the balancing term to the task loss).  The selection (top-k, capacity
 * drops, a selection bias) carries no gradient; it only decides which experts the gradient flows
 * through.  Chain, in the reverse order of the forward steps (every buffer from the forward call
 * is an input):
 *
 *   moe_combine_backward(dy, expert_out, inv, topk_gate)   -> d_out [T*k][d], d_gate [T,k]
 *   moe_expert_backward(x, perm, offsets, w1, w3, w2, d_out) -> dx_rows [T*k][d], dw1, dw3, dw2
 *   moe_expert_backward(x, NULL, NULL, w1s, w3s, w2s, dy)  -> dxs [T][d], dw1s, dw3s, dw2s
 *                                                              (shared expert, gate weight 1)
 *   moe_route_backward(..., d_gate, counts, dx_add = dxs)   -> d_logits [T,E], dw_r [E][d], dx_r
 *   moe_combine(dx_rows, inv, NULL, ..., shared_out = dx_r) -> dx [T][d]
 *
 * bf16 layers only (MOE_ERR_UNSUPPORTED for MOE_F32 where noted); weight gradients are fp32,
 * activation gradients in the layer dtype, accumulation fp32.  Results are bitwise deterministic
 * run to run.  Same argument conventions and errors as the forward calls.
 */

/* Workspace bytes that cover every backward call below for this layer shape (0 for MOE_F32). */
size_t moe_backward_workspace_bytes(int T, int d, int d_ff, int E, int k, moe_dtype dt);

/*
 * moe_combine_backward -- gradient of Combine: for a kept assignment a = t*k+s with row
 * r = inv[a],
 *
 *   d_out[r]    = topk_gate[t,s] * dy[t]          bf16 [T*k][d] (rows r < offsets[E] written)
 *   d_gate[t,s] = sum_i dy[t,i] * expert_out[r,i]  fp32 [T,k], 0 for a dropped assignment
 *
 * dy [T][d], expert_out [T*k][d] (the forward expert rows), inv [T*k], topk_gate [T,k] fp32.
 * MOE_F32 is unsupported.
 */
moe_status moe_combine_backward(const void* dy, const void* expert_out, const int32_t* inv,
                                const float* topk_gate, int T, int d, int k, moe_dtype dt,
                                void* d_out, float* d_gate, void* stream);

/*
 * moe_expert_backward -- gradient of Compute for the SwiGLU experts of moe_expert_ffn, given the
 * gradient d_out of every expert row.  With a = x_t w1_e^T, b = x_t w3_e^T, h = silu(a) * b:
 *
 *   dh      = d_out[r] w2_e                      (recomputing a and b from x, w1, w3)
 *   da      = dh * b * silu'(a),  db = dh * silu(a)
 *   dx_rows[r] = da w1_e + db w3_e               [T*k][d] dtype, one row per expert row r
 *   dw1[e]  = sum_r da_r^T x_t,  dw3[e] = sum_r db_r^T x_t,  dw2[e] = sum_r d_out[r]^T h_r
 *
 * Same row convention, weight storage and dense (perm == NULL, E == 1) mode as moe_expert_ffn;
 * dw1, dw3 [E][d_ff][d] and dw2 [E][d][d_ff] fp32 in that same storage (experts with no rows get
 * zeros).  Rows of dx_rows past offsets[E] are not written.  Intermediates (dh, h, da, db) are
 * rounded to bf16.  The workspace (moe_backward_workspace_bytes) holds the intermediates and
 * transposed copies of the activations (about 8 T k (d + d_ff) bytes); when d_ff is not a
 * multiple of 64 it also holds transposed copies of the weights (3 E d d_ff bf16 more).  MOE_F32 is
 * unsupported.
 */
moe_status moe_expert_backward(const void* x, const int32_t* perm, const int32_t* offsets, int T,
                               int d, int d_ff, int E, int k, const void* w1, const void* w3,
                               const void* w2, const void* d_out, moe_dtype dt, void* dx_rows,
                               float* dw1, float* dw3, float* dw2, void* workspace,
                               size_t ws_bytes, void* stream);

/*
 * Saved activations: the same backward without recomputing a and b.  A training step that can hold
 * 3 * rows * d_ff bf16 values per expert layer (rows = T*k, or T in dense mode) runs the forward
 * Compute step as
 *
 *   moe_expert_ffn_save(x, perm, offsets, ..., out, saved)  -> out as moe_expert_ffn, and
 *       saved [rows][3 * d_ff] bf16: row r holds h_r | a_r | b_r (h exactly the values the down
 *       projection read; a and b rounded to bf16 from the fp32 sums h was computed from)
 *
 * and the Compute gradient as
 *
 *   moe_expert_backward_saved(saved, x, perm, offsets, ...) -> the outputs of moe_expert_backward
 *
 * whose dh product applies the SwiGLU derivative (da = dh * b * silu'(a), db = dh * silu(a), with
 * the saved bf16 a and b) in its epilogue and whose dw2 reads the saved h.  This removes the
 * recomputed up projection (a third of the Compute backward's matrix work) at the price of the
 * stored activations; the results differ from moe_expert_backward only by the bf16 rounding of a
 * and b (dw2 is the same).  Arguments, layouts and errors otherwise as moe_expert_ffn and
 * moe_expert_backward; moe_expert_ffn_save's workspace may be smaller than moe_workspace_bytes
 * (it holds no h) and moe_expert_backward_saved takes moe_backward_workspace_bytes.  bf16 only
 * (MOE_ERR_UNSUPPORTED for MOE_F32, or when saved exceeds 2 GiB); saved must be 16-byte aligned
 * (MOE_ERR_ARG).
 */
moe_status moe_expert_ffn_save(const void* x, const int32_t* perm, const int32_t* offsets, int T,
                               int d, int d_ff, int E, int k, const void* w1, const void* w3,
                               const void* w2, moe_dtype dt, void* out, void* saved,
                               void* workspace, size_t ws_bytes, void* stream);
moe_status moe_expert_backward_saved(const void* saved, const void* x, const int32_t* perm,
                                     const int32_t* offsets, int T, int d, int d_ff, int E, int k,
                                     const void* w1, const void* w3, const void* w2,
                                     const void* d_out, moe_dtype dt, void* dx_rows, float* dw1,
                                     float* dw3, float* dw2, void* workspace, size_t ws_bytes,
                                     void* stream);

/*
 * moe_route_backward -- gradient of Score and of the two router losses:
 *
 *   d_logits[t,.] = (gating function's derivative) applied to d_gate[t,.]
 *                   + p_t (c - <p_t, c>),  c_e = alpha * E * counts[e] / (T*k) / T   (aux)
 *                   + 2 * beta * lse_t * p_t / T                                   (z)
 *   dw_r[e][j]   = sum_t d_logits[t,e] x[t,j]                  fp32 [E][d] (w_r's storage)
 *   dx[t][j]     = sum_e d_logits[t,e] w_r[e][j] (+ dx_add[t][j])        dtype [T][d]
 *
 * where p_t is the full softmax of logits row t and lse_t its logsumexp; the gating derivatives
 * are those of the forward gates (softmax over the selected, softmax over all, or sigmoids
 * renormalised over the selected).  logits [T,E] fp32, topk_idx, topk_gate from moe_route; d_gate
 * from moe_combine_backward; counts from moe_dispatch (may be NULL when alpha == 0); dx_add [T][d]
 * or NULL.  d_logits [T,E] fp32 is an output.  fp32 sums throughout; dw_r is added over token
 * chunks in a fixed order.  For bf16 with E a multiple of 64 the two products run on the matrix
 * cores: d_logits enters as three bf16 terms (hi, mid, lo: their sum is d_logits to within
 * 2^-24 relative), dw_r takes all three and dx the first two (2^-16 relative, below the bf16
 * rounding of dx); dx_add is added before dx is rounded.  Workspace: moe_backward_workspace_bytes.
 */
moe_status moe_route_backward(const void* x, const void* w_r, const float* logits,
                              const int32_t* topk_idx, const float* topk_gate,
                              const float* d_gate, const int32_t* counts, int T, int d, int E,
                              int k, moe_dtype dt, moe_gating gating, float alpha, float beta,
                              const void* dx_add, float* d_logits, float* dw_r, void* dx,
                              void* workspace, size_t ws_bytes, void* stream);

/*
 * Measured ceilings (not part of the layer): the benchmark reports them beside the published
 * peaks of the chip.
 *
 * moe_peak_mfma runs `blocks` blocks of 8 waves; every wave issues iters * 8 bf16 32x32x16 matrix
 * instructions (8 independent fp32 accumulators, operands held in registers), i.e.
 * blocks * 8 * iters * 8 * 32768 FLOPs per call.  operands: 2048 bf16 values (16-byte aligned;
 * two alternating operand sets, 64 lanes x 8 values each for A and B); out: blocks * 512 fp32
 * sums of the accumulators (written so that no instruction is dead; the values carry no meaning).
 *
 * moe_peak_copy copies `bytes` (a multiple of 16, both pointers 16-byte aligned) from src to dst
 * with 16-byte loads and stores: 2 * bytes of HBM traffic per call for buffers larger than the
 * caches.  src and dst must not overlap.
 */
moe_status moe_peak_mfma(const void* operands, int blocks, int iters, float* out, void* stream);
moe_status moe_peak_copy(const void* src, void* dst, size_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBMOE_MOE_H */
