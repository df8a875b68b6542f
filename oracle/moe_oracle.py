"""CPU oracle for the forward and backward passes of one top-k routed Mixture-of-Experts FFN layer,
its Expert Choice and overflow-rerouting variants, and weight-only quantized experts.

TEST INFRASTRUCTURE. Only the test suite, the smoke check and the CPU-baseline leg of the
benchmark may import this module. The product path (the HIP library and its binding) never
imports, links or calls it, and this module imports nothing from the product path: it is plain,
slow, obviously-correct NumPy, written from the pages listed below, in float64 on inputs that are
widened exactly (a bfloat16 value held in a float32 array is exact, and float32 -> float64 is
exact).

Pages (cited by title and section; nothing here copies their code):
  [tirogla]  "Mixture of experts (MoE)" -- tirogla.com/machine-learning/mixture-of-experts.html
             ("How it works" steps 1-6; "Code": route, dispatch, aux_loss, z_loss, combine, main;
             "Complexity and constants"; "Implementation notes").
  [dinesh]   "DL S077 - Mixture of Experts (MoE) Intuition" -- dineshblog.com/blog/session-dl-077-moe
             (1.1 What an "expert" is; 1.2 What the router computes; 2 Top-k gating, step by
             step; 3.1 The auxiliary loss; 3.2 Why not just enforce balance?; 4 The
             parameter-count arithmetic; 8.2 DeepSeek-V2 -> V3 -> R1).
  [starphix] "Mixture of Experts (MoE)" -- learn.starphix.com ... ModelArchitectures/Mixture-of-Experts.md
             (Key Equations; Top-k Gating; Router Variants; Expert Architectures: Shared +
             Specialized; Inference Optimization: Quantization).
  [vanos]    "Mixture of Experts (MoE)" -- vanos001.github.io/placement_prep/llm/moe
             (Load Balancing Loss; Quantized Experts).
  [chipfoundry] "Mixture of Experts (MoE) architecture" glossary entry -- chipfoundryservices.com
             (MoE Architecture Components: the router is trained end to end by gradient descent).

Readings taken where the pages are silent or disagree (each one is also listed with its reason in
the design notes of this repository):
  * W_r is the d x E matrix of [tirogla] How it works, held as its [E, d] transpose (the weight of
    the bias-free linear router of [dinesh] 1.2), logits = x . W_r; no biases except an explicit
    per-expert logit bias input.
  * Ranking is always on the float32 logits, descending, equal logits to the lower expert index
    first (the stable sort of [tirogla] Code `route`); -0.0 == +0.0; -inf ranks last; NaN rejected.
  * Sigmoid gating: g = sigmoid(L_e) / sum over the selected sigmoid(L_s), no extra scale
    ([tirogla] How it works, step 1).
  * f_e = (assignments to e before capacity) / (T*k); P_e = mean over tokens of the full softmax;
    L_aux = alpha * E * sum_e f_e * P_e ([tirogla] step 6 and Code `aux_loss`).  The full softmax
    is used for P in every gating mode.
  * z = beta * mean over tokens of logsumexp(row)^2 ([tirogla] step 6; Code `z_loss`).
  * Capacity C counts assignments per expert; C <= 0 or None means unlimited; overflow is dropped
    in assignment order a = t*k + s, earlier tokens first ([tirogla] Code `dispatch`).
  * y excludes the residual; a dropped assignment contributes 0 ([tirogla] step 5).
  * A shared expert is added to every token with weight 1 ([starphix] Shared + Specialized).
  * token(a) = floor(a / k) for assignment a = t*k + s ([tirogla] Code `combine`).
  * Aux-loss-free balancing ([tirogla] Implementation notes; [dinesh] 8.2): a per-expert selection
    bias is added (float32) to the logits used for ranking only; gates, P and z use the logits.
    After a step each bias moves by a fixed `rate` towards balance: +rate when the expert's load is
    below the mean T*k/E, -rate above it, 0 at it.  [dinesh] 9 mentions an exponential moving
    average of relative load instead; a fixed-size step whose direction comes from the load is the
    plainer reading of [tirogla] and is the one built.

Pins: every function here is checked by the CPU tests against page-printed values (the worked
top-2 example of [dinesh] section 2), closed forms, invariants stated on the pages, library
routines on special cases and brute force on tiny inputs.  The exact float32 bits of gates and y
on the GPU are compared only within tolerances.  Parity unpinned beyond self-consistency: the
sigmoid-mode P_e reading and the Zipf logit-bias input recipe (conventions, no page value).
"""

import math

import numpy as np

# Gating modes (values follow the C header's enum so that test code can pass either).
SOFTMAX_TOPK = 0   # softmax over the k selected logits (Mixtral)
SOFTMAX_ALL = 1    # softmax over all E logits, keep the selected probabilities (Switch / GShard)
SIGMOID_TOPK = 2   # sigmoid affinities renormalised over the selected experts (DeepSeek-V3)


# Working precision of the floating-point arithmetic: float64 (the default, what every check
# uses).  The benchmark's CPU-baseline leg times the same code in float32 (working_precision).
_WORK = [np.float64]


class working_precision:
    """Context manager: run the oracle's floating-point arithmetic in `dtype` (np.float32 or
    np.float64) inside the block.  Only the benchmark's timing of a float32 pass uses it."""

    def __init__(self, dtype):
        self.dtype = np.dtype(dtype).type
        self.prev = None

    def __enter__(self):
        self.prev = _WORK[0]
        _WORK[0] = self.dtype
        return self

    def __exit__(self, *exc):
        _WORK[0] = self.prev
        return False


def _f64(a):
    return np.asarray(a, dtype=_WORK[0])


def router_logits(x, w_r, bias=None, exact=False):
    """Router scores, [tirogla] How it works step 1 (Score) and [dinesh] 1.2 What the router computes.

    logits[t, e] = sum_j x[t, j] * W_r[e, j] (+ bias[e]); x [T, d], W_r [E, d] (the [out][in]
    weight of the bias-free linear layer that [dinesh] 1.2 declares as the router).  Computed in float64
    on the given values and rounded once to float32 (logits are always float32: [tirogla]
    Implementation notes ask for float32 router math).
    """
    L = _f64(x) @ _f64(w_r).T
    if bias is not None:
        L = L + _f64(bias)[None, :]
    return L if exact else L.astype(np.float32)


def select_topk(logits, k, select_bias=None):
    """Top-k experts per token, [tirogla] How it works step 2 (Select) and Code `route`.

    Each row is ordered by a stable descending sort on its float32 logits (equal logits keep the
    lower expert index first) and the first k are kept, in that order.  Returns int32 [T, k].

    select_bias (float32 [E] or None): aux-loss-free balancing ([tirogla] Implementation notes;
    [dinesh] 8.2): the ranking uses the float32 sum logit + select_bias[e]; the gates do not (see
    gate_weights, which takes the logits alone).
    """
    L = np.asarray(logits, dtype=np.float32)
    if select_bias is not None:
        L = L + np.asarray(select_bias, dtype=np.float32)[None, :]   # one float32 rounding
    if L.ndim != 2:
        raise ValueError("logits must be [T, E]")
    T, E = L.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    if np.isnan(L).any():
        raise ValueError("NaN logit: ranking is undefined")
    idx = np.empty((T, k), dtype=np.int32)
    for t in range(T):
        row = [float(v) for v in L[t]]        # python floats: -0.0 == 0.0, -inf sorts last
        order = sorted(range(E), key=lambda e: (-row[e], e))
        idx[t] = order[:k]
    return idx


def row_softmax_lse(logits):
    """Full-row softmax p[t, :] and logsumexp lse[t], [tirogla] Code `route` (probs) and `z_loss`.

    Shifted by the row maximum m: p = exp(L - m) / sum exp(L - m), lse = m + ln sum exp(L - m).
    """
    L = _f64(logits)
    m = L.max(axis=1, keepdims=True)
    ex = np.exp(L - m)
    s = ex.sum(axis=1, keepdims=True)
    return ex / s, m[:, 0] + np.log(s[:, 0])


def gate_weights(logits, idx, mode):
    """Mixture weights of the selected experts, [tirogla] How it works step 1 and Code `route`.

    SOFTMAX_TOPK: exp(L_e - m) / sum over selected exp(L_s - m)  ([dinesh] section 2; [starphix]
                  Top-k Gating).
    SOFTMAX_ALL:  exp(L_e - m) / sum over all j exp(L_j - m)      (Switch / GShard).
    SIGMOID_TOPK: sigmoid(L_e) / sum over selected sigmoid(L_s)    (DeepSeek-V3).
    m is the full-row maximum.  float64 [T, k].
    """
    L = _f64(logits)
    T, E = L.shape
    k = idx.shape[1]
    g = np.empty((T, k), dtype=_WORK[0])
    with np.errstate(over="ignore"):
        for t in range(T):
            row = L[t]
            sel = row[idx[t]]
            m = row.max()
            if mode == SOFTMAX_TOPK:
                w = np.exp(sel - m)
                g[t] = w / w.sum()
            elif mode == SOFTMAX_ALL:
                g[t] = np.exp(sel - m) / np.exp(row - m).sum()
            elif mode == SIGMOID_TOPK:
                s = 1.0 / (1.0 + np.exp(-sel))
                g[t] = s / s.sum()
            else:
                raise ValueError("unknown gating mode %r" % (mode,))
    return g


def dispatch(idx, E, capacity=None):
    """Counting sort of assignments by expert with capacity, [tirogla] How it works step 3 and
    Code `dispatch`; capacity as in [dinesh] 3.2.

    Assignments a = t*k + s are visited in increasing a, so earlier tokens have priority.  Each expert
    keeps its first `capacity` assignments; later ones are dropped.  Returns
      counts   int32 [E]    assignments per expert before capacity,
      offsets  int32 [E+1]  exclusive prefix sum of the kept counts,
      perm     int32 [n_kept] kept assignment ids, expert-major, increasing a within an expert,
      inv      int32 [T*k]  position of a in perm, or -1 when a was dropped,
      n_dropped int.
    capacity None or <= 0 means unlimited.
    """
    flat = np.asarray(idx).reshape(-1)
    A = flat.size
    cap = A if (capacity is None or capacity <= 0) else int(capacity)
    counts = [0] * E
    lists = [[] for _ in range(E)]
    n_dropped = 0
    for a in range(A):
        e = int(flat[a])
        counts[e] += 1
        if len(lists[e]) < cap:
            lists[e].append(a)
        else:
            n_dropped += 1
    offsets = [0]
    for e in range(E):
        offsets.append(offsets[-1] + len(lists[e]))
    perm = np.array([a for e in range(E) for a in lists[e]], dtype=np.int32)
    inv = np.full(A, -1, dtype=np.int32)
    inv[perm] = np.arange(perm.size, dtype=np.int32)
    return (np.array(counts, dtype=np.int32), np.array(offsets, dtype=np.int32), perm, inv,
            n_dropped)


def dispatch_reroute(logits, idx, E, capacity, select_bias=None):
    """Overflow routed to the next-best expert instead of dropped ([chipfoundry] MoE Architecture
    Components, Expert Capacity: tokens past capacity are dropped or sent to their next-best expert;
    [dinesh] 3.2: or routed to their second choice).  Reading, in two rounds:
      round 1: dispatch(idx, E, capacity): each expert keeps its first C assignments;
      round 2: the j-th overflowed slot of token t (slots in order, j = 0, 1, ...) proposes the
               token's expert of rank k + j in its full ranking (the order of select_topk over all
               E, so never one of its top k); proposals take the room each expert has left after
               round 1 (C - kept) in increasing assignment order; a proposal that finds no room, or
               a slot with no rank k + j (k + j >= E), is dropped.
    Returns (idx2, offsets, perm, inv, n_dropped): idx2 [T, k] is idx with each overflowed slot
    replaced by its proposal (kept or not); within an expert the round-1 rows (increasing a) come
    before the round-2 rows (increasing a)."""
    idx = np.asarray(idx)
    T, k = idx.shape
    A = T * k
    cap = A if (capacity is None or capacity <= 0) else int(capacity)
    counts, off1, perm1, inv1, _ = dispatch(idx, E, capacity)
    order = select_topk(logits, E, select_bias)
    idx2 = idx.copy()
    proposal = np.full(A, -1, dtype=np.int64)
    for t in range(T):
        j = 0
        for s in range(k):
            a = t * k + s
            if inv1[a] < 0:
                if k + j < E:
                    proposal[a] = int(order[t, k + j])
                    idx2[t, s] = proposal[a]
                j += 1
    lists = [list(perm1[off1[e]:off1[e + 1]]) for e in range(E)]
    room = [cap - len(lists[e]) for e in range(E)]
    extra = [[] for _ in range(E)]
    for a in range(A):
        e = int(proposal[a])
        if e >= 0 and room[e] > 0:
            extra[e].append(a)
            room[e] -= 1
    offsets = [0]
    for e in range(E):
        offsets.append(offsets[-1] + len(lists[e]) + len(extra[e]))
    perm = np.array([a for e in range(E) for a in lists[e] + extra[e]], dtype=np.int32)
    inv = np.full(A, -1, dtype=np.int32)
    inv[perm] = np.arange(perm.size, dtype=np.int32)
    return (idx2.astype(np.int32), np.array(offsets, dtype=np.int32), perm, inv,
            int(A - offsets[-1]))


def silu(z):
    """silu(z) = z * sigmoid(z) = z / (1 + exp(-z))."""
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu_ffn(X, w1, w3, w2):
    """SwiGLU expert, [dinesh] 1.1 What an "expert" is: w2(silu(w1(x)) * w3(x)), each w a linear
    layer without bias, applied as x -> x W^T.

    X [n, d]; w1, w3 [d_ff, d] (w1 is the gate branch, w3 the up branch); w2 [d, d_ff]: the
    [out][in] weights of those layers.  float64.
    """
    X = _f64(X)
    return (silu(X @ _f64(w1).T) * (X @ _f64(w3).T)) @ _f64(w2).T


def expert_rows(x, perm, offsets, k, w1, w3, w2):
    """Each expert on its contiguous batch, [tirogla] How it works step 4 (Compute).

    Row r of the result is expert e's output for token perm[r] // k, where
    offsets[e] <= r < offsets[e+1].  float64 [offsets[E], d].
    """
    x = np.asarray(x)
    E = len(offsets) - 1
    out = np.zeros((int(offsets[E]), x.shape[1]), dtype=_WORK[0])
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            tok = np.asarray(perm[lo:hi]) // k
            out[lo:hi] = swiglu_ffn(x[tok], w1[e], w3[e], w2[e])
    return out


def combine(out_rows, inv, gate, T, k, shared_out=None):
    """Gate-weighted combine, [tirogla] How it works step 5 and Code `combine`.

    y[t] = sum over slots s with inv[t*k+s] >= 0 of gate[t, s] * out_rows[inv[t*k+s]]; dropped
    assignments add nothing and the residual is not included.  With a shared expert, its output is
    added with weight 1 ([starphix] Shared + Specialized).  float64 [T, d].
    """
    out_rows = _f64(out_rows)
    d = out_rows.shape[1] if out_rows.ndim == 2 and out_rows.shape[0] else (
        shared_out.shape[1] if shared_out is not None else 0)
    inv = np.asarray(inv).reshape(T, k)
    g = _f64(gate).reshape(T, k)
    y = np.zeros((T, d), dtype=_WORK[0])
    for s in range(k):
        keep = inv[:, s] >= 0
        y[keep] += g[keep, s, None] * out_rows[inv[keep, s]]
    if shared_out is not None:
        y += _f64(shared_out)
    return y


def aux_loss(counts, prob_sum, T, E, k, alpha):
    """Load-balancing loss, [tirogla] How it works step 6 and Code `aux_loss`:
    alpha * E * sum_e f_e * P_e with f_e = counts_e / (T*k) and P_e = prob_sum_e / T."""
    f = _f64(counts) / float(T * k)
    P = _f64(prob_sum) / float(T)
    return alpha * E * float(np.sum(f * P))


def z_loss(lse_sq_sum, T, beta):
    """Router z-loss, [tirogla] How it works step 6 and Code `z_loss`: beta * mean_t lse_t^2."""
    return beta * float(lse_sq_sum) / float(T)


def forward(x, w_r, w1, w3, w2, k, mode, capacity=None, bias=None, shared=None,
            alpha=0.01, beta=1e-3, logits=None, select_bias=None, exact_logits=False,
            reroute=False):
    """The whole layer, steps in the order of [tirogla] How it works (Score, Select, Dispatch,
    Compute, Combine, Balance).

    x [T, d]; w_r [E, d]; w1, w3 [E, d_ff, d]; w2 [E, d, d_ff]; shared = (w1s, w3s, w2s) or None.
    `logits` (float32 [T, E]) replaces the router product when given; `select_bias` (float32 [E])
    biases the ranking only (aux-loss-free balancing).  exact_logits keeps the router product in
    float64 instead of rounding it to float32 (for finite-difference checks of the gradients).
    reroute sends overflowed assignments to their next-best expert (dispatch_reroute) instead of
    dropping them; the gates are then those of the final selection and f still counts the router's
    first choices before capacity.
    Returns a dict of every intermediate (float64 except the integer dispatch outputs).
    """
    x = np.asarray(x)
    T = x.shape[0]
    if logits is None:
        logits = router_logits(x, w_r, bias, exact=exact_logits)
    logits = np.asarray(logits, dtype=np.float64 if exact_logits else np.float32)
    E = logits.shape[1]
    idx = select_topk(logits, k, select_bias)
    p, lse = row_softmax_lse(logits)
    counts, offsets, perm, inv, n_dropped = dispatch(idx, E, capacity)
    first_choice = idx
    if reroute:
        idx, offsets, perm, inv, n_dropped = dispatch_reroute(logits, first_choice, E, capacity,
                                                              select_bias)
    gate = gate_weights(logits, idx, mode)
    rows = expert_rows(x, perm, offsets, k, w1, w3, w2)
    shared_out = None
    if shared is not None:
        shared_out = swiglu_ffn(x, *shared)
    y = combine(rows, inv, gate, T, k, shared_out)
    prob_sum = p.sum(axis=0)
    lse_sq_sum = float(np.sum(lse * lse))
    return dict(logits=logits, topk_idx=idx, first_choice=first_choice, topk_gate=gate, probs=p,
                lse=lse,
                prob_sum=prob_sum, lse_sq_sum=lse_sq_sum, counts=counts, offsets=offsets,
                perm=perm, inv=inv, n_dropped=n_dropped, expert_out=rows, shared_out=shared_out,
                y=y, aux=aux_loss(counts, prob_sum, T, E, k, alpha),
                z=z_loss(lse_sq_sum, T, beta))


# ------------------------------------------------------------------------------------------------
# Backward pass.  The objective is J = <dy, y> + L_aux + z: a task loss whose gradient with respect
# to the layer output is dy, plus the two router losses of [tirogla] How it works step 6 (the total
# loss of [vanos] Load Balancing Loss adds the balancing term to the task loss; the router is
# trained end to end by gradient descent, [chipfoundry] MoE Architecture Components).  f_e is a
# count and carries no gradient ([tirogla] step 6 says so); P_e and lse do.  The selection (which
# experts, which assignments are dropped) is piecewise constant in the logits and carries none
# either, so a selection bias only changes which experts the gradient flows through ([dinesh] 8.2:
# the bias acts on routing decisions, not on the gradient path).  Each function below is the chain
# rule of one forward step, run in the reverse order of the steps.
# ------------------------------------------------------------------------------------------------


def combine_backward(dy, out_rows, inv, gate, T, k):
    """Gradient of Combine ([tirogla] How it works step 5): for a kept assignment a = t*k + s with
    row r = inv[a],  d_out[r] = gate[t, s] * dy[t]  and  d_gate[t, s] = <dy[t], out_rows[r]>;
    a dropped assignment gets d_gate = 0.  The shared expert's output enters y with weight 1, so
    its output gradient is dy itself.  float64 ([n_kept, d], [T, k])."""
    dy = _f64(dy)
    out_rows = _f64(out_rows)
    inv = np.asarray(inv).reshape(T, k)
    g = _f64(gate).reshape(T, k)
    d_out = np.zeros(out_rows.shape, dtype=_WORK[0])
    d_gate = np.zeros((T, k), dtype=_WORK[0])
    for s in range(k):
        keep = inv[:, s] >= 0
        rows = inv[keep, s]
        d_out[rows] = g[keep, s, None] * dy[keep]
        d_gate[keep, s] = np.sum(dy[keep] * out_rows[rows], axis=1)
    return d_out, d_gate


def silu_grad(z):
    """d/dz silu(z) = sigmoid(z) * (1 + z * (1 - sigmoid(z)))."""
    with np.errstate(over="ignore"):
        sg = 1.0 / (1.0 + np.exp(-z))
    return sg * (1.0 + z * (1.0 - sg))


def swiglu_ffn_backward(X, w1, w3, w2, dO):
    """Gradient of the SwiGLU expert of [dinesh] 1.1, O = H w2^T with H = silu(A) * B, A = X w1^T,
    B = X w3^T:
        dw2 = dO^T H,  dH = dO w2,  dA = dH * B * silu'(A),  dB = dH * silu(A),
        dw1 = dA^T X,  dw3 = dB^T X,  dX = dA w1 + dB w3.
    Shapes as swiglu_ffn; returns (dX, dw1, dw3, dw2), float64."""
    X = _f64(X)
    w1, w3, w2, dO = _f64(w1), _f64(w3), _f64(w2), _f64(dO)
    A = X @ w1.T
    B = X @ w3.T
    H = silu(A) * B
    dH = dO @ w2
    dA = dH * B * silu_grad(A)
    dB = dH * silu(A)
    return dA @ w1 + dB @ w3, dA.T @ X, dB.T @ X, dO.T @ H


def expert_rows_backward(x, perm, offsets, k, w1, w3, w2, d_out):
    """Gradient of Compute ([tirogla] How it works step 4) given d_out for every kept row.
    Returns dx_rows [n_kept, d] (row r: the input gradient of expert e's batch row, before the
    rows of one token are added), dx [T, d] (those rows added per token), and dw1, dw3 [E, d_ff, d],
    dw2 [E, d, d_ff] (experts with no rows get zeros).  float64."""
    x = _f64(x)
    E = len(offsets) - 1
    dx = np.zeros_like(x)
    dx_rows = np.zeros((int(offsets[E]), x.shape[1]), dtype=_WORK[0])
    dw1 = np.zeros(np.shape(w1), dtype=_WORK[0])
    dw3 = np.zeros(np.shape(w3), dtype=_WORK[0])
    dw2 = np.zeros(np.shape(w2), dtype=_WORK[0])
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            tok = np.asarray(perm[lo:hi]) // k
            dX, dw1[e], dw3[e], dw2[e] = swiglu_ffn_backward(x[tok], w1[e], w3[e], w2[e],
                                                             d_out[lo:hi])
            dx_rows[lo:hi] = dX
            np.add.at(dx, tok, dX)
    return dx_rows, dx, dw1, dw3, dw2


def gate_backward(logits, idx, mode, d_gate):
    """Gradient of the gates (gate_weights) with respect to the logits, per row t:
    SOFTMAX_TOPK: dL[e_s] = g_s (dg_s - sum_s' g_s' dg_s')        (softmax over the selected)
    SOFTMAX_ALL:  dL[j]   = p_j (dp_j - sum_i p_i dp_i), dp = dg on the selected, 0 elsewhere
    SIGMOID_TOPK: dL[e_s] = sigmoid'(L_e_s) (dg_s - sum_s' g_s' dg_s') / sum_s' sigmoid(L_e_s')
    float64 [T, E]; zero on experts that the gate does not depend on."""
    L = _f64(logits)
    T, E = L.shape
    dg_all = _f64(d_gate)
    dL = np.zeros((T, E), dtype=_WORK[0])
    with np.errstate(over="ignore"):
        for t in range(T):
            row, sel, dg = L[t], np.asarray(idx[t]), dg_all[t]
            m = row.max()
            if mode == SOFTMAX_TOPK:
                w = np.exp(row[sel] - m)
                g = w / w.sum()
                dL[t, sel] += g * (dg - np.sum(g * dg))
            elif mode == SOFTMAX_ALL:
                p = np.exp(row - m)
                p /= p.sum()
                dp = np.zeros(E)
                dp[sel] = dg
                dL[t] += p * (dp - np.sum(p * dp))
            elif mode == SIGMOID_TOPK:
                sg = 1.0 / (1.0 + np.exp(-row[sel]))
                S = sg.sum()
                g = sg / S
                dL[t, sel] += sg * (1.0 - sg) * (dg - np.sum(g * dg)) / S
            else:
                raise ValueError("unknown gating mode %r" % (mode,))
    return dL


def balance_backward(logits, counts, T, E, k, alpha, beta):
    """Gradient of L_aux + z with respect to the logits ([tirogla] step 6): with f fixed,
    dL_aux/dp[t, e] = alpha * E * f_e / T =: c_e, so dL[t, j] = p_tj (c_j - sum_e p_te c_e);
    dz/dL[t, j] = 2 * beta * lse_t * p_tj / T.  float64 [T, E]."""
    p, lse = row_softmax_lse(logits)
    c = alpha * E * (_f64(counts) / float(T * k)) / float(T)
    dL = p * (c[None, :] - np.sum(p * c[None, :], axis=1, keepdims=True))
    return dL + (2.0 * beta / float(T)) * lse[:, None] * p


def router_backward(x, w_r, d_logits):
    """Gradient of the router product logits = x W_r^T (+ bias): dW_r = dL^T x, dx = dL W_r.
    float64 ([E, d], [T, d])."""
    dL = _f64(d_logits)
    return dL.T @ _f64(x), dL @ _f64(w_r)


def backward(x, w_r, w1, w3, w2, dy, k, mode, capacity=None, bias=None, shared=None,
             alpha=0.01, beta=1e-3, select_bias=None, exact_logits=False, logits=None):
    """Gradient of J = <dy, y> + L_aux + z with respect to x, W_r and every expert weight, the
    steps of forward() chained in reverse (Combine, Compute, gates and Balance, Score).
    Returns a dict: the forward dict as `fw`, d_out [n_kept, d], d_gate [T, k], dx_rows
    [n_kept, d], d_logits [T, E], dx [T, d], dw_r [E, d], dw1, dw3 [E, d_ff, d], dw2 [E, d, d_ff],
    and dshared = (dw1s, dw3s, dw2s) or None.  `logits` (float32 [T, E]) replaces the router
    product as in forward(); the router gradient still flows through the product.  float64."""
    x = np.asarray(x)
    T = x.shape[0]
    fw = forward(x, w_r, w1, w3, w2, k, mode, capacity=capacity, bias=bias, shared=shared,
                 alpha=alpha, beta=beta, select_bias=select_bias, exact_logits=exact_logits,
                 logits=logits)
    E = fw["logits"].shape[1]
    d_out, d_gate = combine_backward(dy, fw["expert_out"], fw["inv"], fw["topk_gate"], T, k)
    dx_rows, dx, dw1, dw3, dw2 = expert_rows_backward(x, fw["perm"], fw["offsets"], k, w1, w3,
                                                      w2, d_out)
    d_logits = (gate_backward(fw["logits"], fw["topk_idx"], mode, d_gate) +
                balance_backward(fw["logits"], fw["counts"], T, E, k, alpha, beta))
    dw_r, dx_router = router_backward(x, w_r, d_logits)
    dx = dx + dx_router
    dshared = None
    if shared is not None:
        dxs, dw1s, dw3s, dw2s = swiglu_ffn_backward(x, *shared, dy)
        dx = dx + dxs
        dshared = (dw1s, dw3s, dw2s)
    return dict(fw=fw, d_out=d_out, d_gate=d_gate, dx_rows=dx_rows, d_logits=d_logits, dx=dx,
                dw_r=dw_r, dw1=dw1, dw3=dw3, dw2=dw2, dshared=dshared)


def objective(x, w_r, w1, w3, w2, dy, k, mode, capacity=None, bias=None, shared=None,
              alpha=0.01, beta=1e-3, select_bias=None):
    """J = <dy, y> + L_aux + z from forward() with float64 logits (what backward() differentiates)."""
    fw = forward(x, w_r, w1, w3, w2, k, mode, capacity=capacity, bias=bias, shared=shared,
                 alpha=alpha, beta=beta, select_bias=select_bias, exact_logits=True)
    return float(np.sum(_f64(dy) * fw["y"])) + fw["aux"] + fw["z"]


# ------------------------------------------------------------------------------------------------
# Expert Choice routing ([starphix] Router Variants: experts choose tokens, perfect load balance;
# [chipfoundry] Routing Strategies and Variants: experts select their top tokens instead of tokens
# selecting experts, which balances the load by construction and needs no balancing loss).
# Readings: the score of (token t, expert e) is the router's softmax over experts p[t, e] (the router
# is a linear layer followed by a softmax, [chipfoundry] MoE Architecture Components); expert e keeps
# the C tokens with the largest p[:, e], equal scores to the lower token index; the pick's weight in
# y is p[t, e] itself; a token no expert picks gets y = 0 (the residual is outside the layer); an
# expert's rows are listed in increasing token order.
# ------------------------------------------------------------------------------------------------


def expert_choice(scores, C):
    """Per expert, the C tokens with the largest score (ties to the lower token index), listed in
    increasing token order.  scores [T, E] (any float type; compared as given).  Returns
      offsets int32 [E+1] (e * min(C, T)), perm int32 [E * min(C, T)] token ids,
      gate float64 [E * min(C, T)] = scores[perm[r], e], slot int32 [T, E] row of each pick or -1."""
    S = np.asarray(scores)
    T, E = S.shape
    c = min(int(C), T)
    perm = np.empty(E * c, dtype=np.int32)
    gate = np.empty(E * c, dtype=_WORK[0])
    slot = np.full((T, E), -1, dtype=np.int32)
    for e in range(E):
        col = S[:, e]
        # rank: larger score first, then lower token index
        order = sorted(range(T), key=lambda t: (-float(col[t]), t))
        chosen = sorted(order[:c])
        for i, t in enumerate(chosen):
            perm[e * c + i] = t
            gate[e * c + i] = float(col[t])
            slot[t, e] = e * c + i
    offsets = np.arange(E + 1, dtype=np.int32) * c
    return offsets, perm, gate, slot


def forward_expert_choice(x, w_r, w1, w3, w2, C, bias=None, shared=None, logits=None,
                          scores=None):
    """The layer under Expert Choice: router logits, p = softmax over experts, per-expert top-C
    selection, each expert's SwiGLU FFN on its C tokens, y_t = sum over the experts that picked t of
    p[t, e] * FFN_e(x_t) (+ the shared expert).  `scores` (float32 [T, E]) replaces p when given (the
    selection is then taken on those values).  Returns a dict of the intermediates (float64)."""
    x = np.asarray(x)
    T = x.shape[0]
    if logits is None:
        logits = router_logits(x, w_r, bias)
    p, lse = row_softmax_lse(logits)
    S = p if scores is None else np.asarray(scores)
    offsets, perm, gate, slot = expert_choice(S, C)
    E = S.shape[1]
    rows = expert_rows(x, perm, offsets, 1, w1, w3, w2)
    y = np.zeros((T, x.shape[1]), dtype=_WORK[0])
    for e in range(E):
        for r in range(int(offsets[e]), int(offsets[e + 1])):
            y[perm[r]] += gate[r] * rows[r]
    shared_out = None
    if shared is not None:
        shared_out = swiglu_ffn(x, *shared)
        y += shared_out
    return dict(logits=logits, probs=p, scores=S, offsets=offsets, perm=perm, gate=gate,
                slot=slot, expert_out=rows, shared_out=shared_out, y=y)


# ------------------------------------------------------------------------------------------------
# Weight-only quantized experts ([starphix] Inference Optimization, Quantization: experts stored
# in INT8 or INT4 while the router stays 16-bit; [vanos] Quantized Experts: INT4 for a 4x memory
# cut).  Reading: symmetric quantization with one fp32 scale per output channel (per row of a
# [out][in] weight): s = max|w_row| / Q with Q = 127 (INT8) or 7 (INT4), q = round-half-even(w / s)
# in float32 arithmetic, clamped to [-Q, Q]; a zero row has s = 0 and q = 0.  The layer then
# computes with the dequantized weights s * q (activations and accumulation as in the bf16 layer).
# ------------------------------------------------------------------------------------------------


def quantize_rows(w, bits):
    """Per-row symmetric quantization of w [..., rows, cols] (float32 values).  Returns
    (q int8 [..., rows, cols], scale float32 [..., rows])."""
    Q = {8: 127, 4: 7}[bits]
    w = np.asarray(w, dtype=np.float32)
    amax = np.max(np.abs(w), axis=-1)
    scale = (amax / np.float32(Q)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(scale[..., None] > 0, w / scale[..., None], np.float32(0))
    q = np.clip(np.rint(r.astype(np.float32)), -Q, Q).astype(np.int8)
    return q, scale


def pack_int4(q):
    """Two 4-bit two's-complement values per byte along the last axis: column 2j in the low nibble,
    2j + 1 in the high nibble.  q int8 [..., cols] with cols even -> uint8 [..., cols / 2]."""
    q = np.asarray(q, dtype=np.int8).astype(np.int16) & 15
    return (q[..., 0::2] | (q[..., 1::2] << 4)).astype(np.uint8)


def unpack_int4(b):
    """Inverse of pack_int4 (sign-extends each nibble)."""
    b = np.asarray(b, dtype=np.uint8).astype(np.int16)
    lo, hi = b & 15, (b >> 4) & 15
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.int8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def dequantize_rows(q, scale):
    """s * q in float64 (the weights the quantized layer computes with)."""
    return np.asarray(q, dtype=np.float64) * np.asarray(scale, dtype=np.float64)[..., None]


def update_select_bias(select_bias, counts, T, E, k, rate):
    """One aux-loss-free balancing step ([tirogla] Implementation notes: after every step each
    expert's selection bias moves in a direction set by its load; [dinesh] 8.2: it rises for an
    expert that receives too few tokens and falls for one that receives too many).  Reading: the
    step has a fixed size `rate` and the sign of
    (mean load - load), the mean load being T*k/E assignments (counts before capacity):

        b_e <- b_e + rate * sign(T*k - E*counts_e)        (float32, one rounding)
    """
    c = np.asarray(counts, dtype=np.int64)
    sgn = np.sign(np.int64(T) * np.int64(k) - np.int64(E) * c).astype(np.float32)
    return (np.asarray(select_bias, dtype=np.float32) + np.float32(rate) * sgn).astype(np.float32)


def capacity_from_factor(cf, T, k, E):
    """Capacity in assignments per expert, ceil(cf * T * k / E) ([tirogla] Code `main`)."""
    return int(math.ceil(cf * T * k / E))


def routed_flops(T, d, E, d_ff, n_kept, T_shared=0):
    """Algorithmic FLOPs of the layer: router 2*T*d*E ([tirogla] Complexity and constants) plus
    2*3*d*d_ff per expert row (three d x d_ff matrices per expert, [dinesh] section 4)."""
    return 2 * T * d * E + 6 * d * d_ff * (n_kept + T_shared)
