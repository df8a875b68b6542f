"""Brute-force restatements of the layer, used only to pin the oracle on tiny inputs.

Each function states the same definition as the oracle in a different form (rank counting instead
of sorting, pairwise counting instead of a running list, dense evaluation of every expert on every
token followed by a mask) so that a dropped term, a wrong index or a wrong order in either one
shows up as a disagreement.
"""

import numpy as np


def rank_select(logits, k):
    """Slot of expert e for token t = number of experts that beat it (a larger logit, or an equal
    logit with a smaller index); e is selected when that number is below k."""
    L = np.asarray(logits, dtype=np.float64)
    T, E = L.shape
    idx = np.full((T, k), -1, dtype=np.int64)
    for t in range(T):
        for e in range(E):
            beat = sum(1 for j in range(E) if L[t, j] > L[t, e] or (L[t, j] == L[t, e] and j < e))
            if beat < k:
                idx[t, beat] = e
    return idx


def keep_mask(idx, capacity):
    """Assignment a is kept when fewer than C earlier assignments went to the same expert."""
    flat = np.asarray(idx).reshape(-1)
    A = flat.size
    C = A if not capacity or capacity <= 0 else capacity
    keep = np.zeros(A, dtype=bool)
    for a in range(A):
        earlier = sum(1 for b in range(a) if flat[b] == flat[a])
        keep[a] = earlier < C
    return keep


def gates_alt(logits, idx, mode):
    """Gates in an algebraically different but equal form:
    softmax_topk: 1 / sum_s exp(L_s - L_e); softmax_all: 1 / sum_j exp(L_j - L_e);
    sigmoid_topk: (1 / (1 + exp(-L_e))) / sum_s (1 / (1 + exp(-L_s)))."""
    L = np.asarray(logits, dtype=np.float64)
    T, k = idx.shape
    g = np.zeros((T, k))
    for t in range(T):
        for s in range(k):
            e = idx[t, s]
            if mode == 0:
                g[t, s] = 1.0 / sum(np.exp(L[t, idx[t, j]] - L[t, e]) for j in range(k))
            elif mode == 1:
                g[t, s] = 1.0 / np.sum(np.exp(L[t] - L[t, e]))
            else:
                sig = lambda v: 1.0 / (1.0 + np.exp(-v))
                g[t, s] = sig(L[t, e]) / sum(sig(L[t, idx[t, j]]) for j in range(k))
    return g


def swiglu_loops(xrow, w1, w3, w2):
    """One token through a SwiGLU expert with explicit loops over every index.  The weights are
    the [out][in] matrices of bias-free linear layers: w1, w3 [d_ff][d], w2 [d][d_ff]."""
    d_ff, d = w1.shape
    h = np.zeros(d_ff)
    for f in range(d_ff):
        g = sum(xrow[j] * w1[f, j] for j in range(d))
        u = sum(xrow[j] * w3[f, j] for j in range(d))
        h[f] = g / (1.0 + np.exp(-g)) * u
    return np.array([sum(w2[c, f] * h[f] for f in range(d_ff)) for c in range(w2.shape[0])])


def dense_then_mask(x, logits, w1, w3, w2, k, mode, capacity, shared=None):
    """Evaluate every expert on every token, then keep only the selected, non-dropped ones."""
    x = np.asarray(x, dtype=np.float64)
    T, d = x.shape
    E = w1.shape[0]
    idx = rank_select(logits, k)
    g = gates_alt(logits, idx, mode)
    keep = keep_mask(idx, capacity).reshape(T, k)
    dense = np.zeros((E, T, w2.shape[1]))
    for e in range(E):
        for t in range(T):
            dense[e, t] = swiglu_loops(x[t], np.asarray(w1[e], np.float64),
                                       np.asarray(w3[e], np.float64), np.asarray(w2[e], np.float64))
    y = np.zeros((T, w2.shape[1]))
    for t in range(T):
        for s in range(k):
            if keep[t, s]:
                y[t] += g[t, s] * dense[idx[t, s], t]
    if shared is not None:
        for t in range(T):
            y[t] += swiglu_loops(x[t], *[np.asarray(w, np.float64) for w in shared])
    return y, idx, keep
