"""Helpers for the GPU-vs-oracle parity tests: run the oracle on the same seeded inputs, certify
routing flips that are within the float32 rounding bound of the router product, and compare.

Tolerances (the layer's stated bars):
  routing / dispatch  bit-exact (top-k indices with slot order, counts, offsets, perm, inv, drops)
  y                   max|y - y_ref| / max|y_ref| <= 1e-5 (fp32 layers), <= 2e-2 (bf16 layers)
  aux, z              1e-4 relative
  gates               1e-6 absolute (float32 gating arithmetic from the same float32 logits)
"""

import math

import numpy as np
import torch

from oracle import moe_oracle as O

GATE_CODE = {"softmax_topk": O.SOFTMAX_TOPK, "softmax_all": O.SOFTMAX_ALL,
             "sigmoid_topk": O.SIGMOID_TOPK}
U32 = 2.0 ** -24


def y_tol(cfg):
    return 1e-5 if cfg.dtype == "fp32" else 2e-2


def np32(t):
    """Device/host tensor -> numpy float32 (bf16 widens exactly)."""
    return t.detach().float().cpu().numpy()


def npi(t):
    return t.detach().cpu().numpy().astype(np.int64)


def logit_error_bound(x, w_r, bias=None):
    """Per-entry bound on |float32 router logit - exact logit|: the dot-product bound
    gamma_d * sum_j |x_j| |w_je| (fp32 accumulation in any order, exact products of bf16 operands
    or rounded fp32 products) plus the final roundings of the bias add and of the oracle's own
    float32 conversion."""
    d = x.shape[1]
    g = d * U32 / (1 - d * U32)
    ax = np.abs(np.asarray(x, np.float64))
    aw = np.abs(np.asarray(w_r, np.float64)).T          # w_r is [E, d]
    exact = np.asarray(x, np.float64) @ np.asarray(w_r, np.float64).T
    if bias is not None:
        exact = exact + np.asarray(bias, np.float64)[None, :]
    return (g + U32) * (ax @ aw) + 4 * U32 * np.abs(exact) + 1e-30, exact


def certify_routing(gpu_idx, oracle_idx, exact_logits, bound):
    """Tokens whose GPU top-k (with slot order) differs from the oracle's.  Each difference must
    be a near-tie: the GPU's choice at that slot and the oracle's are within the sum of their
    error bounds of each other.  Returns the list of differing tokens (asserts certification)."""
    diff = np.nonzero(np.any(gpu_idx != oracle_idx, axis=1))[0]
    for t in diff:
        for s in range(gpu_idx.shape[1]):
            a, b = int(gpu_idx[t, s]), int(oracle_idx[t, s])
            if a != b:
                gap = abs(exact_logits[t, a] - exact_logits[t, b])
                assert gap <= bound[t, a] + bound[t, b], (
                    "token %d slot %d: GPU chose %d, oracle %d, gap %.3e exceeds bound %.3e"
                    % (t, s, a, b, gap, bound[t, a] + bound[t, b]))
        assert len(set(gpu_idx[t].tolist())) == gpu_idx.shape[1]
    return diff.tolist()


def rel_err(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.max(np.abs(b))
    return float(np.max(np.abs(a - b)) / den) if den > 0 else float(np.max(np.abs(a - b)))


def host_inputs(inp):
    """Host float32 copies (exact widening of bf16) of every input of a workload."""
    sh = None
    if inp.shared is not None:
        sh = tuple(np32(w) for w in inp.shared)
    return dict(x=np32(inp.x), w_r=np32(inp.w_r), w1=np32(inp.w1), w3=np32(inp.w3),
                w2=np32(inp.w2), shared=sh, bias=None if inp.bias is None else np32(inp.bias))


def check_dispatch_exact(b, ref):
    np.testing.assert_array_equal(npi(b.counts), ref["counts"])
    np.testing.assert_array_equal(npi(b.offsets), ref["offsets"])
    n_kept = int(ref["offsets"][-1])
    np.testing.assert_array_equal(npi(b.perm)[:n_kept], ref["perm"])
    np.testing.assert_array_equal(npi(b.inv), ref["inv"])
    assert int(npi(b.n_dropped)[0]) == ref["n_dropped"]


def check_losses(cfg, b, ref):
    aux = float(np32(b.aux)[0])
    z = float(np32(b.z)[0])
    assert math.isclose(aux, ref["aux"], rel_tol=1e-4), (aux, ref["aux"])
    assert math.isclose(z, ref["z"], rel_tol=1e-4, abs_tol=1e-12), (z, ref["z"])


# Near-tie flips seen by the end-to-end parity checks: (case, tokens, flipped tokens).  The test
# session prints them in its summary, so every run reports whether a certified flip occurred.
FLIP_LOG = []


def log_flips(case, T, n_flips):
    FLIP_LOG.append((str(case), int(T), int(n_flips)))
