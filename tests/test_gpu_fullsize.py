"""Parity at the full workload sizes, in the launch configuration the benchmark times (needs an
MI355X).  Inputs are drawn on the device (seed 0).  Routing, dispatch and drops are checked for
every token; y is checked on a sample of tokens whose expert outputs the oracle computes one by one
(float64), plus the shared expert where the workload has one.
"""

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
import parity as P

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def M():
    from sparse_mixture_experts_counting_amd import build
    import os
    if not os.path.exists(build.LIB):
        build.build()
    from sparse_mixture_experts_counting_amd import layer, libmoe, synth
    return dict(layer=layer, lm=libmoe, synth=synth)


def _sample_tokens(T, n, seed):
    rng = np.random.default_rng(seed)
    s = set([0, T - 1]) | set(rng.choice(T, size=min(T, n), replace=False).tolist())
    return np.array(sorted(s))


def sampled_y_ref(inp, cfg, tokens, idx, gate, inv):
    """Oracle y for the given tokens (float64), expert by expert, from host copies of the weights of
    the experts those tokens use."""
    k = cfg.k
    x = P.np32(inp.x[torch.as_tensor(tokens, device=inp.x.device)])
    rows, row_of = [], {}
    need = {}
    for i, t in enumerate(tokens):
        for s in range(k):
            if inv[t * k + s] >= 0:
                need.setdefault(int(idx[t, s]), []).append((i, s))
    out = np.zeros((len(tokens) * k, cfg.d))
    inv_s = np.full(len(tokens) * k, -1, np.int64)
    for e, uses in sorted(need.items()):
        w1, w3, w2 = P.np32(inp.w1[e]), P.np32(inp.w3[e]), P.np32(inp.w2[e])
        ii = [i for i, _ in uses]
        o = O.swiglu_ffn(x[ii], w1, w3, w2)
        for (i, s), row in zip(uses, o):
            inv_s[i * k + s] = i * k + s
            out[i * k + s] = row
    sh = None
    if inp.shared is not None:
        sh = O.swiglu_ffn(x, *[P.np32(w) for w in inp.shared])
    return O.combine(out, inv_s, gate[tokens], len(tokens), k, sh)


@pytest.mark.parametrize("name", ["mixtral_decode", "mixtral_prefill", "deepseek_fine"])
def test_full_size_workload(M, name):
    print("full-size", name, flush=True)
    cfg = M["synth"].CONFIGS[name]
    inp = M["synth"].make_inputs(cfg, seed=0, device="cuda")
    b = M["layer"].alloc_buffers(cfg)
    M["layer"].forward(cfg, inp, b)
    torch.cuda.synchronize()

    x, w_r = P.np32(inp.x), P.np32(inp.w_r)
    bias = None if inp.bias is None else P.np32(inp.bias)
    bound, exact = P.logit_error_bound(x, w_r, bias)
    assert np.all(np.abs(P.np32(b.logits) - exact) <= bound)
    L_ref = exact.astype(np.float32)
    idx_ref = O.select_topk(L_ref, cfg.k)
    flips = P.certify_routing(P.npi(b.topk_idx), idx_ref, exact, bound)
    print("  flips", len(flips), flush=True)
    mode = P.GATE_CODE[cfg.gating]
    gate_ref = O.gate_weights(L_ref, idx_ref, mode)
    ok = np.setdiff1d(np.arange(cfg.T), flips)
    np.testing.assert_allclose(P.np32(b.topk_gate)[ok], gate_ref[ok], atol=1e-6, rtol=0)
    counts, offsets, perm, inv, nd = O.dispatch(idx_ref, cfg.E, cfg.capacity)
    if not flips:
        P.check_dispatch_exact(b, dict(counts=counts, offsets=offsets, perm=perm, inv=inv,
                                       n_dropped=nd))
    p, lse = O.row_softmax_lse(L_ref)
    aux = O.aux_loss(counts, p.sum(axis=0), cfg.T, cfg.E, cfg.k, cfg.alpha)
    z = O.z_loss(float(np.sum(lse * lse)), cfg.T, cfg.beta)
    P.check_losses(cfg, b, dict(aux=aux, z=z))

    tokens = _sample_tokens(cfg.T, 14, seed=5)
    tokens = np.setdiff1d(tokens, flips)
    y_ref = sampled_y_ref(inp, cfg, tokens, idx_ref, gate_ref, inv)
    y_gpu = P.np32(b.y)[tokens]
    err = P.rel_err(y_gpu, y_ref)
    print("  y rel err %.3e on %d tokens" % (err, len(tokens)), flush=True)
    assert err <= P.y_tol(cfg)


BWD_TOL = 2e-2   # the GPU rounds dh, h, da and db to bf16 (as the small-size backward tests)


@pytest.mark.parametrize("save", [False, True], ids=["recomputed", "saved"])
@pytest.mark.parametrize("name", ["mixtral_decode", "mixtral_prefill", "deepseek_fine"])
def test_full_size_expert_backward(M, name, save):
    """moe_expert_backward (save=False) and moe_expert_backward_saved after moe_expert_ffn_save
    (save=True, as the training benchmark runs it) at the full sizes: the input
    gradient of sampled expert rows (full d_ff) and sampled rows / columns of the weight gradients
    of a few experts (all their rows; SwiGLU acts per d_ff index, so restricting d_ff is exact),
    against the oracle fed the GPU's own d_out.  Experts without rows get zero gradients."""
    print("full-size backward", name, "saved" if save else "recomputed", flush=True)
    cfg = M["synth"].CONFIGS[name]
    inp = M["synth"].make_inputs(cfg, seed=0, device="cuda")
    b = M["layer"].alloc_buffers(cfg, save=save)
    M["layer"].forward(cfg, inp, b)
    dy = M["synth"].make_dy(cfg, seed=0, device="cuda")
    g = M["layer"].alloc_grads(cfg)
    M["layer"].backward(cfg, inp, b, dy, g)
    torch.cuda.synchronize()
    k = cfg.k
    offsets, perm = P.npi(b.offsets), P.npi(b.perm)
    counts = np.diff(offsets)
    n_kept = int(offsets[-1])
    rng = np.random.default_rng(11)

    def rows_of(rr):
        rr = np.asarray(sorted(rr))
        return rr, torch.as_tensor(rr, device="cuda")

    # Input gradient of sampled expert rows.
    rows = set([0, n_kept - 1]) | set(rng.choice(n_kept, size=10, replace=False).tolist())
    by_e = {}
    for r in rows:
        by_e.setdefault(int(np.searchsorted(offsets, r, side="right") - 1), []).append(r)
    got, want = [], []
    for e, rr in sorted(by_e.items()):
        rr, rr_d = rows_of(rr)
        tok = torch.as_tensor(perm[rr] // k, device="cuda")
        dX, _, _, _ = O.swiglu_ffn_backward(P.np32(inp.x[tok]), P.np32(inp.w1[e]),
                                            P.np32(inp.w3[e]), P.np32(inp.w2[e]),
                                            P.np32(g.d_out[rr_d]))
        got.append(P.np32(g.dx_rows[rr_d]))
        want.append(dX)
    err = P.rel_err(np.concatenate(got), np.concatenate(want))
    print("  dx_rows rel err %.3e on %d rows" % (err, len(rows)), flush=True)
    assert err <= BWD_TOL

    # Weight gradients: rows f of dw1 / dw3 and columns f of dw2 for a few experts.
    live = np.nonzero(counts > 0)[0]
    experts = sorted(set([int(live[np.argmax(counts[live])]), int(live[np.argmin(counts[live])]),
                          int(rng.choice(live))]))
    fs = np.sort(rng.choice(cfg.d_ff, size=6, replace=False))
    fs_d = torch.as_tensor(fs, device="cuda")
    for e in experts:
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        tok = torch.as_tensor(perm[lo:hi] // k, device="cuda")
        _, w1s, w3s, w2s = O.swiglu_ffn_backward(
            P.np32(inp.x[tok]), P.np32(inp.w1[e][fs_d]), P.np32(inp.w3[e][fs_d]),
            P.np32(inp.w2[e][:, fs_d]), P.np32(g.d_out[lo:hi]))
        errs = (P.rel_err(P.np32(g.dw1[e][fs_d]), w1s), P.rel_err(P.np32(g.dw3[e][fs_d]), w3s),
                P.rel_err(P.np32(g.dw2[e][:, fs_d]), w2s))
        print("  expert %d (%d rows): dw1 %.2e dw3 %.2e dw2 %.2e" % ((e, hi - lo) + errs),
              flush=True)
        assert max(errs) <= BWD_TOL
    empty = np.nonzero(counts == 0)[0]
    if len(empty):
        ed = torch.as_tensor(empty, device="cuda")
        for t in (g.dw1, g.dw3, g.dw2):
            assert bool((t[ed] == 0).all())
