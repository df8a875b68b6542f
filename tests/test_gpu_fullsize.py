"""Parity at the full workload sizes, in the launch configuration the benchmark times (needs an
MI355X).  Inputs are drawn on the device (seed 0).  The forward is compared on every output:
routing, dispatch and drops bit-exact for every token, y on every token against the float64
oracle (shared expert included).  The expert backward is checked on sampled rows and weight
columns that the oracle computes one by one.
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


class DeviceExperts:
    """Host float32 copies of one expert's weight at a time (exact widening of bf16), fetched from
    the device on indexing, so the oracle can walk the experts of a multi-GB layer without holding
    every weight on the host at once."""

    def __init__(self, w):
        self.w = w

    def __getitem__(self, e):
        return P.np32(self.w[e])


@pytest.mark.parametrize("name", ["mixtral_decode", "mixtral_prefill", "deepseek_fine"])
def test_full_size_workload(M, name):
    """The benchmark's workloads at full size, every output compared.  The GPU logits must lie in
    the rounding bound of the exact router product; the oracle then routes, dispatches, gates,
    runs every expert (float64, one expert's weights on the host at a time), combines and forms
    the losses from those float32 logits: top-k and the dispatch layout bit-exact, gates 1e-6, y
    on every token within the bf16 tolerance, losses 1e-4.  Flips against the oracle's own
    rounded logits must be certified near-ties and are logged."""
    print("full-size", name, flush=True)
    cfg = M["synth"].CONFIGS[name]
    inp = M["synth"].make_inputs(cfg, seed=0, device="cuda")
    b = M["layer"].alloc_buffers(cfg)
    M["layer"].forward(cfg, inp, b)
    torch.cuda.synchronize()

    x, w_r = P.np32(inp.x), P.np32(inp.w_r)
    bias = None if inp.bias is None else P.np32(inp.bias)
    bound, exact = P.logit_error_bound(x, w_r, bias)
    gl = P.np32(b.logits)
    assert np.all(np.abs(gl - exact) <= bound)
    flips = P.certify_routing(P.npi(b.topk_idx), O.select_topk(exact.astype(np.float32), cfg.k),
                              exact, bound)
    P.log_flips(name, cfg.T, len(flips))
    print("  flips", len(flips), flush=True)

    sh = None if inp.shared is None else tuple(P.np32(w) for w in inp.shared)
    ref = O.forward(x, w_r, DeviceExperts(inp.w1), DeviceExperts(inp.w3), DeviceExperts(inp.w2),
                    cfg.k, P.GATE_CODE[cfg.gating], capacity=cfg.capacity, bias=bias, shared=sh,
                    alpha=cfg.alpha, beta=cfg.beta, logits=gl)
    np.testing.assert_array_equal(P.npi(b.topk_idx), ref["topk_idx"])
    P.check_dispatch_exact(b, ref)
    np.testing.assert_allclose(P.np32(b.topk_gate), ref["topk_gate"], atol=1e-6, rtol=0)
    P.check_losses(cfg, b, ref)
    err = P.rel_err(P.np32(b.y), ref["y"])
    print("  y rel err %.3e on all %d tokens" % (err, cfg.T), flush=True)
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
