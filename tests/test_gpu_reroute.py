"""GPU parity of overflow rerouting (moe_reroute after moe_route and moe_dispatch) against the CPU
oracle (needs an MI355X).  The final selection, the dispatch layout and the drop count are compared
bit-exactly (the oracle ranks the GPU's own fp32 logits, as moe_route does); gates within 1e-6 and
y within the forward tolerance."""

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
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return dict(layer=layer, lm=libmoe, synth=synth)


def _say(*a):
    print(*a, flush=True)


def _check_layout(r, ref_idx2, ref_off, ref_perm, ref_inv, ref_nd):
    np.testing.assert_array_equal(P.npi(r.topk_idx), ref_idx2)
    np.testing.assert_array_equal(P.npi(r.offsets), ref_off)
    n = int(ref_off[-1])
    np.testing.assert_array_equal(P.npi(r.perm)[:n], ref_perm)
    np.testing.assert_array_equal(P.npi(r.inv), ref_inv)
    assert int(P.npi(r.n_dropped)[0]) == ref_nd


@pytest.mark.parametrize("T,E,k,C,mode", [(40, 3, 2, 5, 0), (300, 8, 2, 40, 0), (257, 16, 4, 30, 2),
                                          (2048, 8, 1, 150, 1), (64, 64, 6, 3, 2), (9, 4, 3, 1, 0)])
def test_reroute_from_given_logits(M, T, E, k, C, mode):
    _say("reroute given logits", T, E, k, C, mode)
    lm, layer, synth = M["lm"], M["layer"], M["synth"]
    rng = np.random.default_rng(T + E + k + C)
    L = rng.normal(0, 1.5, size=(T, E)).astype(np.float32)
    L[:, 0] += 1.0                                          # overload expert 0
    L[::5] = np.round(L[::5])                               # ties
    cfg = synth.tiny_config(T, 8, E, k, 8, "fp32", ["softmax_topk", "softmax_all",
                                                      "sigmoid_topk"][mode], capacity=C)
    b = layer.alloc_buffers(cfg)
    b.logits.copy_(torch.from_numpy(L))
    inp = synth.make_inputs(cfg, seed=0, device="cpu")
    layer.route(cfg, inp, b, logits_in=True)
    layer.dispatch(cfg, b)
    r = layer.alloc_reroute_buffers(cfg)
    lm.reroute(b.logits, None, b.topk_idx, b.topk_gate, b.offsets, b.inv, T, E, k, C, mode,
               r.topk_idx, r.topk_gate, r.offsets, r.perm, r.inv, r.n_dropped, b.workspace)
    torch.cuda.synchronize()
    idx = O.select_topk(L, k)
    np.testing.assert_array_equal(P.npi(b.topk_idx), idx)
    ref = O.dispatch_reroute(L, idx, E, C)
    _check_layout(r, *ref)
    n1 = int(P.npi(b.n_dropped)[0])
    _say("  dropped: %d -> %d" % (n1, ref[4]))
    np.testing.assert_allclose(P.np32(r.topk_gate), O.gate_weights(L, ref[0], mode), atol=1e-6,
                               rtol=0)


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_reroute_gates_with_a_large_logit_gap(M, mode):
    """Every token's first choice (expert 0) sits 300 above the rest, or every other logit lies far
    below zero (sigmoid mode), and expert 0 overflows: the rerouted tokens' selected logits all lie
    far below the row maximum.  Their gates must stay finite and match the oracle's float64 gates
    of the final selection within 1e-6 (the gating of moe_route shifts by the largest selected
    logit; shifting by the row maximum would underflow every term to 0)."""
    _say("reroute large gap, mode", mode)
    lm, layer, synth = M["lm"], M["layer"], M["synth"]
    T, E, k, C = 64, 8, 2, 4
    rng = np.random.default_rng(77 + mode)
    L = rng.normal(0, 1, size=(T, E)).astype(np.float32)
    if mode == 2:
        L[:, 1:] -= 200.0
        L[:, 0] = 5.0
    else:
        L[:, 0] = 300.0
    cfg = synth.tiny_config(T, 8, E, k, 8, "fp32", ["softmax_topk", "softmax_all",
                                                      "sigmoid_topk"][mode], capacity=C)
    b = layer.alloc_buffers(cfg)
    b.logits.copy_(torch.from_numpy(L))
    inp = synth.make_inputs(cfg, seed=0, device="cpu")
    layer.route(cfg, inp, b, logits_in=True)
    layer.dispatch(cfg, b)
    r = layer.alloc_reroute_buffers(cfg)
    lm.reroute(b.logits, None, b.topk_idx, b.topk_gate, b.offsets, b.inv, T, E, k, C, mode,
               r.topk_idx, r.topk_gate, r.offsets, r.perm, r.inv, r.n_dropped, b.workspace)
    torch.cuda.synchronize()
    idx = O.select_topk(L, k)
    ref = O.dispatch_reroute(L, idx, E, C)
    _check_layout(r, *ref)
    got = P.np32(r.topk_gate)
    assert np.all(np.isfinite(got))
    np.testing.assert_allclose(got, O.gate_weights(L, ref[0], mode), atol=1e-6, rtol=0)


REROUTE_LAYER = [
    # T, d, E, k, d_ff, dtype, gating, C, shared, zipf
    (300, 128, 8, 2, 192, "bf16", "softmax_topk", 60, 0, 0.0),
    (257, 136, 16, 4, 264, "bf16", "sigmoid_topk", 50, 1, 1.1),
    (2048, 256, 8, 1, 512, "bf16", "softmax_all", 230, 0, 0.0),
    (64, 32, 4, 2, 64, "fp32", "softmax_topk", 20, 0, 0.0),
]


@pytest.mark.parametrize("case", REROUTE_LAYER, ids=lambda c: "T%d_E%d_k%d_C%d_%s" % (c[0], c[2], c[3], c[7], c[5]))
def test_reroute_layer(M, case):
    T, d, E, k, f, dt, g, C, sh, zipf = case
    _say("reroute layer", case)
    synth, layer = M["synth"], M["layer"]
    cfg = synth.tiny_config(T, d, E, k, f, dt, g, capacity=C, n_shared=sh, zipf_s=zipf,
                            router_scale=3.0)
    inp = synth.make_inputs(cfg, seed=4, device="cpu")
    import dataclasses
    kw = {}
    for fl in dataclasses.fields(inp):
        v = getattr(inp, fl.name)
        if isinstance(v, torch.Tensor):
            v = v.cuda()
        elif isinstance(v, tuple):
            v = tuple(t.cuda() for t in v)
        kw[fl.name] = v
    gi = type(inp)(**kw)
    b = layer.alloc_buffers(cfg)
    r = layer.alloc_reroute_buffers(cfg)
    layer.forward_reroute(cfg, gi, b, r)
    torch.cuda.synchronize()
    h = P.host_inputs(gi)
    logits = P.np32(b.logits)
    mode = P.GATE_CODE[g]
    ref = O.forward(h["x"], h["w_r"], h["w1"], h["w3"], h["w2"], k, mode, capacity=C,
                    bias=h["bias"], shared=h["shared"], alpha=cfg.alpha, beta=cfg.beta,
                    logits=logits, reroute=True)
    _check_layout(r, ref["topk_idx"], ref["offsets"], ref["perm"], ref["inv"], ref["n_dropped"])
    plain = int(P.npi(b.n_dropped)[0])
    _say("  dropped without rerouting %d, with %d" % (plain, ref["n_dropped"]))
    assert ref["n_dropped"] <= plain
    np.testing.assert_allclose(P.np32(r.topk_gate), ref["topk_gate"], atol=1e-6, rtol=0)
    err = P.rel_err(P.np32(b.y), ref["y"])
    assert err <= P.y_tol(cfg), "y relative error %.3e" % err
    P.check_losses(cfg, b, ref)
