"""GPU parity of the backward pass (moe_combine_backward, moe_expert_backward, moe_route_backward
and the unit-gate moe_combine) against the CPU oracle (needs an MI355X).

Two levels per case:
  * end to end, every gradient against oracle.backward() fed the GPU's own fp32 logits (so both
    sides route identically), within the bf16 tolerance of the forward output (2e-2 of the
    largest reference entry): the GPU rounds dh, h, da, db and the activation gradients to bf16;
  * each kernel against a float64 host evaluation of its own formula on the GPU's own inputs
    (d_gate, d_logits, dw_r, dx_route, dx), within fp32 rounding, so that an error in one step is
    not hidden by the bf16 tolerance of the chain.
"""

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
import parity as P

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2


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


def _cuda(inp):
    import dataclasses
    kw = {}
    for f in dataclasses.fields(inp):
        v = getattr(inp, f.name)
        if isinstance(v, torch.Tensor):
            v = v.cuda()
        elif isinstance(v, tuple):
            v = tuple(t.cuda() for t in v)
        kw[f.name] = v
    return type(inp)(**kw)


def _run(M, cfg, seed, zero_dy=False, save=False):
    inp = _cuda(M["synth"].make_inputs(cfg, seed=seed, device="cpu"))
    dy = M["synth"].make_dy(cfg, seed=seed, device="cpu").cuda()
    if zero_dy:
        dy.zero_()
    b = M["layer"].alloc_buffers(cfg, save=save)
    g = M["layer"].alloc_grads(cfg)
    M["layer"].forward(cfg, inp, b)
    M["layer"].backward(cfg, inp, b, dy, g)
    torch.cuda.synchronize()
    return inp, dy, b, g


def _check_case(M, cfg, seed=1, zero_dy=False, save=False):
    inp, dy, b, g = _run(M, cfg, seed, zero_dy, save)
    h = P.host_inputs(inp)
    mode = P.GATE_CODE[cfg.gating]
    T, k = cfg.T, cfg.k
    logits = P.np32(b.logits)
    dyh = P.np32(dy).astype(np.float64)
    ref = O.backward(h["x"], h["w_r"], h["w1"], h["w3"], h["w2"], dyh, k, mode,
                     capacity=cfg.capacity, bias=h["bias"], shared=h["shared"], alpha=cfg.alpha,
                     beta=cfg.beta, logits=logits)
    fw = ref["fw"]
    P.check_dispatch_exact(b, fw)                     # same routing on both sides
    n_kept = int(fw["offsets"][-1])
    inv = fw["inv"].reshape(T, k)

    # Kernel level.
    out_gpu = P.np32(b.expert_out)[:n_kept].astype(np.float64)
    gate_gpu = P.np32(b.topk_gate).astype(np.float64)
    want_dg = np.zeros((T, k))
    for s in range(k):
        keep = inv[:, s] >= 0
        want_dg[keep, s] = np.sum(dyh[keep] * out_gpu[inv[keep, s]], axis=1)
    dg = P.np32(g.d_gate)
    assert P.rel_err(dg, want_dg) <= 1e-5, "d_gate"
    assert np.all(dg[inv < 0] == 0.0)
    want_dout = np.zeros((n_kept, cfg.d))
    for s in range(k):
        keep = inv[:, s] >= 0
        want_dout[inv[keep, s]] = gate_gpu[keep, s, None] * dyh[keep]
    assert P.rel_err(P.np32(g.d_out)[:n_kept], want_dout) <= 4e-3, "d_out (bf16)"
    want_dl = (O.gate_backward(logits, P.npi(b.topk_idx), mode, dg) +
               O.balance_backward(logits, P.npi(b.counts), T, cfg.E, k, cfg.alpha, cfg.beta))
    dl = P.np32(g.d_logits)
    assert P.rel_err(dl, want_dl) <= 1e-4, "d_logits"
    dl64 = dl.astype(np.float64)
    assert P.rel_err(P.np32(g.dw_r), dl64.T @ h["x"]) <= 1e-5, "dw_r"
    want_dxr = dl64 @ h["w_r"]
    if cfg.n_shared:
        want_dxr = want_dxr + P.np32(g.dx_shared)
    assert P.rel_err(P.np32(g.dx_route), want_dxr) <= 4e-3, "dx_route (bf16)"
    want_dx = P.np32(g.dx_route).astype(np.float64)
    rows = P.np32(g.dx_rows).astype(np.float64)
    for s in range(k):
        keep = inv[:, s] >= 0
        want_dx[keep] += rows[inv[keep, s]]
    assert P.rel_err(P.np32(g.dx), want_dx) <= 4e-3, "dx assembly (bf16)"

    # End to end against the oracle.
    errs = dict(d_gate=P.rel_err(dg, ref["d_gate"]), d_logits=P.rel_err(dl, ref["d_logits"]),
                dx_rows=P.rel_err(P.np32(g.dx_rows)[:n_kept], ref["dx_rows"]),
                dx=P.rel_err(P.np32(g.dx), ref["dx"]), dw_r=P.rel_err(P.np32(g.dw_r), ref["dw_r"]),
                dw1=P.rel_err(P.np32(g.dw1), ref["dw1"]), dw3=P.rel_err(P.np32(g.dw3), ref["dw3"]),
                dw2=P.rel_err(P.np32(g.dw2), ref["dw2"]))
    if cfg.n_shared:
        for name, a, r in zip(("dw1s", "dw3s", "dw2s"), g.dshared, ref["dshared"]):
            errs[name] = P.rel_err(P.np32(a), r)
    _say("  %s: %s" % (cfg.name, " ".join("%s=%.1e" % kv for kv in errs.items())))
    for name, e in errs.items():
        assert e <= BF16_TOL, "%s relative error %.3e" % (name, e)
    # Experts without rows get exactly zero weight gradients.
    empty = np.nonzero(np.diff(fw["offsets"]) == 0)[0]
    for e_ in empty:
        assert np.all(P.np32(g.dw1[e_]) == 0) and np.all(P.np32(g.dw2[e_]) == 0)
    return inp, dy, b, g, ref


CASES = [
    # T, d, E, k, d_ff, gating, C, shared, zipf
    (37, 64, 4, 2, 96, "softmax_topk", 0, 0, 0.0),
    (300, 128, 8, 2, 192, "sigmoid_topk", 0, 1, 0.0),
    (257, 136, 8, 2, 264, "softmax_all", 70, 0, 0.0),
    (513, 256, 16, 4, 320, "sigmoid_topk", 0, 1, 1.1),
    (20, 64, 16, 1, 64, "softmax_topk", 0, 0, 1.5),
    (1030, 512, 8, 2, 1024, "softmax_topk", 0, 0, 0.0),
    (2048, 256, 4, 1, 512, "softmax_topk", 0, 1, 0.0),
    # 256 to 512 rows per expert: 256-row tiles for whole blocks, 128-row tiles for the rest
    (700, 256, 4, 2, 512, "softmax_topk", 0, 0, 1.1),
    (1500, 128, 8, 2, 320, "sigmoid_topk", 0, 1, 1.3),
    # E a multiple of 64: the router products on the matrix cores (three-term split of d_logits;
    # token chunks not dividing T; dx with and without the shared expert's addend)
    (300, 128, 64, 4, 192, "sigmoid_topk", 0, 1, 1.1),
    (1030, 256, 128, 2, 256, "softmax_topk", 0, 0, 0.0),
    (96, 64, 256, 8, 64, "sigmoid_topk", 0, 1, 1.1),
    (5, 512, 64, 2, 128, "softmax_all", 0, 0, 0.0),
    # skewed groups with more than two rounds of 256-column tiles (d = 8448): the input-gradient
    # product (weights read transposed) and the forward down projection take the block-sparse
    # launch with one block per CU taking tiles from counters
    (1024, 8448, 8, 2, 128, "softmax_topk", 0, 0, 1.2),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "T%d_d%d_E%d_k%d_f%d_%s_C%d_s%d" % c[:8])
def test_backward_parity(M, case):
    T, d, E, k, f, gating, C, sh, zipf = case
    _say("backward", case)
    cfg = M["synth"].tiny_config(T, d, E, k, f, "bf16", gating, capacity=C, n_shared=sh,
                                 zipf_s=zipf)
    _check_case(M, cfg)


def test_backward_losses_only(M):
    # dy = 0: nothing reaches the experts; the router moves by the balancing and z losses alone
    _say("backward losses only")
    cfg = M["synth"].tiny_config(300, 128, 8, 2, 192, "bf16", "softmax_topk").replace(alpha=0.5,
                                                                              beta=0.2)
    inp, dy, b, g, ref = _check_case(M, cfg, zero_dy=True)
    for t in (g.d_out, g.d_gate, g.dx_rows, g.dw1, g.dw3, g.dw2):
        n = int(P.npi(b.offsets)[-1]) if t.shape[0] == cfg.T * cfg.k else t.shape[0]
        assert np.all(P.np32(t[:n]) == 0)
    assert P.rel_err(P.np32(g.dw_r), ref["dw_r"]) <= 1e-4


def test_backward_deterministic(M):
    _say("backward determinism")
    cfg = M["synth"].tiny_config(513, 256, 16, 4, 320, "bf16", "sigmoid_topk", n_shared=1,
                                 zipf_s=1.1)
    _, _, _, g1 = _run(M, cfg, 3)
    snap = {n: getattr(g1, n).clone() for n in ("dx", "dw_r", "dw1", "dw3", "dw2", "d_logits")}
    _, _, _, g2 = _run(M, cfg, 3)
    for n, v in snap.items():
        assert torch.equal(v, getattr(g2, n)), n


# Saved activations (moe_expert_ffn_save + moe_expert_backward_saved): weights as stored and as
# transposed copies (d_ff % 64), split-K decode shapes, the two-stream tall/short tiling, shared
# experts, capacity drops.
SAVED_CASES = [
    (37, 64, 4, 2, 96, "softmax_topk", 0, 0, 0.0),
    (257, 136, 8, 2, 264, "softmax_all", 70, 0, 0.0),
    (20, 64, 16, 1, 64, "softmax_topk", 0, 0, 1.5),
    (700, 256, 4, 2, 512, "softmax_topk", 0, 0, 1.1),
    (1500, 128, 8, 2, 320, "sigmoid_topk", 0, 1, 1.3),
    (2048, 256, 4, 1, 512, "softmax_topk", 0, 1, 0.0),
]


def _silu(a):
    return a / (1.0 + np.exp(-a))


def _check_saved(saved, x_rows, w1, w3, bounds, f):
    """saved [n][3f] = h | a | b of each row against float64 products of the same bf16 inputs:
    a and b within their bf16 rounding, h within the rounding of the fp32 path."""
    sv = P.np32(saved)[:bounds[-1]].astype(np.float64)
    a = np.zeros((bounds[-1], f))
    b = np.zeros((bounds[-1], f))
    for e in range(len(bounds) - 1):
        r0, r1 = bounds[e], bounds[e + 1]
        a[r0:r1] = x_rows[r0:r1] @ w1[e].T
        b[r0:r1] = x_rows[r0:r1] @ w3[e].T
    assert P.rel_err(sv[:, f:2 * f], a) <= 4e-3, "saved a"
    assert P.rel_err(sv[:, 2 * f:], b) <= 4e-3, "saved b"
    assert P.rel_err(sv[:, :f], _silu(a) * b) <= 4e-3, "saved h"


@pytest.mark.parametrize("case", SAVED_CASES, ids=lambda c: "T%d_d%d_E%d_k%d_f%d_%s_C%d_s%d" % c[:8])
def test_backward_saved_parity(M, case):
    T, d, E, k, f, gating, C, sh, zipf = case
    _say("backward from saved activations", case)
    cfg = M["synth"].tiny_config(T, d, E, k, f, "bf16", gating, capacity=C, n_shared=sh,
                                 zipf_s=zipf)
    # Every gradient against the oracle, end to end and per kernel.
    inp, dy, b, g, ref = _check_case(M, cfg, save=True)
    # The saving forward gives the same outputs as the plain one, bit for bit.
    b0 = M["layer"].alloc_buffers(cfg)
    M["layer"].forward(cfg, inp, b0)
    torch.cuda.synchronize()
    n = int(P.npi(b.offsets)[-1])
    assert torch.equal(b.expert_out[:n], b0.expert_out[:n])
    assert torch.equal(b.y, b0.y)
    if sh:
        assert torch.equal(b.shared_out, b0.shared_out)
    # The saved rows themselves.
    h = P.host_inputs(inp)
    x = h["x"].astype(np.float64)
    perm = P.npi(b.perm)[:n]
    bounds = P.npi(b.offsets)
    _check_saved(b.saved, x[perm // k], h["w1"].astype(np.float64), h["w3"].astype(np.float64),
                 bounds, f)
    if sh:
        w1s, w3s, _ = h["shared"]
        _check_saved(b.saved_shared, x, w1s[None].astype(np.float64),
                     w3s[None].astype(np.float64), np.array([0, T]), f)
    # Against the recomputing backward on the same inputs: only the bf16 rounding of a and b
    # separates the two.
    g0 = M["layer"].alloc_grads(cfg)
    M["layer"].backward(cfg, inp, b0, dy, g0)
    torch.cuda.synchronize()
    for name in ("dx", "dw1", "dw3", "dw2", "dw_r", "d_logits"):
        e_ = P.rel_err(P.np32(getattr(g, name)), P.np32(getattr(g0, name)))
        assert e_ <= 1e-2, "%s saved vs recomputed %.3e" % (name, e_)
