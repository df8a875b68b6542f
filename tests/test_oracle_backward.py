"""Pins of the oracle's backward pass (CPU only).

The gradients are checked against central finite differences of the oracle's forward objective
J = <dy, y> + L_aux + z (the forward is pinned on its own in test_oracle_pins), against a library
autograd on the SwiGLU expert, and against closed forms of single steps: gates that cannot move,
a balancing loss that is constant under uniform routing, and the sum of the z-loss gradient.
"""

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O

MODES = [O.SOFTMAX_TOPK, O.SOFTMAX_ALL, O.SIGMOID_TOPK]


def _case(seed, T=5, d=4, E=4, k=2, f=6, shared=False, bias=False, sbias=False):
    r = np.random.default_rng(seed)
    c = dict(x=r.standard_normal((T, d)), w_r=r.standard_normal((E, d)),
             w1=0.5 * r.standard_normal((E, f, d)), w3=0.5 * r.standard_normal((E, f, d)),
             w2=0.5 * r.standard_normal((E, d, f)), dy=r.standard_normal((T, d)))
    if shared:
        c["w1s"] = 0.5 * r.standard_normal((f, d))
        c["w3s"] = 0.5 * r.standard_normal((f, d))
        c["w2s"] = 0.5 * r.standard_normal((d, f))
    c["bias"] = 0.3 * r.standard_normal(E) if bias else None
    c["select_bias"] = (0.5 * r.standard_normal(E)).astype(np.float32) if sbias else None
    return c


def _shared(c):
    return (c["w1s"], c["w3s"], c["w2s"]) if "w1s" in c else None


def _J(c, k, mode, capacity, alpha, beta):
    return O.objective(c["x"], c["w_r"], c["w1"], c["w3"], c["w2"], c["dy"], k, mode,
                       capacity=capacity, bias=c["bias"], shared=_shared(c), alpha=alpha,
                       beta=beta, select_bias=c["select_bias"])


def _routing(c, k, mode, capacity):
    fw = O.forward(c["x"], c["w_r"], c["w1"], c["w3"], c["w2"], k, mode, capacity=capacity,
                   bias=c["bias"], shared=_shared(c), select_bias=c["select_bias"],
                   exact_logits=True)
    return fw["topk_idx"].tobytes() + fw["perm"].tobytes()


def _fd_check(c, k, mode, capacity, alpha, beta, eps=1e-6, tol=2e-6):
    g = O.backward(c["x"], c["w_r"], c["w1"], c["w3"], c["w2"], c["dy"], k, mode,
                   capacity=capacity, bias=c["bias"], shared=_shared(c), alpha=alpha, beta=beta,
                   select_bias=c["select_bias"], exact_logits=True)
    want = dict(x=g["dx"], w_r=g["dw_r"], w1=g["dw1"], w3=g["dw3"], w2=g["dw2"])
    if g["dshared"] is not None:
        want.update(w1s=g["dshared"][0], w3s=g["dshared"][1], w2s=g["dshared"][2])
    base_route = _routing(c, k, mode, capacity)
    for name, an in want.items():
        arr = c[name]
        fd = np.zeros_like(arr)
        for i in np.ndindex(arr.shape):
            keep = arr[i]
            arr[i] = keep + eps
            jp = _J(c, k, mode, capacity, alpha, beta)
            assert _routing(c, k, mode, capacity) == base_route, "selection moved under the step"
            arr[i] = keep - eps
            jm = _J(c, k, mode, capacity, alpha, beta)
            arr[i] = keep
            fd[i] = (jp - jm) / (2 * eps)
        err = np.max(np.abs(fd - an) / (1.0 + np.abs(an)))
        assert err <= tol, "%s: finite differences disagree (%.3e)" % (name, err)
    return g


@pytest.mark.parametrize("mode", MODES)
def test_fd_all_inputs(mode):
    c = _case(1)
    _fd_check(c, 2, mode, None, 0.3, 0.1)


@pytest.mark.parametrize("mode", MODES)
def test_fd_with_drops_shared_and_biases(mode):
    # capacity 2 with 6 tokens x 2 slots over 4 experts: some assignments are dropped
    c = _case(2, T=6, shared=True, bias=True, sbias=True)
    g = _fd_check(c, 2, mode, 2, 0.3, 0.1)
    assert g["fw"]["n_dropped"] > 0
    inv = g["fw"]["inv"].reshape(6, 2)
    assert np.all(g["d_gate"][inv < 0] == 0.0)       # a dropped slot's gate does not reach y


@pytest.mark.parametrize("mode", MODES)
def test_fd_losses_only(mode):
    # dy = 0: only the balancing and z losses move the router (and nothing reaches the experts)
    c = _case(3, k=1)
    c["dy"][:] = 0.0
    g = _fd_check(c, 1, mode, None, 0.7, 0.4)
    assert np.all(g["dw1"] == 0) and np.all(g["dw3"] == 0) and np.all(g["dw2"] == 0)


def test_fd_top1_of_many():
    c = _case(4, T=4, d=3, E=7, k=3, f=5)
    _fd_check(c, 3, O.SIGMOID_TOPK, None, 0.2, 0.05)


def test_swiglu_backward_matches_autograd():
    r = np.random.default_rng(5)
    X, dO = r.standard_normal((7, 5)), r.standard_normal((7, 5))
    w1, w3, w2 = r.standard_normal((6, 5)), r.standard_normal((6, 5)), r.standard_normal((5, 6))
    got = O.swiglu_ffn_backward(X, w1, w3, w2, dO)
    t = [torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (X, w1, w3, w2)]
    out = (torch.nn.functional.silu(t[0] @ t[1].T) * (t[0] @ t[2].T)) @ t[3].T
    out.backward(torch.tensor(dO))
    for a, b in zip(got, t):
        np.testing.assert_allclose(a, b.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_silu_grad_closed_form():
    z = np.array([-30.0, -2.0, 0.0, 1.5, 40.0])
    sg = 1 / (1 + np.exp(-z))
    np.testing.assert_allclose(O.silu_grad(z), sg + z * sg * (1 - sg), rtol=1e-15, atol=1e-300)
    assert O.silu_grad(np.array([0.0]))[0] == 0.5


@pytest.mark.parametrize("mode", [O.SOFTMAX_TOPK, O.SIGMOID_TOPK])
def test_single_expert_gate_cannot_move(mode):
    # k = 1 with renormalisation over the selection: the gate is 1 whatever the logits
    r = np.random.default_rng(6)
    L = r.standard_normal((4, 5)).astype(np.float32)
    idx = O.select_topk(L, 1)
    assert np.all(O.gate_weights(L, idx, mode) == 1.0)
    assert np.all(O.gate_backward(L, idx, mode, r.standard_normal((4, 1))) == 0.0)


def test_softmax_all_equal_gate_gradient_on_every_expert_is_zero():
    # k = E and the same upstream value on every gate: sum_j p_j is 1, so nothing changes
    r = np.random.default_rng(7)
    L = r.standard_normal((3, 4)).astype(np.float32)
    idx = O.select_topk(L, 4)
    dL = O.gate_backward(L, idx, O.SOFTMAX_ALL, np.full((3, 4), 0.7))
    np.testing.assert_allclose(dL, 0.0, atol=1e-15)


def test_balance_gradient_vanishes_under_uniform_routing():
    # equal counts make L_aux = alpha * sum_e P_e = alpha, a constant
    r = np.random.default_rng(8)
    L = r.standard_normal((6, 4))
    dL = O.balance_backward(L, np.array([3, 3, 3, 3]), 6, 4, 2, 0.5, 0.0)
    np.testing.assert_allclose(dL, 0.0, atol=1e-15)


def test_z_gradient_row_sum():
    # d z / d L[t, j] = 2 beta lse_t p_tj / T, and the p_tj of a row sum to 1
    r = np.random.default_rng(9)
    L = 3 * r.standard_normal((5, 6))
    dL = O.balance_backward(L, np.zeros(6), 5, 6, 2, 0.0, 0.25)
    lse = np.log(np.exp(L).sum(axis=1))
    np.testing.assert_allclose(dL.sum(axis=1), 2 * 0.25 * lse / 5, rtol=1e-12)
