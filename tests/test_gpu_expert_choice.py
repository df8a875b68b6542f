"""GPU parity of Expert Choice routing (moe_expert_choice, moe_expert_ffn_gathered and moe_combine
with one slot per expert) against the CPU oracle (needs an MI355X).

The selection is an integer decision taken on fp32 scores, so both sides take it on the same
values: from given scores (adversarial ties) and, end to end, the oracle selects on the GPU's own
scores (which are compared with the oracle's softmax separately).  Selection outputs are compared
bit-exactly; y within the forward tolerance.
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
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return dict(layer=layer, lm=libmoe, synth=synth)


def _say(*a):
    print(*a, flush=True)


def _select_on_gpu(M, S, C):
    lm = M["lm"]
    T, E = S.shape
    c = min(C, T)
    dev = torch.device("cuda")
    sc = torch.from_numpy(np.ascontiguousarray(S, dtype=np.float32)).to(dev)
    offs = torch.empty(E + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(E * c, dtype=torch.int32, device=dev)
    gate = torch.empty(E * c, dtype=torch.float32, device=dev)
    slot = torch.empty((T, E), dtype=torch.int32, device=dev)
    lm.expert_choice(None, T, E, C, lm.EC_SCORES_IN, sc, offs, perm, gate, slot)
    torch.cuda.synchronize()
    return P.npi(offs), P.npi(perm), P.np32(gate), P.npi(slot)


def _check_selection(got, S, C):
    offs, perm, gate, slot = O.expert_choice(S, C)
    np.testing.assert_array_equal(got[0], offs)
    np.testing.assert_array_equal(got[1], perm)
    np.testing.assert_array_equal(got[2], gate.astype(np.float32))
    np.testing.assert_array_equal(got[3], slot)


@pytest.mark.parametrize("T,E,C", [(1, 1, 1), (7, 3, 2), (300, 8, 90), (2500, 4, 700),
                                   (1030, 64, 17), (64, 256, 2), (50, 5, 50), (40, 6, 100)])
def test_selection_from_given_scores(M, T, E, C):
    _say("ec select", T, E, C)
    rng = np.random.default_rng(T + 7 * E + C)
    S = rng.random((T, E)).astype(np.float32)
    S[::3] = np.round(S[::3] * 4) / 4                 # many exact ties across tokens
    if T > 4:
        S[1] = -0.0
        S[2] = 0.0                                    # -0 and +0 tie, lower token first
        S[3, 0] = np.float32(1e-40)                   # denormal
    _check_selection(_select_on_gpu(M, S, C), S, C)


def test_selection_all_equal_takes_lowest_tokens(M):
    S = np.full((1000, 3), 0.25, dtype=np.float32)
    got = _select_on_gpu(M, S, 10)
    assert got[1].tolist() == list(range(10)) * 3
    _check_selection(got, S, 10)


EC_CASES = [
    # T, d, E, C, d_ff, dtype, shared
    (64, 32, 4, 20, 64, "fp32", 0),
    (300, 128, 8, 90, 192, "bf16", 1),
    (257, 136, 16, 40, 264, "bf16", 0),
    (100, 64, 64, 3, 64, "bf16", 0),
    (37, 64, 4, 50, 96, "bf16", 0),
    (64, 64, 256, 2, 64, "bf16", 0),
    (2048, 256, 8, 320, 512, "bf16", 0),
]


@pytest.mark.parametrize("case", EC_CASES, ids=lambda c: "T%d_d%d_E%d_C%d_f%d_%s_s%d" % c)
def test_expert_choice_layer(M, case):
    T, d, E, C, f, dt, sh = case
    _say("ec layer", case)
    cfg = M["synth"].tiny_config(T, d, E, 1, f, dt, "softmax_all", capacity=C, n_shared=sh)
    inp = M["synth"].make_inputs(cfg, seed=2, device="cpu")
    import dataclasses
    kw = {}
    for fl in dataclasses.fields(inp):
        v = getattr(inp, fl.name)
        if isinstance(v, torch.Tensor):
            v = v.cuda()
        elif isinstance(v, tuple):
            v = tuple(t.cuda() for t in v)
        kw[fl.name] = v
    g = type(inp)(**kw)
    b = M["layer"].alloc_ec_buffers(cfg)
    M["layer"].forward_expert_choice(cfg, g, b)
    torch.cuda.synchronize()
    h = P.host_inputs(g)
    logits = P.np32(b.logits)
    scores = P.np32(b.scores)
    p, _ = O.row_softmax_lse(logits)
    assert np.max(np.abs(scores - p)) <= 2e-6, "scores"
    ref = O.forward_expert_choice(h["x"], h["w_r"], h["w1"], h["w3"], h["w2"], C,
                                  shared=h["shared"], logits=logits, scores=scores)
    np.testing.assert_array_equal(P.npi(b.offsets), ref["offsets"])
    np.testing.assert_array_equal(P.npi(b.perm), ref["perm"])
    np.testing.assert_array_equal(P.npi(b.slot), ref["slot"])
    np.testing.assert_array_equal(P.np32(b.gate), ref["gate"].astype(np.float32))
    counts = np.bincount(ref["perm"], minlength=T)
    _say("  tokens kept by 0 experts: %d, max %d" % (int(np.sum(counts == 0)), int(counts.max())))
    err = P.rel_err(P.np32(b.y), ref["y"])
    assert err <= P.y_tol(cfg), "y relative error %.3e" % err
