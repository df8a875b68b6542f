"""The layer's forward and backward captured into a HIP graph and replayed (needs an MI355X).

Serving loops capture a fixed-shape layer once and replay it.  Every entry point only enqueues
work (no host synchronisation, no allocation, no memset); the grouped products of groups
averaging 256-512 rows fork part of their tiles onto the library's side stream and join it back,
which the capture must follow.  Each replay, with eager work and synchronisations in between,
must reproduce the eager results bit for bit (the kernels are deterministic).
"""

import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def M():
    from sparse_mixture_experts_counting_amd import build
    import os
    if not os.path.exists(build.LIB):
        build.build()
    from sparse_mixture_experts_counting_amd import layer, synth
    return dict(layer=layer, synth=synth)


CASES = [
    # T, d, E, k, d_ff, gating, C, shared, zipf
    (300, 128, 8, 2, 192, "softmax_topk", 0, 0, 0.0),        # 128-row tiles
    (700, 256, 4, 2, 512, "softmax_topk", 0, 1, 1.1),        # tall + short tiles on two streams
    (257, 136, 8, 2, 264, "sigmoid_topk", 70, 0, 0.0),       # capacity drops, ragged shapes
]


def _snapshot(b, g=None):
    out = {n: getattr(b, n).clone() for n in ("y", "topk_idx", "topk_gate", "perm", "inv",
                                              "offsets", "aux", "z")}
    if g is not None:
        for n in ("dx", "dw_r", "dw1", "dw3", "dw2", "d_logits"):
            out["g." + n] = getattr(g, n).clone()
    return out


@pytest.mark.parametrize("save", [False, True], ids=["recomputed", "saved"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "T%d_d%d_E%d_k%d_f%d_%s_C%d_s%d" % c[:8])
def test_graph_replay_matches_eager(M, case, save):
    T, d, E, k, f, gating, C, sh, zipf = case
    print("graph", case, "saved" if save else "recomputed", flush=True)
    L, S = M["layer"], M["synth"]
    cfg = S.tiny_config(T, d, E, k, f, "bf16", gating, capacity=C, n_shared=sh, zipf_s=zipf)
    inp = S.make_inputs(cfg, seed=3, device="cuda")
    dy = S.make_dy(cfg, seed=3, device="cuda")
    b = L.alloc_buffers(cfg, save=save)
    g = L.alloc_grads(cfg)

    def step():
        L.forward(cfg, inp, b)
        L.backward(cfg, inp, b, dy, g)

    step()                                   # eager (also creates the library's side stream)
    torch.cuda.synchronize()
    ref = _snapshot(b, g)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                               # warm-up on the capture stream's side, as torch asks
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    for replay in range(3):
        # Eager work between replays: scribble over the outputs, then replay.
        for t in (b.y, b.topk_gate, g.dx, g.dw1):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = _snapshot(b, g)
        for n, v in ref.items():
            assert torch.equal(got[n], v), "replay %d: %s differs from the eager run" % (replay, n)
