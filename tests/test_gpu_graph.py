"""The layer's forward and backward captured into a HIP graph and replayed (needs an MI355X).

Serving loops capture a fixed-shape layer once and replay it.  Every entry point only enqueues
work on the caller's stream (no host synchronisation, no allocation, no memset, no stream of the
library's own); the warm-up runs on the capture stream itself, as torch asks.  Each replay, with
eager work and synchronisations in between, must reproduce the eager results bit for bit (the
kernels are deterministic).
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
    (700, 256, 4, 2, 512, "softmax_topk", 0, 1, 1.1),        # block-sparse tall and thin tiles
    (257, 136, 8, 2, 264, "sigmoid_topk", 70, 0, 0.0),       # capacity drops, ragged shapes
    # more than two rounds of block-sparse tiles: one block per CU taking tiles from counters that
    # a kernel zeroes in the workspace before every launch, replays included
    (2048, 256, 16, 2, 4096, "softmax_topk", 0, 0, 1.2),
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

    step()                                   # eager
    torch.cuda.synchronize()
    ref = _snapshot(b, g)

    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        step()                               # warm-up on the capture stream (off the default
    torch.cuda.current_stream().wait_stream(cap)   # stream, as torch asks)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cap):
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


@pytest.mark.parametrize("shape", [(700, 256, 4, 2, 512, 1, 1.1), (2048, 256, 16, 2, 4096, 0, 1.2)],
                         ids=["one_block_per_tile", "counters"])
def test_two_caller_streams_concurrently(M, shape):
    """Two streams run the block-sparse tiling (skewed groups) at the same time on different
    buffers (each with its own workspace, which holds the tile counters when there are more than
    two rounds of tiles): each result is bit-identical to the same layer run alone on the default
    stream."""
    print("two caller streams", shape, flush=True)
    L, S = M["layer"], M["synth"]
    T, d, E, k, f, sh, zipf = shape
    cfg = S.tiny_config(T, d, E, k, f, "bf16", "softmax_topk", n_shared=sh, zipf_s=zipf)
    inps = [S.make_inputs(cfg, seed=s, device="cuda") for s in (5, 6)]
    refs = []
    for inp in inps:
        b = L.alloc_buffers(cfg)
        L.forward(cfg, inp, b)
        torch.cuda.synchronize()
        refs.append(b.y.clone())
    bufs = [L.alloc_buffers(cfg) for _ in inps]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for st in streams:
        st.wait_stream(torch.cuda.current_stream())
    for rep in range(3):
        for inp, b, st in zip(inps, bufs, streams):
            with torch.cuda.stream(st):
                L.forward(cfg, inp, b, stream=st)
        torch.cuda.synchronize()
        for b, ref in zip(bufs, refs):
            assert torch.equal(b.y, ref), "repeat %d differs from the lone run" % rep
