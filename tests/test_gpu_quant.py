"""GPU parity of weight-only INT8 / INT4 experts (moe_quantize_weights, moe_expert_ffn_q) against
the CPU oracle (needs an MI355X).  Quantization is an integer decision taken in fp32 on both sides
(the same correctly rounded divisions), so q and the scales are compared bit-exactly; the layer is
compared with the oracle evaluated on the dequantized weights s * q, within the forward tolerance."""

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


@pytest.mark.parametrize("bits", [8, 4])
def test_quantize_exact(M, bits):
    lm = M["lm"]
    rng = np.random.default_rng(bits)
    B, R, C = 3, 70, 512
    w = (rng.standard_normal((B, R, C)) * rng.uniform(1e-3, 5, size=(B, R, 1))).astype(np.float32)
    w[0, 5] = 0.0
    w[1, 7, :3] = [127.0, 2.5, -0.5]                      # ties after scaling (s = 1 when int8)
    w[1, 7, 3:] = 0.0
    wb = torch.from_numpy(w).to(torch.bfloat16)
    wh = wb.float().numpy()                               # the bf16 values both sides quantize
    dev = torch.device("cuda")
    q = torch.empty((B, R, C // (8 // bits)), dtype=torch.uint8, device=dev)
    s = torch.empty((B, R), dtype=torch.float32, device=dev)
    lm.quantize_weights(wb.to(dev), B, R, C, lm.MOE_BF16, bits, q, s)
    torch.cuda.synchronize()
    qo, so = O.quantize_rows(wh, bits)
    np.testing.assert_array_equal(s.cpu().numpy(), so)
    qg = q.cpu().numpy()
    if bits == 8:
        np.testing.assert_array_equal(qg.view(np.int8), qo)
    else:
        np.testing.assert_array_equal(qg, O.pack_int4(qo))


QCASES = [
    # T, d, E, k, d_ff, bits, gating, shared, zipf
    (32, 256, 8, 2, 512, 8, "softmax_topk", 0, 0.0),      # decode-sized: K split
    (32, 256, 8, 2, 512, 4, "softmax_topk", 0, 0.0),
    (300, 128, 8, 2, 384, 8, "sigmoid_topk", 1, 0.0),     # ragged groups past 32 rows
    (300, 128, 8, 2, 384, 4, "softmax_all", 0, 1.1),
    (5, 384, 16, 4, 256, 8, "softmax_topk", 0, 0.0),
    (1024, 256, 4, 1, 640, 4, "softmax_topk", 0, 0.0),
]


@pytest.mark.parametrize("case", QCASES, ids=lambda c: "T%d_d%d_E%d_k%d_f%d_int%d" % c[:6])
def test_quantized_layer(M, case):
    T, d, E, k, f, bits, g, sh, zipf = case
    _say("quantized layer", case)
    synth, layer, lm = M["synth"], M["layer"], M["lm"]
    cfg = synth.tiny_config(T, d, E, k, f, "bf16", g, n_shared=sh, zipf_s=zipf)
    inp = synth.make_inputs(cfg, seed=6, device="cpu")
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
    qw = layer.quantize_experts(cfg, gi, bits)
    b = layer.alloc_buffers(cfg)
    layer.forward_quantized(cfg, gi, b, qw)
    torch.cuda.synchronize()
    h = P.host_inputs(gi)
    deq = []
    for qt, st in ((qw.q1, qw.s1), (qw.q3, qw.s3), (qw.q2, qw.s2)):
        qn = qt.cpu().numpy()
        qn = qn.view(np.int8) if bits == 8 else O.unpack_int4(qn)
        deq.append(O.dequantize_rows(qn, st.cpu().numpy()))
    logits = P.np32(b.logits)
    ref = O.forward(h["x"], h["w_r"], deq[0], deq[1], deq[2], k, P.GATE_CODE[g], bias=h["bias"],
                    shared=h["shared"], alpha=cfg.alpha, beta=cfg.beta, logits=logits)
    P.check_dispatch_exact(b, ref)
    rows = int(ref["offsets"][-1])
    err_rows = P.rel_err(P.np32(b.expert_out)[:rows], ref["expert_out"])
    err = P.rel_err(P.np32(b.y), ref["y"])
    ks = lm.lib()  # noqa: F841
    _say("  expert rows err %.2e, y err %.2e" % (err_rows, err))
    assert err_rows <= P.y_tol(cfg) and err <= P.y_tol(cfg)
    # and the quantized layer stays near the bf16 one (quantization error only)
    b2 = layer.alloc_buffers(cfg)
    layer.forward(cfg, gi, b2)
    torch.cuda.synchronize()
    qerr = P.rel_err(P.np32(b.y), P.np32(b2.y))
    _say("  vs bf16 weights: %.2e" % qerr)
    assert qerr <= (0.05 if bits == 8 else 0.5)
