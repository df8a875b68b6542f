"""One MoE layer forward (and backward) on the GPU through libmoe: buffers plus the C entry points
in order.

Score+Select (moe_route) -> Dispatch (moe_dispatch) -> Compute (moe_expert_ffn, routed experts and
the shared expert when there is one) -> Combine (moe_combine) -> Balance (moe_aux_loss), the step
order of the page "Mixture of experts (MoE)" (tirogla), How it works.  PyTorch only allocates the
device buffers and provides the stream; every step runs in the HIP library.
"""

import dataclasses

import torch

from . import libmoe as lm
from .synth import GATING_CODE


@dataclasses.dataclass
class MoEBuffers:
    logits: torch.Tensor
    topk_idx: torch.Tensor
    topk_gate: torch.Tensor
    prob_sum: torch.Tensor
    lse_sq_sum: torch.Tensor
    counts: torch.Tensor
    offsets: torch.Tensor
    perm: torch.Tensor
    inv: torch.Tensor
    n_dropped: torch.Tensor
    expert_out: torch.Tensor
    shared_out: torch.Tensor
    y: torch.Tensor
    aux: torch.Tensor
    z: torch.Tensor
    workspace: torch.Tensor
    # Saved activations for the backward pass (h | a | b per expert row, bf16), or None: the
    # backward then recomputes a and b.
    saved: torch.Tensor = None
    saved_shared: torch.Tensor = None


def alloc_buffers(cfg, device="cuda", save=False):
    """Device buffers of one forward; save=True adds the saved activations of a training step
    (3 * d_ff bf16 values per expert row and per token of the shared expert)."""
    dev = torch.device(device)
    dt = torch.float32 if cfg.dtype == "fp32" else torch.bfloat16
    code = lm.MOE_F32 if cfg.dtype == "fp32" else lm.MOE_BF16
    T, d, E, k, f = cfg.T, cfg.d, cfg.E, cfg.k, cfg.d_ff
    A = T * k
    i32 = dict(dtype=torch.int32, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    ws = lm.workspace_bytes(T, d, f, E, k, code)
    return MoEBuffers(
        logits=torch.empty((T, E), **f32), topk_idx=torch.empty((T, k), **i32),
        topk_gate=torch.empty((T, k), **f32), prob_sum=torch.empty(E, **f32),
        lse_sq_sum=torch.empty(1, **f32), counts=torch.empty(E, **i32),
        offsets=torch.empty(E + 1, **i32), perm=torch.empty(A, **i32), inv=torch.empty(A, **i32),
        n_dropped=torch.empty(1, **i32), expert_out=torch.empty((A, d), dtype=dt, device=dev),
        shared_out=torch.empty((T, d), dtype=dt, device=dev) if cfg.n_shared else None,
        y=torch.empty((T, d), dtype=dt, device=dev), aux=torch.empty(1, **f32),
        z=torch.empty(1, **f32), workspace=torch.empty(ws, dtype=torch.uint8, device=dev),
        saved=torch.empty((A, 3 * f), dtype=dt, device=dev) if save else None,
        saved_shared=(torch.empty((T, 3 * f), dtype=dt, device=dev)
                      if save and cfg.n_shared else None))


def route(cfg, inp, b, logits_in=False, stream=None):
    code = lm.MOE_F32 if cfg.dtype == "fp32" else lm.MOE_BF16
    lm.route(None if logits_in else inp.x, None if logits_in else inp.w_r,
             None if logits_in else inp.bias, cfg.T, cfg.d, cfg.E, cfg.k, code,
             GATING_CODE[cfg.gating], lm.ROUTE_LOGITS_IN if logits_in else 0, b.logits,
             b.topk_idx, b.topk_gate, b.prob_sum, b.lse_sq_sum, b.workspace, stream,
             select_bias=getattr(inp, "select_bias", None))


def dispatch(cfg, b, stream=None):
    lm.dispatch(b.topk_idx, cfg.T, cfg.E, cfg.k, cfg.capacity, b.counts, b.offsets, b.perm, b.inv,
                b.n_dropped, b.workspace, stream)


def experts(cfg, inp, b, stream=None):
    code = lm.MOE_F32 if cfg.dtype == "fp32" else lm.MOE_BF16
    if b.saved is not None:
        lm.expert_ffn_save(inp.x, b.perm, b.offsets, cfg.T, cfg.d, cfg.d_ff, cfg.E, cfg.k, inp.w1,
                           inp.w3, inp.w2, code, b.expert_out, b.saved, b.workspace, stream)
    else:
        lm.expert_ffn(inp.x, b.perm, b.offsets, cfg.T, cfg.d, cfg.d_ff, cfg.E, cfg.k, inp.w1,
                      inp.w3, inp.w2, code, b.expert_out, b.workspace, stream)
    if cfg.n_shared:
        w1s, w3s, w2s = inp.shared
        if b.saved_shared is not None:
            lm.expert_ffn_save(inp.x, None, None, cfg.T, cfg.d, cfg.d_ff, 1, 1, w1s, w3s, w2s,
                               code, b.shared_out, b.saved_shared, b.workspace, stream)
        else:
            lm.expert_ffn(inp.x, None, None, cfg.T, cfg.d, cfg.d_ff, 1, 1, w1s, w3s, w2s, code,
                          b.shared_out, b.workspace, stream)


def combine(cfg, b, stream=None):
    code = lm.MOE_F32 if cfg.dtype == "fp32" else lm.MOE_BF16
    lm.combine(b.expert_out, b.inv, b.topk_gate, cfg.T, cfg.d, cfg.k, code, b.shared_out, b.y,
               stream)


def losses(cfg, b, stream=None):
    lm.aux_loss(b.counts, b.prob_sum, b.lse_sq_sum, cfg.T, cfg.E, cfg.k, cfg.alpha, cfg.beta,
                b.aux, b.z, stream)


def forward(cfg, inp, b, stream=None, logits_in=False):
    """The whole hot path on one stream; no host synchronisation inside."""
    route(cfg, inp, b, logits_in, stream)
    dispatch(cfg, b, stream)
    experts(cfg, inp, b, stream)
    combine(cfg, b, stream)
    losses(cfg, b, stream)
    return b


@dataclasses.dataclass
class MoEGrads:
    d_out: torch.Tensor       # [T*k, d] gradient of each expert row
    d_gate: torch.Tensor      # [T, k] fp32
    dx_rows: torch.Tensor     # [T*k, d] input gradient of each expert row
    d_logits: torch.Tensor    # [T, E] fp32
    dx_route: torch.Tensor    # [T, d] router (+ shared expert) part of dx
    dx: torch.Tensor          # [T, d]
    dw_r: torch.Tensor        # [E, d] fp32
    dw1: torch.Tensor         # [E, d_ff, d] fp32
    dw3: torch.Tensor
    dw2: torch.Tensor         # [E, d, d_ff] fp32
    dshared: tuple            # (dw1s, dw3s, dw2s) fp32 or None
    dx_shared: torch.Tensor   # [T, d] or None
    workspace: torch.Tensor


def alloc_grads(cfg, device="cuda"):
    dev = torch.device(device)
    if cfg.dtype != "bf16":
        raise ValueError("the backward pass runs bf16 layers only")
    T, d, E, k, f = cfg.T, cfg.d, cfg.E, cfg.k, cfg.d_ff
    bf = dict(dtype=torch.bfloat16, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    ws = lm.backward_workspace_bytes(T, d, f, E, k, lm.MOE_BF16)
    shared = None
    if cfg.n_shared:
        shared = (torch.empty((f, d), **f32), torch.empty((f, d), **f32),
                  torch.empty((d, f), **f32))
    return MoEGrads(
        d_out=torch.empty((T * k, d), **bf), d_gate=torch.empty((T, k), **f32),
        dx_rows=torch.empty((T * k, d), **bf), d_logits=torch.empty((T, E), **f32),
        dx_route=torch.empty((T, d), **bf), dx=torch.empty((T, d), **bf),
        dw_r=torch.empty((E, d), **f32), dw1=torch.empty((E, f, d), **f32),
        dw3=torch.empty((E, f, d), **f32), dw2=torch.empty((E, d, f), **f32), dshared=shared,
        dx_shared=torch.empty((T, d), **bf) if cfg.n_shared else None,
        workspace=torch.empty(ws, dtype=torch.uint8, device=dev))


def backward(cfg, inp, b, dy, g, stream=None):
    """Gradient of <dy, y> + aux + z after forward(cfg, inp, b): the steps in reverse order
    (Combine, Compute of the routed and shared experts, Score and Balance), then the input
    gradient rows added per token.  With saved activations (alloc_buffers(save=True)) the
    expert gradients read them instead of recomputing the up projection.  No host
    synchronisation inside."""
    T, d, f, E, k = cfg.T, cfg.d, cfg.d_ff, cfg.E, cfg.k
    bf = lm.MOE_BF16
    lm.combine_backward(dy, b.expert_out, b.inv, b.topk_gate, T, d, k, bf, g.d_out, g.d_gate,
                        stream)
    if b.saved is not None:
        lm.expert_backward_saved(b.saved, inp.x, b.perm, b.offsets, T, d, f, E, k, inp.w1,
                                 inp.w3, inp.w2, g.d_out, bf, g.dx_rows, g.dw1, g.dw3, g.dw2,
                                 g.workspace, stream)
    else:
        lm.expert_backward(inp.x, b.perm, b.offsets, T, d, f, E, k, inp.w1, inp.w3, inp.w2,
                           g.d_out, bf, g.dx_rows, g.dw1, g.dw3, g.dw2, g.workspace, stream)
    if cfg.n_shared:
        w1s, w3s, w2s = inp.shared
        if b.saved_shared is not None:
            lm.expert_backward_saved(b.saved_shared, inp.x, None, None, T, d, f, 1, 1, w1s, w3s,
                                     w2s, dy, bf, g.dx_shared, *g.dshared, g.workspace, stream)
        else:
            lm.expert_backward(inp.x, None, None, T, d, f, 1, 1, w1s, w3s, w2s, dy, bf,
                               g.dx_shared, *g.dshared, g.workspace, stream)
    lm.route_backward(inp.x, inp.w_r, b.logits, b.topk_idx, b.topk_gate, g.d_gate, b.counts, T, d,
                      E, k, bf, GATING_CODE[cfg.gating], cfg.alpha, cfg.beta, g.dx_shared,
                      g.d_logits, g.dw_r, g.dx_route, g.workspace, stream)
    lm.combine(g.dx_rows, b.inv, None, T, d, k, bf, g.dx_route, g.dx, stream)
    return g


@dataclasses.dataclass
class ECBuffers:
    logits: torch.Tensor      # [T, E] fp32
    topk_idx: torch.Tensor    # [T, 1] (moe_route output, unused by expert choice)
    topk_gate: torch.Tensor
    scores: torch.Tensor      # [T, E] fp32 router probabilities
    offsets: torch.Tensor     # [E + 1]
    perm: torch.Tensor        # [E * c] token of each expert row
    gate: torch.Tensor        # [E * c] fp32
    slot: torch.Tensor        # [T, E] row of each pick or -1
    expert_out: torch.Tensor  # [E * c, d]
    shared_out: torch.Tensor
    y: torch.Tensor
    workspace: torch.Tensor


def ec_rows(cfg):
    """Expert rows under Expert Choice: each expert keeps c = min(C, T) tokens."""
    return cfg.E * min(cfg.capacity, cfg.T)


def alloc_ec_buffers(cfg, device="cuda"):
    dev = torch.device(device)
    dt = torch.float32 if cfg.dtype == "fp32" else torch.bfloat16
    code = lm.MOE_F32 if cfg.dtype == "fp32" else lm.MOE_BF16
    T, d, E, f = cfg.T, cfg.d, cfg.E, cfg.d_ff
    R = ec_rows(cfg)
    i32 = dict(dtype=torch.int32, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    ws = max(lm.gathered_workspace_bytes(R, d, f, E, code), lm.workspace_bytes(T, d, f, E, 1, code))
    return ECBuffers(
        logits=torch.empty((T, E), **f32), topk_idx=torch.empty((T, 1), **i32),
        topk_gate=torch.empty((T, 1), **f32), scores=torch.empty((T, E), **f32),
        offsets=torch.empty(E + 1, **i32), perm=torch.empty(R, **i32), gate=torch.empty(R, **f32),
        slot=torch.empty((T, E), **i32), expert_out=torch.empty((R, d), dtype=dt, device=dev),
        shared_out=torch.empty((T, d), dtype=dt, device=dev) if cfg.n_shared else None,
        y=torch.empty((T, d), dtype=dt, device=dev),
        workspace=torch.empty(ws, dtype=torch.uint8, device=dev))


def forward_expert_choice(cfg, inp, b, stream=None):
    """The layer under Expert Choice routing (cfg.capacity = tokens per expert): router logits
    (moe_route, k = 1, its top-k unused), per-expert top-C selection (moe_expert_choice), the
    experts on their rows (moe_expert_ffn_gathered, plus the shared expert), and the combine with
    one slot per expert (moe_combine, k = E)."""
    code = lm.MOE_F32 if cfg.dtype == "fp32" else lm.MOE_BF16
    T, d, E, f = cfg.T, cfg.d, cfg.E, cfg.d_ff
    lm.route(inp.x, inp.w_r, inp.bias, T, d, E, 1, code, 0, 0, b.logits, b.topk_idx, b.topk_gate,
             None, None, None, stream)
    lm.expert_choice(b.logits, T, E, cfg.capacity, 0, b.scores, b.offsets, b.perm, b.gate, b.slot,
                     stream)
    lm.expert_ffn_gathered(inp.x, b.perm, b.offsets, T, d, f, E, ec_rows(cfg), inp.w1, inp.w3,
                           inp.w2, code, b.expert_out, b.workspace, stream)
    if cfg.n_shared:
        w1s, w3s, w2s = inp.shared
        lm.expert_ffn(inp.x, None, None, T, d, f, 1, 1, w1s, w3s, w2s, code, b.shared_out,
                      b.workspace, stream)
    lm.combine(b.expert_out, b.slot, b.scores, T, d, E, code, b.shared_out, b.y, stream)
    return b


@dataclasses.dataclass
class RerouteBuffers:
    topk_idx: torch.Tensor    # [T, k] final selection
    topk_gate: torch.Tensor   # [T, k] gates over it
    offsets: torch.Tensor
    perm: torch.Tensor
    inv: torch.Tensor
    n_dropped: torch.Tensor


def alloc_reroute_buffers(cfg, device="cuda"):
    dev = torch.device(device)
    T, E, k = cfg.T, cfg.E, cfg.k
    i32 = dict(dtype=torch.int32, device=dev)
    return RerouteBuffers(
        topk_idx=torch.empty((T, k), **i32),
        topk_gate=torch.empty((T, k), dtype=torch.float32, device=dev),
        offsets=torch.empty(E + 1, **i32), perm=torch.empty(T * k, **i32),
        inv=torch.empty(T * k, **i32), n_dropped=torch.empty(1, **i32))


def forward_reroute(cfg, inp, b, r, stream=None):
    """The layer with overflow sent to the next-best expert: route, capacity dispatch (round 1),
    moe_reroute (round 2), then the experts, the combine over the final layout and the losses (f
    from the round-1 counts)."""
    code = lm.MOE_F32 if cfg.dtype == "fp32" else lm.MOE_BF16
    route(cfg, inp, b, stream=stream)
    dispatch(cfg, b, stream)
    lm.reroute(b.logits, getattr(inp, "select_bias", None), b.topk_idx, b.topk_gate, b.offsets,
               b.inv, cfg.T, cfg.E, cfg.k, cfg.capacity, GATING_CODE[cfg.gating], r.topk_idx,
               r.topk_gate, r.offsets, r.perm, r.inv, r.n_dropped, b.workspace, stream)
    lm.expert_ffn(inp.x, r.perm, r.offsets, cfg.T, cfg.d, cfg.d_ff, cfg.E, cfg.k, inp.w1, inp.w3,
                  inp.w2, code, b.expert_out, b.workspace, stream)
    if cfg.n_shared:
        w1s, w3s, w2s = inp.shared
        lm.expert_ffn(inp.x, None, None, cfg.T, cfg.d, cfg.d_ff, 1, 1, w1s, w3s, w2s, code,
                      b.shared_out, b.workspace, stream)
    lm.combine(b.expert_out, r.inv, r.topk_gate, cfg.T, cfg.d, cfg.k, code, b.shared_out, b.y,
               stream)
    losses(cfg, b, stream)
    return b


@dataclasses.dataclass
class QuantWeights:
    bits: int
    q1: torch.Tensor          # int8 [E, d_ff, d] or uint8 [E, d_ff, d / 2]
    s1: torch.Tensor          # fp32 [E, d_ff]
    q3: torch.Tensor
    s3: torch.Tensor
    q2: torch.Tensor          # [E, d, d_ff] or [E, d, d_ff / 2]
    s2: torch.Tensor          # fp32 [E, d]
    workspace: torch.Tensor


def quantize_experts(cfg, inp, bits, device="cuda"):
    """Weight-only INT8 / INT4 copies of the routed experts (moe_quantize_weights), load time."""
    dev = torch.device(device)
    E, d, f = cfg.E, cfg.d, cfg.d_ff
    div = 8 // bits
    mk = lambda rows, cols: (torch.empty((E, rows, cols // div), dtype=torch.uint8, device=dev),
                             torch.empty((E, rows), dtype=torch.float32, device=dev))
    (q1, s1), (q3, s3), (q2, s2) = mk(f, d), mk(f, d), mk(d, f)
    lm.quantize_weights(inp.w1, E, f, d, lm.MOE_BF16, bits, q1, s1)
    lm.quantize_weights(inp.w3, E, f, d, lm.MOE_BF16, bits, q3, s3)
    lm.quantize_weights(inp.w2, E, d, f, lm.MOE_BF16, bits, q2, s2)
    ws = lm.q_workspace_bytes(cfg.T, d, f, E, cfg.k, bits)
    return QuantWeights(bits, q1, s1, q3, s3, q2, s2,
                        torch.empty(ws, dtype=torch.uint8, device=dev))


def forward_quantized(cfg, inp, b, qw, stream=None):
    """The layer with weight-only quantized routed experts (moe_expert_ffn_q); routing, dispatch,
    the shared expert, combine and losses as in forward()."""
    route(cfg, inp, b, stream=stream)
    dispatch(cfg, b, stream)
    lm.expert_ffn_q(inp.x, b.perm, b.offsets, cfg.T, cfg.d, cfg.d_ff, cfg.E, cfg.k, qw.bits,
                    qw.q1, qw.s1, qw.q3, qw.s3, qw.q2, qw.s2, lm.MOE_BF16, b.expert_out,
                    qw.workspace, stream)
    if cfg.n_shared:
        w1s, w3s, w2s = inp.shared
        lm.expert_ffn(inp.x, None, None, cfg.T, cfg.d, cfg.d_ff, 1, 1, w1s, w3s, w2s, lm.MOE_BF16,
                      b.shared_out, b.workspace, stream)
    combine(cfg, b, stream)
    losses(cfg, b, stream)
    return b
