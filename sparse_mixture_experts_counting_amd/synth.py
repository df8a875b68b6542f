"""Seeded synthetic inputs for the MoE layer workloads.

This module only draws and casts random tensors (and builds the one non-random input, the Zipf
logit bias); it holds none of the layer's arithmetic, so both the GPU path and the CPU oracle can
be fed from it without sharing any computation.

Workloads (shapes from the pages' model descriptions: Mixtral d=4096, d_ff=14336, 8 experts, top-2
in "DL S077 - Mixture of Experts (MoE) Intuition", section 4; DeepSeek-V3 256 routed + 1 shared,
top-8 in its section 8.2; Switch top-1 with capacity factor 1.25 in "Mixture of experts (MoE)"
(tirogla), Complexity and constants):

  tiny_fp32          T=64   d=32   E=4   k=2 d_ff=64    fp32 softmax_topk C=64
  switch_top1        T=2048 d=512  E=8   k=1 d_ff=2048  bf16 softmax_all  C=320, router x3
  switch_top1_c256   as switch_top1 with C=256 (capacity factor 1.0: forces drops)
  mixtral_prefill    T=4096 d=4096 E=8   k=2 d_ff=14336 bf16 softmax_topk no capacity
  deepseek_fine      T=8192 d=7168 E=256 k=8 d_ff=2048  bf16 sigmoid_topk no capacity,
                     1 shared expert, Zipf(s=1.1) logit bias
  mixtral_decode     T=32   d=4096 E=8   k=2 d_ff=14336 bf16 softmax_topk no capacity

Weights are held [out][in], as linear layers store them (the expert and router modules of the
"DL S077" page, sections 1.1 and 1.2, are bias-free linear layers).  Draw order for one seed:
x = randn(T, d); W_r = randn(E, d) / sqrt(d) (times router_scale); for each expert e:
w1[e] = randn(d_ff, d) / sqrt(d), w3[e] = randn(d_ff, d) / sqrt(d), w2[e] = randn(d, d_ff) / sqrt(d_ff);
then the shared expert's w1, w3, w2 the same way.  Each tensor is
cast to the layer dtype right after it is drawn (bfloat16 round-to-nearest-even).  On device "cpu"
the draws come from torch's CPU generator; on a GPU device from torch's device generator (much faster
for the multi-GB workloads; a different but equally deterministic stream).
"""

import dataclasses
import math

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int
    d: int
    E: int
    k: int
    d_ff: int
    dtype: str            # "fp32" or "bf16"
    gating: str           # "softmax_topk" | "softmax_all" | "sigmoid_topk"
    capacity: int = 0     # 0 = unlimited
    router_scale: float = 1.0
    n_shared: int = 0
    zipf_s: float = 0.0   # 0 = no logit bias
    alpha: float = 0.01
    beta: float = 1e-3

    def replace(self, **kw):
        return dataclasses.replace(self, **kw)


CONFIGS = {
    c.name: c for c in [
        MoEConfig("tiny_fp32", 64, 32, 4, 2, 64, "fp32", "softmax_topk", capacity=64),
        MoEConfig("switch_top1", 2048, 512, 8, 1, 2048, "bf16", "softmax_all", capacity=320,
                  router_scale=3.0),
        MoEConfig("switch_top1_c256", 2048, 512, 8, 1, 2048, "bf16", "softmax_all", capacity=256,
                  router_scale=3.0),
        MoEConfig("mixtral_prefill", 4096, 4096, 8, 2, 14336, "bf16", "softmax_topk"),
        MoEConfig("deepseek_fine", 8192, 7168, 256, 8, 2048, "bf16", "sigmoid_topk", n_shared=1,
                  zipf_s=1.1),
        MoEConfig("mixtral_decode", 32, 4096, 8, 2, 14336, "bf16", "softmax_topk"),
    ]
}

GATING_CODE = {"softmax_topk": 0, "softmax_all": 1, "sigmoid_topk": 2}


def torch_dtype(cfg):
    return torch.float32 if cfg.dtype == "fp32" else torch.bfloat16


def zipf_logit_bias(E, s):
    """Log of a Zipf(s) pmf over expert ranks 1..E (rank = expert index + 1), as float32.

    b_e = -s * ln(e + 1) - ln(H), H = sum_{r=1..E} r^-s.  This is an input of the layer (a
    per-expert logit offset that skews the load), not part of the method."""
    H = sum(r ** (-s) for r in range(1, E + 1))
    b = [-s * math.log(e + 1) - math.log(H) for e in range(E)]
    return np.asarray(b, dtype=np.float32)


@dataclasses.dataclass
class MoEInputs:
    cfg: MoEConfig
    x: torch.Tensor          # [T, d]
    w_r: torch.Tensor        # [E, d]      (all weights: [out][in], as linear layers hold them)
    w1: torch.Tensor         # [E, d_ff, d]
    w3: torch.Tensor         # [E, d_ff, d]
    w2: torch.Tensor         # [E, d, d_ff]
    shared: tuple = None     # (w1s [d_ff, d], w3s [d_ff, d], w2s [d, d_ff]) or None
    bias: torch.Tensor = None  # float32 [E] or None
    select_bias: torch.Tensor = None  # float32 [E] or None: biases expert selection only


def make_inputs(cfg, seed=0, device="cpu"):
    """Draw every input of one workload in the fixed order described in the module docstring."""
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    dt = torch_dtype(cfg)
    T, d, E, d_ff = cfg.T, cfg.d, cfg.E, cfg.d_ff

    def draw(shape, scale):
        t = torch.randn(shape, generator=gen, device=dev, dtype=torch.float32)
        if scale != 1.0:
            t.mul_(scale)
        return t.to(dt)

    x = draw((T, d), 1.0)
    w_r = draw((E, d), cfg.router_scale / math.sqrt(d))
    w1 = torch.empty((E, d_ff, d), dtype=dt, device=dev)
    w3 = torch.empty((E, d_ff, d), dtype=dt, device=dev)
    w2 = torch.empty((E, d, d_ff), dtype=dt, device=dev)
    for e in range(E):
        w1[e] = draw((d_ff, d), 1.0 / math.sqrt(d))
        w3[e] = draw((d_ff, d), 1.0 / math.sqrt(d))
        w2[e] = draw((d, d_ff), 1.0 / math.sqrt(d_ff))
    shared = None
    if cfg.n_shared:
        if cfg.n_shared != 1:
            raise ValueError("one shared expert supported")
        shared = (draw((d_ff, d), 1.0 / math.sqrt(d)), draw((d_ff, d), 1.0 / math.sqrt(d)),
                  draw((d, d_ff), 1.0 / math.sqrt(d_ff)))
    bias = None
    if cfg.zipf_s:
        bias = torch.from_numpy(zipf_logit_bias(E, cfg.zipf_s)).to(dev)
    return MoEInputs(cfg, x, w_r, w1, w3, w2, shared, bias)


def tiny_config(T, d, E, k, d_ff, dtype="bf16", gating="softmax_topk", capacity=0, n_shared=0,
                zipf_s=0.0, router_scale=1.0):
    """An ad-hoc workload for property sweeps."""
    return MoEConfig("adhoc_T%d_d%d_E%d_k%d_f%d" % (T, d, E, k, d_ff), T, d, E, k, d_ff, dtype,
                     gating, capacity=capacity, n_shared=n_shared, zipf_s=zipf_s,
                     router_scale=router_scale)


def p5_main_logits():
    """The deterministic 64 x 8 logit table of the tirogla page's Code `main`: entry i of the
    row-major table is ((i * 2654435761) >> 7) % 1000 / 250 (64-bit unsigned arithmetic)."""
    i = np.arange(64 * 8, dtype=np.uint64)
    v = ((i * np.uint64(2654435761)) >> np.uint64(7)) % np.uint64(1000)
    return (v.astype(np.float32) / np.float32(250.0)).reshape(64, 8)


def make_dy(cfg, seed=0, device="cpu"):
    """Upstream gradient of the layer output for the backward pass: standard normal [T, d] in the
    layer dtype, from its own generator (seed + 1000003) so the forward inputs are unchanged."""
    gen = torch.Generator(device=torch.device(device))
    gen.manual_seed(seed + 1000003)
    dt = torch.float32 if cfg.dtype == "fp32" else torch.bfloat16
    return torch.randn((cfg.T, cfg.d), generator=gen, device=torch.device(device)).to(dt)
