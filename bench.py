#!/usr/bin/env python3
"""Benchmark of one top-k routed MoE FFN layer forward on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic tokens: router product and
gating (moe_route), counting-sort dispatch (moe_dispatch), the SwiGLU up projection and the down
projection of every expert as grouped GEMMs (moe_expert_up / moe_expert_down; plus the shared
expert when the workload has one), the gate-weighted combine (moe_combine) and the loss reduction
(moe_aux_loss).  Inputs are resident in HBM before timing starts.

Prints ONE JSON line: tokens/s of the layer, per-stage kernel times from HIP events recorded on the
stream the kernels run on, the roofline of the dominant kernel (the fused up projection + SwiGLU
grouped GEMM) against the bf16 matrix-core peak, and the CPU oracle timed on a bounded sample.

    python bench.py [--steps K] [--warmup W] [--workload mixtral_prefill]

The timed steps replay the forward step captured once into a HIP graph (the serving form of a
fixed-shape layer: the same kernels, without the per-kernel launch gaps); --eager times them as
launched one by one.  The per-stage breakdown always comes from eager steps with events between
the stages, and the line also carries the eager step time.

With --pass train a step is the forward followed by the backward pass of the layer (gradients of
<dy, y> + aux + z for x, the router and every expert weight: moe_combine_backward,
moe_expert_backward for the routed and shared experts, moe_route_backward, and moe_combine adding
each token's input-gradient rows); that line reports training-step tokens/s and the roofline of
the expert backward.  The training step saves the experts' activations in the forward pass
(moe_expert_ffn_save, moe_expert_backward_saved); --recompute recomputes them in the backward
pass instead (moe_expert_ffn, moe_expert_backward).  With --routing expert_choice the forward runs under Expert Choice routing
(moe_expert_choice, C = T*k/E tokens per expert) and reports its own line; with --routing reroute
the capacity is C = T*k/E and overflowed assignments go to their next-best expert (moe_reroute);
with --weights int8 / int4 the routed experts are weight-only quantized (moe_expert_ffn_q).
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 matrix-core peak
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E peak
DOMINANT = "expert_up"        # fused up projection + SwiGLU grouped GEMM
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_%s.json")
KERNEL_SRC = os.path.join(ROOT, "sparse_mixture_experts_counting_amd", "csrc", "gemm_bf16.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash():
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def load_traffic(workload):
    """HBM bytes per launch of the dominant kernel from the committed PMC summary, if it was taken
    on the current kernel source; else None."""
    path = TRAFFIC_FILE % workload
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def host_info():
    """The host the CPU oracle runs on: CPU model, logical CPUs, the CPUs this process may use,
    and the BLAS library NumPy calls with its thread count."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    from threadpoolctl import threadpool_info
    blas = [p for p in threadpool_info() if p.get("user_api") == "blas"]
    b = blas[0] if blas else {}
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = None
    return {"cpu_model": model, "host_cpus": os.cpu_count(), "affinity_cpus": affinity,
            "blas": ("%s %s, %s threading" % (b.get("internal_api"), b.get("version"),
                                              b.get("threading_layer"))) if b else None,
            "blas_threads": b.get("num_threads", 1)}


def cpu_baseline(cfg, inp, n_tokens, repeats):
    """The CPU oracle as it stands on the first n_tokens tokens of the same workload (all of them
    when n_tokens <= 0): `repeats` timed runs of its float32 pass (the same code with float32
    working precision), then one float64 pass (the precision every correctness check uses) for
    reference.  Returns the cpu_baseline object."""
    import numpy as np
    from oracle import moe_oracle as O

    n = cfg.T if n_tokens <= 0 else min(n_tokens, cfg.T)
    f = lambda t: t.detach().float().cpu().numpy()
    x = f(inp.x[:n])
    w_r = f(inp.w_r)
    bias = None if inp.bias is None else f(inp.bias)
    mode = {"softmax_topk": 0, "softmax_all": 1, "sigmoid_topk": 2}[cfg.gating]
    # Host copies of the experts this sample touches (copying is not part of the timed work).
    idx = O.select_topk(O.router_logits(x, w_r, bias), cfg.k)
    used = sorted(set(idx.reshape(-1).tolist()))
    w1 = {e: f(inp.w1[e]) for e in used}
    w3 = {e: f(inp.w3[e]) for e in used}
    w2 = {e: f(inp.w2[e]) for e in used}
    shared = tuple(f(w) for w in inp.shared) if inp.shared is not None else None
    cap = cfg.capacity
    if cap > 0:   # same capacity factor on the smaller batch
        cap = max(1, int(math.ceil(cap * n / cfg.T)))

    def run():
        O.forward(x, w_r, w1, w3, w2, cfg.k, mode, capacity=cap, bias=bias, shared=shared,
                  alpha=cfg.alpha, beta=cfg.beta)

    with O.working_precision(np.float32):
        run()                                   # untimed first pass (page-in, BLAS start-up)
        t0 = time.perf_counter()
        for _ in range(repeats):
            run()
        secs32 = time.perf_counter() - t0
    t0 = time.perf_counter()
    run()
    secs64 = time.perf_counter() - t0
    hi = host_info()
    sample = ("first %d of %d tokens of %s, every step of the layer, %d experts touched; "
              "float32 pass of the NumPy oracle, %d timed runs after one untimed"
              % (n, cfg.T, cfg.name, len(used), repeats))
    out = {"value": n * repeats / secs32, "unit": "tokens/s", "cores": hi["blas_threads"],
           "kind": "oracle", "precision": "float32", "sample": sample, "seconds": secs32,
           "float64_pass": {"value": n / secs64, "unit": "tokens/s", "seconds": secs64}}
    out.update(hi)
    return out


def measured_peaks(torch, lm, dev, gemm_shape=None):
    """The chip's measured ceilings beside its published ones: a loop of bf16 32x32x16 matrix
    instructions on random register operands (moe_peak_mfma) and a 1 GiB streaming copy
    (moe_peak_copy), each the best of 10 launches timed with HIP events.  With `gemm_shape`
    (M, N, K), also PyTorch's library GEMM (torch.nn.functional.linear in bf16, weights [N][K]) on
    that dense shape, a reference for what the vendor library reaches at the same size."""
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    g = torch.Generator(device=dev)
    g.manual_seed(12345)
    ops = torch.randn(2048, generator=g, device=dev).to(torch.bfloat16)
    blocks, iters = 4 * cus, 2000
    out = torch.empty(blocks * 512, dtype=torch.float32, device=dev)
    flops = float(blocks) * 8 * iters * 8 * 32768
    nbytes = 1 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(3)
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream(dev)

    def best(fn):
        times = []
        for _ in range(11):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            b.synchronize()
            times.append(a.elapsed_time(b))
        return min(times[1:])

    t_mfma = best(lambda: lm.peak_mfma(ops, blocks, iters, out))
    t_copy = best(lambda: lm.peak_copy(src, dst, nbytes))
    del src, dst
    lib = None
    if gemm_shape is not None:
        M, N, K = gemm_shape
        a = torch.randn(M, K, generator=g, device=dev).to(torch.bfloat16)
        w = torch.randn(N, K, generator=g, device=dev).to(torch.bfloat16)
        c = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
        t_lib = best(lambda: torch.matmul(a, w.t(), out=c))
        lib = {"shape_mnk": [M, N, K], "tflops": 2.0 * M * N * K / (t_lib * 1e-3) / 1e12,
               "ms": t_lib, "how": "torch.matmul(a [M][K], w[N][K].t()) in bf16 (the vendor "
                                   "GEMM library), best of 10"}
        del a, w, c
    return {"mfma_bf16_tflops": flops / (t_mfma * 1e-3) / 1e12,
            "library_gemm_bf16": lib,
            "copy_gbs": 2.0 * nbytes / (t_copy * 1e-3) / 1e9,
            "published_bf16_tflops": PEAK_BF16_TFLOPS, "published_hbm_gbs": PEAK_HBM_GBS,
            "how": "moe_peak_mfma: %d blocks x 8 waves x %d iterations of 8 independent "
                   "32x32x16 bf16 instructions on random register operands; moe_peak_copy: 1 GiB "
                   "copy, 16-byte loads and stores; best of 10 launches" % (blocks, iters)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mixtral_prefill")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-sample-tokens", type=int, default=0,
                    help="tokens of the workload the CPU oracle runs on (0: all)")
    ap.add_argument("--cpu-repeats", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the measured MFMA-loop and copy ceilings")
    ap.add_argument("--cold", action="store_true",
                    help="overwrite a 1 GiB buffer before every timed step (outside the step's "
                         "events), so the step starts with caches holding none of its data; "
                         "ms_per_step is then the mean of the steps' event times")
    ap.add_argument("--eager", action="store_true",
                    help="time the forward steps as launched one by one instead of replaying the "
                         "step captured in a HIP graph (the stage breakdown is eager either way)")
    ap.add_argument("--pass", dest="mode", choices=("forward", "train"), default="forward")
    ap.add_argument("--recompute", action="store_true",
                    help="--pass train: recompute the experts' up projection in the backward "
                         "pass instead of saving its activations in the forward pass")
    ap.add_argument("--weights", choices=("bf16", "int8", "int4"), default="bf16",
                    help="int8 / int4: weight-only quantized routed experts (moe_expert_ffn_q)")
    ap.add_argument("--routing", choices=("topk", "expert_choice", "reroute"), default="topk",
                    help="expert_choice: each expert takes C = T*k/E tokens (same expert work); "
                         "reroute: capacity C = T*k/E with overflow sent to the next-best expert")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py: this build measures one GPU only; --gpus %d is not supported "
              "(run with --gpus 1)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    from sparse_mixture_experts_counting_amd import build as B
    if not os.path.exists(B.LIB):
        B.build()
    from sparse_mixture_experts_counting_amd import layer, libmoe as lm, synth

    cfg = synth.CONFIGS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.mode == "train":
        return train_bench(args, cfg, dev, torch, layer, lm, synth)
    if args.weights != "bf16":
        return quant_bench(args, cfg, dev, torch, layer, lm, synth)
    if args.routing == "expert_choice":
        return expert_choice_bench(args, cfg, dev, torch, layer, lm, synth)
    if args.routing == "reroute":
        return reroute_bench(args, cfg, dev, torch, layer, lm, synth)
    log("bench: workload %s, generating inputs on the device" % cfg.name)
    inp = synth.make_inputs(cfg, seed=args.seed, device=dev)
    buf = layer.alloc_buffers(cfg, dev)
    code = lm.MOE_F32 if cfg.dtype == "fp32" else lm.MOE_BF16
    stream = torch.cuda.current_stream(dev)
    # h between the two expert GEMMs (the workspace holds their split-K scratch, if any)
    h = torch.empty((cfg.T * cfg.k, cfg.d_ff), dtype=synth.torch_dtype(cfg), device=dev)
    ws = buf.workspace

    stages = ["route", "dispatch", "expert_up", "expert_down", "shared_up", "shared_down",
              "combine", "aux_loss"]
    if not cfg.n_shared:
        stages = [s for s in stages if not s.startswith("shared")]

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record(stream)
        mark(0)
        layer.route(cfg, inp, buf)
        mark(1)
        layer.dispatch(cfg, buf)
        mark(2)
        lm.expert_up(inp.x, buf.perm, buf.offsets, cfg.T, cfg.d, cfg.d_ff, cfg.E, cfg.k, inp.w1,
                     inp.w3, code, h, ws)
        mark(3)
        lm.expert_down(h, buf.offsets, cfg.T, cfg.d, cfg.d_ff, cfg.E, cfg.k, inp.w2, code,
                       buf.expert_out, ws)
        mark(4)
        i = 4
        if cfg.n_shared:
            w1s, w3s, w2s = inp.shared
            lm.expert_up(inp.x, None, None, cfg.T, cfg.d, cfg.d_ff, 1, 1, w1s, w3s, code, h, ws)
            mark(5)
            lm.expert_down(h, None, cfg.T, cfg.d, cfg.d_ff, 1, 1, w2s, code, buf.shared_out, ws)
            mark(6)
            i = 6
        layer.combine(cfg, buf)
        mark(i + 1)
        layer.losses(cfg, buf)
        mark(i + 2)

    # A plain copy of known size, untimed: the byte-counter calibration for PMC runs.
    calib_src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
    calib_dst = torch.empty_like(calib_src)
    calib_dst.copy_(calib_src)
    del calib_src, calib_dst

    scrub = torch.empty(1 << 30, dtype=torch.uint8, device=dev) if args.cold else None
    for w in range(args.warmup):
        if scrub is not None:
            scrub.fill_(w & 0xff)
        step()
    torch.cuda.synchronize(dev)
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
              for _ in range(args.steps)]
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    for s in range(args.steps):
        if scrub is not None:
            scrub.fill_((s + 7) & 0xff)
        step(events[s])
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0
    del scrub

    stage_ms = {}
    for j, name in enumerate(stages):
        stage_ms[name] = sum(events[s][j].elapsed_time(events[s][j + 1])
                             for s in range(args.steps)) / args.steps
    gpu_ms = sum(events[s][0].elapsed_time(events[s][-1]) for s in range(args.steps)) / args.steps
    ms_per_step = gpu_ms if args.cold else wall * 1e3 / args.steps
    eager = {"ms_per_step": ms_per_step, "gpu_event_ms": gpu_ms}
    launch = "eager: every kernel launched per step"
    if not args.eager:
        # The step captured once into a HIP graph (warm-up on the capture stream itself) and
        # replayed: the serving form of a fixed-shape layer.  The same kernels run; only the
        # per-kernel launch gaps go.  The stage breakdown above stays the eager one.
        cap = torch.cuda.Stream(dev)
        cap.wait_stream(stream)
        with torch.cuda.stream(cap):
            step()
        torch.cuda.synchronize(dev)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=cap):
            step()
        torch.cuda.synchronize(dev)
        scrub = torch.empty(1 << 30, dtype=torch.uint8, device=dev) if args.cold else None
        for w in range(args.warmup):
            if scrub is not None:
                scrub.fill_(w & 0xff)
            graph.replay()
        torch.cuda.synchronize(dev)
        gev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        torch.cuda.synchronize(dev)
        t0 = time.perf_counter()
        for s in range(args.steps):
            if scrub is not None:
                scrub.fill_((s + 7) & 0xff)
            gev[s][0].record(stream)
            graph.replay()
            gev[s][1].record(stream)
        torch.cuda.synchronize(dev)
        wall = time.perf_counter() - t0
        del scrub, graph
        gpu_ms = sum(a.elapsed_time(b) for a, b in gev) / args.steps
        ms_per_step = gpu_ms if args.cold else wall * 1e3 / args.steps
        launch = "hip graph: the step captured once and replayed"

    counts = buf.counts.cpu().tolist()
    n_kept = int(buf.offsets[-1].item())
    n_dropped = int(buf.n_dropped.item())
    touched = sum(1 for c in counts if c > 0)
    T, d, E, k, f = cfg.T, cfg.d, cfg.E, cfg.k, cfg.d_ff
    sb = 4 if cfg.dtype == "fp32" else 2
    up_flops = 4.0 * d * f * n_kept
    down_flops = 2.0 * d * f * n_kept
    layer_flops = 2.0 * T * d * E + 6.0 * d * f * (n_kept + T * cfg.n_shared)
    layer_bytes = sb * (3.0 * d * f * (touched + cfg.n_shared) + 2.0 * T * d + d * E)
    up_ms = stage_ms["expert_up"]
    # The up projection's bound: matrix cores when its FLOPs per byte of touched expert weights
    # (w1 and w3) exceed the chip's ridge point (2.5 PFLOP/s / 8 TB/s), else the weight stream.
    up_weight_bytes = 2.0 * sb * d * f * touched
    if up_flops / max(up_weight_bytes, 1.0) >= PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9):
        roof = {"bound": "mfma", "achieved": up_flops / (up_ms * 1e-3) / 1e12,
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s"}
    else:   # algorithmic bytes: touched w1 and w3, the token rows read, h written
        up_bytes = up_weight_bytes + sb * (T * d + n_kept * f)
        roof = {"bound": "hbm", "achieved": up_bytes / (up_ms * 1e-3) / 1e9,
                "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    # The up projection's launch: the block-sparse tall/thin tiling when the groups fill 256-row
    # tiles (gemm_bs_persistent_kernel: one block per CU taking tiles from per-XCD counters, which
    # zero_tickets_kernel clears in the workspace first), else the grouped tiles (gemm_bf16_kernel,
    # with a finish kernel for split partial sums); the fp32 layers run gemm_f32_kernel.
    if cfg.dtype == "fp32":
        up_kernel = "moe_expert_up: gemm_f32_kernel (SwiGLU epilogue)"
    elif T * k >= 256 * E:
        up_kernel = ("moe_expert_up: gemm_bs_persistent_kernel (block-sparse tall/thin tiles, one "
                     "block per CU, SwiGLU epilogue) + zero_tickets_kernel")
    else:
        up_kernel = ("moe_expert_up: gemm_bf16_kernel (SwiGLU epilogue) + its split-K finish "
                     "kernel")
    traffic = load_traffic(cfg.name)
    gg_ms = stage_ms["expert_up"] + stage_ms["expert_down"]
    result = {
        "metric": "MoE layer tokens/s at 1 GPU; expert grouped-GEMM % bf16 MFMA peak",
        "value": T / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic (seeded randn inputs and random-init expert weights of the workload's "
                "shapes, drawn on the device)",
        "config": {"workload": cfg.name, "T": T, "d": d, "E": E, "k": k, "d_ff": f,
                   "gating": cfg.gating, "capacity": cfg.capacity or None,
                   "shared_experts": cfg.n_shared, "parallelism": "none (1 GPU)",
                   "cache": ("cold: a 1 GiB buffer overwritten before every step, outside its "
                             "events" if args.cold else "warm: steps back to back"),
                   "launch": launch},
        "roofline": dict(roof, kernel=up_kernel, traffic=traffic),
        "grouped_gemm": {"ms": gg_ms, "tflops": (up_flops + down_flops) / (gg_ms * 1e-3) / 1e12,
                         "frac_bf16_peak": (up_flops + down_flops) / (gg_ms * 1e-3) / 1e12
                         / PEAK_BF16_TFLOPS},
        "eager": eager,
        "layer": {"gpu_event_ms": gpu_ms, "tflops": layer_flops / (ms_per_step * 1e-3) / 1e12,
                  "hbm_gbs_algorithmic": layer_bytes / (ms_per_step * 1e-3) / 1e9,
                  "algorithmic_flops": layer_flops, "algorithmic_bytes": layer_bytes,
                  "kept_assignments": n_kept, "dropped": n_dropped, "experts_touched": touched},
        "stage_ms": stage_ms,
    }
    del h
    if not args.no_peaks:
        log("bench: measuring the MFMA-loop and copy ceilings")
        # The library reference: the up projection's kept rows as one dense GEMM against both
        # stacked weight matrices of one expert (the same FLOPs, none of the grouping or gather).
        shape = (n_kept, 2 * f, d) if roof["bound"] == "mfma" and sb == 2 else None
        result["measured_peaks"] = measured_peaks(torch, lm, dev, shape)
    if not args.no_cpu_baseline:
        log("bench: timing the CPU oracle on a sample")
        result["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_sample_tokens, args.cpu_repeats)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


def expert_choice_bench(args, cfg, dev, torch, layer, lm, synth):
    """The layer under Expert Choice routing with C = T*k/E tokens per expert (the same number of
    expert rows as the top-k workload)."""
    C = cfg.T * cfg.k // cfg.E
    cfg = cfg.replace(capacity=C, name=cfg.name + "_expert_choice")
    log("bench: workload %s (expert choice, C = %d), generating inputs on the device" % (cfg.name, C))
    inp = synth.make_inputs(cfg, seed=args.seed, device=dev)
    b = layer.alloc_ec_buffers(cfg, dev)
    stream = torch.cuda.current_stream(dev)
    T, d, E, f = cfg.T, cfg.d, cfg.E, cfg.d_ff
    code = lm.MOE_F32 if cfg.dtype == "fp32" else lm.MOE_BF16
    R = layer.ec_rows(cfg)
    stages = ["route", "select", "experts", "shared", "combine"]
    if not cfg.n_shared:
        stages.remove("shared")

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record(stream)
        mark(0)
        lm.route(inp.x, inp.w_r, inp.bias, T, d, E, 1, code, 0, 0, b.logits, b.topk_idx,
                 b.topk_gate, None, None, None)
        mark(1)
        lm.expert_choice(b.logits, T, E, C, 0, b.scores, b.offsets, b.perm, b.gate, b.slot)
        mark(2)
        lm.expert_ffn_gathered(inp.x, b.perm, b.offsets, T, d, f, E, R, inp.w1, inp.w3, inp.w2,
                               code, b.expert_out, b.workspace)
        mark(3)
        i = 3
        if cfg.n_shared:
            w1s, w3s, w2s = inp.shared
            lm.expert_ffn(inp.x, None, None, T, d, f, 1, 1, w1s, w3s, w2s, code, b.shared_out,
                          b.workspace)
            i += 1
            mark(i)
        lm.combine(b.expert_out, b.slot, b.scores, T, d, E, code, b.shared_out, b.y)
        mark(i + 1)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize(dev)
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
              for _ in range(args.steps)]
    t0 = time.perf_counter()
    for s_ in range(args.steps):
        step(events[s_])
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0
    stage_ms = {name: sum(events[s_][j].elapsed_time(events[s_][j + 1])
                          for s_ in range(args.steps)) / args.steps
                for j, name in enumerate(stages)}
    ms_per_step = wall * 1e3 / args.steps
    exp_flops = 6.0 * d * f * R
    achieved = exp_flops / (stage_ms["experts"] * 1e-3) / 1e12
    kept_by = torch.bincount(b.perm.long(), minlength=T)
    result = {
        "metric": "MoE layer tokens/s at 1 GPU, Expert Choice routing",
        "value": T / (ms_per_step * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic (seeded randn inputs and random-init expert weights of the workload's "
                "shapes, drawn on the device)",
        "config": {"workload": cfg.name, "routing": "expert_choice", "T": T, "d": d, "E": E,
                   "C": C, "d_ff": f, "shared_experts": cfg.n_shared,
                   "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma",
                     "kernel": "moe_expert_ffn_gathered: up (SwiGLU) + down grouped GEMMs",
                     "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": None},
        "routing": {"expert_rows": R, "tokens_kept_by_no_expert": int((kept_by == 0).sum()),
                    "max_experts_per_token": int(kept_by.max())},
        "stage_ms": stage_ms,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        from oracle import moe_oracle as O
        n = args.cpu_sample_tokens if args.cpu_sample_tokens > 0 else 512
        fl = lambda t: t.detach().float().cpu().numpy()
        x, w_r = fl(inp.x[:n]), fl(inp.w_r)
        w1, w3, w2 = fl(inp.w1), fl(inp.w3), fl(inp.w2)
        c_s = max(1, n * cfg.k // E)
        t1 = time.perf_counter()
        for _ in range(args.cpu_repeats):
            O.forward_expert_choice(x, w_r, w1, w3, w2, c_s)
        secs = time.perf_counter() - t1
        hi = host_info()
        result["cpu_baseline"] = dict({
            "value": n * args.cpu_repeats / secs, "unit": "tokens/s", "cores": hi["blas_threads"],
            "kind": "oracle", "precision": "float64", "seconds": secs,
            "sample": "first %d of %d tokens, expert choice with C = %d, float64 NumPy oracle, "
                      "%d runs" % (n, T, c_s, args.cpu_repeats)}, **hi)
    print(json.dumps(result), flush=True)


def quant_bench(args, cfg, dev, torch, layer, lm, synth):
    """The layer with weight-only INT8 / INT4 routed experts (quantized once, untimed)."""
    bits = 8 if args.weights == "int8" else 4
    log("bench: workload %s with %s experts" % (cfg.name, args.weights))
    inp = synth.make_inputs(cfg, seed=args.seed, device=dev)
    qw = layer.quantize_experts(cfg, inp, bits, dev)
    b = layer.alloc_buffers(cfg, dev)
    stream = torch.cuda.current_stream(dev)
    T, d, E, k, f = cfg.T, cfg.d, cfg.E, cfg.k, cfg.d_ff
    stages = ["route", "dispatch", "experts", "shared", "combine", "aux_loss"]
    if not cfg.n_shared:
        stages.remove("shared")

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record(stream)
        mark(0)
        layer.route(cfg, inp, b)
        mark(1)
        layer.dispatch(cfg, b)
        mark(2)
        lm.expert_ffn_q(inp.x, b.perm, b.offsets, T, d, f, E, k, bits, qw.q1, qw.s1, qw.q3, qw.s3,
                        qw.q2, qw.s2, lm.MOE_BF16, b.expert_out, qw.workspace)
        mark(3)
        i = 3
        if cfg.n_shared:
            w1s, w3s, w2s = inp.shared
            lm.expert_ffn(inp.x, None, None, T, d, f, 1, 1, w1s, w3s, w2s, lm.MOE_BF16,
                          b.shared_out, b.workspace)
            i += 1
            mark(i)
        layer.combine(cfg, b)
        mark(i + 1)
        layer.losses(cfg, b)
        mark(i + 2)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize(dev)
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
              for _ in range(args.steps)]
    t0 = time.perf_counter()
    for s_ in range(args.steps):
        step(events[s_])
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0
    stage_ms = {name: sum(events[s_][j].elapsed_time(events[s_][j + 1])
                          for s_ in range(args.steps)) / args.steps
                for j, name in enumerate(stages)}
    ms_per_step = wall * 1e3 / args.steps
    touched = int((b.counts > 0).sum().item())
    # Algorithmic bytes of the quantized expert GEMMs: the touched experts' three weight matrices
    # (bits / 8 bytes per weight) and their fp32 scales.
    wbytes = touched * (3.0 * d * f * bits / 8 + 4.0 * (2 * f + d))
    achieved = wbytes / (stage_ms["experts"] * 1e-3) / 1e9
    result = {
        "metric": "MoE layer tokens/s at 1 GPU with %s weight-only experts" % args.weights.upper(),
        "value": T / (ms_per_step * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 activations, %s weights" % args.weights,
        "data": "synthetic (seeded randn inputs and random-init expert weights of the workload's "
                "shapes, drawn on the device, quantized per output channel)",
        "config": {"workload": cfg.name, "weights": args.weights, "T": T, "d": d, "E": E, "k": k,
                   "d_ff": f, "gating": cfg.gating, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "kernel": "moe_expert_ffn_q: up (SwiGLU) + down GEMMs",
                     "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": None},
        "stage_ms": stage_ms,
        "cpu_baseline": None,
    }
    print(json.dumps(result), flush=True)


def reroute_bench(args, cfg, dev, torch, layer, lm, synth):
    """Top-k routing with capacity C = T*k/E (capacity factor 1) and overflow sent to the
    next-best expert (moe_reroute after moe_dispatch)."""
    C = cfg.T * cfg.k // cfg.E
    cfg = cfg.replace(capacity=C, name=cfg.name + "_reroute")
    log("bench: workload %s (capacity %d, overflow rerouted)" % (cfg.name, C))
    inp = synth.make_inputs(cfg, seed=args.seed, device=dev)
    b = layer.alloc_buffers(cfg, dev)
    r = layer.alloc_reroute_buffers(cfg, dev)
    stream = torch.cuda.current_stream(dev)
    code = lm.MOE_F32 if cfg.dtype == "fp32" else lm.MOE_BF16
    from sparse_mixture_experts_counting_amd.synth import GATING_CODE
    T, d, E, k, f = cfg.T, cfg.d, cfg.E, cfg.k, cfg.d_ff
    stages = ["route", "dispatch", "reroute", "experts", "shared", "combine", "aux_loss"]
    if not cfg.n_shared:
        stages.remove("shared")

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record(stream)
        mark(0)
        layer.route(cfg, inp, b)
        mark(1)
        layer.dispatch(cfg, b)
        mark(2)
        lm.reroute(b.logits, None, b.topk_idx, b.topk_gate, b.offsets, b.inv, T, E, k, C,
                   GATING_CODE[cfg.gating], r.topk_idx, r.topk_gate, r.offsets, r.perm, r.inv,
                   r.n_dropped, b.workspace)
        mark(3)
        lm.expert_ffn(inp.x, r.perm, r.offsets, T, d, f, E, k, inp.w1, inp.w3, inp.w2, code,
                      b.expert_out, b.workspace)
        mark(4)
        i = 4
        if cfg.n_shared:
            w1s, w3s, w2s = inp.shared
            lm.expert_ffn(inp.x, None, None, T, d, f, 1, 1, w1s, w3s, w2s, code, b.shared_out,
                          b.workspace)
            i += 1
            mark(i)
        lm.combine(b.expert_out, r.inv, r.topk_gate, T, d, k, code, b.shared_out, b.y)
        mark(i + 1)
        layer.losses(cfg, b)
        mark(i + 2)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize(dev)
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
              for _ in range(args.steps)]
    t0 = time.perf_counter()
    for s_ in range(args.steps):
        step(events[s_])
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0
    stage_ms = {name: sum(events[s_][j].elapsed_time(events[s_][j + 1])
                          for s_ in range(args.steps)) / args.steps
                for j, name in enumerate(stages)}
    ms_per_step = wall * 1e3 / args.steps
    kept = int(r.offsets[-1].item())
    exp_flops = 6.0 * d * f * kept
    achieved = exp_flops / (stage_ms["experts"] * 1e-3) / 1e12
    result = {
        "metric": "MoE layer tokens/s at 1 GPU, capacity factor 1 with overflow rerouted",
        "value": T / (ms_per_step * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic (seeded randn inputs and random-init expert weights of the workload's "
                "shapes, drawn on the device)",
        "config": {"workload": cfg.name, "routing": "topk+reroute", "T": T, "d": d, "E": E,
                   "k": k, "capacity": C, "d_ff": f, "gating": cfg.gating,
                   "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "kernel": "moe_expert_ffn: up (SwiGLU) + down grouped GEMMs",
                     "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": None},
        "routing": {"dropped_without_reroute": int(b.n_dropped.item()),
                    "dropped_with_reroute": int(r.n_dropped.item()), "kept": kept},
        "stage_ms": stage_ms,
        "cpu_baseline": None,
    }
    print(json.dumps(result), flush=True)


def cpu_baseline_train(cfg, inp, dy, n_tokens, repeats):
    """The CPU oracle's forward + backward (float64 NumPy, as it stands) on the first n_tokens
    tokens, `repeats` times.  Returns tokens/s, BLAS threads, the sample and the seconds spent."""
    from oracle import moe_oracle as O

    n = min(n_tokens, cfg.T)
    f = lambda t: t.detach().float().cpu().numpy()
    x, w_r, dyh = f(inp.x[:n]), f(inp.w_r), f(dy[:n]).astype("float64")
    bias = None if inp.bias is None else f(inp.bias)
    mode = {"softmax_topk": 0, "softmax_all": 1, "sigmoid_topk": 2}[cfg.gating]
    w1, w3, w2 = f(inp.w1), f(inp.w3), f(inp.w2)
    shared = tuple(f(w) for w in inp.shared) if inp.shared is not None else None
    t0 = time.perf_counter()
    for _ in range(repeats):
        O.backward(x, w_r, w1, w3, w2, dyh, cfg.k, mode, capacity=cfg.capacity or None,
                   bias=bias, shared=shared, alpha=cfg.alpha, beta=cfg.beta)
    secs = time.perf_counter() - t0
    sample = ("first %d of %d tokens of %s, forward + backward, float64 NumPy oracle, %d runs"
              % (n, cfg.T, cfg.name, repeats))
    hi = host_info()
    return dict({"value": n * repeats / secs, "unit": "tokens/s", "cores": hi["blas_threads"],
                 "kind": "oracle", "precision": "float64", "sample": sample, "seconds": secs},
                **hi)


def train_bench(args, cfg, dev, torch, layer, lm, synth):
    if cfg.dtype != "bf16":
        print("bench.py: the backward pass runs bf16 layers only", file=sys.stderr)
        sys.exit(2)
    log("bench: workload %s (forward + backward), generating inputs on the device" % cfg.name)
    inp = synth.make_inputs(cfg, seed=args.seed, device=dev)
    dy = synth.make_dy(cfg, seed=args.seed, device=dev)
    save = not args.recompute
    buf = layer.alloc_buffers(cfg, dev, save=save)
    g = layer.alloc_grads(cfg, dev)
    stream = torch.cuda.current_stream(dev)
    T, d, E, k, f = cfg.T, cfg.d, cfg.E, cfg.k, cfg.d_ff
    bf = lm.MOE_BF16
    from sparse_mixture_experts_counting_amd.synth import GATING_CODE
    stages = ["forward", "combine_bwd", "expert_bwd", "shared_bwd", "route_bwd", "dx_combine"]
    if not cfg.n_shared:
        stages.remove("shared_bwd")

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record(stream)
        mark(0)
        layer.forward(cfg, inp, buf)
        mark(1)
        lm.combine_backward(dy, buf.expert_out, buf.inv, buf.topk_gate, T, d, k, bf, g.d_out,
                            g.d_gate)
        mark(2)
        if save:
            lm.expert_backward_saved(buf.saved, inp.x, buf.perm, buf.offsets, T, d, f, E, k,
                                     inp.w1, inp.w3, inp.w2, g.d_out, bf, g.dx_rows, g.dw1,
                                     g.dw3, g.dw2, g.workspace)
        else:
            lm.expert_backward(inp.x, buf.perm, buf.offsets, T, d, f, E, k, inp.w1, inp.w3,
                               inp.w2, g.d_out, bf, g.dx_rows, g.dw1, g.dw3, g.dw2, g.workspace)
        mark(3)
        i = 3
        if cfg.n_shared:
            w1s, w3s, w2s = inp.shared
            if save:
                lm.expert_backward_saved(buf.saved_shared, inp.x, None, None, T, d, f, 1, 1, w1s,
                                         w3s, w2s, dy, bf, g.dx_shared, *g.dshared, g.workspace)
            else:
                lm.expert_backward(inp.x, None, None, T, d, f, 1, 1, w1s, w3s, w2s, dy, bf,
                                   g.dx_shared, *g.dshared, g.workspace)
            i += 1
            mark(i)
        lm.route_backward(inp.x, inp.w_r, buf.logits, buf.topk_idx, buf.topk_gate, g.d_gate,
                          buf.counts, T, d, E, k, bf, GATING_CODE[cfg.gating], cfg.alpha,
                          cfg.beta, g.dx_shared, g.d_logits, g.dw_r, g.dx_route, g.workspace)
        mark(i + 1)
        lm.combine(g.dx_rows, buf.inv, None, T, d, k, bf, g.dx_route, g.dx)
        mark(i + 2)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize(dev)
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
              for _ in range(args.steps)]
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(events[s])
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0
    stage_ms = {name: sum(events[s][j].elapsed_time(events[s][j + 1])
                          for s in range(args.steps)) / args.steps
                for j, name in enumerate(stages)}
    ms_per_step = wall * 1e3 / args.steps
    n_kept = int(buf.offsets[-1].item())
    # Algorithmic FLOPs of the expert backward: dh (2 d d_ff per row), dx (4), dw1 + dw3 (4),
    # dw2 (2); the recomputed up projection (4 more, --recompute) is not counted.
    bwd_flops = 12.0 * d * f * n_kept
    achieved = bwd_flops / (stage_ms["expert_bwd"] * 1e-3) / 1e12
    fwd_flops = 2.0 * T * d * E + 6.0 * d * f * (n_kept + T * cfg.n_shared)
    train_flops = fwd_flops + 2.0 * 2 * T * d * E + 12.0 * d * f * (n_kept + T * cfg.n_shared)
    result = {
        "metric": "MoE layer training step (forward + backward) tokens/s at 1 GPU",
        "value": T / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded randn inputs, upstream gradient and random-init expert "
                "weights of the workload's shapes, drawn on the device)",
        "config": {"workload": cfg.name, "pass": "forward+backward",
                   "activations": "recomputed" if args.recompute else "saved",
                   "T": T, "d": d, "E": E,
                   "k": k, "d_ff": f, "gating": cfg.gating, "capacity": cfg.capacity or None,
                   "shared_experts": cfg.n_shared, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma",
                     "kernel": ("moe_expert_backward (routed): 6 grouped GEMMs + row gather"
                                if args.recompute else
                                "moe_expert_backward_saved (routed): 5 grouped GEMMs + row "
                                "gather"),
                     "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": None},
        "layer": {"algorithmic_flops": train_flops,
                  "tflops": train_flops / (ms_per_step * 1e-3) / 1e12,
                  "kept_assignments": n_kept},
        "stage_ms": stage_ms,
    }
    if not args.no_cpu_baseline:
        log("bench: timing the CPU oracle (forward + backward) on a sample")
        n = args.cpu_sample_tokens if args.cpu_sample_tokens > 0 else 256
        result["cpu_baseline"] = cpu_baseline_train(cfg, inp, dy, n, args.cpu_repeats)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
