#!/usr/bin/env python3
"""Benchmark: the routed-MoE layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--procs 3]

A step is one pass of the whole hot path over one batch: route -> permute
(small batches group the pairs inside the FFN kernels) -> routed and shared
expert FFN (gate/up + SwiGLU, down) -> combine, all through the C ABI, with
inputs and weights resident in HBM before timing starts.

Default run: the Kimi-shaped decode step (T=8, d=2304, E=256, top-8,
I=2048, int8 per-row experts and shared expert) is the line's `value`; the
same line carries, each with its own roofline, the Kimi-shaped prefill
(T=1024, and as 4 chunks of 256), the Qwen3-shaped int4 layer (T=1, T=128),
and the 26-layer Kimi-shaped stack at T=4096 prefill and T=1 decode (~95 GB
of weights, Zipf-skewed routing).

Timing protocol (after the pages' own: warm-up first, several iterations,
several processes, the median): every workload runs in --procs separate
processes (default 3); in each, W warm-up steps, then exactly K steps, each
bracketed by HIP events on the launch stream between two synchronisations;
a process reports the median step, the line reports the median of the
process medians and p10/p90 over all timed steps.  Single layers are timed
with eager launches and, at decode sizes, also as HIP-graph replays (one
graph per weight copy); the line takes the faster and names it (timed_as):
one-token steps are bound by the host's launch rate when launched eagerly,
longer ones run ahead of the GPU.  The stack's decode step is replayed as
one HIP graph of all its layers.

Weight copies: a single-layer step alternates between identical copies of
the expert weights in separate HBM allocations, as many as make the bytes a
step touches, times (copies - 1), exceed 600 MB, so that no step finds its
experts in the 256 MB last-level cache from the steps before.  The stack is
cold by size.

Per-kernel durations for the rooflines come from a pass of their own after
the timed region, in which every launch records its kernel's start and stop
timestamps on a pair of HIP events (moe_timing, through hipExtLaunchKernel);
kernels_note gives their sum per step beside the timed step.

Attainable peaks: after the workloads, a fresh process runs the library's
probes (moe_probe_read, moe_probe_mfma): a non-temporal streaming read of
each HBM-bound roofline's bytes per launch, from regions the previous
launches did not touch, and int8 MFMA loops of both shapes.  Each roofline
then carries `attainable` (the probe's figure and achieved / attainable)
beside the published peak it is priced against.
cpu_baseline: the CPU oracle, as it stands, on a bounded sample of the
primary workload, all host threads and one thread; other_configs holds the
same for the other single-layer configurations on shorter samples.
"""
from __future__ import annotations

import argparse
import gc
import json
import math
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s + HBM GB/s (decode) / TFLOP/s (prefill), % roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 MFMA, published (5.0 POP/s)
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published (2.5 PFLOP/s)
LLC_BYTES = 256e6              # MI355X last-level (Infinity) cache
ROTATION_BYTES = 600e6         # touched bytes x (copies - 1) must exceed this

WORKLOADS = {
    # name: (layer spec, chunks, description[, spec overrides])
    "kimi_decode": ("kimi_decode", 1,
                    "Kimi-shaped MoE layer decode step: T=8, d=2304, E=256, top-8, "
                    "sigmoid+bias router x2.446, I=2048 SwiGLU, int8 per-row experts, "
                    "int8 shared expert I=2048"),
    "kimi_prefill": ("kimi_prefill", 1,
                     "Kimi-shaped MoE layer prefill: T=1024, same layer as kimi_decode"),
    "kimi_prefill_4x256": ("kimi_prefill", 4,
                           "Kimi-shaped MoE layer prefill, T=1024 as 4 chunks of 256"),
    "qwen_decode": ("qwen_decode", 1,
                    "Qwen3-shaped MoE layer decode: T=1, d=2048, E=128, top-8 softmax, "
                    "I=768 SwiGLU, int4 block-32 experts, no shared expert"),
    "qwen_prefill": ("qwen_prefill", 1, "Qwen3-shaped MoE layer, T=128"),
    "qwen_prefill_1024": ("qwen_prefill", 1,
                          "Qwen3-shaped MoE layer prefill, T=1024 (the pages' prefill length): "
                          "d=2048, E=128, top-8 softmax, I=768 SwiGLU, int4 block-32 experts, "
                          "no shared expert", {"T": 1024}),
    "qwen_prefill_1024_b128": ("qwen_prefill", 1,
                               "Qwen3-shaped MoE layer prefill, T=1024, int4 block-128 experts",
                               {"T": 1024, "fmt": "int4_b128"}),
    "qwen_decode_b128": ("qwen_decode", 1,
                         "Qwen3-shaped MoE layer decode as qwen_decode, int4 experts with one "
                         "scale per block of 128 inputs", {"fmt": "int4_b128"}),
    "qwen_prefill_b128": ("qwen_prefill", 1,
                          "Qwen3-shaped MoE layer, T=128, int4 block-128 experts",
                          {"fmt": "int4_b128"}),
    "tiny": ("tiny", 1, "tiny MoE layer: T=32, d=512, E=32, top-8, I=256"),
}

STACK_WORKLOADS = {
    # name: (T, description)
    "kimi_stack_decode": (1, "stack of 26 distinct Kimi-shaped MoE layers with the residual "
                             "between layers, T=1 decode, Zipf-skewed selection bias (64 "
                             "experts take ~73% of selections), int8 experts and shared "
                             "expert, ~95 GB of weights; the 26 layers replayed as one HIP "
                             "graph"),
    "kimi_stack_prefill": (4096, "stack of 26 distinct Kimi-shaped MoE layers with the residual "
                                 "between layers, T=4096 prefill, Zipf-skewed selection bias, "
                                 "int8 experts and shared expert, ~95 GB of weights"),
    "qwen_stack_decode": (1, "stack of 48 distinct Qwen3-shaped MoE layers with the residual "
                             "between layers, T=1 decode, d=2048, E=128, softmax top-8, I=768, "
                             "int4 block-32 experts, no shared expert, ~18 GB of weights; the "
                             "48 layers replayed as one HIP graph"),
}

QUANT_WORKLOADS = {
    # name: (layer spec whose routed expert set is quantized, format, description)
    "kimi_quantize": ("kimi_decode", "int8_row",
                      "weight quantizer: the Kimi-shaped routed expert set (E=256, d=2304, "
                      "I=2048; 3.62e9 weights) from bf16 to int8 per output row, "
                      "gate/up and down in one launch each"),
    "qwen_quantize": ("qwen_decode", "int4_b32",
                      "weight quantizer: the Qwen3-shaped routed expert set (E=128, d=2048, "
                      "I=768; 6.04e8 weights) from bf16 to int4 block-32"),
}

PRIMARY = "kimi_decode"
DEFAULT_EXTRAS = ["kimi_prefill", "kimi_prefill_4x256", "qwen_decode", "qwen_prefill",
                  "kimi_stack_prefill", "kimi_stack_decode"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def dtype_of(fmt: str) -> str:
    """The arithmetic type the FFN computes in: the integer matrix cores take the
    stored codes (int8, or int4 unpacked to int8 operands) against int8 digits."""
    return {"int8_row": "int8", "int4_b32": "int4", "int4_b128": "int4"}.get(fmt, "f32")


def expert_bytes(ew, e_list):
    """Codes + scales of the listed experts (host arrays), gate_up and down separately."""
    if ew.fmt in ("int4_b32", "int4_b128"):
        gu = ew.gu_packed[0].nbytes + ew.gu_s[0].nbytes
        dn = ew.dn_packed[0].nbytes + ew.dn_s[0].nbytes
    elif ew.fmt == "int8_row":
        gu = ew.gu[0].nbytes + ew.gu_s[0].nbytes
        dn = ew.dn[0].nbytes + ew.dn_s[0].nbytes
    else:
        gu, dn = ew.gu[0].nbytes, ew.dn[0].nbytes
    n = len(e_list)
    return gu * n, dn * n


def counter_traffic(workload: str, kernel_prefix: str, source: str = "ffn.hip"):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3
    counter summary (profiles/<workload>__*.md, FETCH_SIZE + WRITE_SIZE
    calibrated), or None when no summary matches or it was taken from a
    different version of the kernel source."""
    import glob
    import hashlib
    src = os.path.join(ROOT, "sparse_moe_expert_sigmoid_amd", "csrc", source)
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", f"{workload}__*.md"))):
        fields = {}
        for line in open(path):
            if ":" in line and not line.startswith(("|", "#", "`")):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
        if (fields.get("kernel_source_sha256") == sha
                and fields.get("dominant_kernel", "").startswith(kernel_prefix)
                and "traffic_bytes_per_launch" in fields):
            return int(fields["traffic_bytes_per_launch"])
    return None


# ---------------------------------------------------------------------------------------
# GPU side (child processes)

def timed_steps(step, steps: int, warmup: int, stream):
    """W untimed steps, then exactly `steps` steps between two synchronisations,
    each bracketed by HIP events on the launch stream.  Returns the per-step
    milliseconds and the total."""
    import torch
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for i in range(steps):
        step(warmup + i)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    return per, ev[0].elapsed_time(ev[-1])


def capture(fn, stream):
    """fn() recorded as a HIP graph (after one eager run on a side stream, so that
    every buffer exists before capture)."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        fn()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def kernel_pass(ctx, run, n: int) -> dict:
    """Per-kernel launch counts and durations over n eager runs, from the start
    and stop timestamps each launch records on a pair of HIP events."""
    import torch
    ctx.moe_timing(64 * n * 64)
    for i in range(n):
        run(i)
    torch.cuda.synchronize()
    kt = ctx.moe_timing_read()
    ctx.moe_timing(0)
    return {name: {"launches": int(c), "total_ms": t} for name, (c, t) in kt.items()}


def measure_layer(name: str, args) -> dict:
    import torch
    from sparse_moe_expert_sigmoid_amd import Context, MoELayer, synth as S

    spec_name, chunks, desc, *spec_kw = WORKLOADS[name]
    spec = S.spec(spec_name, **(spec_kw[0] if spec_kw else {}))
    decode = spec.T <= 16
    steps = args.steps or (200 if decode else 40)
    warmup = args.warmup if args.warmup is not None else (20 if decode else 5)
    log(f"[bench] {name}: generating inputs")
    inputs = S.make_layer(spec)
    dev = torch.device("cuda:0")
    ctx = Context(0)
    base = MoELayer.from_inputs(ctx, inputs, dev, act=args.act)
    x = torch.from_numpy(inputs.x).to(dev)
    Tc = spec.T // chunks
    xs = [x[i * Tc:(i + 1) * Tc].contiguous() for i in range(chunks)]
    stream = torch.cuda.current_stream()

    # routing of every chunk (the same on every weight copy): touched experts
    touched = []
    for c in range(chunks):
        base.forward_fused(xs[c], stream=stream)
        torch.cuda.synchronize()
        touched.append(np.unique(base.idx.cpu().numpy()))
    d, I, k, E = spec.d, spec.inter, spec.k, spec.E
    gu_b = dn_b = 0
    for t in touched:
        a, b = expert_bytes(inputs.experts, t)
        gu_b += a
        dn_b += b
    sh_gu = sh_dn = 0
    if inputs.shared is not None:
        sh_gu, sh_dn = expert_bytes(inputs.shared, [0])
        sh_gu *= chunks
        sh_dn *= chunks
    touched_bytes = gu_b + dn_b + sh_gu + sh_dn
    layer_bytes = base.experts.nbytes + (base.shared.nbytes if base.shared else 0)
    copies = args.copies or max(2, min(64, math.ceil(ROTATION_BYTES / touched_bytes) + 1,
                                       int(60e9 // layer_bytes)))
    layers = [base] + [base.with_weights(base.experts.clone(),
                                         base.shared.clone() if base.shared else None)
                       for _ in range(copies - 1)]
    for L in layers:
        L.alloc(Tc)
    log(f"[bench] {name}: {copies} weight copies of {layer_bytes / 1e9:.3f} GB "
        f"({touched_bytes / 1e6:.1f} MB touched per step); T={spec.T} ({chunks} chunk(s)); "
        f"warmup {warmup}, steps {steps}")

    def run_eager(i):
        L = layers[i % copies]
        for c in range(chunks):
            if args.path == "fused":
                L.forward_fused(xs[c], stream=stream)
            else:
                L.forward(xs[c], stream=stream)

    # Steps are timed with eager launches and, for decode (T <= 16), also as
    # HIP-graph replays (one graph per weight copy).  The line reports the faster
    # of the two and names it: a short step (one token) is bound by the host's
    # launch rate when launched eagerly, while for longer steps the eager
    # launches run ahead of the GPU and the graph's inter-node gaps cost more.
    per, total = timed_steps(run_eager, steps, warmup, stream)
    eager_ms, graph_ms, timed_as = float(np.median(per)), None, "eager launches"
    use_graph = decode and chunks == 1 and not args.no_graph
    if use_graph:
        graphs = [capture(lambda L=L: L.forward_fused(xs[0]) if args.path == "fused"
                          else L.forward(xs[0]), stream) for L in layers]
        gper, gtotal = timed_steps(lambda i: graphs[i % copies].replay(), steps, warmup, stream)
        graph_ms = float(np.median(gper))
        del graphs
        if graph_ms < eager_ms:
            per, total, timed_as = gper, gtotal, "HIP-graph replays"

    act_bytes = spec.T * d * 4 * 2                      # x read once, y written once
    router_bytes = (E * d + (E if inputs.bias is not None else 0)) * 4 * chunks
    step_bytes = touched_bytes + act_bytes + router_bytes
    Is = spec.shared_inter if inputs.shared is not None else 0
    step_flops = 2.0 * (spec.T * k * 3 * d * I + spec.T * 3 * d * Is + spec.T * d * E)

    kernels = {} if args.no_kernel_timing else kernel_pass(ctx, run_eager, steps)
    roofline = None
    dom = "ffn_i4_gate_up" if spec.fmt.startswith("int4") else "ffn_i8_gate_up"
    gemm = next((n for n in ("ffn_i8_gate_up_gemm", "ffn_i4_gate_up_gemm") if n in kernels),
                None)
    if gemm:
        dom = gemm
    if dom in kernels:
        launches = kernels[dom]["launches"] / steps
        R = spec.T * k
        # algorithmic bytes of the gate/up launches of one step: codes + scales of
        # every touched routed expert and the shared expert, x read once as 2-byte
        # digits, h written once as 2-byte digits + one fp32 scale per 64 columns
        per_step = (gu_b + sh_gu + spec.T * d * 2
                    + (R * I + spec.T * Is) * 2 + (R * I + spec.T * Is) // 64 * 4)
        roofline = {"bound": "hbm", "kernel": dom, "bytes_per_launch": int(per_step / launches),
                    "launches_per_step": launches,
                    "traffic": counter_traffic(name, "gate_up_kernel<" if not gemm else
                                               "gemm4_kernel" if "i4" in gemm
                                               else "gate_up_gemm_kernel")}
        if gemm:
            roofline["flops_per_launch"] = 2.0 * (R * 2 * I * d + spec.T * 2 * Is * d) / launches
    config = {"workload": desc, "T": spec.T, "chunks": chunks, "d": d, "E": E, "k": k,
              "inter": I, "router": spec.router, "expert_format": spec.fmt,
              "shared_expert": spec.shared, "weight_copies": copies,
              "touched_bytes_per_step": int(touched_bytes), "activation": args.act,
              "timed_as": timed_as,
              "entry_point": "moe_forward" if args.path == "fused" else
              "moe_route+moe_permute+moe_expert_ffn x2+moe_combine",
              "parallelism": "single GPU"}
    out = {"workload": name, "T": spec.T, "steps": steps, "warmup": warmup, "step_ms": per,
           "total_ms": total, "step_bytes": int(step_bytes), "step_flops": step_flops,
           "roofline": roofline, "kernels": kernels, "config": config,
           "dtype": dtype_of(spec.fmt), "graph_ms": graph_ms, "eager_ms": eager_ms,
           "data": "synthetic (seeded generator; random weights of the stated shapes)"}
    return out


def measure_stack(name: str, args) -> dict:
    import torch
    from sparse_moe_expert_sigmoid_amd import Context, MoEStack, synth as S

    T, desc = STACK_WORKLOADS[name]
    decode = T <= 16
    steps = args.steps or (50 if decode else 5)
    warmup = args.warmup if args.warmup is not None else (5 if decode else 1)
    st = S.qwen_stack_spec(T) if name.startswith("qwen") else S.stack_spec(T)
    if args.layers is not None:
        st = S.StackSpec(st.name, args.layers, st.T, st.alpha, st.base)
    dev = torch.device("cuda:0")
    ctx = Context(0)
    log(f"[bench] {name}: drawing {st.layers} layers on the GPU")
    stk = MoEStack.from_synth(ctx, st, dev, log=log)
    x0 = torch.from_numpy(S.stack_x(st)).to(dev)
    stream = torch.cuda.current_stream()
    stk.forward(x0, stream=stream)
    torch.cuda.synchronize()
    use_graph = decode and not args.no_graph
    if use_graph:
        g = capture(lambda: stk.forward(x0), stream)

        def step(i):
            g.replay()
    else:
        def step(i):
            stk.forward(x0, stream=stream)
    log(f"[bench] {name}: {stk.weight_bytes / 1e9:.1f} GB of weights; T={T}; "
        f"{'HIP graph' if use_graph else 'eager'}; warmup {warmup}, steps {steps}")
    per, total = timed_steps(step, steps, warmup, stream)

    s0 = st.layer(0)
    d, I, Is, E, k = s0.d, s0.inter, s0.shared_inter, s0.E, s0.k
    int4 = s0.fmt in S.INT4_BLOCK
    if int4:  # packed codes + one fp32 scale per block
        B = S.INT4_BLOCK[s0.fmt]
        e_gu, e_dn = I * d + 2 * I * (d // B) * 4, d * I // 2 + d * (I // B) * 4
    else:     # codes + fp32 row scales
        e_gu, e_dn = 2 * I * d + 2 * I * 4, d * I + d * 4
    sh_gu, sh_dn = (2 * Is * d + 2 * Is * 4, d * Is + d * 4) if Is else (0, 0)
    touched, masses = [], []
    for l in range(st.layers):
        counts = np.bincount(stk.idx[l].cpu().numpy().ravel(), minlength=E)
        touched.append(int((counts > 0).sum()))
        masses.append(round(float(np.sort(counts)[::-1][:64].sum()) / counts.sum(), 4))
    router_b = (E * d + (E if s0.router == "sigmoid_bias" else 0)) * 4
    step_bytes = sum(n * (e_gu + e_dn) + sh_gu + sh_dn + router_b + T * d * 4 * 2
                     for n in touched)
    step_flops = st.layers * 2.0 * (T * k * 3 * d * I + T * 3 * d * Is + T * d * E)

    kernels = {} if args.no_kernel_timing else kernel_pass(
        ctx, lambda i: stk.forward(x0, stream=stream), steps)
    roofline = None
    R = T * k
    gemm = next((n for n in ("ffn_i8_gate_up_gemm", "ffn_i4_gate_up_gemm") if n in kernels),
                None)
    if gemm:
        launches = kernels[gemm]["launches"] / steps
        roofline = {"bound": "mfma", "kernel": gemm,
                    "flops_per_launch": st.layers * 2.0 * (R * 2 * I * d + T * 2 * Is * d)
                    / launches, "launches_per_step": launches,
                    "traffic": counter_traffic(name, "gemm4_kernel" if "i4" in gemm
                                               else "gate_up_gemm_kernel")}
    else:
        kname = "ffn_i4_gate_up" if int4 else "ffn_i8_gate_up"
        if kname in kernels:
            launches = kernels[kname]["launches"] / steps
            per_step = sum(n * e_gu + sh_gu + T * d * 2 + (R * I + T * Is) * 2
                           + (R * I + T * Is) // 64 * 4 for n in touched)
            roofline = {"bound": "hbm", "kernel": kname,
                        "bytes_per_launch": int(per_step / launches),
                        "launches_per_step": launches,
                        "traffic": counter_traffic(name, "gate_up_kernel<")}
    config = {"workload": desc, "T": T, "layers": st.layers, "d": d, "E": E, "k": k,
              "inter": I, "router": s0.router, "expert_format": s0.fmt,
              "shared_expert": s0.shared, "zipf_alpha": st.alpha, "hip_graph": use_graph,
              "entry_point": "moe_forward per layer", "parallelism": "single GPU",
              "top64_mass_per_layer": masses, "touched_experts_per_layer": touched}
    out = {"workload": name, "T": T, "steps": steps, "warmup": warmup, "step_ms": per,
           "total_ms": total, "step_bytes": int(step_bytes), "step_flops": step_flops,
           "roofline": roofline, "kernels": kernels, "config": config,
           "dtype": "int4" if int4 else "int8",
           "data": "synthetic (seeded generator, weights drawn on the GPU; random weights of "
                   "the stated shapes)"}
    if use_graph:
        del g
    return out


def measure_quant(name: str, args) -> dict:
    import torch
    from sparse_moe_expert_sigmoid_amd import Context, binding as B, synth as S

    spec_name, fmt, desc = QUANT_WORKLOADS[name]
    spec = S.spec(spec_name)
    E, d, I = spec.E, spec.d, spec.inter
    steps = args.steps or 10
    warmup = args.warmup if args.warmup is not None else 2
    dev = torch.device("cuda:0")
    ctx = Context(0)
    log(f"[bench] {name}: uploading bf16 weights of {E} experts")
    gu = torch.empty((E * 2 * I, d), dtype=torch.bfloat16, device=dev)
    dn = torch.empty((E * d, I), dtype=torch.bfloat16, device=dev)
    for e in range(E):
        gu[e * 2 * I:(e + 1) * 2 * I] = torch.from_numpy(
            S.bf16_bits(S.float_expert(spec, e, "gu")).view(np.int16)).view(torch.bfloat16)
        dn[e * d:(e + 1) * d] = torch.from_numpy(
            S.bf16_bits(S.float_expert(spec, e, "dn")).view(np.int16)).view(torch.bfloat16)
    per_b = 1 if fmt == "int8_row" else 2
    f = B.MOE_W_INT8_ROW if fmt == "int8_row" else B.MOE_W_INT4_B32
    cdt = torch.int8 if per_b == 1 else torch.uint8
    cg = torch.empty((E * 2 * I, d // per_b), dtype=cdt, device=dev)
    cd = torch.empty((E * d, I // per_b), dtype=cdt, device=dev)
    sg = torch.empty((E * 2 * I) * (1 if per_b == 1 else d // 32), dtype=torch.float32,
                     device=dev)
    sd = torch.empty((E * d) * (1 if per_b == 1 else I // 32), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def step(i):
        ctx.moe_quantize(f, gu, cg, sg, stream)
        ctx.moe_quantize(f, dn, cd, sd, stream)

    per, total = timed_steps(step, steps, warmup, stream)
    n_w = gu.numel() + dn.numel()
    step_bytes = (n_w * 2 + cg.numel() + cd.numel() + (sg.numel() + sd.numel()) * 4)
    kernels = {} if args.no_kernel_timing else kernel_pass(ctx, step, steps)
    kname = "quant_i8_rows" if per_b == 1 else "quant_i4_blocks"
    roofline = None
    if kname in kernels:
        launches = kernels[kname]["launches"] / steps
        roofline = {"bound": "hbm", "kernel": kname,
                    "bytes_per_launch": int(step_bytes / launches), "launches_per_step": launches,
                    "traffic": counter_traffic(name, "quant_", "quant.hip")}
    config = {"workload": desc, "E": E, "d": d, "inter": I, "format": fmt, "input": "bf16",
              "entry_point": "moe_quantize x2", "parallelism": "single GPU",
              "weights_per_step": n_w}
    return {"workload": name, "T": None, "steps": steps, "warmup": warmup, "step_ms": per,
            "total_ms": total, "step_bytes": int(step_bytes), "step_flops": None,
            "roofline": roofline, "kernels": kernels, "config": config, "dtype": "f32",
            "data": "synthetic (seeded N(0, 0.02^2) weights rounded to bf16)"}


PROBE_BUFFER_BYTES = 4 << 30       # the read probe's source, far above the 256 MB MALL
PROBE_BLOCKS_PER_CU = (4, 8, 16)   # read-probe grids tried; the fastest counts
PROBE_REPS = 20


def measure_peaks(sizes) -> dict:
    """Attainable ceilings on this GPU: a plain streaming read of each size in
    `sizes` (bytes; each launch reads a region the previous launches did not
    touch, so no launch finds its bytes in the MALL), and int8 MFMA loops of
    both shapes.  Each figure is the median of PROBE_REPS event-timed launches;
    the read takes the fastest of a few grid sizes."""
    import torch
    from sparse_moe_expert_sigmoid_amd import Context
    from sparse_moe_expert_sigmoid_amd.binding import (MOE_PROBE_MFMA_16X16X64,
                                                       MOE_PROBE_MFMA_32X32X32)
    ctx = Context(0)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    stream = torch.cuda.current_stream()
    sink = torch.zeros(4, dtype=torch.int32, device="cuda:0")
    buf = torch.empty(PROBE_BUFFER_BYTES, dtype=torch.uint8, device="cuda:0")
    buf.fill_(1)

    def timed(launch, reps=PROBE_REPS):
        for i in range(3):
            launch(i)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * reps)]
        for i in range(reps):
            ev[2 * i].record(stream)
            launch(3 + i)
            ev[2 * i + 1].record(stream)
        torch.cuda.synchronize()
        return float(np.median([ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(reps)]))

    reads = []
    for size in sorted(set(int(x) for x in sizes)):
        nbytes = max(16, min(size, PROBE_BUFFER_BYTES) // 16 * 16)
        slots = max(1, PROBE_BUFFER_BYTES // nbytes)
        best = None
        for bpc in PROBE_BLOCKS_PER_CU:
            def launch(i, bpc=bpc):
                off = (i % slots) * nbytes
                ctx.moe_probe_read(buf[off:off + nbytes], nbytes, sink, blocks=bpc * cus,
                                   stream=stream)
            ms = timed(launch)
            if best is None or ms < best[0]:
                best = (ms, bpc)
        reads.append({"bytes": nbytes, "us": round(best[0] * 1e3, 2),
                      "gbps": round(nbytes / (best[0] / 1e3) / 1e9, 1),
                      "blocks_per_cu": best[1]})
    del buf
    mfma = {}
    for shape, label, ops in ((MOE_PROBE_MFMA_16X16X64, "i8_16x16x64", 16 * 16 * 64 * 2),
                              (MOE_PROBE_MFMA_32X32X32, "i8_32x32x32", 32 * 32 * 32 * 2)):
        iters, blocks = 512, 8 * cus
        ms = timed(lambda i: ctx.moe_probe_mfma(shape, iters, sink, blocks=blocks,
                                                stream=stream))
        total = blocks * 4 * iters * 32 * ops
        mfma[label] = {"tops": round(total / (ms / 1e3) / 1e12, 1), "us": round(ms * 1e3, 1),
                       "ops_per_launch": total}
    return {"workload": "peaks", "read": reads, "mfma": mfma,
            "probe": "moe_probe_read / moe_probe_mfma (streaming read, each wavefront "
                     "8 KB contiguous per step with 8 loads of 16 B in flight per lane; "
                     "MFMA loop of 4 independent accumulator chains per wavefront, "
                     "8 workgroups of 256 threads per CU); median of %d event-timed "
                     "launches" % PROBE_REPS}


def child(args):
    import torch
    if args.child == "peaks":
        sizes = [int(x) for x in (args.probe_sizes or "").split(",") if x]
        print("@@RESULT " + json.dumps(measure_peaks(sizes + [2 << 30])), flush=True)
        return
    for name in args.child.split(","):
        if name in STACK_WORKLOADS:
            r = measure_stack(name, args)
        elif name in QUANT_WORKLOADS:
            r = measure_quant(name, args)
        else:
            r = measure_layer(name, args)
        print("@@RESULT " + json.dumps(r), flush=True)
        gc.collect()
        torch.cuda.synchronize()
        torch.cuda.empty_cache()


# ---------------------------------------------------------------------------------------
# aggregation and the CPU oracle (parent process; it never touches the GPU)

def summarize(runs: list) -> dict:
    """One workload over its processes: the median of the process medians, p10 and
    p90 over every timed step, and the roofline of the dominant kernel from the
    median over processes of its mean event-timed launch."""
    r0 = runs[0]
    med = [float(np.median(r["step_ms"])) for r in runs]
    pooled = np.concatenate([np.asarray(r["step_ms"]) for r in runs])
    ms = float(np.median(med))
    s = ms / 1e3
    out = {"ms_per_step": round(ms, 5),
           "ms_p10": round(float(np.percentile(pooled, 10)), 5),
           "ms_p90": round(float(np.percentile(pooled, 90)), 5),
           "ms_per_process": [round(m, 5) for m in med],
           "mean_ms_per_step": round(float(np.median([r["total_ms"] / r["steps"]
                                                      for r in runs])), 5),
           "steps": r0["steps"], "warmup": r0["warmup"], "processes": len(runs)}
    if r0.get("graph_ms"):
        out["hip_graph_ms_per_step"] = round(float(np.median([r["graph_ms"] for r in runs])), 5)
        out["eager_ms_per_step"] = round(float(np.median([r["eager_ms"] for r in runs])), 5)
    if r0["T"]:
        out["tokens_per_s"] = round(r0["T"] / s, 1)
    else:
        out["weights_per_s"] = round(r0["config"]["weights_per_step"] / s, 1)
    out["hbm_gbps_algorithmic"] = round(r0["step_bytes"] / s / 1e9, 1)
    out["hbm_frac_algorithmic"] = round(r0["step_bytes"] / s / 1e9 / HBM_PEAK_GBS, 4)
    out["step_bytes_algorithmic"] = r0["step_bytes"]
    if r0["step_flops"]:
        out["tflops_algorithmic"] = round(r0["step_flops"] / s / 1e12, 3)
        out["step_flops_algorithmic"] = r0["step_flops"]
    kernels = {}
    for kname in r0["kernels"]:
        avg = [r["kernels"][kname]["total_ms"] / r["kernels"][kname]["launches"] * 1e3
               for r in runs if kname in r["kernels"]]
        kernels[kname] = {"launches": r0["kernels"][kname]["launches"],
                          "avg_us": round(float(np.median(avg)), 2)}
    out["kernels"] = kernels
    if kernels:
        ksum = sum(v["launches"] * v["avg_us"] for v in kernels.values()) / r0["steps"] / 1e3
        out["kernels_note"] = (
            "avg_us per kernel from the start and stop timestamps of each dispatch "
            "(hipExtLaunchKernel with an event pair, moe_timing), in a pass of its own after "
            f"the timed steps: they sum to {ksum:.4f} ms per step against the {ms:.4f} ms "
            "timed step; the gaps between kernels make up the rest")
    rl = r0["roofline"]
    if rl and rl["kernel"] in kernels:
        avg_s = kernels[rl["kernel"]]["avg_us"] / 1e6
        roof = {"bound": rl["bound"], "kernel": rl["kernel"]}
        if rl["bound"] == "mfma":
            achieved = rl["flops_per_launch"] / avg_s / 1e12
            roof.update({"achieved": round(achieved, 1), "peak": INT8_PEAK_TOPS,
                         "unit": "TFLOP/s", "frac": round(achieved / INT8_PEAK_TOPS, 4),
                         "frac_of_bf16_peak": round(achieved / BF16_PEAK_TFLOPS, 4),
                         "flops_per_launch": rl["flops_per_launch"]})
        else:
            achieved = rl["bytes_per_launch"] / avg_s / 1e9
            roof.update({"achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(achieved / HBM_PEAK_GBS, 4),
                         "bytes_per_launch": rl["bytes_per_launch"]})
            if "flops_per_launch" in rl:  # a grouped GEMM: its matrix-core rate as well
                t = rl["flops_per_launch"] / avg_s / 1e12
                roof["mfma_tflops"] = round(t, 1)
                roof["mfma_frac_int8"] = round(t / INT8_PEAK_TOPS, 4)
        roof["traffic"] = rl["traffic"]
        roof["avg_launch_us"] = round(avg_s * 1e6, 2)
        roof["launches_per_step"] = rl["launches_per_step"]
        roof["duration_source"] = ("each dispatch's start and stop timestamps (hipExtLaunchKernel "
                                   "with HIP events, moe_timing), a pass of its own after the "
                                   "timed steps; median over processes of the mean launch")
        out["roofline"] = roof
    else:
        out["roofline"] = None
    out["config"] = r0["config"]
    out["dtype"] = r0["dtype"]
    out["data"] = r0["data"]
    return out


def host_info() -> dict:
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "cpu_model": model,
            "omp_threads": int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))}


def _oracle_layer_rate(inputs, tokens, budget_s: float, act: str):
    import oracle
    s = inputs.spec
    ex = oracle.Experts.of(inputs.experts, act)
    sh = oracle.Experts.of(inputs.shared, act) if inputs.shared is not None else None
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.layer(s.router, s.k, s.scale, inputs.x, inputs.wr, inputs.bias, ex, sh,
                     tokens=tokens)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or el / reps * (reps + 1) > 3 * budget_s:
            return len(tokens) * reps / el, reps, el


def cpu_baseline(name: str, budget_s: float, act: str) -> dict:
    """The oracle, as it stands, on the same layer and tokens of the workload
    (bounded repeat count): OpenMP over the tokens with every host thread, then
    one token on one thread."""
    from sparse_moe_expert_sigmoid_amd import synth as S
    spec_name, chunks, desc, *spec_kw = WORKLOADS[name]
    inputs = S.make_layer(S.spec(spec_name, **(spec_kw[0] if spec_kw else {})))
    info = host_info()
    n_tok = min(inputs.spec.T, info["omp_threads"])
    rate, reps, el = _oracle_layer_rate(inputs, np.arange(n_tok), budget_s, act)
    import oracle
    oracle.set_threads(1)
    rate1, reps1, el1 = _oracle_layer_rate(inputs, np.arange(1), budget_s / 3, act)
    oracle.set_threads(info["omp_threads"])
    return {"value": rate, "unit": "tokens/s", "cores": min(n_tok, info["omp_threads"]),
            "kind": "oracle",
            "sample": f"{reps} x oracle layer on tokens 0..{n_tok - 1} of {name} (fp64 C, "
                      f"OpenMP over tokens, one thread per token), {el:.1f} s",
            "one_thread": {"value": rate1, "unit": "tokens/s", "cores": 1,
                           "sample": f"{reps1} x oracle layer on token 0, one thread, "
                                     f"{el1:.1f} s"},
            **info}


def cpu_baseline_stack(name: str, budget_s: float) -> dict:
    """The oracle on the first tokens of the stack's input, layer after layer
    until the budget is spent; tokens/s extrapolated to all layers.  Only the
    oracle calls are timed (the host draws each layer's selected experts
    between them)."""
    import oracle
    from sparse_moe_expert_sigmoid_amd import synth as S
    T, _ = STACK_WORKLOADS[name]
    st = S.qwen_stack_spec(T) if name.startswith("qwen") else S.stack_spec(T)
    info = host_info()
    n_tok = min(st.T, info["omp_threads"], 16)
    x = np.ascontiguousarray(S.stack_x(st)[:n_tok])
    spent, layers_done = 0.0, 0
    for l in range(st.layers):
        s = st.layer(l)
        wr, bias = S.stack_router(st, l)
        t0 = time.perf_counter()
        idx, w, _ = oracle.route(s.router, x, wr, bias, s.k, s.scale)
        spent += time.perf_counter() - t0
        uniq = np.unique(idx)
        remap = np.full(s.E, -1, np.int64)
        remap[uniq] = np.arange(len(uniq))
        ex = oracle.Experts.of(S.expert_slice(s, uniq))
        sh = (oracle.Experts.of(S.expert_slice(s, [0], shared=True))
              if s.shared is not None else None)
        t0 = time.perf_counter()
        offsets, row_token, token_row = oracle.permute(remap[idx].astype(np.int32), len(uniq))
        rows = oracle.expert_rows(ex, x, row_token, offsets)
        shr = (oracle.expert_rows(sh, x, None, np.array([0, n_tok], np.int32))
               if sh is not None else None)
        y = oracle.combine(rows, token_row, w, shared=shr, residual=x)
        spent += time.perf_counter() - t0
        x = y.astype(np.float32)
        layers_done += 1
        if spent >= budget_s:
            break
    per_layer = spent / layers_done
    return {"value": n_tok / (per_layer * st.layers), "unit": "tokens/s",
            "cores": n_tok, "kind": "oracle",
            "sample": f"tokens 0..{n_tok - 1} through layers 0..{layers_done - 1} of the "
                      f"{st.layers}-layer stack ({spent:.1f} s of oracle time), extrapolated "
                      f"to {st.layers} layers", **info}


def attach_peaks(summaries: dict) -> None:
    """Runs the peak probes in a fresh process and adds to each roofline the
    attainable ceiling beside the published one: for an HBM-bound kernel the
    probe's streaming read of that kernel's algorithmic bytes per launch, for a
    matrix-core-bound one the 16x16x64 int8 MFMA loop."""
    sizes = sorted({int(sm["roofline"]["bytes_per_launch"]) for sm in summaries.values()
                    if sm.get("roofline") and sm["roofline"].get("bytes_per_launch")})
    log("[bench] attainable-peak probes")
    r = subprocess.run([sys.executable, os.path.abspath(__file__), "--child", "peaks",
                        "--probe-sizes", ",".join(str(x) for x in sizes)],
                       stdout=subprocess.PIPE, text=True)
    peaks = None
    for line in r.stdout.splitlines():
        if line.startswith("@@RESULT "):
            peaks = json.loads(line[len("@@RESULT "):])
        elif line.strip():
            log(line)
    if r.returncode != 0 or peaks is None:
        log(f"[bench] peak probes failed with status {r.returncode}; stopping")
        sys.exit(r.returncode if r.returncode > 0 else 1)
    by_size = {x["bytes"]: x for x in peaks["read"]}
    probe_bytes = lambda n: max(16, min(int(n), PROBE_BUFFER_BYTES) // 16 * 16)
    for sm in summaries.values():
        roof = sm.get("roofline")
        if not roof:
            continue
        if roof["bound"] == "hbm":
            rd = by_size.get(probe_bytes(roof["bytes_per_launch"]))
            if rd:
                roof["attainable"] = {"value": rd["gbps"], "unit": "GB/s",
                                      "frac": round(roof["achieved"] / rd["gbps"], 4),
                                      "probe": f"streaming read of {rd['bytes']} B, "
                                               f"{rd['us']} us"}
        else:
            m = peaks["mfma"]["i8_16x16x64"]
            roof["attainable"] = {"value": m["tops"], "unit": "TFLOP/s",
                                  "frac": round(roof["achieved"] / m["tops"], 4),
                                  "probe": "int8 16x16x64 MFMA loop"}
    summaries["_peaks"] = peaks


def run_children(names, args) -> dict:
    """Runs the workloads in args.procs fresh processes, one after the other;
    returns {name: [result per process]}.  Stops at the first failure."""
    results = {n: [] for n in names}
    fwd = []
    for flag, val in (("--steps", args.steps), ("--warmup", args.warmup),
                      ("--copies", args.copies), ("--layers", args.layers)):
        if val is not None:
            fwd += [flag, str(val)]
    fwd += ["--path", args.path, "--act", args.act]
    for flag in ("no_graph", "no_kernel_timing"):
        if getattr(args, flag):
            fwd.append("--" + flag.replace("_", "-"))
    for p in range(args.procs):
        log(f"[bench] process {p + 1}/{args.procs}: {','.join(names)}")
        r = subprocess.run([sys.executable, os.path.abspath(__file__), "--child", ",".join(names),
                            *fwd], stdout=subprocess.PIPE, text=True)
        for line in r.stdout.splitlines():
            if line.startswith("@@RESULT "):
                res = json.loads(line[len("@@RESULT "):])
                results[res["workload"]].append(res)
            elif line.strip():
                log(line)
        if r.returncode != 0:
            log(f"[bench] process {p + 1} failed with status {r.returncode}; stopping")
            sys.exit(r.returncode if r.returncode > 0 else 1)
    return results


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default=None,
                    choices=sorted(WORKLOADS) + sorted(STACK_WORKLOADS) +
                    sorted(QUANT_WORKLOADS),
                    help="one workload alone (default: the Kimi-shaped decode step as the "
                         "value, with the prefill, Qwen-shaped and stack workloads beside it)")
    ap.add_argument("--extras", default=None,
                    help="comma-separated workloads to carry beside the default one "
                         "(default: " + ",".join(DEFAULT_EXTRAS) + "; 'none' for none)")
    ap.add_argument("--procs", type=int, default=3, help="processes per workload")
    ap.add_argument("--layers", type=int, default=None,
                    help="stack workloads: run only the first N layers")
    ap.add_argument("--no-graph", action="store_true",
                    help="decode: launch eagerly instead of replaying HIP graphs")
    ap.add_argument("--copies", type=int, default=None)
    ap.add_argument("--path", default="fused", choices=["fused", "staged"],
                    help="fused: one moe_forward call per step; staged: moe_route, "
                         "moe_permute, moe_expert_ffn (routed, shared), moe_combine")
    ap.add_argument("--act", default="silu", choices=["silu", "gelu_tanh"],
                    help="gate activation of the layer workloads")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-kernel-timing", action="store_true")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the attainable-peak probes (streaming read, MFMA loop)")
    ap.add_argument("--child", default=None, help=argparse.SUPPRESS)
    ap.add_argument("--probe-sizes", default=None, help=argparse.SUPPRESS)
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library runs the layer on a single MI355X and "
              "has no multi-GPU path (run with --gpus 1).", file=sys.stderr)
        sys.exit(2)
    if args.child:
        return child(args)

    primary = args.workload or PRIMARY
    if args.workload:
        extras = [] if args.extras is None else [e for e in args.extras.split(",")
                                                 if e and e != "none"]
    else:
        extras = DEFAULT_EXTRAS if args.extras is None else [
            e for e in args.extras.split(",") if e and e != "none"]
    names = [primary] + [e for e in extras if e != primary]
    results = run_children(names, args)
    summaries = {n: summarize(results[n]) for n in names}
    p = summaries[primary]
    if not args.no_peaks:
        attach_peaks(summaries)

    cpu = None
    if not args.no_cpu:
        log("[bench] timing the CPU oracle on a bounded sample")
        if primary in STACK_WORKLOADS:
            cpu = cpu_baseline_stack(primary, args.cpu_budget)
        elif primary in WORKLOADS:
            cpu = cpu_baseline(primary, args.cpu_budget, args.act)
            # the other single-layer configurations (tiny; the Kimi-shaped
            # layer at prefill size; the Qwen-shaped layer at T = 1 and 128),
            # each on a shorter sample, all host threads and one thread
            info_keys = set(host_info())
            cpu["other_configs"] = {
                n: {k: v for k, v in cpu_baseline(n, args.cpu_budget / 6, args.act).items()
                    if k not in info_keys}
                for n in ("tiny", "kimi_prefill", "qwen_decode", "qwen_prefill") if n != primary}

    quant = primary in QUANT_WORKLOADS
    out = {
        "metric": ("weights quantized per second (bf16 -> expert format), % HBM roofline"
                   if quant else METRIC),
        "value": p["weights_per_s"] if quant else p["tokens_per_s"],
        "unit": "weights/s" if quant else "tokens/s",
        "n_gpus": 1,
        "steps": p["steps"],
        "warmup": p["warmup"],
        "ms_per_step": p["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": p["dtype"],
        "data": p["data"],
        "config": p["config"],
        "timing": {"processes": p["processes"], "ms_per_process": p["ms_per_process"],
                   "ms_p10": p["ms_p10"], "ms_p90": p["ms_p90"],
                   "mean_ms_per_step": p["mean_ms_per_step"],
                   "hip_graph_ms_per_step": p.get("hip_graph_ms_per_step"),
                   "eager_ms_per_step": p.get("eager_ms_per_step"),
                   "protocol": "median over processes of each process's median step; "
                               "p10/p90 over every timed step; per-step HIP events on the "
                               "launch stream"},
        "hbm_gbps_algorithmic": p["hbm_gbps_algorithmic"],
        "hbm_frac_algorithmic": p["hbm_frac_algorithmic"],
        "tflops_algorithmic": p.get("tflops_algorithmic"),
        "step_bytes_algorithmic": p["step_bytes_algorithmic"],
        "step_flops_algorithmic": p.get("step_flops_algorithmic"),
        "roofline": p["roofline"],
        "cpu_baseline": cpu,
        "kernels": p["kernels"],
        "kernels_note": p.get("kernels_note"),
        "attainable_peaks": summaries.get("_peaks"),
        "workloads": {n: summaries[n] for n in names[1:]},
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
