#!/usr/bin/env python3
"""Benchmark: one routed-MoE layer step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload kimi_decode]

A step is the whole hot path over one batch: route -> permute -> routed expert
FFN -> shared expert FFN -> combine, all through the C ABI.  Inputs and
weights are resident in HBM before timing starts.  The default workload is
the Kimi-shaped decode step (T=8 tokens, d=2304, 256 experts, top 8, I=2048,
int8 per-row experts, int8 shared expert).

Weight copies: the step alternates between `--copies` identical copies of the
expert weights (and the shared expert) in separate HBM allocations, so no
step finds its weights in the 256 MB last-level cache from the step before.

Stack workloads (--workload kimi_stack_decode | kimi_stack_prefill): 26
distinct Kimi-shaped layers (about 95 GB of weights, drawn on the GPU, so cold
by size) with the residual between layers and a Zipf-skewed selection bias; a
step is one pass through all 26 layers, replayed as one HIP graph at T=1.

Quantizer workloads (--workload kimi_quantize | qwen_quantize): a step
quantizes a whole routed expert set from bf16 (moe_quantize, gate/up and
down); value = weights per second.

Output: one JSON line (metric, value = tokens/s, ms_per_step, roofline of the
dominant kernel measured with HIP events on its own stream in a second,
separately timed pass, and the CPU oracle timed on a bounded sample).
"""
from __future__ import annotations

import argparse
import json
import math
import os
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

WORKLOADS = {
    # name: (layer spec, chunks, description)
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


def log(*a):
    print(*a, file=sys.stderr, flush=True)


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
                and fields.get("dominant_kernel", "").startswith(kernel_prefix)):
            return int(fields["traffic_bytes_per_launch"])
    return None


def cpu_baseline(inputs, budget_s: float, act: str = "silu"):
    """The oracle, as it stands, on the same layer and tokens; bounded repeat count."""
    import oracle
    s = inputs.spec
    ex = oracle.Experts.of(inputs.experts, act)
    sh = oracle.Experts.of(inputs.shared, act) if inputs.shared is not None else None
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    T_sample = min(s.T, 8)
    tokens = np.arange(T_sample)
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.layer(s.router, s.k, s.scale, inputs.x, inputs.wr, inputs.bias, ex, sh,
                     tokens=tokens)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or el / reps * (reps + 1) > 3 * budget_s:
            break
    return {"value": T_sample * reps / el, "unit": "tokens/s", "cores": min(threads, T_sample),
            "kind": "oracle",
            "sample": f"{reps} x oracle layer on tokens 0..{T_sample - 1} of this workload "
                      f"(fp64 C, OpenMP over tokens), {el:.1f} s"}


def cpu_baseline_stack(st, budget_s: float):
    """The oracle on the first tokens of the stack's input, layer after layer
    until the budget is spent; tokens/s extrapolated to all layers.  Only the
    oracle calls are timed (the host draws each layer's selected experts
    between them)."""
    import oracle
    from sparse_moe_expert_sigmoid_amd import synth as S
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    n_tok = min(st.T, threads, 16)
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
            "cores": min(threads, n_tok), "kind": "oracle",
            "sample": f"tokens 0..{n_tok - 1} through layers 0..{layers_done - 1} of the "
                      f"{st.layers}-layer stack ({spent:.1f} s of oracle time), extrapolated "
                      f"to {st.layers} layers"}


def run_stack(args):
    import torch
    from sparse_moe_expert_sigmoid_amd import Context, MoEStack, synth as S

    T, desc = STACK_WORKLOADS[args.workload]
    decode = T <= 16
    steps = args.steps or (50 if decode else 5)
    warmup = args.warmup if args.warmup is not None else (5 if decode else 1)
    st = S.qwen_stack_spec(T) if args.workload.startswith("qwen") else S.stack_spec(T)
    if args.layers is not None:
        st = S.StackSpec(st.name, args.layers, st.T, st.alpha, st.base)
    dev = torch.device("cuda:0")
    ctx = Context(0)
    log(f"[bench] workload {args.workload}: drawing {st.layers} layers on the GPU")
    stk = MoEStack.from_synth(ctx, st, dev, log=log)
    x0 = torch.from_numpy(S.stack_x(st)).to(dev)
    stream = torch.cuda.current_stream()
    stk.forward(x0, stream=stream)
    torch.cuda.synchronize()
    use_graph = decode and not args.no_graph
    if use_graph:
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            stk.forward(x0)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            stk.forward(x0)
        step = g.replay
    else:
        def step():
            stk.forward(x0, stream=stream)
    log(f"[bench] {stk.weight_bytes / 1e9:.1f} GB of weights; T={T}; "
        f"{'HIP graph' if use_graph else 'eager'}; warmup {warmup}, steps {steps}")
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    ev0.record(stream)
    for _ in range(steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms_per_step = ev0.elapsed_time(ev1) / steps
    tok_s = T / (ms_per_step / 1e3)
    log(f"[bench] {ms_per_step:.3f} ms/step, {tok_s:,.1f} tokens/s (wall {wall:.3f} s)")

    # ---- algorithmic work, from each layer's actual routing
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
    gbs = step_bytes / (ms_per_step / 1e3) / 1e9
    tflops = step_flops / (ms_per_step / 1e3) / 1e12

    kernels, roofline = {}, None
    if not args.no_kernel_timing:
        ctx.moe_timing(64 * st.layers * steps)
        for _ in range(steps):
            stk.forward(x0, stream=stream)
        torch.cuda.synchronize()
        kt = ctx.moe_timing_read()
        ctx.moe_timing(0)
        kernels = {n: {"launches": int(c), "avg_us": t / c * 1e3} for n, (c, t) in kt.items()}
        R = T * k
        if "ffn_i8_gate_up_gemm" in kt:
            launches, tot_ms = kt["ffn_i8_gate_up_gemm"]
            per_step_flops = st.layers * 2.0 * (R * 2 * I * d + T * 2 * Is * d)
            per_launch = per_step_flops / (launches / steps)
            avg_s = tot_ms / launches / 1e3
            achieved = per_launch / avg_s / 1e12
            roofline = {"bound": "mfma", "kernel": "ffn_i8_gate_up_gemm",
                        "achieved": round(achieved, 1), "peak": INT8_PEAK_TOPS,
                        "unit": "TFLOP/s", "frac": round(achieved / INT8_PEAK_TOPS, 4),
                        "traffic": counter_traffic(args.workload, "gate_up_gemm_kernel"),
                        "traffic_scope": "median launch of the first 2 layers (profiles/)",
                        "flops_per_launch": per_launch,
                        "avg_launch_us": round(avg_s * 1e6, 2),
                        "frac_of_bf16_peak": round(achieved / BF16_PEAK_TFLOPS, 4)}
        elif "ffn_i8_gate_up" in kt or "ffn_i4_gate_up" in kt:
            kname = "ffn_i4_gate_up" if int4 else "ffn_i8_gate_up"
            launches, tot_ms = kt[kname]
            per_step = sum(n * e_gu + sh_gu + T * d * 2 + (R * I + T * Is) * 2
                           + (R * I + T * Is) // 64 * 4 for n in touched)
            per_launch = per_step / (launches / steps)
            avg_s = tot_ms / launches / 1e3
            achieved = per_launch / avg_s / 1e9
            roofline = {"bound": "hbm", "kernel": kname,
                        "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(achieved / HBM_PEAK_GBS, 4),
                        "traffic": counter_traffic(args.workload, "gate_up_kernel<"),
                        "traffic_scope": "median launch of the first 2 layers (profiles/)",
                        "bytes_per_launch": int(per_launch),
                        "avg_launch_us": round(avg_s * 1e6, 2)}

    cpu = None
    if not args.no_cpu:
        log("[bench] timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline_stack(st, args.cpu_budget)

    out = {
        "metric": METRIC,
        "value": round(tok_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4" if int4 else "int8",
        "data": "synthetic (seeded generator, weights drawn on the GPU; random weights of the "
                "stated shapes)",
        "config": {"workload": desc, "T": T, "layers": st.layers, "d": d, "E": E, "k": k,
                   "inter": I, "router": s0.router, "expert_format": s0.fmt,
                   "shared_expert": s0.shared, "zipf_alpha": st.alpha,
                   "hip_graph": use_graph, "entry_point": "moe_forward per layer",
                   "parallelism": "single GPU"},
        "hbm_gbps_algorithmic": round(gbs, 1),
        "hbm_frac_algorithmic": round(gbs / HBM_PEAK_GBS, 4),
        "tflops_algorithmic": round(tflops, 3),
        "step_bytes_algorithmic": int(step_bytes),
        "step_flops_algorithmic": step_flops,
        "top64_mass_per_layer": masses,
        "touched_experts_per_layer": touched,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernels": kernels,
    }
    print(json.dumps(out), flush=True)


def cpu_baseline_quant(spec, fmt, budget_s: float):
    """The oracle's quantizer on whole experts of the same workload (host copies of
    the same bf16 values), bounded repeat count."""
    import oracle
    from sparse_moe_expert_sigmoid_amd import synth as S
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    w = [oracle.bf16_to_f32(S.bf16_bits(S.float_expert(spec, e, p)))
         for e in range(2) for p in ("gu", "dn")]
    n = sum(a.size for a in w)
    reps = 0
    t0 = time.perf_counter()
    while True:
        for a in w:
            oracle.quantize(fmt, a)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or el / reps * (reps + 1) > 3 * budget_s:
            break
    return {"value": n * reps / el, "unit": "weights/s", "cores": threads, "kind": "oracle",
            "sample": f"{reps} x oracle quantizer on experts 0 and 1 (gate/up and down, "
                      f"{n} weights) of this workload (C, OpenMP over rows), {el:.1f} s"}


def run_quant(args):
    import torch
    from sparse_moe_expert_sigmoid_amd import Context, binding as B, synth as S

    spec_name, fmt, desc = QUANT_WORKLOADS[args.workload]
    spec = S.spec(spec_name)
    E, d, I = spec.E, spec.d, spec.inter
    steps = args.steps or 10
    warmup = args.warmup if args.warmup is not None else 2
    dev = torch.device("cuda:0")
    ctx = Context(0)
    log(f"[bench] workload {args.workload}: uploading bf16 weights of {E} experts")
    gu = torch.empty((E * 2 * I, d), dtype=torch.bfloat16, device=dev)
    dn = torch.empty((E * d, I), dtype=torch.bfloat16, device=dev)
    for e in range(E):
        gu[e * 2 * I:(e + 1) * 2 * I] = torch.from_numpy(
            S.bf16_bits(S.float_expert(spec, e, "gu")).view(np.int16)).view(torch.bfloat16)
        dn[e * d:(e + 1) * d] = torch.from_numpy(
            S.bf16_bits(S.float_expert(spec, e, "dn")).view(np.int16)).view(torch.bfloat16)
    per = 1 if fmt == "int8_row" else 2
    f = B.MOE_W_INT8_ROW if fmt == "int8_row" else B.MOE_W_INT4_B32
    cdt = torch.int8 if per == 1 else torch.uint8
    cg = torch.empty((E * 2 * I, d // per), dtype=cdt, device=dev)
    cd = torch.empty((E * d, I // per), dtype=cdt, device=dev)
    sg = torch.empty((E * 2 * I) * (1 if per == 1 else d // 32), dtype=torch.float32, device=dev)
    sd = torch.empty((E * d) * (1 if per == 1 else I // 32), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        ctx.moe_quantize(f, gu, cg, sg, stream)
        ctx.moe_quantize(f, dn, cd, sd, stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    ev0.record(stream)
    for _ in range(steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms_per_step = ev0.elapsed_time(ev1) / steps
    n_w = gu.numel() + dn.numel()
    w_s = n_w / (ms_per_step / 1e3)
    step_bytes = (n_w * 2 + cg.numel() + cd.numel() + (sg.numel() + sd.numel()) * 4)
    gbs = step_bytes / (ms_per_step / 1e3) / 1e9
    log(f"[bench] {ms_per_step:.3f} ms/step, {w_s / 1e9:.1f} G weights/s, {gbs:.0f} GB/s "
        f"(wall {wall:.3f} s)")

    kernels, roofline = {}, None
    if not args.no_kernel_timing:
        ctx.moe_timing(4 * steps)
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
        kt = ctx.moe_timing_read()
        ctx.moe_timing(0)
        kernels = {n: {"launches": int(c), "avg_us": t / c * 1e3} for n, (c, t) in kt.items()}
        name = "quant_i8_rows" if per == 1 else "quant_i4_blocks"
        if name in kt:
            launches, tot_ms = kt[name]
            per_launch = step_bytes / (launches / steps)
            avg_s = tot_ms / launches / 1e3
            achieved = per_launch / avg_s / 1e9
            roofline = {"bound": "hbm", "kernel": name, "achieved": round(achieved, 1),
                        "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(achieved / HBM_PEAK_GBS, 4),
                        "traffic": counter_traffic(args.workload, "quant_", "quant.hip"),
                        "bytes_per_launch": int(per_launch),
                        "avg_launch_us": round(avg_s * 1e6, 2)}

    cpu = None
    if not args.no_cpu:
        log("[bench] timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline_quant(spec, fmt, args.cpu_budget)

    out = {
        "metric": "weights quantized per second (bf16 -> expert format), % HBM roofline",
        "value": round(w_s, 1),
        "unit": "weights/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded N(0, 0.02^2) weights rounded to bf16)",
        "config": {"workload": desc, "E": E, "d": d, "inter": I, "format": fmt,
                   "input": "bf16", "entry_point": "moe_quantize x2",
                   "parallelism": "single GPU"},
        "hbm_gbps_algorithmic": round(gbs, 1),
        "step_bytes_algorithmic": int(step_bytes),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernels": kernels,
    }
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="kimi_decode",
                    choices=sorted(WORKLOADS) + sorted(STACK_WORKLOADS) +
                    sorted(QUANT_WORKLOADS))
    ap.add_argument("--layers", type=int, default=None,
                    help="stack workloads: run only the first N of the 26 layers")
    ap.add_argument("--no-graph", action="store_true",
                    help="stack decode: launch the layers eagerly instead of replaying a HIP graph")
    ap.add_argument("--copies", type=int, default=None)
    ap.add_argument("--path", default="fused", choices=["fused", "staged"],
                    help="fused: one moe_forward call per step; staged: moe_route, "
                         "moe_permute, moe_expert_ffn (routed, shared), moe_combine")
    ap.add_argument("--act", default="silu", choices=["silu", "gelu_tanh"],
                    help="gate activation of the layer workloads")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-kernel-timing", action="store_true")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="after timing, copy BYTES once device-to-device (a kernel of known "
                         "traffic, used to calibrate hardware byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library runs the layer on a single MI355X and "
              "has no multi-GPU path (run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    if args.workload in STACK_WORKLOADS:
        return run_stack(args)
    if args.workload in QUANT_WORKLOADS:
        return run_quant(args)

    import torch
    from sparse_moe_expert_sigmoid_amd import Context, MoELayer, synth as S

    spec_name, chunks, desc, *spec_kw = WORKLOADS[args.workload]
    spec = S.spec(spec_name, **(spec_kw[0] if spec_kw else {}))
    decode = spec.T <= 16
    steps = args.steps or (200 if decode else 40)
    warmup = args.warmup if args.warmup is not None else (20 if decode else 5)

    log(f"[bench] workload {args.workload}: generating inputs")
    inputs = S.make_layer(spec)
    dev = torch.device("cuda:0")
    ctx = Context(0)
    base = MoELayer.from_inputs(ctx, inputs, dev, act=args.act)
    layer_bytes = base.experts.nbytes + (base.shared.nbytes if base.shared else 0)
    # enough copies that one step's weights are never cache-resident from the last
    copies = args.copies or max(2, min(32, math.ceil(2.0e9 / layer_bytes) + 1))
    layers = [base]
    for _ in range(copies - 1):
        layers.append(base.with_weights(base.experts.clone(),
                                        base.shared.clone() if base.shared else None))
    x = torch.from_numpy(inputs.x).to(dev)
    Tc = spec.T // chunks
    xs = [x[i * Tc:(i + 1) * Tc].contiguous() for i in range(chunks)]
    for L in layers:
        L.alloc(Tc)
    stream = torch.cuda.current_stream()
    log(f"[bench] {copies} weight copies of {layer_bytes / 1e9:.3f} GB; T={spec.T} "
        f"({chunks} chunk(s)); warmup {warmup}, steps {steps}")

    def step(i):
        L = layers[i % copies]
        for c in range(chunks):
            if args.path == "fused":
                L.forward_fused(xs[c], stream=stream)
            else:
                L.forward(xs[c], stream=stream)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()

    # ---- timed region: exactly `steps` steps
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    ev0.record(stream)
    for i in range(steps):
        step(warmup + i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms = ev0.elapsed_time(ev1)
    ms_per_step = ms / steps
    tok_s = spec.T / (ms_per_step / 1e3)
    log(f"[bench] {ms_per_step * 1e3:.1f} us/step, {tok_s:,.0f} tokens/s (wall {wall:.3f} s)")

    # ---- algorithmic work of one step, from the actual routing
    idx = layers[0].idx.cpu().numpy() if chunks == 1 else None
    if chunks > 1:
        idx_all = []
        for c in range(chunks):
            layers[0].forward(xs[c], stream=stream)
            torch.cuda.synchronize()
            idx_all.append(layers[0].idx.cpu().numpy().copy())
        touched_per_chunk = [np.unique(a) for a in idx_all]
    else:
        touched_per_chunk = [np.unique(idx)]
    d, I, k, E = spec.d, spec.inter, spec.k, spec.E
    gu_b = dn_b = 0
    for t in touched_per_chunk:
        a, b = expert_bytes(inputs.experts, t)
        gu_b += a
        dn_b += b
    sh_gu = sh_dn = 0
    if inputs.shared is not None:
        sh_gu, sh_dn = expert_bytes(inputs.shared, [0])
        sh_gu *= chunks
        sh_dn *= chunks
    act_bytes = spec.T * d * 4 * 2                      # x read once, y written once
    router_bytes = (E * d + (E if inputs.bias is not None else 0)) * 4 * chunks
    step_bytes = gu_b + dn_b + sh_gu + sh_dn + act_bytes + router_bytes
    Is = spec.shared_inter if inputs.shared is not None else 0
    step_flops = 2.0 * (spec.T * k * 3 * d * I + spec.T * 3 * d * Is + spec.T * d * E)
    gbs = step_bytes / (ms_per_step / 1e3) / 1e9
    tflops = step_flops / (ms_per_step / 1e3) / 1e12

    # ---- second pass: per-kernel durations from HIP events on the launch stream
    kernels = {}
    roofline = None
    if not args.no_kernel_timing:
        ctx.moe_timing(64 * steps)
        for i in range(steps):
            step(warmup + i)
        torch.cuda.synchronize()
        kt = ctx.moe_timing_read()
        ctx.moe_timing(0)
        kernels = {n: {"launches": int(c), "avg_us": t / c * 1e3} for n, (c, t) in kt.items()}
        dom = "ffn_i4_gate_up" if spec.fmt.startswith("int4") else "ffn_i8_gate_up"
        gemm = "ffn_i8_gate_up_gemm" in kt
        if gemm:
            dom = "ffn_i8_gate_up_gemm"
        if dom in kt:
            launches, tot_ms = kt[dom]
            # algorithmic bytes of the gate/up launches of one step: codes + scales of
            # every touched expert (routed) or the shared expert, activation digits
            # read once (2 bytes per input), h written once (fp32)
            R = spec.T * k
            # (x as 2-byte digits; h written as 2-byte digits + one fp32 scale per 64)
            per_step = (gu_b + sh_gu + spec.T * d * 2
                        + (R * I + spec.T * Is) * 2 + (R * I + spec.T * Is) // 64 * 4)
            launches_per_step = launches / steps
            bytes_per_launch = per_step / launches_per_step
            avg_s = tot_ms / launches / 1e3
            achieved = bytes_per_launch / avg_s / 1e9
            traffic = counter_traffic(args.workload,
                                      "gate_up_gemm_kernel" if gemm else "gate_up_kernel<")
            roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
                        "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                        "bytes_per_launch": int(bytes_per_launch),
                        "avg_launch_us": round(avg_s * 1e6, 2)}
            if gemm:  # the grouped GEMM's matrix-core rate beside its HBM rate
                gflops = 2.0 * (R * 2 * I * d + spec.T * 2 * Is * d) / launches_per_step
                roofline["mfma_tflops"] = round(gflops / avg_s / 1e12, 1)
                roofline["mfma_frac_int8"] = round(gflops / avg_s / 1e12 / INT8_PEAK_TOPS, 4)

    if args.copy_probe > 0:
        # a fill kernel (writes N bytes) and an elementwise kernel (reads N, writes N)
        src = torch.empty(args.copy_probe, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        src.fill_(1)
        torch.add(src, 0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    cpu = None
    if not args.no_cpu:
        log("[bench] timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline(inputs, args.cpu_budget, args.act)

    out = {
        "metric": METRIC,
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8" if spec.fmt != "fp32" else "f32",
        "data": "synthetic (seeded generator; random weights of the stated shapes)",
        "config": {"workload": desc, "T": spec.T, "chunks": chunks, "d": d, "E": E, "k": k,
                   "inter": I, "router": spec.router, "expert_format": spec.fmt,
                   "shared_expert": spec.shared, "weight_copies": copies,
                   "activation": args.act,
                   "entry_point": "moe_forward" if args.path == "fused" else
                   "moe_route+moe_permute+moe_expert_ffn x2+moe_combine",
                   "parallelism": "single GPU"},
        "hbm_gbps_algorithmic": round(gbs, 1),
        "tflops_algorithmic": round(tflops, 3),
        "step_bytes_algorithmic": int(step_bytes),
        "step_flops_algorithmic": step_flops,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernels": kernels,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
