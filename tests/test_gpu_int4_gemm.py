"""GPU parity of the int4 grouped GEMM (prefill: at least 16 rows per expert on
average, tiled int4 codes) against the oracle.

* The Qwen3-shaped layer at the pages' prefill length, T = 1024 (d = 2048,
  E = 128, I = 768, softmax top-8, 64 rows per expert on average), blocks of
  32 and of 128, on sampled tokens, through moe_forward and the separate calls.
* Ragged shapes on the small layer: d = 384 and I = 384 (three 128-input
  spans; the 256-column gate/up blocks and the 512-column down blocks half
  empty), experts with several 64-row tiles and a partial last one, experts
  with no rows, an int4 shared expert in the same launches (group 1), and a
  layer whose int8 shared expert runs apart.
* Block scales at, below and far below 2^-14 (the generator's clamp cases).
Bound: max|err| <= 2e-3 max|y| (the fp32 bound; the arithmetic is exact
integer sums of int4 codes and two int8 digits, folded in fp32).
"""
import numpy as np
import pytest

import oracle
from sparse_moe_expert_sigmoid_amd import synth as S
from tests.parity import compare_outputs, compare_route, log_result, oracle_keys

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ctx(gpu):
    from sparse_moe_expert_sigmoid_amd import Context
    return Context(0)


def _run(ctx, inp, tag, tokens=None, expect_gemm=True):
    import torch
    from sparse_moe_expert_sigmoid_amd import MoELayer
    s = inp.spec
    L = MoELayer.from_inputs(ctx, inp)
    xd = torch.from_numpy(np.ascontiguousarray(inp.x)).to("cuda:0")
    sel = np.arange(s.T) if tokens is None else np.asarray(tokens)
    print(f"[int4 gemm] {tag} T={s.T} tokens={len(sel)}", flush=True)
    oy, oidx, ow, ogap = oracle.layer_of(inp, tokens=tokens)
    _, _, _, logits = oracle.route(s.router, inp.x[sel], inp.wr, inp.bias, s.k, s.scale,
                                   want_logits=True)
    keys = oracle_keys(s.router, logits, inp.bias)
    for path in ("forward", "staged"):
        ctx.moe_timing(64)
        y = L.forward_fused(xd) if path == "forward" else L(xd)
        torch.cuda.synchronize()
        kt = ctx.moe_timing_read()
        ctx.moe_timing(0)
        if expect_gemm:
            assert "ffn_i4_gate_up_gemm" in kt and "ffn_i4_down_gemm" in kt, sorted(kt)
        exc = compare_route(L.idx.cpu().numpy()[sel], L.w.cpu().numpy()[sel], oidx, ow, ogap,
                            keys, s.scale)
        ratio = compare_outputs(y.cpu().numpy()[sel], oy, np.setdiff1d(np.arange(len(sel)), exc))
        log_result(test="int4_gemm", case=tag, path=path, T=s.T, excused=len(exc),
                   err_over_max=ratio)


@pytest.mark.parametrize("fmt", ["int4_b32", "int4_b128"])
def test_qwen_prefill_1024(ctx, fmt):
    inp = S.make_layer(S.spec("qwen_prefill", T=1024, fmt=fmt))
    tokens = np.unique(np.concatenate([np.arange(0, 1024, 37), [1, 2, 511, 1022, 1023]]))
    _run(ctx, inp, f"qwen_T1024_{fmt}", tokens=tokens)


@pytest.mark.parametrize("fmt", ["int4_b32", "int4_b128"])
def test_ragged_spans_and_tiles(ctx, fmt):
    # 8 experts, top 2 of 600 tokens: about 150 rows each (three 64-row tiles,
    # the last partial); d = I = 384: three spans, half-empty column blocks
    kw = dict(T=600, d=384, E=8, k=2, inter=384, fmt=fmt, shared=None, shared_inter=0,
              router="softmax", scale=1.0, xseed=0x4D6F4540)
    _run(ctx, S.make_layer(S.spec("tiny", **kw)), f"ragged_{fmt}")


def test_int4_shared_expert_in_the_launch(ctx):
    # the int4 shared expert (one expert over every token) as group 1 of the
    # same gate/up and down launches; 2 experts get no rows (bias -1)
    kw = dict(T=300, d=512, E=16, k=4, inter=256, fmt="int4_b32", shared="int4_b32",
              shared_inter=384, xseed=0x4D6F4541)
    inp = S.make_layer(S.spec("tiny", **kw))
    b = inp.bias.copy()
    b[[3, 11]] = -1.0
    inp2 = S.LayerInputs(inp.spec, inp.x, inp.wr, b, inp.experts, inp.shared)
    _run(ctx, inp2, "int4_shared")


def test_int8_shared_expert_apart(ctx):
    # int4 routed experts with an int8 shared expert: the routed experts take
    # the int4 GEMM, the shared expert its own launches
    kw = dict(T=400, d=512, E=8, k=4, inter=256, fmt="int4_b128", shared="int8_row",
              shared_inter=256, xseed=0x4D6F4542)
    _run(ctx, S.make_layer(S.spec("tiny", **kw)), "int8_shared_apart")


def test_int4_gemm_repeatable(ctx):
    import torch
    from sparse_moe_expert_sigmoid_amd import MoELayer
    inp = S.make_layer(S.spec("qwen_prefill", T=512))
    L = MoELayer.from_inputs(ctx, inp)
    xd = torch.from_numpy(inp.x).to("cuda:0")
    ys = [L.forward_fused(xd).clone() for _ in range(3)]
    torch.cuda.synchronize()
    assert all(torch.equal(ys[0], y) for y in ys[1:])
