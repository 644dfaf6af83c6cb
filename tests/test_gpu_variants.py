"""GPU: the layer variants the pages name beside the main path.

* The gelu_tanh gate activation (the moe op's other activation attribute,
  LiteRT-LM details, "Runtime") through every FFN path: pairs grouped
  in-kernel (T <= 16), 16-row tiles, the int8 grouped GEMM, int4 experts and
  the fp32 shared expert; separate calls and moe_forward.
* int4 experts with one scale per block of 128 inputs (the block width the
  Kimi-Linear LiteRT-LM model card measures beside 32): layers of the
  Qwen3-shaped sizes at decode and prefill, both code layouts, and the
  quantizer for that format.
Each against the oracle under the usual rules (expert sets exact except at
oracle near-ties, outputs within 2e-3 of max|y|; quantizer bit-exact).
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


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def _layer_case(ctx, name, act="silu", tokens=None, tiled=True, fused_too=True, **kw):
    import torch
    from sparse_moe_expert_sigmoid_amd import MoELayer
    spec = S.spec(name, **kw)
    inp = S.make_layer(spec)
    print(f"[variant] {name} act={act} {kw} tiled={tiled}", flush=True)
    L = MoELayer.from_inputs(ctx, inp, tiled=tiled, act=act)
    xd = _dev(inp.x)
    sel = np.arange(spec.T) if tokens is None else np.asarray(tokens)
    ex = oracle.Experts.of(inp.experts, act)
    sh = oracle.Experts.of(inp.shared, act) if inp.shared is not None else None
    oy, oidx, ow, ogap = oracle.layer(spec.router, spec.k, spec.scale, inp.x, inp.wr, inp.bias,
                                      ex, sh, tokens=tokens)
    _, _, _, logits = oracle.route(spec.router, inp.x[sel], inp.wr, inp.bias, spec.k,
                                   spec.scale, want_logits=True)
    keys = oracle_keys(spec.router, logits, inp.bias)
    for fused in ((False, True) if fused_too else (False,)):
        y = L.forward_fused(xd) if fused else L(xd)
        torch.cuda.synchronize()
        exc = compare_route(L.idx.cpu().numpy()[sel], L.w.cpu().numpy()[sel], oidx, ow, ogap,
                            keys, spec.scale)
        keep = np.setdiff1d(np.arange(len(sel)), exc)
        ratio = compare_outputs(y.cpu().numpy()[sel], oy, keep)
        log_result(test="variant", config=name, act=act, fmt=spec.fmt, T=spec.T, fused=fused,
                   tiled=tiled, excused=len(exc), err_over_max=ratio)
    return L


# ------------------------------------------------------------------ gelu_tanh

@pytest.mark.parametrize("kw", [
    dict(T=5, E=16, k=4, shared="int8_row", shared_inter=128),     # pairs, fused shared
    dict(T=40),                                                    # 16-row tiles, fp32 shared
    dict(T=300, E=16, k=4, shared="int8_row", shared_inter=256),   # grouped GEMM (75 rows/expert)
    dict(T=24, fmt="int4_b32", d=256, inter=128, shared=None, shared_inter=0),
    dict(T=3, fmt="int4_b128", d=256, inter=256, shared=None, shared_inter=0),
    # one token: the gate/up launch selects and encodes for itself
    dict(T=1, E=16, k=4, shared="int8_row", shared_inter=128),
    dict(T=1, fmt="int4_b32", d=256, inter=128, shared=None, shared_inter=0),
])
def test_gelu_tanh_layer_matches_oracle(ctx, kw):
    _layer_case(ctx, "tiny", act="gelu_tanh", xseed=0x6E4C0000 + kw["T"], **kw)


def test_gelu_tanh_kimi_prefill_sampled(ctx):
    tokens = [0, 17, 511, 1023]
    _layer_case(ctx, "kimi_prefill", act="gelu_tanh", tokens=tokens)


def test_gelu_tanh_differs_from_silu(ctx):
    import torch
    from sparse_moe_expert_sigmoid_amd import MoELayer
    inp = S.make_layer(S.spec("tiny", T=8))
    a = MoELayer.from_inputs(ctx, inp, act="silu").forward_fused(_dev(inp.x)).clone()
    b = MoELayer.from_inputs(ctx, inp, act="gelu_tanh").forward_fused(_dev(inp.x)).clone()
    torch.cuda.synchronize()
    assert not torch.allclose(a, b, rtol=1e-3, atol=1e-3)


# ------------------------------------------------------------------ int4 block 128

@pytest.mark.parametrize("name", ["qwen_decode", "qwen_prefill"])
@pytest.mark.parametrize("tiled", [True, False])
def test_int4_b128_qwen_layers(ctx, name, tiled):
    # (the fused call at T = 1 splits gate/up K over 2 workgroups)
    _layer_case(ctx, name, fmt="int4_b128", tiled=tiled, fused_too=True)


@pytest.mark.parametrize("T", [1, 16, 37, 200])
def test_int4_b128_small_layers_and_clamp(ctx, T):
    # scales at, below and far below 2^-14 are drawn among the block scales
    spec = S.spec("tiny", T=T, fmt="int4_b128", d=384, inter=256, E=24, k=6,
                  shared=None, shared_inter=0, xseed=0x6E4D0000 + T)
    inp = S.make_layer(spec)
    assert (inp.experts.gu_s < 2.0 ** -14).any() or (inp.experts.dn_s < 2.0 ** -14).any()
    _layer_case(ctx, "tiny", fmt="int4_b128", d=384, inter=256, E=24, k=6, shared=None,
                shared_inter=0, T=T, xseed=0x6E4D0000 + T)


def _unpack_i4(b, K):
    b = b.astype(np.uint8)
    lo = (b & 0xF).astype(np.int8)
    hi = (b >> 4).astype(np.int8)
    q = np.empty(b.shape[:-1] + (K,), np.int8)
    q[..., 0::2] = np.where(lo > 7, lo - 16, lo)
    q[..., 1::2] = np.where(hi > 7, hi - 16, hi)
    return q


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("rows,K", [(41, 128), (7, 2048), (130, 640), (3, 16384), (5, 768)])
def test_quantize_int4_b128_matches_oracle(ctx, rows, K, dtype):
    import torch
    from sparse_moe_expert_sigmoid_amd import binding as B
    w = S.normal(0x6E4E0000 + K, rows, (rows, K), 0.02)
    w[rows // 2] *= 1e-5                      # every block under the 2^-14 floor
    w[rows // 3, :K // 2] = 0.0
    if dtype == "bf16":
        bits = S.bf16_bits(w)
        wv = oracle.bf16_to_f32(bits)
        wd = torch.from_numpy(bits.view(np.int16)).to("cuda:0").view(torch.bfloat16)
    else:
        wv, wd = w, _dev(w)
    codes = torch.empty((rows, K // 2), dtype=torch.uint8, device="cuda:0")
    scales = torch.empty((rows, K // 128), dtype=torch.float32, device="cuda:0")
    ctx.moe_quantize(B.MOE_W_INT4_B128, wd, codes, scales)
    torch.cuda.synchronize()
    oq, os_ = oracle.quantize("int4_b128", wv)
    assert np.array_equal(_unpack_i4(codes.cpu().numpy(), K), oq)
    assert np.array_equal(scales.cpu().numpy().view(np.uint32), os_.view(np.uint32))


# ------------------------------------------------------------------ errors

def test_variant_abi_errors(ctx):
    import torch
    from sparse_moe_expert_sigmoid_amd import MoELayer, binding as B
    inp = S.make_layer(S.spec("tiny", T=4))
    L = MoELayer.from_inputs(ctx, inp)
    L.alloc(4)
    with pytest.raises(B.MoeError) as e:
        ctx.moe_expert_ffn(L.experts, 2, _dev(inp.x), 4, None, None, 4, L.rows, L.ws)
    assert e.value.status == B.MOE_E_UNSUPPORTED and "activation=2" in str(e.value)
    w = torch.zeros((4, 96), dtype=torch.float32, device="cuda:0")
    c = torch.empty((4, 48), dtype=torch.uint8, device="cuda:0")
    s = torch.empty(4, dtype=torch.float32, device="cuda:0")
    with pytest.raises(B.MoeError) as e:
        ctx.moe_quantize(B.MOE_W_INT4_B128, w, c, s)      # 96 is not a multiple of 128
    assert e.value.status == B.MOE_E_UNSUPPORTED and "multiple of 128" in str(e.value)
