"""GPU: moe_forward_chained through the C ABI on single layers.

Two layers chained (the first from x, the second from the first's pending
output) must give, bit for bit, what moe_forward gives for the two layers one
after the other with the first layer's output as the second's input and
residual: the second layer's input formed by its router launch (x_out), both
layers' routing, and the completed output.  Cases: the Kimi-shaped layer
(int8, int8 shared expert, sigmoid router) at T = 1, 5 and 16, the
Qwen-shaped int4 layer without a shared expert (softmax router) at blocks of
32 and 128, and small layers with k up to 16 and E up to 1024.  Calls the
chained path cannot serve are refused before any launch.
"""
import numpy as np
import pytest

from sparse_moe_expert_sigmoid_amd import synth as S

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ctx(gpu):
    from sparse_moe_expert_sigmoid_amd import Context
    return Context(0)


def _two_layers(ctx, name, **kw):
    from sparse_moe_expert_sigmoid_amd import MoELayer
    a = S.make_layer(S.spec(name, **kw))
    b = S.make_layer(S.spec(name, **dict(kw, wseed=S.spec(name, **kw).wseed + 17)))
    return a, MoELayer.from_inputs(ctx, a), MoELayer.from_inputs(ctx, b)


def _check(ctx, name, T, **kw):
    import torch
    inp, A, B = _two_layers(ctx, name, T=T, **kw)
    s = inp.spec
    d, k = s.d, s.k
    print(f"[chained] {name} T={T} {kw}", flush=True)
    x = torch.from_numpy(np.ascontiguousarray(inp.x)).to("cuda:0")
    dev = dict(device="cuda:0")
    # reference: moe_forward twice, the first output as input and residual
    ws = [torch.empty(max(ctx.moe_layer_workspace_size(L.desc, T), 1), dtype=torch.uint8, **dev)
          for L in (A, B)]
    y1 = torch.empty((T, d), dtype=torch.float32, **dev)
    y2 = torch.empty((T, d), dtype=torch.float32, **dev)
    idx = [torch.empty((T, k), dtype=torch.int32, **dev) for _ in range(4)]
    w = [torch.empty((T, k), dtype=torch.float32, **dev) for _ in range(4)]
    ctx.moe_forward(A.desc, A.act, x, T, x, y1, idx[0], w[0], ws[0])
    ctx.moe_forward(B.desc, B.act, y1, T, y1, y2, idx[1], w[1], ws[1])
    # chained: A leaves its output pending, B forms it into x_out
    x_out = torch.full((T, d), float("nan"), dtype=torch.float32, **dev)
    y = torch.full((T, d), float("nan"), dtype=torch.float32, **dev)
    ws2 = [torch.empty_like(t) for t in ws]
    p1 = ctx.moe_forward_chained(A.desc, A.act, x, None, None, T, idx[2], w[2], ws2[0])
    p2 = ctx.moe_forward_chained(B.desc, B.act, None, p1, x_out, T, idx[3], w[3], ws2[1])
    ctx.moe_combine_pending(p2, y)
    torch.cuda.synchronize()
    assert torch.equal(idx[0], idx[2]) and torch.equal(w[0], w[2])
    assert torch.equal(idx[1], idx[3]) and torch.equal(w[1], w[3])
    assert torch.equal(x_out, y1)
    assert torch.equal(y, y2)
    assert p2.T == T and p2.k == k and p2.d == d and p2.residual == x_out.data_ptr()


@pytest.mark.parametrize("T", [1, 5, 16])
def test_chained_kimi_shaped(ctx, T):
    _check(ctx, "kimi_decode", T)


@pytest.mark.parametrize("fmt", ["int4_b32", "int4_b128"])
def test_chained_qwen_shaped(ctx, fmt):
    _check(ctx, "qwen_decode", 3, fmt=fmt)


@pytest.mark.parametrize("E,k,T,d", [(1024, 16, 4, 512), (40, 1, 16, 256), (24, 8, 9, 1088)])
def test_chained_small_layers(ctx, E, k, T, d):
    _check(ctx, "tiny", T, E=E, k=k, d=d, inter=256, shared="int8_row", shared_inter=256)


def test_chained_refusals(ctx):
    import torch
    from sparse_moe_expert_sigmoid_amd import binding as B
    inp, A, _ = _two_layers(ctx, "tiny", T=32)        # fp32 shared expert: runs apart
    x = torch.from_numpy(np.ascontiguousarray(inp.x)).to("cuda:0")
    ws = torch.empty(ctx.moe_layer_workspace_size(A.desc, 32), dtype=torch.uint8,
                     device="cuda:0")
    with pytest.raises(B.MoeError) as e:
        ctx.moe_forward_chained(A.desc, A.act, x[:4].contiguous(), None, None, 4, None, None,
                                ws)
    assert e.value.status == B.MOE_E_UNSUPPORTED
    inp, K, _ = _two_layers(ctx, "kimi_decode", T=17)
    x = torch.from_numpy(np.ascontiguousarray(inp.x)).to("cuda:0")
    ws = torch.empty(ctx.moe_layer_workspace_size(K.desc, 17), dtype=torch.uint8,
                     device="cuda:0")
    with pytest.raises(B.MoeError) as e:          # past the small-batch size
        ctx.moe_forward_chained(K.desc, K.act, x, None, None, 17, None, None, ws)
    assert e.value.status == B.MOE_E_UNSUPPORTED
    p = ctx.moe_forward_chained(K.desc, K.act, x[:2].contiguous(), None, None, 2, None, None, ws)
    with pytest.raises(B.MoeError) as e:          # x and a pending input both given
        ctx.moe_forward_chained(K.desc, K.act, x[:2].contiguous(), p, x[2:4].contiguous(), 2,
                                None, None, ws)
    assert e.value.status == B.MOE_E_INVALID
    torch.cuda.synchronize()
