"""moe_forward_noalloc: the layer with the library's own scratch array as its
workspace (for callers that cannot allocate), against moe_forward with a
caller's workspace and against the oracle.

Two calls in a row on the Kimi-shaped decode layer, the second with fewer
tokens (T = 8, then T = 1, whose shared expert splits K across workgroups
that meet in the scratch array's join area), then the Qwen-shaped int4 layer
at T = 3 on the same array.  Every call must give moe_forward's routing and
output bit for bit, and match the oracle (expert sets exact, outputs within
2e-3 of max|y|).  A layer too large for the array is refused before any launch.
The T = 8 call is also captured in a HIP graph and replayed, with other
calls on the same array between the replays.
"""
import numpy as np
import pytest

import oracle
from sparse_moe_expert_sigmoid_amd import synth as S
from tests.parity import compare_outputs, compare_route, log_result, oracle_keys

pytestmark = pytest.mark.gpu


def _check(ctx, L, inp, T):
    import torch
    s = inp.spec
    x = torch.from_numpy(np.ascontiguousarray(inp.x[:T])).to("cuda:0")
    print(f"[noalloc] {s.name} T={T}", flush=True)
    y_ref = L.forward_fused(x).clone()
    idx_ref, w_ref = L.idx.clone(), L.w.clone()
    y = torch.full((T, s.d), float("nan"), dtype=torch.float32, device="cuda:0")
    idx = torch.full((T, s.k), -1, dtype=torch.int32, device="cuda:0")
    w = torch.full((T, s.k), float("nan"), dtype=torch.float32, device="cuda:0")
    ctx.moe_forward_noalloc(L.desc, L.act, x, T, None, y, idx, w)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx_ref) and torch.equal(w, w_ref)
    assert torch.equal(y, y_ref)
    tokens = np.arange(T)
    oy, oidx, ow, ogap = oracle.layer_of(inp, tokens=tokens)
    _, _, _, logits = oracle.route(s.router, inp.x[:T], inp.wr, inp.bias, s.k, s.scale,
                                   want_logits=True)
    exc = compare_route(idx.cpu().numpy(), w.cpu().numpy(), oidx, ow, ogap,
                        oracle_keys(s.router, logits, inp.bias), s.scale)
    ratio = compare_outputs(y.cpu().numpy(), oy, np.setdiff1d(tokens, exc))
    log_result(test="forward_noalloc", config=s.name, T=T, excused=len(exc), err_over_max=ratio)


def test_forward_noalloc_matches_forward(gpu):
    from sparse_moe_expert_sigmoid_amd import Context, MoELayer
    from sparse_moe_expert_sigmoid_amd import binding as B
    ctx = Context(0)
    kimi = S.make_layer(S.spec("kimi_decode"))
    L = MoELayer.from_inputs(ctx, kimi)
    _check(ctx, L, kimi, 8)
    _check(ctx, L, kimi, 1)
    # a layer whose workspace exceeds the scratch array: refused, nothing launched
    import torch
    T = 300
    x = torch.zeros((T, kimi.spec.d), dtype=torch.float32, device="cuda:0")
    y = torch.empty_like(x)
    with pytest.raises(B.MoeError) as e:
        ctx.moe_forward_noalloc(L.desc, L.act, x, T, None, y, None, None)
    assert e.value.status == B.MOE_E_UNSUPPORTED and "scratch" in str(e.value)
    del L
    qwen = S.make_layer(S.spec("qwen_decode", T=3))
    Q = MoELayer.from_inputs(ctx, qwen)
    _check(ctx, Q, qwen, 3)


def test_forward_noalloc_in_a_hip_graph(gpu):
    # The callers this entry point is for include code under HIP graph
    # capture: the Kimi-shaped T = 8 call captured once, replayed four times
    # with eager work between the replays (a T = 1 call that leaves other
    # contents in the shared scratch array, and y and the routing outputs
    # overwritten), each replay equal to the eager call bit for bit.
    import torch
    from sparse_moe_expert_sigmoid_amd import Context, MoELayer
    ctx = Context(0)
    kimi = S.make_layer(S.spec("kimi_decode"))
    L = MoELayer.from_inputs(ctx, kimi)
    d, k = kimi.spec.d, kimi.spec.k
    x = torch.from_numpy(np.ascontiguousarray(kimi.x[:8])).to("cuda:0")
    x1 = x[:1].contiguous()
    y = torch.empty((8, d), dtype=torch.float32, device="cuda:0")
    idx = torch.empty((8, k), dtype=torch.int32, device="cuda:0")
    w = torch.empty((8, k), dtype=torch.float32, device="cuda:0")
    y1 = torch.empty((1, d), dtype=torch.float32, device="cuda:0")
    print("[noalloc] graph capture, Kimi-shaped T=8", flush=True)
    ctx.moe_forward_noalloc(L.desc, L.act, x, 8, x, y, idx, w)
    torch.cuda.synchronize()
    y_ref, idx_ref, w_ref = y.clone(), idx.clone(), w.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):           # warm-up on the capture stream
        ctx.moe_forward_noalloc(L.desc, L.act, x, 8, x, y, idx, w, stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ctx.moe_forward_noalloc(L.desc, L.act, x, 8, x, y, idx, w,
                                stream=torch.cuda.current_stream())
    for rep in range(4):
        ctx.moe_forward_noalloc(L.desc, L.act, x1, 1, None, y1, None, None)
        y.fill_(float("nan"))
        idx.fill_(-1)
        w.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, idx_ref) and torch.equal(w, w_ref), f"replay {rep}"
        assert torch.equal(y, y_ref), f"replay {rep}"
    del g
    log_result(test="forward_noalloc_graph", replays=4)
