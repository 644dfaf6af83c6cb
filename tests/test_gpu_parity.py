"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Every input comes from the seeded generator; both sides read the same
arrays.  Shapes follow the layer workloads (tiny, Kimi-shaped decode and
prefill, Qwen3-shaped int4 decode and prefill) plus edge cases: T = 0 and 1,
ragged expert row counts, every token on the same experts (many tiles per
expert), E = k, and int4 scales at, below and far below 2^-14.
"""
import numpy as np
import pytest

import oracle
from sparse_moe_expert_sigmoid_amd import synth as S
from tests.parity import compare_outputs, compare_route, log_result, oracle_keys

pytestmark = pytest.mark.gpu

_CACHE = {}


_log = log_result


def inputs(name, **kw):
    key = (name, tuple(sorted(kw.items())))
    if key not in _CACHE:
        _CACHE[key] = S.make_layer(S.spec(name, **kw))
    return _CACHE[key]


@pytest.fixture(scope="module")
def ctx(gpu):
    from sparse_moe_expert_sigmoid_amd import Context
    return Context(0)


_LAYERS = {}


def device_layer(ctx, name, tiled=True, **kw):
    import torch
    from sparse_moe_expert_sigmoid_amd import MoELayer
    key = (name, tiled, tuple(sorted(kw.items())))
    if key not in _LAYERS:
        _LAYERS.clear()
        torch.cuda.empty_cache()
        _LAYERS[key] = MoELayer.from_inputs(ctx, inputs(name, **kw), tiled=tiled)
    return _LAYERS[key]


def to_dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def run_route(ctx, L, x):
    import torch
    T = x.shape[0]
    layer = L
    layer.alloc(T)
    xd = to_dev(x)
    ctx.moe_route(layer.router, xd, layer.w_router, layer.bias, T, layer.d, layer.E, layer.k,
                  layer.scale, layer.idx, layer.w, layer.ws)
    torch.cuda.synchronize()
    return layer.idx.cpu().numpy().copy(), layer.w.cpu().numpy().copy()


# ------------------------------------------------------------------ router

@pytest.mark.parametrize("name", ["tiny", "kimi_decode", "kimi_prefill", "qwen_decode",
                                  "qwen_prefill"])
def test_route_parity(ctx, name):
    inp = inputs(name)
    s = inp.spec
    L = device_layer(ctx, name)
    print(f"[route] {name} T={s.T} E={s.E} d={s.d}", flush=True)
    gidx, gw = run_route(ctx, L, inp.x)
    oidx, ow, ogap, logits = oracle.route(s.router, inp.x, inp.wr, inp.bias, s.k, s.scale,
                                          want_logits=True)
    keys = oracle_keys(s.router, logits, inp.bias)
    exc = compare_route(gidx, gw, oidx, ow, ogap, keys, s.scale)
    _log(test="route", config=name, T=s.T, excused=len(exc),
         near_ties=int((ogap < 1e-6).sum()))


def test_route_batch_invariance(ctx):
    inp = inputs("kimi_prefill")
    L = device_layer(ctx, "kimi_prefill")
    idx_full, w_full = run_route(ctx, L, inp.x)
    for c in range(4):
        idx_c, w_c = run_route(ctx, L, inp.x[256 * c: 256 * (c + 1)])
        assert np.array_equal(idx_c, idx_full[256 * c: 256 * (c + 1)])
        assert np.array_equal(w_c, w_full[256 * c: 256 * (c + 1)])
    for t in (0, 5, 1023):
        idx_1, w_1 = run_route(ctx, L, inp.x[t:t + 1])
        assert np.array_equal(idx_1[0], idx_full[t]) and np.array_equal(w_1[0], w_full[t])


@pytest.mark.parametrize("d", [64, 320])
def test_route_short_last_slice(ctx, d):
    # d not a multiple of the 256-wide logit slice: the last slice is short.
    # Small T (the per-chain logits kernel) and T > 32 (the 64x64 tile
    # kernel, 64 inputs staged at a time) must both match the oracle and each
    # other bit for bit.
    got = {}
    for T in (1, 8, 40):
        inp = inputs("tiny", d=d, T=T, E=24, k=4, xseed=0x4D6F45A0)
        s = inp.spec
        L = device_layer(ctx, "tiny", d=d, T=T, E=24, k=4, xseed=0x4D6F45A0)
        gidx, gw = run_route(ctx, L, inp.x)
        oidx, ow, ogap, logits = oracle.route(s.router, inp.x, inp.wr, inp.bias, s.k, s.scale,
                                              want_logits=True)
        exc = compare_route(gidx, gw, oidx, ow, ogap, oracle_keys(s.router, logits, inp.bias),
                            s.scale)
        assert np.isfinite(gw).all()
        got[T] = (gidx, gw)
        _log(test="route_short_slice", d=d, T=T, excused=len(exc))
    for T in (1, 8):
        assert np.array_equal(got[T][0], got[40][0][:T])
        assert np.array_equal(got[T][1], got[40][1][:T])


@pytest.mark.parametrize("E,k,d", [(300, 16, 512), (1024, 16, 256), (40, 8, 4096), (40, 8, 4160)])
def test_layer_router_edges(ctx, E, k, d):
    # E > 256 (2 and 4 experts per selecting thread), k = 16, and d at and past
    # the small-batch tail's limits (16 logit slices, 4096 inputs held in
    # registers); both the small-batch path (T = 5) and the permuted one (T = 40)
    for T in (5, 40):
        kw = dict(E=E, k=k, d=d, T=T, inter=64, shared=None, shared_inter=0,
                  xseed=0x4D6F45B0 + T)
        _forward_vs_oracle(ctx, "tiny", **kw)


# ------------------------------------------------------------------ permute

def _check_permute(ctx, idx, E):
    import torch
    T, k = idx.shape
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda:0")
    row_token = torch.empty(T * k, dtype=torch.int32, device="cuda:0")
    token_row = torch.empty(T * k, dtype=torch.int32, device="cuda:0")
    ctx.moe_permute(to_dev(idx.astype(np.int32)), T, k, E, offsets, row_token, token_row)
    torch.cuda.synchronize()
    oo, ort, otr = oracle.permute(idx, E)
    assert np.array_equal(offsets.cpu().numpy(), oo)
    assert np.array_equal(row_token.cpu().numpy(), ort)
    assert np.array_equal(token_row.cpu().numpy(), otr)


@pytest.mark.parametrize("name", ["tiny", "kimi_decode", "kimi_prefill", "qwen_prefill"])
def test_permute_parity(ctx, name):
    inp = inputs(name)
    s = inp.spec
    idx, _, _ = oracle.route(s.router, inp.x, inp.wr, inp.bias, s.k, s.scale)
    _check_permute(ctx, idx, s.E)


@pytest.mark.parametrize("T,k,E", [(1, 8, 256), (37, 8, 32), (4096, 8, 256), (300, 16, 1024),
                                   (5, 3, 3), (70, 1, 7), (1000, 7, 13), (16384, 8, 256),
                                   (70000, 16, 64)])
def test_permute_synthetic(ctx, T, k, E):
    # (the list is cut into chunks of up to 1024 pairs, one workgroup each, and
    # past 512 chunks into longer segments: T = 70000, k = 16 takes 192-pair
    # segments)
    # distinct experts per token drawn from the generator; includes skew
    u = S.uniform(77, T, (T, E), 0, 1).astype(np.float64)
    u[:, : min(E, 4)] += 0.5                       # four popular experts
    idx = np.argsort(-u, axis=1, kind="stable")[:, :k].astype(np.int32)
    _check_permute(ctx, idx, E)


def test_permute_all_same_experts(ctx):
    idx = np.tile(np.array([9, 3, 200, 17, 0, 255, 128, 64], np.int32), (500, 1))
    _check_permute(ctx, idx, 256)


# ------------------------------------------------------------------ expert FFN

def _ffn_case(ctx, experts_host, dev_experts, x, idx, E):
    import torch
    T = x.shape[0]
    k = idx.shape[1]
    offsets, row_token, token_row = oracle.permute(idx, E)
    R = T * k
    rows = torch.full((R, dev_experts.d), float("nan"), dtype=torch.float32, device="cuda:0")
    need = ctx.moe_workspace_size(T, k, E, dev_experts.d, dev_experts.inter, dev_experts.fmt)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda:0")
    ctx.moe_expert_ffn(dev_experts, 0, to_dev(x), T, to_dev(row_token), to_dev(offsets), R, rows,
                       ws)
    torch.cuda.synchronize()
    g = rows.cpu().numpy()
    o = oracle.expert_rows(oracle.Experts.of(experts_host), x, row_token, offsets)
    return compare_outputs(g, o)


@pytest.mark.parametrize("name", ["tiny", "kimi_decode", "qwen_decode", "qwen_prefill"])
def test_expert_ffn_parity(ctx, name):
    inp = inputs(name)
    s = inp.spec
    L = device_layer(ctx, name)
    idx, _, _ = oracle.route(s.router, inp.x, inp.wr, inp.bias, s.k, s.scale)
    ratio = _ffn_case(ctx, inp.experts, L.experts, inp.x, idx, s.E)
    _log(test="expert_ffn", config=name, fmt=s.fmt, err_over_max=ratio)


def test_expert_ffn_kimi_prefill_sampled(ctx):
    # full T=1024 routing on the GPU; oracle rows for the rows of 3 experts
    import torch
    inp = inputs("kimi_prefill")
    s = inp.spec
    L = device_layer(ctx, "kimi_prefill")
    idx, _, _ = oracle.route(s.router, inp.x, inp.wr, inp.bias, s.k, s.scale)
    offsets, row_token, token_row = oracle.permute(idx, s.E)
    R = s.T * s.k
    rows = torch.empty((R, s.d), dtype=torch.float32, device="cuda:0")
    L.alloc(s.T)
    ctx.moe_expert_ffn(L.experts, 0, to_dev(inp.x), s.T, to_dev(row_token), to_dev(offsets), R,
                       rows, L.ws)
    torch.cuda.synchronize()
    g = rows.cpu().numpy()
    counts = np.diff(offsets)
    picks = [int(np.argmax(counts)), int(np.argmin(np.where(counts > 0, counts, 1 << 30))),
             int(np.flatnonzero(counts > 0)[len(np.flatnonzero(counts > 0)) // 2])]
    picks = sorted(set(picks))
    sel = np.concatenate([np.arange(offsets[e], offsets[e + 1]) for e in picks])
    sub_off = np.zeros(s.E + 1, np.int32)
    for e in picks:
        sub_off[e + 1] = counts[e]
    sub_off = np.cumsum(sub_off).astype(np.int32)
    order = np.concatenate([np.arange(offsets[e], offsets[e + 1]) for e in sorted(set(picks))])
    o = oracle.expert_rows(oracle.Experts.of(inp.experts), inp.x, row_token[order], sub_off)
    ratio = compare_outputs(g[order], o)
    _log(test="expert_ffn_sampled", config="kimi_prefill", rows=int(sel.size),
         err_over_max=ratio)


def test_shared_expert_identity_rows(ctx):
    import torch
    inp = inputs("kimi_decode")
    s = inp.spec
    L = device_layer(ctx, "kimi_decode")
    out = torch.empty((s.T, s.d), dtype=torch.float32, device="cuda:0")
    L.alloc(s.T)
    ctx.moe_expert_ffn(L.shared, 0, to_dev(inp.x), s.T, None, None, s.T, out, L.ws)
    torch.cuda.synchronize()
    o = oracle.expert_rows(oracle.Experts.of(inp.shared), inp.x, None,
                           np.array([0, s.T], np.int32))
    compare_outputs(out.cpu().numpy(), o)


# ------------------------------------------------------------------ combine

@pytest.mark.parametrize("T,k,d,with_shared,with_res", [(8, 8, 2304, True, False),
                                                        (37, 8, 512, True, True),
                                                        (5, 3, 64, False, True)])
def test_combine_parity(ctx, T, k, d, with_shared, with_res):
    import torch
    R = T * k
    rows = S.normal(5, 1, (R, d), 1.0)
    perm = np.argsort(S.uniform(5, 2, (R,), 0, 1)).astype(np.int32)
    w = S.uniform(5, 3, (T, k), 0, 1)
    sh = S.normal(5, 4, (T, d), 1.0) if with_shared else None
    res = S.normal(5, 6, (T, d), 1.0) if with_res else None
    y = torch.empty((T, d), dtype=torch.float32, device="cuda:0")
    ctx.moe_combine(to_dev(rows), to_dev(perm), to_dev(w), to_dev(sh) if sh is not None else None,
                    to_dev(res) if res is not None else None, T, k, d, y)
    torch.cuda.synchronize()
    o = oracle.combine(rows, perm, w, sh, res)
    assert np.allclose(y.cpu().numpy(), o, rtol=1e-6, atol=1e-6 * np.abs(o).max())


# ------------------------------------------------------------------ whole layer

def _layer_vs_oracle(ctx, name, tokens=None, tiled=True, **kw):
    import torch
    inp = inputs(name, **kw)
    s = inp.spec
    L = device_layer(ctx, name, tiled=tiled, **kw)
    xd = to_dev(inp.x)
    y = L(xd)
    torch.cuda.synchronize()
    gy = y.cpu().numpy()
    gidx = L.idx.cpu().numpy()
    gw = L.w.cpu().numpy()
    oy, oidx, ow, ogap = oracle.layer_of(inp, tokens=tokens)
    sel = np.arange(s.T) if tokens is None else np.asarray(tokens)
    _, _, _, logits = oracle.route(s.router, inp.x[sel], inp.wr, inp.bias, s.k, s.scale,
                                   want_logits=True)
    keys = oracle_keys(s.router, logits, inp.bias)
    exc = compare_route(gidx[sel], gw[sel], oidx, ow, ogap, keys, s.scale)
    keep = np.setdiff1d(np.arange(len(sel)), exc)
    ratio = compare_outputs(gy[sel], oy, keep)
    _log(test="layer", config=name, T=s.T, E=s.E, checked_tokens=len(sel), excused=len(exc),
         err_over_max=ratio)
    return gy


@pytest.mark.parametrize("name", ["tiny", "kimi_decode", "qwen_decode", "qwen_prefill"])
def test_layer_parity(ctx, name):
    print(f"[layer] {name}", flush=True)
    _layer_vs_oracle(ctx, name)


@pytest.mark.parametrize("name", ["tiny", "kimi_decode", "qwen_prefill"])
def test_layer_parity_row_layout(ctx, name):
    _layer_vs_oracle(ctx, name, tiled=False)


def _tile_reference(codes_rows, fmt):
    """Byte order of the tiled layout, written from its definition in include/moe.h."""
    N, nbytes = codes_rows.shape
    out = np.empty(N * nbytes, np.uint8)
    pos = 0
    if fmt == "int8_row":
        K = nbytes
        for n16 in range(N // 16):
            for st in range(K // 64):
                for lane in range(64):
                    i, g = lane % 16, lane // 16
                    out[pos:pos + 16] = codes_rows[16 * n16 + i, 64 * st + 16 * g:64 * st + 16 * g + 16]
                    pos += 16
    else:
        K = 2 * nbytes
        for n16 in range(N // 16):
            for sp in range(K // 128):
                for lane in range(64):
                    i, g = lane % 16, lane // 16
                    for q in range(4):          # the span's 4 blocks of 32
                        b = 4 * sp + q
                        o = (32 * b + 8 * g) // 2
                        out[pos:pos + 4] = codes_rows[16 * n16 + i, o:o + 4]
                        pos += 4
    return out


@pytest.mark.parametrize("fmt", ["int8_row", "int4_b32"])
def test_tile_weights_layout(ctx, fmt):
    import torch
    from sparse_moe_expert_sigmoid_amd.binding import DeviceExperts
    E, d, I = 2, 256, 128
    w = S.make_experts(fmt, E, d, I, 31, (4, 5, 6, 7, 12, 13))
    dev = DeviceExperts.upload(w, "cuda:0")
    t = dev.tiled(ctx)
    torch.cuda.synchronize()
    gu_rows = (w.gu_packed if fmt == "int4_b32" else w.gu.view(np.uint8)).reshape(E * 2 * I, -1)
    dn_rows = (w.dn_packed if fmt == "int4_b32" else w.dn.view(np.uint8)).reshape(E * d, -1)
    got_gu = t.w_gate_up.cpu().numpy().view(np.uint8).reshape(-1)
    got_dn = t.w_down.cpu().numpy().view(np.uint8).reshape(-1)
    assert np.array_equal(got_gu, _tile_reference(np.ascontiguousarray(gu_rows), fmt))
    assert np.array_equal(got_dn, _tile_reference(np.ascontiguousarray(dn_rows), fmt))


def test_layer_parity_kimi_prefill_sampled(ctx):
    tokens = np.unique(np.concatenate([np.arange(0, 1024, 41), [1, 2, 511, 1022, 1023]]))
    _layer_vs_oracle(ctx, "kimi_prefill", tokens=tokens)


def test_layer_ragged_tiny_T37(ctx):
    _layer_vs_oracle(ctx, "tiny", T=37, xseed=0x4D6F4599)


def test_layer_single_token(ctx):
    _layer_vs_oracle(ctx, "tiny", T=1, xseed=0x4D6F4598)


def test_layer_every_token_on_same_experts(ctx):
    # bias +1 on 8 experts: they win for every token (64 rows each: 4 tiles per expert)
    import torch
    inp = inputs("tiny", T=64, xseed=0x4D6F4597)
    forced = inp.bias.copy()
    forced[[1, 4, 6, 10, 11, 20, 25, 31]] = 1.0
    inp2 = S.LayerInputs(inp.spec, inp.x, inp.wr, forced, inp.experts, inp.shared)
    from sparse_moe_expert_sigmoid_amd import MoELayer, Context
    L = MoELayer.from_inputs(ctx, inp2)
    y = L(to_dev(inp.x))
    torch.cuda.synchronize()
    oy, oidx, ow, ogap = oracle.layer_of(inp2)
    assert np.array_equal(np.sort(L.idx.cpu().numpy(), 1), np.sort(oidx, 1))
    compare_outputs(y.cpu().numpy(), oy)


def test_layer_gemm_path_edges(ctx):
    # >= 16 rows per expert selects the GEMM tiles (128 rows for gate/up, 64
    # for down); d = 320 and I = 192 leave short K tails and half-empty column
    # blocks; about 150 rows per expert take two gate/up tiles and three down
    # tiles, the last ones partial; the int8 shared expert (I = 128) rides along.
    kw = dict(T=600, d=320, E=8, k=2, inter=192, shared="int8_row", shared_inter=128,
              xseed=0x4D6F4595)
    _layer_vs_oracle(ctx, "tiny", **kw)
    _forward_vs_oracle(ctx, "tiny", **kw)


def test_layer_E_equals_k(ctx):
    _layer_vs_oracle(ctx, "tiny", E=8, T=20, xseed=0x4D6F4596)


def test_layer_zero_tokens_is_noop(ctx):
    import torch
    L = device_layer(ctx, "tiny")
    x = torch.empty((0, 512), dtype=torch.float32, device="cuda:0")
    y = L(x)
    torch.cuda.synchronize()
    assert y.shape == (0, 512)


def test_int4_clamp_inputs_present():
    inp = inputs("qwen_decode")
    s = inp.experts.gu_s
    assert np.count_nonzero(s < S.TWO_M14) > 0 and np.count_nonzero(s == S.TWO_M14) > 0


def test_layer_determinism(ctx):
    import torch
    inp = inputs("kimi_decode")
    L = device_layer(ctx, "kimi_decode")
    xd = to_dev(inp.x)
    a = L(xd).clone()
    b = L(xd).clone()
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# ------------------------------------------------------------------ moe_forward (one call)

def _forward_vs_oracle(ctx, name, tokens=None, residual=False, **kw):
    import torch
    inp = inputs(name, **kw)
    s = inp.spec
    L = device_layer(ctx, name, **kw)
    xd = to_dev(inp.x)
    res = S.normal(0x5EED, 9, (s.T, s.d), 1.0) if residual else None
    y = L.forward_fused(xd, residual=to_dev(res) if residual else None)
    torch.cuda.synchronize()
    gy = y.cpu().numpy()
    oy, oidx, ow, ogap = oracle.layer_of(inp, tokens=tokens)
    sel = np.arange(s.T) if tokens is None else np.asarray(tokens)
    if residual:
        oy = oy + res[sel].astype(np.float64)
    _, _, _, logits = oracle.route(s.router, inp.x[sel], inp.wr, inp.bias, s.k, s.scale,
                                   want_logits=True)
    keys = oracle_keys(s.router, logits, inp.bias)
    exc = compare_route(L.idx.cpu().numpy()[sel], L.w.cpu().numpy()[sel], oidx, ow, ogap, keys,
                        s.scale)
    keep = np.setdiff1d(np.arange(len(sel)), exc)
    ratio = compare_outputs(gy[sel], oy, keep)
    _log(test="forward", config=name, T=s.T, checked_tokens=len(sel), excused=len(exc),
         err_over_max=ratio, residual=residual)


@pytest.mark.parametrize("name", ["tiny", "kimi_decode", "qwen_decode", "qwen_prefill"])
def test_forward_parity(ctx, name):
    _forward_vs_oracle(ctx, name)


def test_forward_kimi_prefill_sampled_with_residual(ctx):
    tokens = np.unique(np.concatenate([np.arange(3, 1024, 53), [0, 1023]]))
    _forward_vs_oracle(ctx, "kimi_prefill", tokens=tokens, residual=True)


def test_forward_small_batch_edges(ctx):
    # T <= 16 groups the (token, slot) pairs inside the FFN kernels: few experts
    # with many rows each, an int8 shared expert in the same launches, T = 16.
    kw = dict(T=16, E=8, k=4, shared="int8_row", shared_inter=128, xseed=0x4D6F4594)
    _forward_vs_oracle(ctx, "tiny", **kw)
    kw1 = dict(T=3, E=8, k=8, shared="int8_row", shared_inter=128, xseed=0x4D6F4593)
    _forward_vs_oracle(ctx, "tiny", **kw1)


def test_forward_small_batch_all_tokens_same_experts(ctx):
    import torch
    from sparse_moe_expert_sigmoid_amd import MoELayer
    inp = inputs("tiny", T=16, shared="int8_row", shared_inter=128, xseed=0x4D6F4592)
    forced = inp.bias.copy()
    forced[[2, 3, 5, 7, 11, 13, 17, 19]] = 1.0
    inp2 = S.LayerInputs(inp.spec, inp.x, inp.wr, forced, inp.experts, inp.shared)
    L = MoELayer.from_inputs(ctx, inp2)
    y = L.forward_fused(to_dev(inp.x))
    torch.cuda.synchronize()
    oy, oidx, ow, ogap = oracle.layer_of(inp2)
    assert np.array_equal(np.sort(L.idx.cpu().numpy(), 1), np.sort(oidx, 1))
    compare_outputs(y.cpu().numpy(), oy)


def test_combine_identity_rows(ctx):
    import torch
    T, k, d = 6, 4, 128
    rows = S.normal(8, 1, (T * k, d), 1.0)
    w = S.uniform(8, 3, (T, k), 0, 1)
    y = torch.empty((T, d), dtype=torch.float32, device="cuda:0")
    ctx.moe_combine(to_dev(rows), None, to_dev(w), None, None, T, k, d, y)
    torch.cuda.synchronize()
    o = oracle.combine(rows, np.arange(T * k, dtype=np.int32), w)
    assert np.allclose(y.cpu().numpy(), o, rtol=1e-6, atol=1e-6 * np.abs(o).max())


def test_forward_matches_staged_router_outputs(ctx):
    import torch
    inp = inputs("kimi_decode")
    L = device_layer(ctx, "kimi_decode")
    xd = to_dev(inp.x)
    L(xd)
    torch.cuda.synchronize()
    idx_a, w_a = L.idx.clone(), L.w.clone()
    L.forward_fused(xd)
    torch.cuda.synchronize()
    assert torch.equal(idx_a, L.idx) and torch.equal(w_a, L.w)


def test_forward_ragged_and_single_token(ctx):
    _forward_vs_oracle(ctx, "tiny", T=37, xseed=0x4D6F4599)
    _forward_vs_oracle(ctx, "tiny", T=1, xseed=0x4D6F4598)


# ------------------------------------------------------------------ errors through the ABI

def test_abi_errors(ctx):
    import torch
    from sparse_moe_expert_sigmoid_amd import binding as B
    L = device_layer(ctx, "tiny")
    L.alloc(4)
    x = torch.zeros((4, 512), dtype=torch.float32, device="cuda:0")
    with pytest.raises(B.MoeError) as e:
        ctx.moe_route(0, x, L.w_router, L.bias, 4, 512, 32, 33, 2.446, L.idx, L.w, L.ws)
    assert e.value.status == B.MOE_E_INVALID and "k=33" in str(e.value)
    with pytest.raises(B.MoeError) as e:
        ctx.moe_route(1, x, L.w_router, L.bias, 4, 512, 32, 8, 1.0, L.idx, L.w, L.ws)
    assert e.value.status == B.MOE_E_INVALID and "bias" in str(e.value)
    with pytest.raises(B.MoeError) as e:
        ctx.moe_route(0, x, L.w_router, L.bias, 4, 512, 32, 8, 2.446, L.idx, L.w, L.ws,
                      ws_bytes=16)
    assert e.value.status == B.MOE_E_WORKSPACE
    with pytest.raises(B.MoeError) as e:
        ctx.moe_expert_ffn(L.experts, 7, x, 4, L.row_token, L.offsets, 32, L.rows, L.ws)
    assert e.value.status == B.MOE_E_UNSUPPORTED and "activation" in str(e.value)
    with pytest.raises(B.MoeError) as e:
        ctx.moe_combine(L.rows, L.token_row, L.w, None, None, 4, 8, 510, L.y)
    assert e.value.status == B.MOE_E_UNSUPPORTED
    # widths past the supported maximum are refused before any launch
    wide = B.DeviceExperts(L.experts.fmt, L.experts.n_experts, 16448, L.experts.inter,
                           L.experts.w_gate_up, L.experts.w_down, L.experts.s_gate_up,
                           L.experts.s_down, L.experts.layout)
    with pytest.raises(B.MoeError) as e:
        ctx.moe_expert_ffn(wide, 0, x, 4, L.row_token, L.offsets, 32, L.rows, L.ws)
    assert e.value.status == B.MOE_E_UNSUPPORTED and "16384" in str(e.value)


# K split across workgroups (decode launches with fewer work units than CUs).
# The T = 1 cases are sized so the launcher splits (256 CUs); the arithmetic:
#  int8 gate/up: 9 tiles (8 slots + shared) x 512/64 column blocks = 72 units,
#    36 K-steps: split 3 ways (integer partials, exact).
#  int8 down: 9 tiles x 512/64 output blocks = 72 units, I = 2048: 3 ways
#    (fp32 partials added in workgroup order).
#  int4 down: 8 tiles x 512/64 = 64 units, I = 2048 (16 spans): 2 ways.
#  int8 gate/up at T = 2 (pairs grouped in-kernel): 17 tiles x 384/64 = 102
#    units: 2 ways.
# At T = 2 and 3 the other shapes have too many tiles to split: those cases
# check the unsplit path of the same shapes.
_SPLIT_CASES = {
    "i8_gate_up": dict(d=2304, E=64, k=8, inter=512, shared="int8_row", shared_inter=512),
    "i8_down": dict(d=512, E=64, k=8, inter=2048, shared="int8_row", shared_inter=2048),
    "i8_gate_up_pairs": dict(d=2304, E=64, k=8, inter=384, shared="int8_row", shared_inter=384),
}


@pytest.mark.parametrize("case", sorted(_SPLIT_CASES))
@pytest.mark.parametrize("T", [1, 2, 3])
def test_forward_split_k(ctx, case, T):
    print(f"[split] {case} T={T}", flush=True)
    _forward_vs_oracle(ctx, "tiny", T=T, xseed=0x4D6F4580 + T, **_SPLIT_CASES[case])


@pytest.mark.parametrize("T", [1, 3])
def test_forward_split_k_int4_down(ctx, T):
    print(f"[split] int4 down T={T}", flush=True)
    _forward_vs_oracle(ctx, "qwen_decode", T=T, d=512, inter=2048, xseed=0x4D6F4590 + T)


def test_forward_split_k_repeatable(ctx):
    # the join adds partials in workgroup order: repeated calls agree bit for bit
    import torch
    for name, kw in (("tiny", _SPLIT_CASES["i8_down"]), ("qwen_decode", dict(d=512, inter=2048))):
        inp = inputs(name, T=2, xseed=0x4D6F4577, **kw)
        L = device_layer(ctx, name, T=2, xseed=0x4D6F4577, **kw)
        xd = to_dev(inp.x)
        ys = [L.forward_fused(xd).clone() for _ in range(3)]
        torch.cuda.synchronize()
        assert all(torch.equal(ys[0], y) for y in ys[1:])


def test_layer_gemm_path_wide_inter(ctx):
    # I = 4224 (33 scale blocks of 128) is above what the ring down GEMM
    # stages in LDS: the register-staged down GEMM runs; 64 rows per expert
    # select the GEMM path
    kw = dict(T=128, d=256, E=4, k=2, inter=4224, shared="int8_row", shared_inter=4224,
              xseed=0x4D6F4594)
    _forward_vs_oracle(ctx, "tiny", **kw)


# ------------------------------------------------------------------ T = 1024 as 4 x 256 chunks

def test_forward_kimi_prefill_4x256_chunks(ctx):
    # The Kimi-shaped prefill (d = 2304, E = 256, I = 2048, int8 shared
    # expert) run as four chunks of 256 tokens, the way the chunked prefill is
    # timed.  At T = 256 the rows per expert (2048 over 256 experts) stay below
    # the grouped GEMM's threshold, so this takes the 16-row tile kernels with
    # the shared expert in the same launches, at the layer's real width.  Both
    # the one-call layer and the five separate calls are compared with the
    # oracle on sampled tokens of every chunk (tokens are independent, so the
    # oracle of token 256 c + t is the chunk's token t).
    import torch
    inp = inputs("kimi_prefill")
    s = inp.spec
    L = device_layer(ctx, "kimi_prefill")
    local = np.array([0, 1, 37, 100, 128, 199, 254, 255])
    for c in range(4):
        xc = to_dev(inp.x[256 * c: 256 * (c + 1)])
        tokens = 256 * c + local
        oy, oidx, ow, ogap = oracle.layer_of(inp, tokens=tokens)
        _, _, _, logits = oracle.route(s.router, inp.x[tokens], inp.wr, inp.bias, s.k, s.scale,
                                       want_logits=True)
        keys = oracle_keys(s.router, logits, inp.bias)
        for path in ("forward", "staged"):
            print(f"[chunk] kimi_prefill chunk {c} path {path}", flush=True)
            y = L.forward_fused(xc) if path == "forward" else L(xc)
            torch.cuda.synchronize()
            gy = y.cpu().numpy()[local]
            exc = compare_route(L.idx.cpu().numpy()[local], L.w.cpu().numpy()[local], oidx, ow,
                                ogap, keys, s.scale)
            keep = np.setdiff1d(np.arange(len(local)), exc)
            ratio = compare_outputs(gy, oy, keep)
            _log(test="forward_4x256", config="kimi_prefill", chunk=c, path=path, T=256,
                 checked_tokens=len(local), excused=len(exc), err_over_max=ratio)


# ------------------------------------------------------------------ a large batch

@pytest.mark.parametrize("name", ["kimi_prefill", "qwen_prefill"])
def test_forward_T65536_sampled(ctx, name):
    # A layer at T = 65536 through moe_forward: 524288 routed rows, so the
    # expert rows (4.8 GB of fp32 for the Kimi-shaped layer, 4.3 GB for the
    # Qwen-shaped one) span more than 2^31 bytes and every row offset into
    # them needs 64-bit arithmetic (int8 grouped GEMM and int4 grouped GEMM).
    # Sampled tokens: both ends, the middle, and tokens whose experts (as the
    # GPU routed them) sit at the top of the permuted rows, checked against
    # the oracle token by token (tokens are independent).
    import torch
    T = 65536
    try:
        inp = inputs(name, T=T)
        s = inp.spec
        L = device_layer(ctx, name, T=T)
        print(f"[large] {name} T={T} forward", flush=True)
        y = L.forward_fused(to_dev(inp.x))
        torch.cuda.synchronize()
        gidx = L.idx.cpu().numpy()
        top = np.flatnonzero((gidx >= s.E - 3).any(axis=1))
        tokens = np.unique(np.concatenate([[0, 1, T // 2 - 1, T // 2, T - 2, T - 1],
                                           top[:4], top[-4:]]))
        gy = y.cpu().numpy()[tokens]
        gw = L.w.cpu().numpy()[tokens]
        del y
        oy, oidx, ow, ogap = oracle.layer_of(inp, tokens=tokens)
        _, _, _, logits = oracle.route(s.router, inp.x[tokens], inp.wr, inp.bias, s.k, s.scale,
                                       want_logits=True)
        keys = oracle_keys(s.router, logits, inp.bias)
        exc = compare_route(gidx[tokens], gw, oidx, ow, ogap, keys, s.scale)
        keep = np.setdiff1d(np.arange(len(tokens)), exc)
        ratio = compare_outputs(gy, oy, keep)
        _log(test="forward_large", config=name, T=T, checked_tokens=len(tokens),
             excused=len(exc), err_over_max=ratio)
    finally:
        _LAYERS.clear()
        _CACHE.pop((name, (("T", T),)), None)
        torch.cuda.empty_cache()


# ------------------------------------------------------------------ path boundaries

@pytest.mark.parametrize("name,T,kernel,permute", [
    ("kimi_prefill", 16, "ffn_i8_gate_up", False),       # small batch: pairs grouped in-kernel
    ("kimi_prefill", 17, "ffn_i8_gate_up", True),        # 16-row tiles over the permutation
    ("kimi_prefill", 511, "ffn_i8_gate_up", True),       # R = 4088 < 16 E: still the tiles
    ("kimi_prefill", 512, "ffn_i8_gate_up_gemm", True),  # R = 4096 = 16 E: the grouped GEMM
    ("qwen_prefill", 255, "ffn_i4_gate_up", True),       # R = 2040 < 16 E
    ("qwen_prefill", 256, "ffn_i4_gate_up_gemm", True),  # R = 2048: the int4 grouped GEMM
])
def test_forward_path_boundaries(ctx, name, T, kernel, permute):
    # moe_forward on either side of each switch between kernel families (by
    # batch size, and by rows per expert R / E against 16), checked against the
    # oracle on sampled tokens; the kernel timer shows which family ran.
    # Tokens are independent, so the first T tokens of a longer seeded batch
    # serve as the batch.
    import torch
    kw = {} if name == "kimi_prefill" else {"T": 1024}  # (kimi_prefill is T = 1024)
    inp = inputs(name, **kw)
    s = inp.spec
    L = device_layer(ctx, name, **kw)
    x = np.ascontiguousarray(inp.x[:T])
    print(f"[boundary] {name} T={T}", flush=True)
    ctx.moe_timing(256)
    try:
        y = L.forward_fused(to_dev(x))
        torch.cuda.synchronize()
        names = set(ctx.moe_timing_read())
    finally:
        ctx.moe_timing(0)
    assert kernel in names, sorted(names)
    assert ("permute" in names) == permute, sorted(names)
    tokens = np.unique(np.concatenate([np.arange(0, T, max(1, T // 12)), [T - 1]]))
    gy = y.cpu().numpy()[tokens]
    oy, oidx, ow, ogap = oracle.layer_of(inp, tokens=tokens)
    _, _, _, logits = oracle.route(s.router, inp.x[tokens], inp.wr, inp.bias, s.k, s.scale,
                                   want_logits=True)
    keys = oracle_keys(s.router, logits, inp.bias)
    exc = compare_route(L.idx.cpu().numpy()[tokens], L.w.cpu().numpy()[tokens], oidx, ow, ogap,
                        keys, s.scale)
    keep = np.setdiff1d(np.arange(len(tokens)), exc)
    ratio = compare_outputs(gy, oy, keep)
    _log(test="forward_boundary", config=name, T=T, kernel=kernel, checked_tokens=len(tokens),
         excused=len(exc), err_over_max=ratio)
