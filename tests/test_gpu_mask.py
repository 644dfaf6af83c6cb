"""GPU: expert restriction (moe_route_masked, moe_layer.expert_mask) and routing
statistics (moe_expert_counts).

Restricting a layer to an expert subset is the same as masking the other
experts at run time (Kimi-Linear-48B-A3B-Code-CMF listing, "How it was made",
step 3), so each masked result is checked against the oracle on the sliced
layer: router rows, bias and expert weights of the allowed experts only,
renumbered 0..n-1, with the oracle's ids mapped back to the full numbering.
The oracle's own mask-equals-slice pin is a CPU test.  The per-expert routing
frequencies (step 2 of the same listing) are checked against a bincount of the
selected ids, accumulated over two calls, and the kept set chosen from them
(moe_coverage_set, step 3) against the oracle's greedy choice.
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


def _keep_mask(E, n, seed):
    keep = np.sort(np.argsort(S.uniform(seed, 1, (E,), 0.0, 1.0))[:n]).astype(np.int64)
    m = np.zeros(E, np.uint8)
    m[keep] = 1
    return keep, m


def _sliced(inp, keep):
    ex = inp.experts
    exs = oracle.Experts(ex.fmt, ex.gu[keep], ex.dn[keep],
                         None if ex.gu_s is None else ex.gu_s[keep],
                         None if ex.dn_s is None else ex.dn_s[keep])
    wr = np.ascontiguousarray(inp.wr[keep])
    bias = None if inp.bias is None else np.ascontiguousarray(inp.bias[keep])
    return wr, bias, exs


def _remap(keep, E):
    r = np.full(E, -1, np.int64)
    r[keep] = np.arange(len(keep))
    return r


CASES = [
    # (router, E, k, kept, T, d, fmt)
    ("sigmoid_bias", 32, 4, 12, 5, 128, "int8_row"),        # small-batch tail path
    ("sigmoid_bias", 32, 4, 12, 40, 128, "int8_row"),       # 16-row decode tiles
    ("sigmoid_bias", 256, 8, 40, 300, 256, "int8_row"),     # grouped GEMM, 60 rows/expert
    ("sigmoid_bias", 300, 8, 8, 9, 256, "int4_b32"),        # E > 256, exactly k allowed
    ("softmax", 128, 8, 33, 24, 256, "int4_b32"),
    ("softmax", 40, 4, 9, 3, 64, "int8_row"),
    # one token, every expert set reading digits: the gate/up launch selects itself
    ("softmax", 128, 8, 33, 1, 256, "int4_b32"),
    ("softmax", 40, 4, 9, 1, 64, "int8_row"),
    ("sigmoid_bias", 64, 8, 20, 1, 128, "int8_row", "int8_row"),
]


@pytest.mark.parametrize("case", CASES)
def test_masked_layer_equals_oracle_on_slice(ctx, case):
    import torch
    from sparse_moe_expert_sigmoid_amd import MoELayer
    router, E, k, kept, T, d, fmt = case[:7]
    # shared expert: fp32 beside the sigmoid router unless the case names one
    shared = case[7] if len(case) > 7 else ("fp32" if router == "sigmoid_bias" else None)
    scale = 2.446 if router == "sigmoid_bias" else 1.0
    step = 128 if fmt == "int4_b32" else 64
    spec = S.spec("tiny", T=T, d=d, E=E, k=k, inter=step, router=router,
                  scale=float(np.float32(scale)), fmt=fmt, shared=shared,
                  shared_inter=step if shared else 0,
                  xseed=0x4D61534B + T, wseed=0x4D61534C + E)
    inp = S.make_layer(spec)
    keep, m = _keep_mask(E, kept, 0x4D61 + E)
    print(f"[mask] {router} E={E} k={k} kept={kept} T={T} d={d} {fmt}", flush=True)
    base = MoELayer.from_inputs(ctx, inp)
    md = _dev(m)
    L = base.with_mask(md)
    xd = _dev(inp.x)
    # oracle on the slice, ids mapped back
    wr_s, bias_s, ex_s = _sliced(inp, keep)
    sh = oracle.Experts.of(inp.shared) if inp.shared is not None else None
    oy, oidx_s, ow, ogap = oracle.layer(router, k, spec.scale, inp.x, wr_s, bias_s, ex_s, sh)
    _, _, _, logits = oracle.route(router, inp.x, wr_s, bias_s, k, spec.scale, want_logits=True)
    keys = oracle_keys(router, logits, bias_s)
    remap = _remap(keep, E)
    for fused in (False, True):
        y = L.forward_fused(xd) if fused else L(xd)
        torch.cuda.synchronize()
        gidx = L.idx.cpu().numpy()
        assert np.isin(gidx, keep).all(), "a masked expert was selected"
        exc = compare_route(remap[gidx].astype(np.int32), L.w.cpu().numpy(), oidx_s, ow, ogap,
                            keys, spec.scale)
        keepr = np.setdiff1d(np.arange(T), exc)
        ratio = compare_outputs(y.cpu().numpy(), oy, keepr)
        log_result(test="masked_layer", router=router, E=E, k=k, kept=kept, T=T, fmt=fmt,
                   fused=fused, excused=len(exc), err_over_max=ratio)
    # the unmasked layer does select outside the subset (the mask is doing work)
    base(xd)
    torch.cuda.synchronize()
    assert not np.isin(base.idx.cpu().numpy(), keep).all()


def test_masked_route_equals_sliced_route_bit_exact(ctx):
    # Sigmoid router: the mask and the sliced router give the same ids (mapped)
    # and the same fp32 weights, bit for bit: the logits are per-expert sums in
    # a fixed order and the weight sums run in slot order.
    import torch
    from sparse_moe_expert_sigmoid_amd import MoELayer
    for T in (4, 64):
        spec = S.spec("tiny", T=T, d=256, E=256, k=8, xseed=0x4D61535B + T)
        inp = S.make_layer(spec)
        keep, m = _keep_mask(256, 50, 0x4D62)
        L = MoELayer.from_inputs(ctx, inp)
        L.alloc(T)
        xd = _dev(inp.x)
        ctx.moe_route_masked(L.router, xd, L.w_router, L.bias, _dev(m), T, spec.d, 256, 8,
                             L.scale, L.idx, L.w, L.ws)
        torch.cuda.synchronize()
        gidx, gw = L.idx.cpu().numpy().copy(), L.w.cpu().numpy().copy()
        wr_s = _dev(inp.wr[keep])
        b_s = _dev(inp.bias[keep])
        idx_s = torch.empty((T, 8), dtype=torch.int32, device="cuda:0")
        w_s = torch.empty((T, 8), dtype=torch.float32, device="cuda:0")
        ctx.moe_route(L.router, xd, wr_s, b_s, T, spec.d, len(keep), 8, L.scale, idx_s, w_s, L.ws)
        torch.cuda.synchronize()
        assert np.array_equal(gidx, keep[idx_s.cpu().numpy()])
        assert np.array_equal(gw.view(np.uint32), w_s.cpu().numpy().view(np.uint32))


def test_mask_all_allowed_equals_unmasked(ctx):
    import torch
    from sparse_moe_expert_sigmoid_amd import MoELayer
    for name, T in (("tiny", 24), ("tiny", 3)):
        spec = S.spec(name, T=T, router="softmax", scale=1.0, shared=None, shared_inter=0,
                      xseed=0x4D61536B + T)
        inp = S.make_layer(spec)
        L = MoELayer.from_inputs(ctx, inp)
        xd = _dev(inp.x)
        y0 = L.forward_fused(xd).clone()
        i0 = L.idx.clone()
        Lm = L.with_mask(_dev(np.ones(spec.E, np.uint8)))
        y1 = Lm.forward_fused(xd)
        torch.cuda.synchronize()
        assert torch.equal(i0, Lm.idx) and torch.equal(y0, y1)


def test_fewer_allowed_than_k_stays_in_range(ctx):
    # Outside the contract (fewer than k allowed): the call still returns ids in
    # [0, E), the allowed experts first, the rest with weight 0.
    import torch
    from sparse_moe_expert_sigmoid_amd import MoELayer
    spec = S.spec("tiny", T=6, E=16, k=4, xseed=0x4D61537B)
    inp = S.make_layer(spec)
    L = MoELayer.from_inputs(ctx, inp)
    L.alloc(6)
    m = np.zeros(16, np.uint8)
    m[[3, 9]] = 1
    ctx.moe_route_masked(L.router, _dev(inp.x), L.w_router, L.bias, _dev(m), 6, spec.d, 16, 4,
                         L.scale, L.idx, L.w, L.ws)
    torch.cuda.synchronize()
    idx, w = L.idx.cpu().numpy(), L.w.cpu().numpy()
    assert ((idx >= 0) & (idx < 16)).all()
    for t in range(6):
        assert set(idx[t, :2]) == {3, 9}
        assert list(idx[t, 2:]) == [0, 1]
        assert (w[t, 2:] == 0).all() and np.isclose(w[t, :2].sum(), spec.scale, rtol=1e-6)


def test_expert_counts_accumulate(ctx):
    import torch
    E, k = 256, 8
    a = S.randint8(0x4D63, 1, (3001, k), 0, 127).astype(np.int32) * 2 + 1   # odd ids < 256
    b = np.asarray(S.uniform(0x4D63, 2, (17, k), 0, E), np.float64).astype(np.int32)
    b[0, 0], b[1, 1] = -1, E + 5                      # outside [0, E): not counted
    counts = torch.zeros(E, dtype=torch.int64, device="cuda:0")
    ctx.moe_expert_counts(_dev(a), a.shape[0], k, E, counts)
    ctx.moe_expert_counts(_dev(b), b.shape[0], k, E, counts)
    ctx.moe_expert_counts(_dev(b), 0, k, E, counts)   # T = 0: nothing
    torch.cuda.synchronize()
    bv = b[(b >= 0) & (b < E)]
    want = np.bincount(a.ravel(), minlength=E) + np.bincount(bv, minlength=E)
    assert np.array_equal(counts.cpu().numpy(), want)
    # E above 256 (several LDS words per thread) and many blocks
    E2 = 1000
    c = np.asarray(S.uniform(0x4D63, 3, (100003, 4), 0, E2), np.float64).astype(np.int32)
    counts2 = torch.zeros(E2, dtype=torch.int64, device="cuda:0")
    ctx.moe_expert_counts(_dev(c), c.shape[0], 4, E2, counts2)
    torch.cuda.synchronize()
    cv = c[(c >= 0) & (c < E2)]
    assert np.array_equal(counts2.cpu().numpy(), np.bincount(cv, minlength=E2))


def test_expert_counts_of_a_routed_batch(ctx):
    # the statistics the restriction is built from: counts of the ids the
    # router chose, equal to the oracle's selection counts
    import torch
    from sparse_moe_expert_sigmoid_amd import MoELayer
    spec = S.spec("tiny", T=200, E=64, k=6, xseed=0x4D61538B)
    inp = S.make_layer(spec)
    L = MoELayer.from_inputs(ctx, inp)
    L(_dev(inp.x))
    counts = torch.zeros(64, dtype=torch.int64, device="cuda:0")
    ctx.moe_expert_counts(L.idx, 200, 6, 64, counts)
    torch.cuda.synchronize()
    oidx, _, ogap = oracle.route(spec.router, inp.x, inp.wr, inp.bias, 6, spec.scale)
    if (ogap < 1e-6).any():
        pytest.skip("oracle near-tie in this draw")
    assert np.array_equal(counts.cpu().numpy(), np.bincount(oidx.ravel(), minlength=64))


def _tiny_stack(ctx, layers=3, T=256, d=256, E=64, k=6, inter=128):
    from sparse_moe_expert_sigmoid_amd import MoELayer, MoEStack
    out, inps = [], []
    for l in range(layers):
        spec = S.spec("tiny", T=T, d=d, E=E, k=k, inter=inter, shared="int8_row",
                      shared_inter=inter, wseed=0x4D615300 + l, xseed=0x4D6153F0)
        inp = S.make_layer(spec)
        # skewed selection bias, as the calibration statistics of a real model
        bias = S.zipf_bias(spec.wseed, E, 1.0)
        inp = S.LayerInputs(spec, inp.x, inp.wr, bias, inp.experts, inp.shared)
        inps.append(inp)
        out.append(MoELayer.from_inputs(ctx, inp))
    return MoEStack(ctx, out), inps


def test_coverage_set_matches_oracle(ctx):
    # moe_coverage_set against the oracle's greedy choice on random and
    # adversarial counts: ties (few distinct values), zeros, counts above 2^40,
    # covers 0 and 1, k above and below the set size, E up to the 1024 maximum
    from sparse_moe_expert_sigmoid_amd.restrict import coverage_set
    n = 0
    for trial in range(160):
        E = [1, 2, 7, 32, 128, 256, 300, 1000, 1024][trial % 9]
        hi = [0, 1, 3, 100, 127][trial % 5]
        c = S.randint8(0xC0FF, trial, (E,), 0, hi).astype(np.uint64)
        if trial % 11 == 0:
            c = c * np.uint64(1 << 40)                   # large counts
        cd = _dev(c.view(np.int64))
        for cover in (0.0, 0.3, 0.73, 0.95, 1.0):
            for k in (1, 8, 16):
                got = coverage_set(ctx, cd, cover, k)
                want = oracle.coverage_set(c, cover, k)
                assert np.array_equal(got, want), (trial, E, cover, k)
                n += 1
    log_result(test="coverage_set", cases=n)


def test_coverage_set_rejects_bad_arguments(ctx):
    import torch
    from sparse_moe_expert_sigmoid_amd import MoeError
    from sparse_moe_expert_sigmoid_amd.restrict import coverage_set
    c = torch.ones(4, dtype=torch.int64, device="cuda:0")
    for cover, k in ((1.2, 1), (-0.1, 1), (0.5, 0)):
        with pytest.raises(MoeError):
            coverage_set(ctx, c, cover, k)
    with pytest.raises(MoeError):
        coverage_set(ctx, torch.ones(1025, dtype=torch.int64, device="cuda:0"), 0.5, 1)
    with pytest.raises(ValueError):
        coverage_set(ctx, torch.ones(0, dtype=torch.int64, device="cuda:0"), 0.5, 1)


def test_restriction_from_recorded_counts(ctx):
    # Calibrate: run a batch through a 3-layer stack recording per-layer
    # counts; restrict each layer to the smallest set carrying 95% of its
    # selections; the sliced stack and the masked full stack then agree on
    # another batch (ids through the renumbering, outputs within the bound),
    # and layer 0 of the sliced stack matches the oracle on the slice.
    import torch
    stk, inps = _tiny_stack(ctx)
    E, k, T = 64, 6, 256
    x_cal = _dev(inps[0].x)
    counts = torch.zeros((3, E), dtype=torch.int64, device="cuda:0")
    stk.forward(x_cal, counts=counts)
    torch.cuda.synchronize()
    c = counts.cpu().numpy()
    for l in range(3):
        assert np.array_equal(c[l], np.bincount(stk.idx[l].cpu().numpy().ravel(), minlength=E))
    cut, keeps = stk.restricted(counts, 0.95)
    masked, keeps_m = stk.restricted(counts, 0.95, masked=True)
    for l in range(3):
        assert np.array_equal(keeps[l], oracle.coverage_set(c[l], 0.95, k))
        assert np.array_equal(keeps[l], keeps_m[l])
        assert k <= len(keeps[l]) < E
    x = S.normal(0x4D6153F1, 1, (T, 256), 1.0)
    xd = _dev(x)
    y_cut = cut.forward(xd).clone()
    idx_cut = [i.cpu().numpy() for i in cut.idx]
    y_mask = masked.forward(xd).clone()
    torch.cuda.synchronize()
    assert np.array_equal(keeps[0][idx_cut[0]], masked.idx[0].cpu().numpy())
    a, b = y_cut.cpu().numpy(), y_mask.cpu().numpy()
    err = float(np.abs(a - b).max()) / float(np.abs(b).max())
    assert err <= 2e-3
    # layer 0 of the cut stack against the oracle on the slice
    inp = inps[0]
    keep = keeps[0]
    exs = oracle.Experts(inp.experts.fmt, inp.experts.gu[keep], inp.experts.dn[keep],
                         inp.experts.gu_s[keep], inp.experts.dn_s[keep])
    wr_s, b_s = np.ascontiguousarray(inp.wr[keep]), np.ascontiguousarray(inp.bias[keep])
    oy, oidx, ow, ogap = oracle.layer("sigmoid_bias", k, inp.spec.scale, x, wr_s, b_s, exs,
                                      oracle.Experts.of(inp.shared))
    _, _, _, logits = oracle.route("sigmoid_bias", x, wr_s, b_s, k, inp.spec.scale,
                                   want_logits=True)
    cut0 = cut.layers[0]
    y0 = cut0.forward_fused(xd)
    torch.cuda.synchronize()
    exc = compare_route(cut0.idx.cpu().numpy(), cut0.w.cpu().numpy(), oidx, ow, ogap,
                        oracle_keys("sigmoid_bias", logits, b_s), inp.spec.scale)
    ratio = compare_outputs(y0.cpu().numpy(), oy, np.setdiff1d(np.arange(T), exc))
    log_result(test="restriction", kept=[len(kp) for kp in keeps], cut_vs_masked=err,
               bit_identical=bool(np.array_equal(a, b)), layer0_err_over_max=ratio)
