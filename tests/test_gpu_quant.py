"""GPU: the weight quantizers (moe_quantize) against the oracle's, bit for bit.

Codes and scales are integers and fp32 values decided by fp32 arithmetic, so
both sides take the same decisions and must agree exactly (codes, and scale
bit patterns).  Inputs: seeded normal weights in fp32 and in bf16, plus rows
built to hit every rule: exact halfway quotients (rounded away from zero),
all-zero rows, a negative largest magnitude, int4 blocks below the 2^-14
floor, rows short enough to sit in registers and long enough to be read
twice, and ragged row counts.  At the full Kimi-shaped expert set the output
is checked on sampled experts.
"""
import numpy as np
import pytest

import oracle
from sparse_moe_expert_sigmoid_amd import synth as S

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ctx(gpu):
    from sparse_moe_expert_sigmoid_amd import Context
    return Context(0)


def _special_rows(K, fmt, seed):
    """Rows whose quotients are exact halves, zeros, a negative maximum, and
    (int4) blocks under the scale floor."""
    rows = []
    u = 2.0 ** -9
    qmax = 127 if fmt == "int8_row" else 7
    n = S.randint8(seed, 1, (K,), -qmax + 1, qmax - 2).astype(np.float64)
    r = (n + 0.5) * u                                   # every quotient an exact half
    if fmt == "int8_row":
        r[K // 3] = qmax * u                            # the row maximum: s = u exactly
    else:
        r[0::32] = qmax * u                             # each block's maximum
    rows.append(r)
    rows.append(-r)                                     # negative maxima, negative halves
    rows.append(np.zeros(K))
    t = S.normal(seed, 2, (K,), 1.0).astype(np.float64) * 2.0 ** -17   # below 7 * 2^-14
    rows.append(t)
    m = S.normal(seed, 3, (K,), 1.0).astype(np.float64)
    m[::7] = 0.0
    rows.append(m)
    return np.asarray(rows, np.float32)


def _unpack_i4(b, K):
    b = b.astype(np.uint8)
    lo = (b & 0xF).astype(np.int8)
    hi = (b >> 4).astype(np.int8)
    q = np.empty(b.shape[:-1] + (K,), np.int8)
    q[..., 0::2] = np.where(lo > 7, lo - 16, lo)
    q[..., 1::2] = np.where(hi > 7, hi - 16, hi)
    return q


def _run(ctx, fmt, w32, dtype):
    """GPU quantizer on w (fp32 values; bf16 input if dtype == 'bf16')."""
    import torch
    from sparse_moe_expert_sigmoid_amd import binding as B
    rows, K = w32.shape
    if dtype == "bf16":
        bits = S.bf16_bits(w32)
        wv = oracle.bf16_to_f32(bits)                   # the values the GPU reads
        wd = torch.from_numpy(bits.view(np.int16)).to("cuda:0").view(torch.bfloat16)
    else:
        wv = w32
        wd = torch.from_numpy(np.ascontiguousarray(w32)).to("cuda:0")
    f = B.MOE_W_INT8_ROW if fmt == "int8_row" else B.MOE_W_INT4_B32
    if fmt == "int8_row":
        codes = torch.empty((rows, K), dtype=torch.int8, device="cuda:0")
        scales = torch.empty(rows, dtype=torch.float32, device="cuda:0")
    else:
        codes = torch.empty((rows, K // 2), dtype=torch.uint8, device="cuda:0")
        scales = torch.empty((rows, K // 32), dtype=torch.float32, device="cuda:0")
    ctx.moe_quantize(f, wd.reshape(rows, K), codes, scales)
    torch.cuda.synchronize()
    q = codes.cpu().numpy()
    if fmt == "int4_b32":
        q = _unpack_i4(q, K)
    return wv, q, scales.cpu().numpy()


def _check(ctx, fmt, w32, dtype):
    wv, q, s = _run(ctx, fmt, w32, dtype)
    oq, os_ = oracle.quantize(fmt, wv)
    bad = np.argwhere(q != oq)
    assert bad.size == 0, f"{len(bad)} codes differ, first at {bad[0]}: {q[tuple(bad[0])]} " \
                          f"vs {oq[tuple(bad[0])]}"
    assert np.array_equal(s.view(np.uint32), os_.view(np.uint32))
    return q, s


SHAPES_I8 = [(37, 8), (5, 2304), (130, 520), (3, 4096), (2, 4104), (3, 16384), (9, 768)]
SHAPES_I4 = [(41, 32), (7, 2048), (130, 544), (3, 16384), (5, 768)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("rows,K", SHAPES_I8)
def test_quantize_int8_matches_oracle(ctx, rows, K, dtype):
    print(f"[quant] int8 rows={rows} K={K} {dtype}", flush=True)
    w = S.normal(0x51A0 + K, rows, (rows, K), 0.02)
    w = np.concatenate([w, _special_rows(K, "int8_row", 0x51B0 + K)])
    q, s = _check(ctx, "int8_row", w, dtype)
    assert (s[rows + 2] == 0) and (q[rows + 2] == 0).all()     # the zero row
    if dtype == "f32":                                          # halves went away from zero
        assert np.array_equal(np.abs(q[rows]), np.abs(q[rows + 1]))
        assert (q[rows] == -q[rows + 1]).all()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("rows,K", SHAPES_I4)
def test_quantize_int4_matches_oracle(ctx, rows, K, dtype):
    print(f"[quant] int4 rows={rows} K={K} {dtype}", flush=True)
    w = S.normal(0x51C0 + K, rows, (rows, K), 0.02)
    w = np.concatenate([w, _special_rows(K, "int4_b32", 0x51D0 + K)])
    q, s = _check(ctx, "int4_b32", w, dtype)
    assert (s[rows + 3] == np.float32(2.0 ** -14)).all()       # every block under the floor
    assert (s[rows + 2] == np.float32(2.0 ** -14)).all() and (q[rows + 2] == 0).all()


def test_quantize_empty_and_errors(ctx):
    import torch
    from sparse_moe_expert_sigmoid_amd import binding as B
    w = torch.zeros((0, 64), dtype=torch.float32, device="cuda:0")
    c = torch.empty((0, 64), dtype=torch.int8, device="cuda:0")
    s = torch.empty(0, dtype=torch.float32, device="cuda:0")
    ctx.moe_quantize(B.MOE_W_INT8_ROW, w, c, s)                # rows = 0: no-op
    w = torch.zeros((4, 48), dtype=torch.float32, device="cuda:0")
    c = torch.empty((4, 48), dtype=torch.int8, device="cuda:0")
    s = torch.empty(4 * 2, dtype=torch.float32, device="cuda:0")
    with pytest.raises(B.MoeError) as e:
        ctx.moe_quantize(B.MOE_W_INT4_B32, w, c, s)            # 48 is not a multiple of 32
    assert e.value.status == B.MOE_E_UNSUPPORTED and "multiple of 32" in str(e.value)
    with pytest.raises(B.MoeError) as e:
        ctx.moe_quantize(B.MOE_W_FP32, w, c, s)
    assert e.value.status == B.MOE_E_UNSUPPORTED
    with pytest.raises(B.MoeError) as e:
        ctx.moe_quantize(B.MOE_W_INT8_ROW, w[:, 1:45], c, s)  # misaligned and K=44
    assert e.value.status in (B.MOE_E_UNSUPPORTED, B.MOE_E_INVALID)


def test_quantized_experts_run_through_the_layer(ctx):
    # Quantize float experts on the GPU, tile them, and run the layer: the same
    # as the oracle's layer on the oracle's quantization of the same floats.
    import torch
    from sparse_moe_expert_sigmoid_amd import DeviceExperts, MoELayer, binding as B
    from tests.parity import compare_outputs
    for fmt in ("int8_row", "int4_b32"):
        spec = S.spec("tiny", T=40, d=256, E=12, k=4, inter=128, fmt=fmt, shared=None,
                      shared_inter=0)
        inp = S.make_layer(spec)
        E, d, I = spec.E, spec.d, spec.inter
        gu = np.stack([S.float_expert(spec, e, "gu") for e in range(E)])
        dn = np.stack([S.float_expert(spec, e, "dn") for e in range(E)])
        f = B.MOE_W_INT8_ROW if fmt == "int8_row" else B.MOE_W_INT4_B32
        per = 1 if fmt == "int8_row" else 2
        gud, dnd = torch.from_numpy(gu).to("cuda:0"), torch.from_numpy(dn).to("cuda:0")
        cg = torch.empty((E, 2 * I, d // per), dtype=torch.int8 if per == 1 else torch.uint8,
                         device="cuda:0")
        cd = torch.empty((E, d, I // per), dtype=cg.dtype, device="cuda:0")
        sg = torch.empty((E, 2 * I) + (() if per == 1 else (d // 32,)), dtype=torch.float32,
                         device="cuda:0")
        sd = torch.empty((E, d) + (() if per == 1 else (I // 32,)), dtype=torch.float32,
                         device="cuda:0")
        ctx.moe_quantize(f, gud.reshape(E * 2 * I, d), cg.reshape(E * 2 * I, -1), sg)
        ctx.moe_quantize(f, dnd.reshape(E * d, I), cd.reshape(E * d, -1), sd)
        ex = DeviceExperts(f, E, d, I, cg, cd, sg, sd).tiled(ctx)
        L = MoELayer(ctx, spec.router, spec.k, spec.scale,
                     torch.from_numpy(inp.wr).to("cuda:0"),
                     torch.from_numpy(inp.bias).to("cuda:0"), ex)
        y = L.forward_fused(torch.from_numpy(inp.x).to("cuda:0"))
        torch.cuda.synchronize()
        qg, qsg = oracle.quantize(fmt, gu.reshape(E * 2 * I, d))
        qd, qsd = oracle.quantize(fmt, dn.reshape(E * d, I))
        shp = (lambda a, n: a.reshape(E, n)) if per == 1 else (lambda a, n: a.reshape(E, n, -1))
        oex = oracle.Experts(fmt, qg.reshape(E, 2 * I, d), qd.reshape(E, d, I), shp(qsg, 2 * I),
                             shp(qsd, d))
        oy, oidx, _, ogap = oracle.layer(spec.router, spec.k, spec.scale, inp.x, inp.wr,
                                         inp.bias, oex)
        keep = np.nonzero(ogap >= 1e-6)[0]
        assert np.array_equal(L.idx.cpu().numpy()[keep], oidx[keep])
        compare_outputs(y.cpu().numpy(), oy, keep)


@pytest.mark.parametrize("name,fmt", [("kimi_decode", "int8_row"), ("qwen_decode", "int4_b32")])
def test_quantize_full_expert_set_sampled(ctx, name, fmt):
    # The whole routed expert set of the layer from bf16 in two launches (the
    # benchmarked configuration); sampled experts checked bit for bit.
    import torch
    from sparse_moe_expert_sigmoid_amd import binding as B
    spec = S.spec(name)
    E, d, I = spec.E, spec.d, spec.inter
    per = 1 if fmt == "int8_row" else 2
    f = B.MOE_W_INT8_ROW if fmt == "int8_row" else B.MOE_W_INT4_B32
    print(f"[quant] full {name} {fmt}: uploading bf16 weights", flush=True)
    gu = torch.empty((E, 2 * I, d), dtype=torch.bfloat16, device="cuda:0")
    dn = torch.empty((E, d, I), dtype=torch.bfloat16, device="cuda:0")
    for e in range(E):
        gu[e] = torch.from_numpy(S.bf16_bits(S.float_expert(spec, e, "gu")).view(np.int16)) \
            .view(torch.bfloat16)
        dn[e] = torch.from_numpy(S.bf16_bits(S.float_expert(spec, e, "dn")).view(np.int16)) \
            .view(torch.bfloat16)
    cdt = torch.int8 if per == 1 else torch.uint8
    cg = torch.empty((E * 2 * I, d // per), dtype=cdt, device="cuda:0")
    cd = torch.empty((E * d, I // per), dtype=cdt, device="cuda:0")
    sg = torch.empty((E * 2 * I,) + (() if per == 1 else (d // 32,)), dtype=torch.float32,
                     device="cuda:0")
    sd = torch.empty((E * d,) + (() if per == 1 else (I // 32,)), dtype=torch.float32,
                     device="cuda:0")
    ctx.moe_quantize(f, gu.reshape(E * 2 * I, d), cg, sg)
    ctx.moe_quantize(f, dn.reshape(E * d, I), cd, sd)
    torch.cuda.synchronize()
    for e in (0, E // 2 + 3, E - 1):
        for part, c, s, n, K in (("gu", cg, sg, 2 * I, d), ("dn", cd, sd, d, I)):
            wv = oracle.bf16_to_f32(S.bf16_bits(S.float_expert(spec, e, part)))
            oq, os_ = oracle.quantize(fmt, wv)
            q = c[e * n:(e + 1) * n].cpu().numpy()
            if per == 2:
                q = _unpack_i4(q, K)
            assert np.array_equal(q, oq), (e, part)
            assert np.array_equal(s[e * n:(e + 1) * n].cpu().numpy().view(np.uint32),
                                  os_.view(np.uint32)), (e, part)
    del gu, dn, cg, cd
    torch.cuda.empty_cache()
