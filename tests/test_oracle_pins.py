"""Pins for the CPU oracle: checks against what the pages and mathematics fix.

None of these compares the oracle with itself.  Each test names the mistake
it would catch.  Sources: the Kimi-Linear LiteRT-LM DETAILS.md (Conversion
notes: the mixture-of-experts and int8-quantization bullets), the Qwen3-30B-A3B
LiteRT model card (Available Artifacts; Conversion Notes), and the
Kimi-Linear Code-CMF listing (How it was made, steps 2-3).
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from sparse_moe_expert_sigmoid_amd import synth as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
K_SCALE = float(np.float32(2.446))


def silu(z):
    return z / (1.0 + math.exp(-z))


# ---------------------------------------------------------------- generator

def test_splitmix64_published_vector():
    # SplitMix64 from state 1234567 (the reference implementation's test vector).
    assert list(S.splitmix64(1234567, 5)) == [
        6457827717110365317, 3203168211198807973, 9817491932198370423,
        4593380528125082431, 16408922859458223821]


def test_generator_ranges_and_determinism():
    a = S.randint8(7, 4, (200000,), -127, 127)
    assert a.min() == -127 and a.max() == 127
    b = S.randint8(7, 4, (200000,), -8, 7)
    assert b.min() == -8 and b.max() == 7
    assert np.array_equal(a, S.randint8(7, 4, (200000,), -127, 127))
    u = S.uniform(7, 3, (100000,), -0.1, 0.1)
    assert u.min() >= -0.1 and u.max() < 0.1
    z = S.normal(7, 1, (200000,), 1.0)
    assert abs(z.mean()) < 0.01 and abs(z.std() - 1.0) < 0.01
    s = S.scales(7, 5, (1 << 16,), 1.0 / (8 * math.sqrt(2048)), special_tid=12)
    assert np.count_nonzero(s == S.TWO_M14) > 20
    assert np.count_nonzero(s < S.TWO_M14) > 20
    codes = S.randint8(1, 1, (4, 64), -8, 7)
    p = S.pack_int4(codes)
    lo = (p & 0x0F).astype(np.int16)
    hi = (p >> 4).astype(np.int16)
    lo[lo > 7] -= 16
    hi[hi > 7] -= 16
    assert np.array_equal(lo, codes[:, 0::2]) and np.array_equal(hi, codes[:, 1::2])


# ---------------------------------------------------------------- golden case

def _golden():
    with open(os.path.join(GOLDEN, "tiny_sigmoid_int8.json")) as f:
        return json.load(f)


def test_golden_tiny_sigmoid_int8_closed_form():
    g = _golden()
    experts = oracle.Experts("int8_row",
                             np.array(g["gu_codes"], np.int8), np.array(g["dn_codes"], np.int8),
                             np.array(g["gu_scales"], np.float32),
                             np.array(g["dn_scales"], np.float32))
    shared = oracle.Experts("fp32", np.array(g["shared_gu"], np.float32),
                            np.array(g["shared_dn"], np.float32))
    y, idx, w, gap = oracle.layer("sigmoid_bias", g["k"], K_SCALE, np.array(g["x"], np.float32),
                                  np.array(g["wr"], np.float32),
                                  np.array(g["bias"], np.float32), experts, shared)
    assert idx.tolist() == g["expected_idx"]
    assert np.allclose(gap, g["expected_gap"], rtol=0, atol=1e-7)
    wj = 0.5 / 1.0 * K_SCALE
    assert np.allclose(w, wj, rtol=1e-15, atol=0)
    # token 0
    h1 = silu(2.0) * 1.5
    h3 = silu(0.25) * 0.5
    hs = silu(0.5) * 0.5
    y0 = [wj * h1 + wj * 1.5 * h3 + 2 * hs, wj * (-0.5 * h1) + wj * 2 * h3 - hs]
    # token 1
    h3b = silu(-1.0) * 2.0
    y1 = [wj * 1.5 * h3b, wj * 2 * h3b]
    assert np.allclose(y, [y0, y1], rtol=1e-14, atol=1e-15)


# ---------------------------------------------------------------- brute force

def _dense_reference(router, k, scale, x, wr, bias, ex, sh):
    """Dense-gated definition: every expert on every token, gate zero unless
    selected.  Independent code: numpy matmuls, full sort for selection."""
    x64 = x.astype(np.float64)
    logits = x64 @ wr.astype(np.float64).T                      # [T, E]
    T, E = logits.shape
    if router == "sigmoid_bias":
        s = 1.0 / (1.0 + np.exp(-logits))
        key = (s + (bias.astype(np.float64) if bias is not None else 0.0)).astype(np.float32)
    else:
        m = logits.max(axis=1, keepdims=True)
        p = np.exp(logits - m)
        s = p / p.sum(axis=1, keepdims=True)
        key = s.astype(np.float32)
    G = np.zeros((T, E))
    idx = np.zeros((T, k), np.int64)
    for t in range(T):
        order = np.lexsort((np.arange(E), -key[t].astype(np.float64)))  # key desc, index asc
        sel = order[:k]
        idx[t] = sel
        G[t, sel] = scale * s[t, sel] / s[t, sel].sum()

    def deq(mat, sc, fmt):
        if fmt == "fp32":
            return mat.astype(np.float64)
        if fmt == "int8_row":
            return mat.astype(np.float64) * sc.astype(np.float64)[..., None]
        sc = np.maximum(sc.astype(np.float64), 2.0 ** -14)
        return mat.astype(np.float64) * np.repeat(sc, 32, axis=-1)

    def all_experts(w):
        gu = deq(w.gu, w.gu_s, w.fmt)            # [E, 2I, d]
        dn = deq(w.dn, w.dn_s, w.fmt)            # [E, d, I]
        I = gu.shape[1] // 2
        gate = np.einsum("end,td->ten", gu[:, :I], x64)
        up = np.einsum("end,td->ten", gu[:, I:], x64)
        h = gate / (1.0 + np.exp(-gate)) * up
        return np.einsum("emn,ten->tem", dn, h)   # [T, E, d]

    y = np.einsum("te,ted->td", G, all_experts(ex))
    if sh is not None:
        y = y + all_experts(sh)[:, 0]
    return y, idx, G


@pytest.mark.parametrize("router,fmt,shared", [
    ("sigmoid_bias", "int8_row", "fp32"),
    ("sigmoid_bias", "int8_row", "int8_row"),
    ("softmax", "int4_b32", None),
    ("sigmoid_bias", "fp32", None),
])
def test_sparse_equals_dense_gating_bruteforce(router, fmt, shared):
    # Only the k routed experts are computed per token (Qwen3 card, Conversion
    # Notes): the sparse result must equal the dense sum with zero gates.
    T, d, E, k, I = 12, 64, 10, 4, 32
    scale = K_SCALE if router == "sigmoid_bias" else 1.0
    seed = 99
    x = S.normal(seed, 1, (T, d), 1.0)
    wr = S.normal(seed, 2, (E, d), 1.0 / math.sqrt(d))
    bias = S.uniform(seed, 3, (E,), -0.1, 0.1) if router == "sigmoid_bias" else None
    ex = S.make_experts(fmt, E, d, I, seed, (4, 5, 6, 7, 12, 13))
    sh = S.make_experts(shared, 1, d, 32, seed, (8, 9, 10, 11, 14, 15)) if shared else None
    y, idx, w, gap = oracle.layer(router, k, scale, x, wr, bias, oracle.Experts.of(ex),
                                  oracle.Experts.of(sh) if sh else None)
    yd, idxd, G = _dense_reference(router, k, scale, x, wr, bias, ex, sh)
    assert np.array_equal(idx, idxd)
    for t in range(T):
        assert np.allclose(w[t], G[t, idx[t]], rtol=1e-14, atol=0)
    assert np.allclose(y, yd, rtol=1e-12, atol=1e-12 * np.abs(yd).max())


# ---------------------------------------------------------------- router

def _router_inputs(seed=5, T=64, d=128, E=32):
    x = S.normal(seed, 1, (T, d), 1.0)
    wr = S.normal(seed, 2, (E, d), 1.0 / math.sqrt(d))
    bias = S.uniform(seed, 3, (E,), -0.1, 0.1)
    return x, wr, bias


def test_selection_is_full_sort_of_keys_and_gap():
    x, wr, bias = _router_inputs()
    k = 8
    idx, w, gap, logits = oracle.route("sigmoid_bias", x, wr, bias, k, K_SCALE, want_logits=True)
    s = 1.0 / (1.0 + np.exp(-logits))
    key = (s + bias.astype(np.float64)).astype(np.float32)
    for t in range(x.shape[0]):
        order = np.argsort(-key[t], kind="stable")   # descending, ties keep lower index first
        assert idx[t].tolist() == order[:k].tolist()
        assert gap[t] == float(key[t, order[k - 1]]) - float(key[t, order[k]])
        assert gap[t] >= 0


def test_logits_are_the_plain_dot_products():
    x, wr, bias = _router_inputs()
    _, _, _, logits = oracle.route("sigmoid_bias", x, wr, bias, 8, K_SCALE, want_logits=True)
    ref = x.astype(np.float64) @ wr.astype(np.float64).T
    assert np.allclose(logits, ref, rtol=1e-13, atol=1e-13)


def test_sigmoid_weights_sum_to_scale_and_use_raw_scores():
    # Weights renormalised then scaled by 2.446: sum is 2.446 and each weight
    # is proportional to sigmoid(l) (not to sigmoid(l) + b).
    x, wr, bias = _router_inputs()
    idx, w, gap, logits = oracle.route("sigmoid_bias", x, wr, bias, 8, K_SCALE, want_logits=True)
    assert np.all(w > 0)
    assert np.allclose(w.sum(1), K_SCALE, rtol=1e-14)
    s = 1.0 / (1.0 + np.exp(-np.take_along_axis(logits, idx, 1)))
    assert np.allclose(w, K_SCALE * s / s.sum(1, keepdims=True), rtol=1e-13)


def test_softmax_weights_are_softmax_of_selected_logits():
    x, wr, _ = _router_inputs()
    idx, w, gap, logits = oracle.route("softmax", x, wr, None, 8, 1.0, want_logits=True)
    assert np.allclose(w.sum(1), 1.0, rtol=1e-14)
    sel = np.take_along_axis(logits, idx, 1)
    ref = np.exp(sel - sel.max(1, keepdims=True))
    ref /= ref.sum(1, keepdims=True)
    assert np.allclose(w, ref, rtol=1e-12)
    # selection on probabilities = selection on logits (softmax is monotone)
    for t in range(x.shape[0]):
        assert set(idx[t]) == set(np.argsort(-logits[t], kind="stable")[:8])


def test_zero_bias_selects_top_scores():
    x, wr, _ = _router_inputs()
    E = wr.shape[0]
    idx, w, gap, logits = oracle.route("sigmoid_bias", x, wr, np.zeros(E, np.float32), 8,
                                       K_SCALE, want_logits=True)
    for t in range(x.shape[0]):
        assert set(idx[t]) == set(np.argsort(-logits[t], kind="stable")[:8])


def test_bias_forces_selection_but_not_weights():
    # The correction bias only steers selection (CMF listing: "noaux selection
    # bias"; DETAILS.md: top 8 on scores plus bias, weights from the scores).
    x, wr, bias = _router_inputs()
    E = wr.shape[0]
    chosen = np.array([3, 7, 8, 15, 16, 22, 29, 31])
    b1 = bias.copy()
    b1[chosen] = 1.0                      # sigmoid < 1, so these 8 always win
    idx1, w1, _ = oracle.route("sigmoid_bias", x, wr, b1, 8, K_SCALE)
    b2 = S.uniform(17, 3, (E,), -0.1, 0.1)
    b2[chosen] = 1.0
    idx2, w2, _ = oracle.route("sigmoid_bias", x, wr, b2, 8, K_SCALE)
    for t in range(x.shape[0]):
        assert set(idx1[t]) == set(chosen)
        assert idx1[t].tolist() == idx2[t].tolist()
    assert np.array_equal(w1, w2)


def test_ties_go_to_lower_index():
    T, d, E = 3, 8, 12
    x = np.ones((T, d), np.float32)
    wr = np.zeros((E, d), np.float32)          # all scores 0.5
    bias = np.zeros(E, np.float32)
    bias[[2, 9]] = 0.25
    idx, w, gap = oracle.route("sigmoid_bias", x, wr, bias, 5, K_SCALE)
    assert idx.tolist() == [[2, 9, 0, 1, 3]] * T
    assert np.allclose(gap, 0.0)
    assert np.allclose(w, K_SCALE / 5, rtol=1e-15)


def test_all_experts_selected_when_k_equals_E():
    x, wr, bias = _router_inputs(E=8)
    idx, w, gap, logits = oracle.route("sigmoid_bias", x, wr, bias, 8, K_SCALE, want_logits=True)
    for t in range(x.shape[0]):
        assert sorted(idx[t]) == list(range(8))
    assert np.all(np.isinf(gap))
    s = 1.0 / (1.0 + np.exp(-logits))
    assert np.allclose(np.take_along_axis(w, np.argsort(idx, 1), 1),
                       K_SCALE * s / s.sum(1, keepdims=True), rtol=1e-13)


# ---------------------------------------------------------------- permutation

def test_permute_is_stable_counting_sort():
    rng_idx = np.stack([np.argsort(S.uniform(3, 50 + t, (40,), 0, 1))[:8] for t in range(37)])
    idx = rng_idx.astype(np.int32)
    E = 40
    offsets, row_token, token_row = oracle.permute(idx, E)
    flat = idx.ravel()
    order = np.argsort(flat, kind="stable")
    assert np.array_equal(row_token, order // 8)
    inv = np.empty_like(order)
    inv[order] = np.arange(order.size)
    assert np.array_equal(token_row, inv)
    assert np.array_equal(offsets, np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))]))


# ---------------------------------------------------------------- dequantisation

def _one_hot_down(d, I, perm):
    dn = np.zeros((1, d, I), np.int8)
    for m in range(d):
        dn[0, m, perm[m]] = 1
    return dn


def test_int8_row_dequant_integer_exact():
    # w = q * s[row] (one scale per output row and expert): with power-of-two
    # scales and small integers, gate and up sums are exact.
    d, I = 8, 4
    x = np.array([1, -2, 3, 0, 1, 1, -1, 2], np.float32)
    gu = np.zeros((1, 2 * I, d), np.int8)
    gu[0, :, :] = np.arange(2 * I * d).reshape(2 * I, d) % 7 - 3
    gu_s = np.array([[0.5, 0.25, 2.0, 1.0, 0.125, 1.0, 0.5, 4.0]], np.float32)
    perm = [0, 1, 2, 3, 0, 1, 2, 3]
    dn = _one_hot_down(d, I, perm)
    dn_s = np.ones((1, d), np.float32)
    out = oracle.ffn(oracle.Experts("int8_row", gu, dn, gu_s, dn_s), 0, x)
    q = gu[0].astype(np.int64) @ x.astype(np.int64)              # exact integers
    g = q[:I] * gu_s[0, :I].astype(np.float64)
    u = q[I:] * gu_s[0, I:].astype(np.float64)
    h = [silu(g[n]) * u[n] for n in range(I)]
    assert np.allclose(out, [h[p] for p in perm], rtol=1e-15, atol=0)


def test_int8_down_uses_row_scale_of_output():
    d, I = 4, 2
    x = np.array([1, 0, 0, 0], np.float32)
    gu = np.zeros((1, 4, d), np.int8)
    gu[0, 0, 0] = 3      # gate 0 = 3
    gu[0, 1, 0] = -2     # gate 1 = -2
    gu[0, 2, 0] = 1      # up 0 = 1
    gu[0, 3, 0] = 5      # up 1 = 5
    gu_s = np.ones((1, 4), np.float32)
    dn = np.array([[[1, 0], [0, 1], [2, 3], [-1, 1]]], np.int8)
    dn_s = np.array([[1.0, 0.5, 0.25, 8.0]], np.float32)
    out = oracle.ffn(oracle.Experts("int8_row", gu, dn, gu_s, dn_s), 0, x)
    h0, h1 = silu(3.0) * 1, silu(-2.0) * 5
    ref = [h0, 0.5 * h1, 0.25 * (2 * h0 + 3 * h1), 8.0 * (-h0 + h1)]
    assert np.allclose(out, ref, rtol=1e-15)


def test_int4_block_scales_along_input_and_clamp():
    # int4 blockwise, block 32 along the input, fp32 scales; scales below
    # 2^-14 are raised to 2^-14 (Qwen3 card, Conversion Notes).
    d, I = 64, 32
    x = np.ones(d, np.float32)
    gu = np.zeros((1, 2 * I, d), np.int8)
    gu[0, :, :32] = 1
    gu[0, :, 32:] = -1
    f = 2.0 ** -14
    cases = [(2.0 ** -3, 2.0 ** -5), (2.0 ** -3, 0.0), (2.0 ** -3, 1e-40),
             (2.0 ** -3, 2.0 ** -20), (2.0 ** -3, 0.999 * f), (2.0 ** -3, f), (1.0, 2.0 ** -13)]
    gu_s = np.ones((1, 2 * I, 2), np.float32)
    for n, (s0, s1) in enumerate(cases):
        gu_s[0, n] = (s0, s1)
        gu_s[0, I + n] = (1.0, 0.0)            # up row n = 32*1 - 32*2^-14
    perm = list(range(I)) * 2
    dn = _one_hot_down(d, I, perm)
    dn_s = np.ones((1, d, 1), np.float32)
    out = oracle.ffn(oracle.Experts("int4_b32", gu, dn, gu_s, dn_s), 0, x)
    u = 32.0 - 32.0 * f
    for n, (s0, s1) in enumerate(cases):
        eff1 = max(float(np.float32(s1)), f)
        g = 32.0 * s0 - 32.0 * eff1
        assert out[n] == pytest.approx(silu(g) * u, rel=1e-15, abs=0)
    assert out[1] == pytest.approx(silu(4.0 - 32 * f) * u, rel=1e-15)
    # the clamp touches the down projection's scales too
    dn_s0 = np.zeros((1, d, 1), np.float32)
    out0 = oracle.ffn(oracle.Experts("int4_b32", gu, dn, gu_s, dn_s0), 0, x)
    assert np.allclose(out0, out * f, rtol=1e-15)


def test_silu_identities():
    # silu(z) - silu(-z) = z; silu(0) = 0; sigmoid(0) = 1/2.
    for z in [0.0, 1e-8, 0.3, 1.0, 2.5, 10.0, 30.0]:
        assert oracle.silu(z) - oracle.silu(-z) == pytest.approx(z, rel=1e-15, abs=1e-300)
    assert oracle.silu(0.0) == 0.0
    assert oracle.sigmoid(0.0) == 0.5
    assert oracle.silu(50.0) == 50.0
    assert 0 > oracle.silu(-50.0) > -1e-19


# ---------------------------------------------------------------- invariances

def _tiny_layer(seed=11, T=24, d=64, E=16, k=4, I=32):
    x = S.normal(seed, 1, (T, d), 1.0)
    wr = S.normal(seed, 2, (E, d), 1.0 / math.sqrt(d))
    bias = S.uniform(seed, 3, (E,), -0.1, 0.1)
    ex = S.make_experts("int8_row", E, d, I, seed, (4, 5, 6, 7, 12, 13))
    sh = S.make_experts("int8_row", 1, d, I, seed, (8, 9, 10, 11, 14, 15))
    return x, wr, bias, ex, sh, k


def test_expert_mask_equals_slice_bit_identical():
    # CMF listing, step 3: restricting to an expert subset (renumbered dense
    # prefix, router rows and selection bias sliced) equals the runtime mask.
    x, wr, bias, ex, sh, k = _tiny_layer()
    E = wr.shape[0]
    keep = np.array([0, 2, 3, 5, 8, 9, 11, 14])
    bm = bias.copy()
    bm[np.setdiff1d(np.arange(E), keep)] = -np.inf
    ym, idxm, wm, _ = oracle.layer("sigmoid_bias", k, K_SCALE, x, wr, bm,
                                   oracle.Experts.of(ex), oracle.Experts.of(sh))
    exs = oracle.Experts("int8_row", ex.gu[keep], ex.dn[keep], ex.gu_s[keep], ex.dn_s[keep])
    ys, idxs, ws, _ = oracle.layer("sigmoid_bias", k, K_SCALE, x, np.ascontiguousarray(wr[keep]),
                                   np.ascontiguousarray(bias[keep]), exs, oracle.Experts.of(sh))
    assert np.array_equal(idxm, keep[idxs])
    assert np.array_equal(wm, ws)
    assert np.array_equal(ym, ys)


def test_token_permutation_permutes_outputs_bit_exactly():
    x, wr, bias, ex, sh, k = _tiny_layer()
    perm = np.argsort(S.uniform(4, 4, (x.shape[0],), 0, 1))
    y, idx, w, gap = oracle.layer("sigmoid_bias", k, K_SCALE, x, wr, bias,
                                  oracle.Experts.of(ex), oracle.Experts.of(sh))
    yp, idxp, wp, gapp = oracle.layer("sigmoid_bias", k, K_SCALE, np.ascontiguousarray(x[perm]),
                                      wr, bias, oracle.Experts.of(ex), oracle.Experts.of(sh))
    assert np.array_equal(yp, y[perm]) and np.array_equal(idxp, idx[perm])
    assert np.array_equal(wp, w[perm]) and np.array_equal(gapp, gap[perm])


def test_layer_equals_staged_pipeline():
    # route -> permute -> expert rows -> combine reproduces the per-token layer
    # (weights rounded to fp32 in between, as the staged interface stores them).
    x, wr, bias, ex, sh, k = _tiny_layer()
    y, idx, w, _ = oracle.layer("sigmoid_bias", k, K_SCALE, x, wr, bias,
                                oracle.Experts.of(ex), oracle.Experts.of(sh))
    idx2, w2, _ = oracle.route("sigmoid_bias", x, wr, bias, k, K_SCALE)
    assert np.array_equal(idx, idx2) and np.array_equal(w, w2)
    E = wr.shape[0]
    offsets, row_token, token_row = oracle.permute(idx2, E)
    rows = oracle.expert_rows(oracle.Experts.of(ex), x, row_token, offsets)
    shr = oracle.expert_rows(oracle.Experts.of(sh), x, None,
                             np.array([0, x.shape[0]], np.int32))
    ys = oracle.combine(rows.astype(np.float32), token_row, w2.astype(np.float32),
                        shr.astype(np.float32))
    assert np.allclose(ys, y, rtol=1e-5, atol=1e-6 * np.abs(y).max())


def test_combine_one_hot_and_linear():
    T, k, d = 5, 3, 16
    rows = S.normal(1, 1, (T * k, d), 1.0)
    token_row = np.arange(T * k, dtype=np.int32)[::-1].copy()
    w = np.zeros((T, k), np.float32)
    w[:, 1] = 1.0
    sh = S.normal(1, 2, (T, d), 1.0)
    res = S.normal(1, 3, (T, d), 1.0)
    y = oracle.combine(rows, token_row, w, sh, res)
    for t in range(T):
        ref = rows[token_row[t * k + 1]].astype(np.float64) + sh[t] + res[t]
        assert np.array_equal(y[t], ref)
    w2 = S.uniform(1, 4, (T, k), 0, 1)
    y2 = oracle.combine(rows, token_row, w2)
    ref2 = np.einsum("tk,tkd->td", w2.astype(np.float64),
                     rows.astype(np.float64)[token_row].reshape(T, k, d))
    assert np.allclose(y2, ref2, rtol=1e-14)


# ------------------------------------------------------------ expert restriction

def _min_cover_size_bruteforce(counts, cover):
    import itertools
    E = len(counts)
    total = int(counts.sum())
    need = cover * float(total)
    for n in range(0, E + 1):
        for sub in itertools.combinations(range(E), n):
            if float(int(counts[list(sub)].sum())) >= need:
                return n
    return E


def test_coverage_set_is_a_smallest_cover_bruteforce():
    # CMF listing, step 3: the smallest expert set reaching the covered share
    # of the recorded routing mass.  Every subset of tiny layers is tried.
    for trial in range(60):
        E = 3 + trial % 7
        counts = S.randint8(0xC0FE, trial, (E,), 0, 20).astype(np.uint64)
        if trial % 5 == 0:
            counts[:] = counts[0]                        # all equal
        for cover in (0.0, 0.5, 0.73, 0.95, 1.0):
            for k in (1, 2, 4):
                keep = oracle.coverage_set(counts, cover, k)
                n_min = _min_cover_size_bruteforce(counts, cover)
                assert len(keep) == max(n_min, min(k, E)), (counts, cover, k, keep)
                assert np.all(np.diff(keep) > 0)         # ascending, distinct
                assert float(counts[keep].sum()) >= cover * float(counts.sum())
                # greedy by count: no expert left out has more selections than
                # one kept (ties go to the lower id)
                out = np.setdiff1d(np.arange(E), keep)
                if len(out):
                    c_in = counts[keep].astype(np.int64)
                    assert counts[out].max() <= c_in.min()
                    tie_out = out[counts[out] == c_in.min()]
                    tie_in = keep[c_in == c_in.min()]
                    if len(tie_out):
                        assert tie_in.max() < tie_out.min()


def test_coverage_set_worked_example_and_edges():
    c = np.array([5, 1, 9, 0, 9, 3], np.uint64)      # total 27
    assert list(oracle.coverage_set(c, 0.80, 2)) == [0, 2, 4]      # 9+9+5 = 23 >= 21.6
    assert list(oracle.coverage_set(c, 18 / 27, 1)) == [2, 4]      # exactly the share
    assert list(oracle.coverage_set(c, 1.0, 1)) == [0, 1, 2, 4, 5]  # every expert ever chosen
    assert list(oracle.coverage_set(c, 0.0, 3)) == [0, 2, 4]      # only the k floor
    assert list(oracle.coverage_set(np.zeros(4, np.uint64), 0.95, 2)) == [0, 1]
    assert list(oracle.coverage_set(c, 0.5, 9)) == [0, 1, 2, 3, 4, 5]   # k > E: all
    for bad in (-0.1, 1.5, float("nan")):
        with pytest.raises(ValueError):
            oracle.coverage_set(c, bad, 2)


# ------------------------------------------------------------ weight quantizers

def test_quantize_int8_worked_example():
    # The row's largest magnitude is 127 * 2^-7, so s = 2^-7 exactly and every
    # quotient below is exact: codes are the quotients rounded, halves away
    # from zero (2.5 -> 3, -63.5 -> -64, 1.5 -> 2).
    u = 2.0 ** -7
    row = np.array([[127 * u, 0.5, 2.5 * u, -2.5 * u, 1.5 * u, -63.5 * u, 0.0, 0.49 * u,
                     -127 * u, 0.51 * u]], np.float32)
    q, s = oracle.quantize("int8_row", row)
    assert s[0] == np.float32(u)
    assert list(q[0]) == [127, 64, 3, -3, 2, -64, 0, 0, -127, 1]
    z, sz = oracle.quantize("int8_row", np.zeros((2, 16), np.float32))
    assert (z == 0).all() and (sz == 0).all()


def test_quantize_int4_worked_example_and_clamp():
    # block 0: max 7 * 2^-3 -> s = 2^-3, quotients exact: 3.5 -> 4, -0.5 -> -1
    # block 1: max 3 * 2^-15 -> max/7 < 2^-14, so s = 2^-14: codes w * 2^14
    #          (1.5 -> 2, 0.25 -> 0, -1.5 -> -2)
    # block 2: zero -> s = 2^-14, codes 0
    b0 = np.zeros(32, np.float32)
    b0[:4] = [7 * 0.125, 3.5 * 0.125, -0.5 * 0.125, -7 * 0.125]
    b1 = np.zeros(32, np.float32)
    b1[:3] = [3 * 2.0 ** -15, 2.0 ** -16, -3 * 2.0 ** -15]
    row = np.concatenate([b0, b1, np.zeros(32, np.float32)])[None, :]
    q, s = oracle.quantize("int4_b32", row)
    assert list(s[0]) == [0.125, 2.0 ** -14, 2.0 ** -14]
    assert list(q[0, :4]) == [7, 4, -1, -7] and (q[0, 4:32] == 0).all()
    assert list(q[0, 32:35]) == [2, 0, -2] and (q[0, 35:] == 0).all()


@pytest.mark.parametrize("fmt", ["int8_row", "int4_b32"])
def test_quantize_round_trip_range_and_extremes(fmt):
    # |q s - w| <= s/2 (plus the fp32 rounding of the quotient), codes in range,
    # each row's (block's) largest magnitude on the end code, and codes
    # non-decreasing in w within a row (block).
    w = S.normal(0x5151, 1, (64, 256), 0.02)
    w[3] *= 1e-4                                  # int4: every block below the floor
    w[5, :40] = 0.0
    q, s = oracle.quantize(fmt, w)
    qmax = 127 if fmt == "int8_row" else 7
    B = 256 if fmt == "int8_row" else 32
    sb = np.repeat(s.reshape(64, -1), B, axis=1).astype(np.float64)
    err = np.abs(q * sb - w.astype(np.float64))
    assert (err <= sb * (0.5 + 2.0 ** -20)).all()
    assert q.min() >= -qmax and q.max() <= qmax
    for r in range(64):
        for b in range(256 // B):
            wb, qb = w[r, b * B:(b + 1) * B], q[r, b * B:(b + 1) * B]
            o = np.argsort(wb, kind="stable")
            assert (np.diff(qb[o].astype(int)) >= 0).all()
            if sb[r, b * B] > 2.0 ** -14:
                assert np.abs(qb).max() == qmax
                assert qb[np.argmax(np.abs(wb))] == qmax * np.sign(wb[np.argmax(np.abs(wb))])
    if fmt == "int4_b32":
        assert (s[3] == np.float32(2.0 ** -14)).all()


@pytest.mark.parametrize("fmt", ["int8_row", "int4_b32"])
def test_quantize_power_of_two_scaling(fmt):
    # scaling a row by 2^j scales s by 2^j and keeps the codes (exact in fp32)
    w = S.normal(0x5152, 1, (8, 128), 1.0)
    q, s = oracle.quantize(fmt, w)
    for j in (-3, 5):
        q2, s2 = oracle.quantize(fmt, w * np.float32(2.0 ** j))
        assert np.array_equal(q2, q) and np.array_equal(s2, s * np.float32(2.0 ** j))


def test_quantized_experts_reproduce_the_float_layer():
    # Format wiring: fp32 experts quantized by the oracle and read back as
    # int8 per-row / int4 block-32 experts give nearly the fp32 layer (a
    # transposed scale or a wrong block index would not).
    T, d, E, k, I = 12, 128, 6, 2, 64
    x = S.normal(0x5153, 1, (T, d), 1.0)
    wr = S.normal(0x5153, 2, (E, d), 1.0 / math.sqrt(d))
    bias = S.uniform(0x5153, 3, (E,), -0.1, 0.1)
    gu = S.normal(0x5153, 4, (E, 2 * I, d), 1.0 / math.sqrt(d))
    dn = S.normal(0x5153, 5, (E, d, I), 1.0 / math.sqrt(I))
    yf, idxf, _, _ = oracle.layer("sigmoid_bias", k, K_SCALE, x, wr, bias,
                                  oracle.Experts("fp32", gu, dn))
    for fmt, tol in (("int8_row", 0.02), ("int4_b32", 0.25)):
        qg, sg = oracle.quantize(fmt, gu.reshape(E * 2 * I, d))
        qd, sd = oracle.quantize(fmt, dn.reshape(E * d, I))
        shp = (lambda a, n: a.reshape(E, n)) if fmt == "int8_row" else \
              (lambda a, n: a.reshape(E, n, -1))
        ex = oracle.Experts(fmt, qg.reshape(E, 2 * I, d), qd.reshape(E, d, I),
                            shp(sg, 2 * I), shp(sd, d))
        yq, idxq, _, _ = oracle.layer("sigmoid_bias", k, K_SCALE, x, wr, bias, ex)
        assert np.array_equal(idxq, idxf)
        rel = np.abs(yq - yf).max() / np.abs(yf).max()
        assert rel < tol, (fmt, rel)


def test_bf16_bits_to_f32():
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x7F7F, 0x0001], np.uint16)
    v = oracle.bf16_to_f32(bits)
    assert v[0] == 1.0 and v[1] == -2.0 and v[2] == 0.0 and np.signbit(v[3])
    assert v[4] == np.float32(3.3895314e38) and v[5] == np.float32(2.0 ** -133)


# ------------------------------------------------------------ gelu_tanh, int4 block 128

def test_gelu_tanh_identities_and_erf_form():
    # odd part: f(z) - f(-z) = z exactly (tanh is odd); f(0) = 0; the tails go
    # to z and 0; and the tanh form stays within 5e-4 of the erf form z Phi(z)
    for z in (0.0, 0.3, 1.0, 2.5, 7.0):
        assert abs(oracle.gelu_tanh(z) - oracle.gelu_tanh(-z) - z) <= 1e-15 * max(1.0, z)
    assert oracle.gelu_tanh(0.0) == 0.0
    assert abs(oracle.gelu_tanh(12.0) - 12.0) < 1e-12 and abs(oracle.gelu_tanh(-12.0)) < 1e-12
    zs = np.linspace(-8.0, 8.0, 4001)
    gap = max(abs(oracle.gelu_tanh(z) - 0.5 * z * (1.0 + math.erf(z / math.sqrt(2.0))))
              for z in zs)
    assert 1e-4 < gap < 5e-4                    # an approximation, and a close one
    # slope 1/2 at 0 (central difference)
    h = 1e-6
    assert abs((oracle.gelu_tanh(h) - oracle.gelu_tanh(-h)) / (2 * h) - 0.5) < 1e-9


def test_gelu_tanh_layer_uses_the_activation():
    # A layer run with gelu_tanh equals the staged pipeline with h computed by
    # gelu_tanh: checked through one expert, gate row n, by the oracle's FFN
    # on a one-hot weight layout (down = identity rows pick h_n out).
    d, I = 32, 32
    x = S.normal(0x6E10, 1, (d,), 1.0)
    gu = np.zeros((1, 2 * I, d), np.float32)
    gu[0, :I] = np.eye(I, d, dtype=np.float32)            # gate_n = x_n
    gu[0, I:] = np.eye(I, d, dtype=np.float32)            # up_n = x_n
    dn = np.eye(d, I, dtype=np.float32)[None]             # out_m = h_m
    for act, f in (("silu", oracle.silu), ("gelu_tanh", oracle.gelu_tanh)):
        out = oracle.ffn(oracle.Experts("fp32", gu, dn, act=act), 0, x)
        want = np.array([f(float(v)) * float(v) for v in x])
        assert np.allclose(out, want, rtol=1e-15, atol=0)


def test_int4_b128_equals_b32_with_repeated_scales():
    # A block-128 scale is the block-32 scale of each of its four sub-blocks:
    # the layer with block-128 experts equals the layer with block-32 experts
    # whose scales repeat each block-128 scale four times (clamp included).
    T, d, E, k, I = 9, 256, 6, 2, 128
    x = S.normal(0x6E20, 1, (T, d), 1.0)
    wr = S.normal(0x6E20, 2, (E, d), 1.0 / math.sqrt(d))
    bias = S.uniform(0x6E20, 3, (E,), -0.1, 0.1)
    gu = S.randint8(0x6E20, 4, (E, 2 * I, d), -8, 7)
    dn = S.randint8(0x6E20, 5, (E, d, I), -8, 7)
    sg = S.scales(0x6E20, 6, (E, 2 * I, d // 128), 0.02)
    sd = S.scales(0x6E20, 7, (E, d, I // 128), 0.02)
    sg[:, 3, 1] = 1e-6                                    # below the 2^-14 floor
    sd[:, 5, 0] = 0.0
    e128 = oracle.Experts("int4_b128", gu, dn, sg, sd)
    e32 = oracle.Experts("int4_b32", gu, dn, np.repeat(sg, 4, axis=2), np.repeat(sd, 4, axis=2))
    y1, i1, w1, _ = oracle.layer("sigmoid_bias", k, K_SCALE, x, wr, bias, e128)
    y2, i2, w2, _ = oracle.layer("sigmoid_bias", k, K_SCALE, x, wr, bias, e32)
    assert np.array_equal(i1, i2) and np.array_equal(y1, y2)
    # and differs from reading the scales as block-32 (the first quarter)
    e_wrong = oracle.Experts("int4_b32", gu, dn, np.repeat(sg, 4, axis=2)[:, :, ::-1].copy(),
                             np.repeat(sd, 4, axis=2))
    y3, _, _, _ = oracle.layer("sigmoid_bias", k, K_SCALE, x, wr, bias, e_wrong)
    assert not np.allclose(y1, y3)


def test_quantize_int4_b128_scale_is_max_of_b32_scales():
    # RN(max/7) is monotone in the maximum, so a block-128 scale is the largest
    # of its four block-32 scales (before and after the 2^-14 floor), and the
    # round trip stays within half a scale.
    w = S.normal(0x6E30, 1, (40, 512), 0.02)
    w[7] *= 1e-5
    q128, s128 = oracle.quantize("int4_b128", w)
    q32, s32 = oracle.quantize("int4_b32", w)
    assert np.array_equal(s128, s32.reshape(40, -1, 4).max(axis=2))
    sb = np.repeat(s128, 128, axis=1).astype(np.float64)
    assert (np.abs(q128 * sb - w) <= sb * (0.5 + 2.0 ** -20)).all()
    assert q128.min() >= -7 and q128.max() <= 7 and (s128[7] == np.float32(2.0 ** -14)).all()
