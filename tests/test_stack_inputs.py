"""CPU checks of the inputs of the 26-layer Kimi-shaped stack.

* Drawing a subset of experts (by element offset) gives exactly the rows that
  drawing the whole tensor gives, for int8 per-row and int4 block-32 layers.
* The Zipf ranks are a permutation of 1..E and the bias moves by the Zipf
  term alone.
* The stored amplitude alpha (tests/golden/kimi_stack_zipf.json, written by
  make_stack_zipf.py with the oracle's router) still puts 73% +- 1% of layer
  0's selections at T=4096 on its 64 most-selected experts — the concentration
  of the code-corpus routing statistics in the Kimi-Linear-48B-A3B-Code-CMF
  listing ("How it was made").
"""
import json

import numpy as np
import pytest

import oracle
from sparse_moe_expert_sigmoid_amd import synth as S


@pytest.mark.parametrize("name,experts", [("tiny", [5, 0, 31]), ("qwen_decode", [127, 7, 64])])
def test_expert_slice_equals_whole_draw(name, experts):
    s = S.spec(name)
    full = S.make_layer(s, with_x=False).experts
    sl = S.expert_slice(s, experts)
    for a in ("gu", "dn", "gu_s", "dn_s", "gu_packed", "dn_packed"):
        fa, sa = getattr(full, a), getattr(sl, a)
        if fa is None:
            assert sa is None
            continue
        assert np.array_equal(fa[experts], sa), a


def test_shared_slice_equals_whole_draw():
    s = S.spec("kimi_decode", E=16, d=256, inter=128, shared_inter=192)
    full = S.make_layer(s, with_x=False).shared
    sl = S.expert_slice(s, [0], shared=True)
    for a in ("gu", "dn", "gu_s", "dn_s"):
        assert np.array_equal(getattr(full, a), getattr(sl, a)), a


def test_offset_draws_match_whole_tensor():
    whole = S.randint8(7, 4, (1000,), -127, 127)
    part = S.randint8(7, 4, (333,), -127, 127, start=555)
    assert np.array_equal(whole[555:888], part)
    ws = S.scales(7, 5, (1000,), 0.01, special_tid=12)
    ps = S.scales(7, 5, (100,), 0.01, special_tid=12, start=900)
    assert np.array_equal(ws[900:], ps)


def test_zipf_ranks_and_bias():
    E = 256
    seen = set()
    for l in range(S.STACK_LAYERS):
        r = S.zipf_ranks(S.stack_wseed(l), E)
        assert sorted(r.tolist()) == list(range(1, E + 1))
        seen.add(int(np.argmin(r)))
    assert len(seen) > 10          # layers favour different experts
    st = S.stack_spec(1, alpha=0.5)
    s0 = st.layer(0)
    b0 = S.zipf_bias(s0.wseed, E, 0.0)
    b1 = S.zipf_bias(s0.wseed, E, 0.5)
    assert np.array_equal(b0, S.uniform(s0.wseed, S.TID_BIAS, (E,), -0.1, 0.1))
    r = S.zipf_ranks(s0.wseed, E)
    np.testing.assert_allclose(b1.astype(np.float64) - b0, 0.5 * r ** -1.1, atol=1e-7)


def test_stack_layers_have_distinct_weights():
    st = S.stack_spec(1)
    w0, _ = S.stack_router(st, 0)
    w1, _ = S.stack_router(st, 1)
    assert not np.array_equal(w0, w1)
    e0 = S.expert_slice(st.layer(0), [3])
    e1 = S.expert_slice(st.layer(1), [3])
    assert not np.array_equal(e0.gu, e1.gu)


def test_stored_zipf_alpha_gives_target_mass():
    with open(S.ZIPF_FILE) as f:
        rec = json.load(f)
    st = S.stack_spec(4096)
    assert st.alpha == rec["alpha"]
    s0 = st.layer(0)
    wr, bias = S.stack_router(st, 0)
    idx, _, _ = oracle.route(s0.router, S.stack_x(st), wr, bias, s0.k, s0.scale)
    counts = np.bincount(idx.ravel(), minlength=s0.E)
    mass = np.sort(counts)[::-1][:64].sum() / idx.size
    assert abs(mass - 0.73) <= 0.01, mass
    assert abs(mass - rec["mass_layer0_T4096"]) < 1e-4


def test_qwen_stack_spec_layers():
    st = S.qwen_stack_spec(1)
    assert st.layers == 48 and st.base.fmt == "int4_b32" and st.base.shared is None
    seeds = {st.layer(l).wseed for l in range(48)}
    assert len(seeds) == 48
    s = st.layer(7)
    assert (s.d, s.E, s.k, s.inter, s.router) == (2048, 128, 8, 768, "softmax")
    wr, bias = S.stack_router(st, 7)
    assert wr.shape == (128, 2048) and bias is None
    # distinct from the Kimi stack's seeds
    assert not seeds & {S.stack_spec(1).layer(l).wseed for l in range(26)}
    x = S.stack_x(st)
    assert x.shape == (1, 2048)
    assert np.array_equal(S.stack_x(S.qwen_stack_spec(4))[:1], x)
