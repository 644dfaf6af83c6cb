"""GPU property tests: random small layer shapes against the oracle.

Hypothesis draws the shape and options of one layer — T, d, E, k, I, router,
expert format, shared expert, weight layout — and both the separate calls
(route, permute, expert FFN, combine) and the single moe_forward call must
match the oracle under the usual rules (expert sets exact except at oracle
near-ties, outputs within 2e-3 of max|y|).  The draws cover the three FFN
paths: pairs grouped in-kernel (T <= 16), 16-row decode tiles, and the
grouped GEMM (int8 with at least 16 rows per expert on average).  A second
draw covers int4 layers (blocks of 32 and 128) with enough rows per expert
for the int4 grouped GEMM, with the shared expert int4 (in the same
launches), int8 or fp32.  The example lists are derandomised, so every run
checks the same shapes.
"""
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from tests.test_gpu_parity import _forward_vs_oracle, _layer_vs_oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ctx(gpu):
    from sparse_moe_expert_sigmoid_amd import Context
    return Context(0)


@st.composite
def layer_shapes(draw):
    fmt = draw(st.sampled_from(["int8_row", "int8_row", "int4_b32"]))
    step = 128 if fmt == "int4_b32" else 64
    wide = draw(st.integers(0, 5)) == 0      # now and then a wide layer, few tokens
    d = step * (draw(st.integers(16, 96)) if wide else draw(st.integers(1, 4)))
    inter = step * draw(st.integers(1, 3))
    k = draw(st.integers(1, 8))
    E = draw(st.integers(k, 40))
    # small batches, 16-row tiles, or enough rows per expert for the GEMM tiles
    T = draw(st.one_of(st.integers(1, 16), st.integers(17, 64),
                       st.integers(max(17, (16 * E + k - 1) // k), 16 * E // k + 64)))
    if wide:
        T = min(T, 40)
    router = draw(st.sampled_from(["sigmoid_bias", "softmax"]))
    shared = draw(st.sampled_from([None, "fp32", fmt if fmt == "int8_row" else None]))
    shared_inter = step * draw(st.integers(1, 2)) if shared else 0
    tiled = draw(st.booleans())
    seed = draw(st.integers(0, 2 ** 16))
    return dict(T=T, d=d, E=E, k=k, inter=inter, router=router,
                scale=2.446 if router == "sigmoid_bias" else 1.0, fmt=fmt, shared=shared,
                shared_inter=shared_inter, wseed=0x5EED0000 + seed, xseed=0x5EED8000 + seed,
                tiled=tiled)


@settings(max_examples=40, deadline=None, derandomize=True, database=None,
          suppress_health_check=[HealthCheck.function_scoped_fixture,
                                 HealthCheck.too_slow])
@given(case=layer_shapes())
def test_random_layers_match_oracle(ctx, case):
    import numpy as np
    case = dict(case)
    tiled = case.pop("tiled")
    case["scale"] = float(np.float32(case["scale"]))
    print(f"[property] {case} tiled={tiled}", flush=True)
    _layer_vs_oracle(ctx, "tiny", tiled=tiled, **case)
    _forward_vs_oracle(ctx, "tiny", **case)


@st.composite
def int4_gemm_shapes(draw):
    # int4 layers (blocks of 32 or 128) with enough rows per expert for the
    # int4 grouped GEMM (tiled codes), and now and then a decode-sized batch;
    # the shared expert int4 (in the same launches), int8 or fp32 (apart)
    fmt = draw(st.sampled_from(["int4_b32", "int4_b128"]))
    d = 128 * draw(st.integers(1, 6))
    inter = 128 * draw(st.integers(1, 4))
    k = draw(st.integers(1, 8))
    E = draw(st.integers(k, 24))
    gemm_T = st.integers(max(17, (16 * E + k - 1) // k), 16 * E // k + 200)
    T = draw(st.one_of(gemm_T, gemm_T, st.integers(1, 16)))
    router = draw(st.sampled_from(["sigmoid_bias", "softmax"]))
    shared = draw(st.sampled_from([None, fmt, "int8_row", "fp32"]))
    shared_inter = 128 * draw(st.integers(1, 3)) if shared else 0
    seed = draw(st.integers(0, 2 ** 16))
    return dict(T=T, d=d, E=E, k=k, inter=inter, router=router,
                scale=2.446 if router == "sigmoid_bias" else 1.0, fmt=fmt, shared=shared,
                shared_inter=shared_inter, wseed=0x5EED4000 + seed, xseed=0x5EEDC000 + seed)


@settings(max_examples=24, deadline=None, derandomize=True, database=None,
          suppress_health_check=[HealthCheck.function_scoped_fixture,
                                 HealthCheck.too_slow])
@given(case=int4_gemm_shapes())
def test_random_int4_layers_match_oracle(ctx, case):
    import numpy as np
    case = dict(case)
    case["scale"] = float(np.float32(case["scale"]))
    print(f"[property int4] {case}", flush=True)
    _layer_vs_oracle(ctx, "tiny", tiled=True, **case)
    _forward_vs_oracle(ctx, "tiny", **case)
