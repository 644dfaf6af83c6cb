"""Host logic of the expert restriction: the package's kept-set choice equals
the oracle's on random and adversarial counts (ties, zeros, tiny covers)."""
import numpy as np
import pytest

import oracle
from sparse_moe_expert_sigmoid_amd import synth as S
from sparse_moe_expert_sigmoid_amd.restrict import coverage_set


def test_coverage_set_matches_oracle():
    for trial in range(300):
        E = [1, 2, 7, 32, 128, 256, 300][trial % 7]
        hi = [0, 1, 3, 100, 127][trial % 5]
        c = S.randint8(0xC0FF, trial, (E,), 0, hi).astype(np.uint64)
        if trial % 11 == 0:
            c = c * np.uint64(1 << 40)                   # large counts
        for cover in (0.0, 0.3, 0.73, 0.95, 1.0):
            for k in (1, 8):
                got = coverage_set(c, cover, k)
                want = oracle.coverage_set(c, cover, k)
                assert np.array_equal(got, want), (trial, cover, k)


def test_coverage_set_rejects_bad_arguments():
    with pytest.raises(ValueError):
        coverage_set(np.array([1, 2]), 1.2, 1)
    with pytest.raises(ValueError):
        coverage_set(np.array([1, 2]), 0.5, 0)
    with pytest.raises(ValueError):
        coverage_set(np.array([], np.int64), 0.5, 1)
