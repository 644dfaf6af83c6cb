#!/usr/bin/env python3
"""Writes tests/golden/kimi_stack_zipf.json: the Zipf amplitude alpha of the
26-layer Kimi-shaped stack's selection bias.

The stack's layer l draws its selection bias as u_l + alpha * r_l^-1.1 (see
the input generator).  alpha is the value for which, on layer 0 at T=4096
tokens, the 64 most-selected experts receive 73% of the T*8 selections: the
concentration that the routing statistics of the Kimi-Linear-48B-A3B-Code-CMF
listing ("How it was made", the routing-frequency step) report for code.

The selections are the oracle's (its router, on the generator's x_0, router
weights and bias); alpha is found by bisection on that fraction.  Only the
oracle and the input generator are used.

    python tests/golden/make_stack_zipf.py
"""
from __future__ import annotations

import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from sparse_moe_expert_sigmoid_amd import synth  # noqa: E402

T_CAL = 4096
TOP = 64
TARGET = 0.73


def top_mass(idx: np.ndarray, E: int, top: int = TOP) -> float:
    counts = np.bincount(idx.ravel(), minlength=E)
    return float(np.sort(counts)[::-1][:top].sum()) / idx.size


def mass_at(alpha: float, x, wr, E: int) -> float:
    s = synth.stack_spec(T_CAL, alpha=alpha).layer(0)
    bias = synth.zipf_bias(s.wseed, E, alpha)
    idx, _, _ = oracle.route(s.router, x, wr, bias, s.k, s.scale)
    return top_mass(idx, E)


def main():
    st = synth.stack_spec(T_CAL, alpha=0.0)
    s0 = st.layer(0)
    x = synth.stack_x(st)
    wr, _ = synth.stack_router(st, 0)
    lo, hi = 0.0, 2.0
    m_lo, m_hi = mass_at(lo, x, wr, s0.E), mass_at(hi, x, wr, s0.E)
    print(f"alpha {lo}: {m_lo:.4f}   alpha {hi}: {m_hi:.4f}", flush=True)
    assert m_lo < TARGET < m_hi
    alpha, mass = hi, m_hi
    for _ in range(30):
        mid = 0.5 * (lo + hi)
        m = mass_at(mid, x, wr, s0.E)
        print(f"alpha {mid:.6f}: {m:.4f}", flush=True)
        alpha, mass = mid, m
        if abs(m - TARGET) < 0.002:
            break
        if m < TARGET:
            lo = mid
        else:
            hi = mid
    rec = {
        "alpha": round(alpha, 6),
        "zipf_exponent": synth.ZIPF_S,
        "top_experts": TOP,
        "target_mass": TARGET,
        "mass_layer0_T4096": round(mass_at(round(alpha, 6), x, wr, s0.E), 4),
        "method": "bisection on alpha; selections from oracle.route on layer 0, x_0 at T=4096",
    }
    with open(os.path.join(HERE, "kimi_stack_zipf.json"), "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(rec)


if __name__ == "__main__":
    main()
