"""Comparison rules shared by the GPU parity tests (test-side only).

* Expert indices: each token's set of k experts must equal the oracle's
  bit-exactly, except where the oracle's gap between its k-th and (k+1)-th
  selection key is below 1e-6 (a near tie that fp32 rounding order may flip);
  such tokens are counted, reported and left out of the output check.
  Within a token, the order must match wherever adjacent oracle keys differ
  by at least 1e-6.
* Weights: |w_gpu - w_oracle| <= 1e-6 * scale per slot (weights sum to scale).
* Outputs: max |y_gpu - y_oracle| <= 2e-3 * max |y_oracle| (the fp32 bound),
  with the maximum taken over the whole oracle output.
"""
from __future__ import annotations

import json
import os

import numpy as np

GAP_TOL = 1e-6
Y_TOL = 2e-3


def oracle_keys(router, logits, bias):
    if router == "sigmoid_bias":
        s = 1.0 / (1.0 + np.exp(-logits))
        return (s + (bias.astype(np.float64) if bias is not None else 0.0)).astype(np.float32)
    m = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - m)
    return (p / p.sum(axis=1, keepdims=True)).astype(np.float32)


def compare_route(gidx, gw, oidx, ow, ogap, keys, scale):
    """Returns the list of excused tokens; asserts everything else."""
    T, k = oidx.shape
    excused = []
    for t in range(T):
        if set(gidx[t].tolist()) != set(oidx[t].tolist()):
            assert ogap[t] < GAP_TOL, (
                f"token {t}: experts {sorted(gidx[t])} vs oracle {sorted(oidx[t])}, "
                f"oracle gap {ogap[t]:.3e}")
            excused.append(t)
            continue
        kt = keys[t, oidx[t]].astype(np.float64)
        for j in range(k):
            if gidx[t, j] != oidx[t, j]:
                # allowed only inside a run of near-equal keys
                near = (j > 0 and kt[j - 1] - kt[j] < GAP_TOL) or \
                       (j + 1 < k and kt[j] - kt[j + 1] < GAP_TOL)
                assert near, f"token {t} slot {j}: order {gidx[t]} vs oracle {oidx[t]}"
        om = dict(zip(oidx[t].tolist(), ow[t].tolist()))
        for j in range(k):
            ref = om[int(gidx[t, j])]
            assert abs(float(gw[t, j]) - ref) <= GAP_TOL * scale, (
                f"token {t} slot {j}: w {gw[t, j]} vs oracle {ref}")
    return excused


def compare_outputs(gy, oy, keep=None, tol=Y_TOL):
    """max |gy - oy| over rows `keep` <= tol * max|oy| (whole tensor); returns the ratio."""
    scale = float(np.abs(oy).max())
    assert scale > 0
    if keep is None:
        keep = np.arange(oy.shape[0])
    keep = np.asarray(keep)
    if keep.size == 0:
        return 0.0
    err = float(np.abs(gy[keep].astype(np.float64) - oy[keep]).max())
    ratio = err / scale
    assert ratio <= tol, f"max|err| = {err:.3e} = {ratio:.3e} x max|y| (bound {tol})"
    return ratio


def log_result(**kw):
    """Print one result record and append it to $MOE_PARITY_LOG (JSON lines)."""
    path = os.environ.get("MOE_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(kw) + "\n")
    print(kw, flush=True)
