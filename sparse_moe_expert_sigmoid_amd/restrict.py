"""Expert restriction from recorded routing statistics.

Kimi-Linear-48B-A3B-Code-CMF listing, "How it was made": step 2 records, per
layer, how often each expert is selected on a calibration run (here the
moe_expert_counts call); step 3 keeps, per layer, the smallest expert set that
carries a given share of those selections, renumbers the kept experts into a
dense prefix and slices the router rows and the selection bias to match.  The
result equals routing the full layer under a mask of the kept experts
(moe_route_masked / moe_layer.expert_mask), so either form can be served.

The kept set is chosen on the host from E counters; the sliced weights are
device-to-device gathers of whole experts.
"""
from __future__ import annotations

import numpy as np
import torch


def coverage_set(counts, cover: float = 0.95, k: int = 1) -> np.ndarray:
    """Ascending ids of the smallest expert set whose counts reach `cover` of
    the total: experts by descending count, equal counts by ascending id, until
    the running sum reaches cover * total, then at least min(k, E) experts so
    that a token can still select k.  counts: [E] non-negative integers."""
    c = np.asarray(counts)
    if c.ndim != 1 or c.size == 0:
        raise ValueError("counts must be a non-empty 1-D array")
    if not (0.0 <= cover <= 1.0):
        raise ValueError(f"cover={cover} outside [0, 1]")
    if k < 1:
        raise ValueError(f"k={k} must be positive")
    c = c.astype(np.uint64)
    E = c.size
    order = np.lexsort((np.arange(E), -c.astype(np.float64)))   # count desc, id asc
    running = np.cumsum(c[order], dtype=np.uint64).astype(np.float64)
    need = cover * float(c.sum(dtype=np.uint64))
    reached = np.nonzero(running >= need)[0]
    n = 0 if need <= 0.0 else (int(reached[0]) + 1 if reached.size else E)
    n = max(n, min(k, E))
    return np.sort(order[:n]).astype(np.int64)


def expert_mask(keep, E: int, device) -> torch.Tensor:
    """[E] uint8 device mask, 1 for the kept experts."""
    m = torch.zeros(E, dtype=torch.uint8)
    m[torch.as_tensor(np.asarray(keep), dtype=torch.long)] = 1
    return m.to(device)
