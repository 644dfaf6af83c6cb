"""Expert restriction from recorded routing statistics.

Kimi-Linear-48B-A3B-Code-CMF listing, "How it was made": step 2 records, per
layer, how often each expert is selected on a calibration run (here the
moe_expert_counts call); step 3 keeps, per layer, the smallest expert set that
carries a given share of those selections, renumbers the kept experts into a
dense prefix and slices the router rows and the selection bias to match.  The
result equals routing the full layer under a mask of the kept experts
(moe_route_masked / moe_layer.expert_mask), so either form can be served.

The kept set is chosen on the GPU by moe_coverage_set from the device
counters; the sliced weights are device-to-device gathers of whole experts.
"""
from __future__ import annotations

import numpy as np
import torch


def coverage_set(ctx, counts, cover: float = 0.95, k: int = 1) -> np.ndarray:
    """Ascending ids of the smallest expert set whose counts reach `cover` of
    the total (moe_coverage_set: experts by descending count, equal counts by
    ascending id, until the running sum reaches cover * total, then at least
    min(k, E) experts).  counts: [E] non-negative integers, a device tensor
    (int64 or uint64 bits, as moe_expert_counts accumulates them) or host
    values; waits for the result."""
    if isinstance(counts, torch.Tensor):
        c = counts.detach()
    else:
        c = torch.from_numpy(np.ascontiguousarray(np.asarray(counts).astype(np.uint64))
                             .view(np.int64))
    if c.dim() != 1 or c.numel() == 0:
        raise ValueError("counts must be a non-empty 1-D array")
    if c.dtype not in (torch.int64, torch.uint64):
        raise ValueError(f"counts must hold 64-bit integers (got {c.dtype})")
    dev = torch.device("cuda", ctx.device)
    c = c.to(dev).contiguous()
    E = c.numel()
    keep = torch.empty(E, dtype=torch.int32, device=dev)
    n = torch.empty(4, dtype=torch.int32, device=dev)
    ctx.moe_coverage_set(c, E, cover, k, keep, n)
    torch.cuda.synchronize(dev)
    m = int(n[0].item())
    return keep[:m].cpu().numpy().astype(np.int64)


def expert_mask(keep, E: int, device) -> torch.Tensor:
    """[E] uint8 device mask, 1 for the kept experts."""
    m = torch.zeros(E, dtype=torch.uint8)
    m[torch.as_tensor(np.asarray(keep), dtype=torch.long)] = 1
    return m.to(device)
