"""A stack of routed-MoE layers with the residual outside each layer:

    x_{l+1} = x_l + MoE_l(x_l)            (one moe_forward call per layer)

The residual add sits after the moe op (Qwen3-30B-A3B model card,
"Conversion Notes"), so each layer passes its input as moe_forward's
residual.  Activations ping-pong between two [T, d] buffers; the input x_0 is
never written, so a captured HIP graph of the whole stack can be replayed on
the same input.  All buffers, including the workspaces, are allocated by
alloc(T), never inside forward().

At decode sizes (T <= 16, every layer on the small-batch path) the layers
chain (moe_forward_chained): each layer leaves its output pending and the
next layer's router launch forms it, so a layer takes one launch fewer; the
last layer's output is completed by moe_combine.  The results are bit for
bit those of one moe_forward per layer.  Two workspaces alternate (a layer
reads the previous one's rows from its workspace).
"""
from __future__ import annotations

from typing import Callable, List, Optional

import torch

from .binding import Context, DeviceExperts, MOE_W_FP32, MOE_W_INT8_ROW
from .layer import MoELayer


class MoEStack:
    def __init__(self, ctx: Context, layers: List[MoELayer]):
        assert layers, "empty stack"
        self.ctx = ctx
        self.layers = layers
        self.d, self.k = layers[0].d, layers[0].k
        self.device = layers[0].device
        self._T = None

    @property
    def weight_bytes(self) -> int:
        n = 0
        for L in self.layers:
            n += L.experts.nbytes + (L.shared.nbytes if L.shared is not None else 0)
            n += L.w_router.numel() * 4 + (L.bias.numel() * 4 if L.bias is not None else 0)
        return n

    def alloc(self, T: int):
        if self._T == T:
            return
        dev, k, d = self.device, self.k, self.d
        self.buf = [torch.empty((T, d), dtype=torch.float32, device=dev) for _ in range(2)]
        self.idx = [torch.empty((T, k), dtype=torch.int32, device=dev) for _ in self.layers]
        self.w = [torch.empty((T, k), dtype=torch.float32, device=dev) for _ in self.layers]
        need = max(self.ctx.moe_layer_workspace_size(L.desc, T) for L in self.layers)
        self.ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        self.chain = 0 < T <= 16 and all(_chains(L) for L in self.layers)
        self.ws2 = (torch.empty(max(need, 1), dtype=torch.uint8, device=dev) if self.chain
                    else None)
        self._T = T

    def forward(self, x0: torch.Tensor, stream=None,
                before_layer: Optional[Callable[[int, torch.Tensor], None]] = None,
                after_layer: Optional[Callable[[int, torch.Tensor, torch.Tensor], None]] = None,
                counts: Optional[torch.Tensor] = None) -> torch.Tensor:
        """Runs every layer on x0 [T, d]; returns x_L (one of the two buffers).

        before_layer(l, x_l) may modify x_l in place before layer l reads it
        (x_0 itself is passed for l = 0); after_layer(l, x_l, x_{l+1}) sees
        each layer's input and output.  Both run on the host between the
        enqueues, so they are for tests, not for timed or captured runs.
        counts: optional [layers, E] int64 device tensor; each layer's expert
        selections are added to its row (the routing statistics of a
        calibration run)."""
        T, d = x0.shape
        assert d == self.d and x0.dtype == torch.float32 and x0.is_contiguous()
        self.alloc(T)
        if self.chain and before_layer is None and after_layer is None:
            return self._forward_chained(x0, stream, counts)
        cur = x0
        for l, L in enumerate(self.layers):
            if before_layer is not None:
                before_layer(l, cur)
            out = self.buf[l % 2]
            self.ctx.moe_forward(L.desc, L.act, cur, T, cur, out, self.idx[l], self.w[l],
                                 self.ws, stream)
            if counts is not None:
                self.ctx.moe_expert_counts(self.idx[l], T, L.k, L.E, counts[l], stream)
            if after_layer is not None:
                after_layer(l, cur, out)
            cur = out
        return cur

    def _forward_chained(self, x0, stream, counts):
        T = x0.shape[0]
        ws = (self.ws, self.ws2)
        pend = None
        for l, L in enumerate(self.layers):
            if pend is None:
                pend = self.ctx.moe_forward_chained(L.desc, L.act, x0, None, None, T, self.idx[l],
                                                    self.w[l], ws[l % 2], stream)
            else:
                # the input x_l is formed into buf[(l - 1) % 2], the buffer the
                # unchained run writes layer l - 1's output to
                pend = self.ctx.moe_forward_chained(L.desc, L.act, None, pend,
                                                    self.buf[(l - 1) % 2], T, self.idx[l],
                                                    self.w[l], ws[l % 2], stream)
            if counts is not None:
                self.ctx.moe_expert_counts(self.idx[l], T, L.k, L.E, counts[l], stream)
        out = self.buf[(len(self.layers) - 1) % 2]
        self.ctx.moe_combine_pending(pend, out, stream)
        return out

    __call__ = forward


    def restricted(self, counts, cover: float = 0.95, masked: bool = False):
        """Per layer, the smallest expert set carrying `cover` of the recorded
        selections (counts: [layers, E], host or device), as a new stack of
        sliced layers, or of masked full layers with masked=True.  Returns
        (stack, [kept ids per layer])."""
        from .restrict import coverage_set, expert_mask
        if len(counts) != len(self.layers):
            raise ValueError("counts needs one row per layer")
        keeps, layers = [], []
        for l, L in enumerate(self.layers):
            keep = coverage_set(self.ctx, counts[l][:L.E], cover, L.k)
            keeps.append(keep)
            layers.append(L.with_mask(expert_mask(keep, L.E, L.device)) if masked
                          else L.restricted(keep))
        return MoEStack(self.ctx, layers), keeps

    # ------------------------------------------------------------------
    @staticmethod
    def from_synth(ctx: Context, st, device="cuda:0", layers: Optional[int] = None,
                   log: Optional[Callable[[str], None]] = None) -> "MoEStack":
        """Builds the stack `st` (a synth.StackSpec: the Kimi-shaped int8 stack
        or the Qwen3-shaped int4 one): router weights and biases drawn on the
        host, expert codes and scales drawn on the GPU by the generator's
        device twin, codes converted to the tiled layout."""
        from . import synth
        from .binding import FMT
        n = st.layers if layers is None else layers
        out = []
        for l in range(n):
            s = st.layer(l)
            wr, bias = synth.stack_router(st, l)
            if s.fmt == synth.FMT_INT8_ROW:
                gu, gu_s, dn, dn_s = synth.dev_int8_experts(s, device)
            else:
                gu, gu_s, dn, dn_s = synth.dev_int4_experts(s, device)
            rows = DeviceExperts(FMT[s.fmt], s.E, s.d, s.inter, gu, dn, gu_s, dn_s)
            routed = rows.tiled(ctx)
            del rows, gu, dn
            shared = None
            if s.shared is not None:
                gu, gu_s, dn, dn_s = synth.dev_int8_experts(s, device, shared=True)
                rows = DeviceExperts(MOE_W_INT8_ROW, 1, s.d, s.shared_inter, gu, dn, gu_s, dn_s)
                shared = rows.tiled(ctx)
                del rows, gu, dn
            L = MoELayer(ctx, s.router, s.k, s.scale, torch.from_numpy(wr).to(device),
                         torch.from_numpy(bias).to(device) if bias is not None else None,
                         routed, shared)
            out.append(L)
            if log is not None and (l == 0 or (l + 1) % 8 == 0 or l + 1 == n):
                torch.cuda.synchronize()
                log(f"[stack] layer {l + 1}/{n} built")
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        return MoEStack(ctx, out)


def _chains(L) -> bool:
    """Whether the layer runs on the chained (small-batch) path: quantised
    routed experts and no shared expert, or one in their format and layout."""
    if L.experts.fmt == MOE_W_FP32:
        return False
    sh = L.shared
    return sh is None or (sh.fmt == L.experts.fmt and sh.layout == L.experts.layout)
