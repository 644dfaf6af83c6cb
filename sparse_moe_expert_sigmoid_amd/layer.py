"""One routed-MoE layer on the GPU: the five calls of the C ABI in order.

    y = combine(expert_ffn(permute(route(x))), shared_ffn(x)) [+ residual]

(route -> permute -> routed expert FFN -> shared expert FFN -> combine).  This
class only owns device buffers and issues the calls on one stream; all
arithmetic is in the HIP library.  Buffers are allocated when the layer is
built or when T changes, never inside forward() at a fixed T.
"""
from __future__ import annotations

from typing import Optional

import torch

from .binding import ACT, Context, DeviceExperts, ROUTER, moe_layer, moe_weights


class MoELayer:
    def __init__(self, ctx: Context, router: str, k: int, scale: float, w_router: torch.Tensor,
                 bias: Optional[torch.Tensor], experts: DeviceExperts,
                 shared: Optional[DeviceExperts] = None,
                 expert_mask: Optional[torch.Tensor] = None, act: str = "silu"):
        self.ctx = ctx
        self.act_name = act
        self.act = ACT[act]  # gate activation of the routed and shared experts
        self.router = ROUTER[router]
        self.k, self.scale = k, float(scale)
        self.w_router, self.bias = w_router, bias
        self.experts, self.shared = experts, shared
        self.E, self.d = experts.n_experts, experts.d
        self.device = w_router.device
        self._T = None
        self._fused_T = None
        self.expert_mask = expert_mask  # [E] uint8 on the device, nonzero = allowed
        self.desc = moe_layer(self.router, k, self.scale, w_router.data_ptr(),
                              bias.data_ptr() if bias is not None else None, experts.struct(),
                              shared.struct() if shared is not None else moe_weights(),
                              expert_mask.data_ptr() if expert_mask is not None else None)

    @staticmethod
    def from_inputs(ctx: Context, inputs, device="cuda:0", tiled: bool = True,
                    act: str = "silu") -> "MoELayer":
        """Upload a synth.LayerInputs; quantised codes go to the tiled layout unless
        tiled=False."""
        s = inputs.spec
        wr = torch.from_numpy(inputs.wr).to(device)
        bias = torch.from_numpy(inputs.bias).to(device) if inputs.bias is not None else None
        ex = DeviceExperts.upload(inputs.experts, device)
        sh = DeviceExperts.upload(inputs.shared, device) if inputs.shared is not None else None
        if tiled:
            ex = ex.tiled(ctx)
            sh = sh.tiled(ctx) if sh is not None else None
        return MoELayer(ctx, s.router, s.k, s.scale, wr, bias, ex, sh, act=act)

    def with_weights(self, experts: DeviceExperts, shared: Optional[DeviceExperts]) -> "MoELayer":
        """Same router, other expert weights (e.g. a copy in other HBM pages)."""
        return MoELayer(self.ctx, self._router_name(), self.k, self.scale, self.w_router,
                        self.bias, experts, shared, self.expert_mask, self.act_name)

    def _router_name(self) -> str:
        return [k for k, v in ROUTER.items() if v == self.router][0]

    def with_mask(self, expert_mask: Optional[torch.Tensor]) -> "MoELayer":
        """Same layer restricted to the experts whose mask entry is nonzero."""
        return MoELayer(self.ctx, self._router_name(), self.k, self.scale, self.w_router,
                        self.bias, self.experts, self.shared, expert_mask, self.act_name)

    def restricted(self, keep) -> "MoELayer":
        """The layer cut to the experts `keep` (ascending ids), renumbered
        0..n-1: router rows, selection bias and expert weights sliced, the
        shared expert unchanged.  Equal to with_mask() of the same set, with
        ids mapped through keep (Kimi-Linear-48B-A3B-Code-CMF listing, "How it
        was made", step 3)."""
        keep = [int(e) for e in keep]
        if sorted(set(keep)) != keep:
            raise ValueError("keep must be strictly ascending expert ids")
        ix = torch.as_tensor(keep, dtype=torch.long, device=self.device)
        wr = self.w_router.index_select(0, ix).contiguous()
        bias = self.bias.index_select(0, ix).contiguous() if self.bias is not None else None
        return MoELayer(self.ctx, self._router_name(), self.k, self.scale, wr, bias,
                        self.experts.select(keep), self.shared, act=self.act_name)

    def alloc(self, T: int):
        if self._T == T:
            return
        dev, k, d, E = self.device, self.k, self.d, self.E
        i32 = dict(dtype=torch.int32, device=dev)
        f32 = dict(dtype=torch.float32, device=dev)
        R = T * k
        self.idx = torch.empty((T, k), **i32)
        self.w = torch.empty((T, k), **f32)
        self.offsets = torch.empty(E + 1, **i32)
        self.row_token = torch.empty(R, **i32)
        self.token_row = torch.empty(R, **i32)
        self.rows = torch.empty((R, d), **f32)
        self.sh_out = torch.empty((T, d), **f32) if self.shared is not None else None
        self.y = torch.empty((T, d), **f32)
        need = self.ctx.moe_workspace_size(T, k, E, d, self.experts.inter, self.experts.fmt)
        if self.shared is not None:
            need = max(need, self.ctx.moe_workspace_size(T, 1, 1, d, self.shared.inter,
                                                         self.shared.fmt))
        self.ws = torch.empty(need, dtype=torch.uint8, device=dev)
        self._T = T

    def forward(self, x: torch.Tensor, residual: Optional[torch.Tensor] = None, stream=None,
                out: Optional[torch.Tensor] = None) -> torch.Tensor:
        T, d = x.shape
        self.alloc(T)
        c, k, E = self.ctx, self.k, self.E
        c.moe_route_masked(self.router, x, self.w_router, self.bias, self.expert_mask, T, d, E, k,
                           self.scale, self.idx, self.w, self.ws, stream)
        c.moe_permute(self.idx, T, k, E, self.offsets, self.row_token, self.token_row, stream)
        c.moe_expert_ffn(self.experts, self.act, x, T, self.row_token, self.offsets, T * k,
                         self.rows, self.ws, stream)
        if self.shared is not None:
            c.moe_expert_ffn(self.shared, self.act, x, T, None, None, T, self.sh_out,
                             self.ws, stream)
        y = self.y if out is None else out
        c.moe_combine(self.rows, self.token_row, self.w, self.sh_out, residual, T, k, d, y,
                      stream)
        return y

    def forward_fused(self, x: torch.Tensor, residual: Optional[torch.Tensor] = None,
                      stream=None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
        """The same layer through the single moe_forward call."""
        T, d = x.shape
        self.alloc(T)
        if self._fused_T != T:
            need = self.ctx.moe_layer_workspace_size(self.desc, T)
            self.fws = torch.empty(need, dtype=torch.uint8, device=self.device)
            self._fused_T = T
        y = self.y if out is None else out
        self.ctx.moe_forward(self.desc, self.act, x, T, residual, y, self.idx, self.w,
                             self.fws, stream)
        return y

    __call__ = forward
