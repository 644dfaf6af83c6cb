"""ctypes binding over libmoe_mi355x.so (the C ABI in include/moe.h).

Argument marshalling only: every step of the layer runs in the HIP library.
Functions carry the C names (moe_route, moe_permute, moe_expert_ffn,
moe_combine, ...) and take torch tensors on the GPU (their data pointers are
passed through) plus plain integers.  If the library is missing this module
raises at import of the context; there is no fallback of any kind.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_mi355x.so")

MOE_OK, MOE_E_INVALID, MOE_E_UNSUPPORTED, MOE_E_DEVICE, MOE_E_WORKSPACE = range(5)
MOE_ROUTER_SIGMOID_BIAS, MOE_ROUTER_SOFTMAX = 0, 1
MOE_W_FP32, MOE_W_INT8_ROW, MOE_W_INT4_B32, MOE_W_INT4_B128 = 0, 1, 2, 3
MOE_ACT_SILU, MOE_ACT_GELU_TANH = 0, 1
ACT = {"silu": MOE_ACT_SILU, "gelu_tanh": MOE_ACT_GELU_TANH}
MOE_LAYOUT_ROWS, MOE_LAYOUT_TILED = 0, 1
MOE_IN_F32, MOE_IN_BF16 = 0, 1
MOE_PROBE_MFMA_16X16X64, MOE_PROBE_MFMA_32X32X32 = 0, 1

ROUTER = {"sigmoid_bias": MOE_ROUTER_SIGMOID_BIAS, "softmax": MOE_ROUTER_SOFTMAX}
FMT = {"fp32": MOE_W_FP32, "int8_row": MOE_W_INT8_ROW, "int4_b32": MOE_W_INT4_B32,
       "int4_b128": MOE_W_INT4_B128}

EXPORTS = ("moe_create", "moe_destroy", "moe_last_error", "moe_status_string",
           "moe_workspace_size", "moe_route", "moe_permute", "moe_expert_ffn", "moe_combine",
           "moe_timing", "moe_timing_read", "moe_layer_workspace_size", "moe_forward",
           "moe_tile_weights", "moe_route_masked", "moe_expert_counts", "moe_quantize",
           "moe_forward_noalloc", "moe_probe_read", "moe_probe_mfma", "moe_coverage_set",
           "moe_forward_chained")
MOE_NOALLOC_SCRATCH_BYTES = 40 * 1024 * 1024


class MoeError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} [status {status}]")
        self.status = status


class moe_weights(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int), ("layout", ctypes.c_int), ("n_experts", ctypes.c_int),
                ("d", ctypes.c_int),
                ("inter", ctypes.c_int), ("w_gate_up", ctypes.c_void_p),
                ("s_gate_up", ctypes.c_void_p), ("w_down", ctypes.c_void_p),
                ("s_down", ctypes.c_void_p)]


class moe_layer(ctypes.Structure):
    _fields_ = [("router", ctypes.c_int), ("k", ctypes.c_int), ("scale", ctypes.c_float),
                ("w_router", ctypes.c_void_p), ("bias", ctypes.c_void_p),
                ("experts", moe_weights), ("shared", moe_weights),
                ("expert_mask", ctypes.c_void_p)]


class moe_pending(ctypes.Structure):
    """A layer's output left pending by moe_forward_chained (device pointers)."""
    _fields_ = [("rows", ctypes.c_void_p), ("shared", ctypes.c_void_p), ("w", ctypes.c_void_p),
                ("residual", ctypes.c_void_p), ("T", ctypes.c_int), ("k", ctypes.c_int),
                ("d", ctypes.c_int)]


class moe_kernel_time(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("launches", ctypes.c_longlong),
                ("total_ms", ctypes.c_double)]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m sparse_moe_expert_sigmoid_amd.build`")
    lib = ctypes.CDLL(path)
    vp, ci, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.moe_create.argtypes = [ci, ctypes.POINTER(vp)]
    lib.moe_destroy.argtypes = [vp]
    lib.moe_destroy.restype = None
    lib.moe_last_error.argtypes = [vp]
    lib.moe_last_error.restype = ctypes.c_char_p
    lib.moe_status_string.argtypes = [ci]
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_workspace_size.argtypes = [vp, ci, ci, ci, ci, ci, ci, ctypes.POINTER(sz)]
    lib.moe_route.argtypes = [vp, ci, vp, vp, vp, ci, ci, ci, ci, ctypes.c_float, vp, vp, vp, sz,
                              vp]
    lib.moe_route_masked.argtypes = [vp, ci, vp, vp, vp, vp, ci, ci, ci, ci, ctypes.c_float, vp,
                                     vp, vp, sz, vp]
    lib.moe_expert_counts.argtypes = [vp, vp, ci, ci, ci, vp, vp]
    lib.moe_quantize.argtypes = [vp, ci, ci, vp, ctypes.c_longlong, ci, vp, vp, vp]
    lib.moe_permute.argtypes = [vp, vp, ci, ci, ci, vp, vp, vp, vp]
    lib.moe_expert_ffn.argtypes = [vp, ctypes.POINTER(moe_weights), ci, vp, ci, vp, vp, ci, vp,
                                   vp, sz, vp]
    lib.moe_combine.argtypes = [vp, vp, vp, vp, vp, vp, ci, ci, ci, vp, vp]
    lib.moe_layer_workspace_size.argtypes = [vp, ctypes.POINTER(moe_layer), ci,
                                             ctypes.POINTER(sz)]
    lib.moe_forward.argtypes = [vp, ctypes.POINTER(moe_layer), ci, vp, ci, vp, vp, vp, vp, vp, sz,
                                vp]
    lib.moe_forward_noalloc.argtypes = [vp, ctypes.POINTER(moe_layer), ci, vp, ci, vp, vp, vp, vp,
                                        vp]
    lib.moe_tile_weights.argtypes = [vp, ctypes.POINTER(moe_weights), vp, vp, vp]
    lib.moe_probe_read.argtypes = [vp, vp, sz, ci, vp, vp]
    lib.moe_coverage_set.argtypes = [vp, vp, ci, ctypes.c_double, ci, vp, vp, vp]
    lib.moe_forward_chained.argtypes = [vp, ctypes.POINTER(moe_layer), ci, vp,
                                        ctypes.POINTER(moe_pending), vp, ci,
                                        ctypes.POINTER(moe_pending), vp, vp, vp, sz, vp]
    lib.moe_probe_mfma.argtypes = [vp, ci, ci, ci, vp, vp]
    lib.moe_timing.argtypes = [vp, ci]
    lib.moe_timing_read.argtypes = [vp, ctypes.POINTER(moe_kernel_time), ci,
                                    ctypes.POINTER(ci)]
    for f in ("moe_create", "moe_workspace_size", "moe_route", "moe_permute", "moe_expert_ffn",
              "moe_combine", "moe_timing", "moe_timing_read", "moe_layer_workspace_size",
              "moe_forward", "moe_tile_weights", "moe_route_masked", "moe_expert_counts",
              "moe_quantize", "moe_forward_noalloc", "moe_probe_read", "moe_probe_mfma",
              "moe_coverage_set", "moe_forward_chained"):
        getattr(lib, f).restype = ci
    _lib = lib
    return lib


def _p(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("device tensor expected")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


class Context:
    """A moe_ctx on one device."""

    def __init__(self, device: int = 0):
        self.lib = load_library()
        h = ctypes.c_void_p()
        st = self.lib.moe_create(device, ctypes.byref(h))
        if st != MOE_OK:
            raise MoeError(st, self.lib.moe_last_error(None).decode())
        self.handle = h
        self.device = device

    def close(self):
        if getattr(self, "handle", None):
            self.lib.moe_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _check(self, st: int):
        if st != MOE_OK:
            raise MoeError(st, self.lib.moe_last_error(self.handle).decode())

    # ---- the C calls, same names ----
    def moe_workspace_size(self, T, k, E, d, inter, fmt) -> int:
        n = ctypes.c_size_t()
        self._check(self.lib.moe_workspace_size(self.handle, T, k, E, d, inter, fmt,
                                                ctypes.byref(n)))
        return n.value

    def moe_route(self, router, x, w_router, bias, T, d, E, k, scale, topk_idx, topk_w, ws,
                  stream=None, ws_bytes=None):
        self._check(self.lib.moe_route(
            self.handle, router, _p(x), _p(w_router), _p(bias), T, d, E, k, scale, _p(topk_idx),
            _p(topk_w), _p(ws), ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes,
            _stream(stream)))

    def moe_route_masked(self, router, x, w_router, bias, mask, T, d, E, k, scale, topk_idx,
                         topk_w, ws, stream=None, ws_bytes=None):
        self._check(self.lib.moe_route_masked(
            self.handle, router, _p(x), _p(w_router), _p(bias), _p(mask), T, d, E, k, scale,
            _p(topk_idx), _p(topk_w), _p(ws),
            ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes, _stream(stream)))

    def moe_expert_counts(self, topk_idx, T, k, E, counts, stream=None):
        self._check(self.lib.moe_expert_counts(self.handle, _p(topk_idx), T, k, E, _p(counts),
                                               _stream(stream)))

    def moe_coverage_set(self, counts, E, cover, k, keep, n_keep, stream=None):
        self._check(self.lib.moe_coverage_set(self.handle, _p(counts), E, float(cover), k,
                                              _p(keep), _p(n_keep), _stream(stream)))

    def moe_quantize(self, fmt, w, codes, scales, stream=None):
        """w: [rows, K] fp32 or bf16 device tensor; fmt MOE_W_INT8_ROW or
        MOE_W_INT4_B32; codes / scales preallocated (see moe.h)."""
        if w.dtype == torch.float32:
            in_type = MOE_IN_F32
        elif w.dtype == torch.bfloat16:
            in_type = MOE_IN_BF16
        else:
            raise TypeError(f"moe_quantize takes fp32 or bf16 weights, not {w.dtype}")
        rows, K = w.shape
        self._check(self.lib.moe_quantize(self.handle, fmt, in_type, _p(w), rows, K, _p(codes),
                                          _p(scales), _stream(stream)))

    def moe_permute(self, topk_idx, T, k, E, offsets, row_token, token_row, stream=None):
        self._check(self.lib.moe_permute(self.handle, _p(topk_idx), T, k, E, _p(offsets),
                                         _p(row_token), _p(token_row), _stream(stream)))

    def moe_expert_ffn(self, weights: "DeviceExperts", act, x, T, row_token, offsets, R_max,
                       rows_out, ws, stream=None, ws_bytes=None):
        w = weights.struct()
        self._check(self.lib.moe_expert_ffn(
            self.handle, ctypes.byref(w), act, _p(x), T, _p(row_token), _p(offsets), R_max,
            _p(rows_out), _p(ws),
            ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes, _stream(stream)))

    def moe_layer_workspace_size(self, layer: "moe_layer", T) -> int:
        n = ctypes.c_size_t()
        self._check(self.lib.moe_layer_workspace_size(self.handle, ctypes.byref(layer), T,
                                                      ctypes.byref(n)))
        return n.value

    def moe_forward(self, layer: "moe_layer", act, x, T, residual, y, topk_idx, topk_w, ws,
                    stream=None, ws_bytes=None):
        self._check(self.lib.moe_forward(
            self.handle, ctypes.byref(layer), act, _p(x), T, _p(residual), _p(y), _p(topk_idx),
            _p(topk_w), _p(ws), ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes,
            _stream(stream)))

    def moe_forward_noalloc(self, layer: "moe_layer", act, x, T, residual, y, topk_idx, topk_w,
                            stream=None):
        self._check(self.lib.moe_forward_noalloc(
            self.handle, ctypes.byref(layer), act, _p(x), T, _p(residual), _p(y), _p(topk_idx),
            _p(topk_w), _stream(stream)))

    def moe_forward_chained(self, layer: "moe_layer", act, x, pending_in, x_out, T, topk_idx,
                            topk_w, ws, stream=None, ws_bytes=None) -> "moe_pending":
        """One chained layer: input x (a tensor) or pending_in (the moe_pending of
        the previous call, whose sum goes to x_out); returns this layer's
        moe_pending."""
        out = moe_pending()
        self._check(self.lib.moe_forward_chained(
            self.handle, ctypes.byref(layer), act, _p(x),
            ctypes.byref(pending_in) if pending_in is not None else None, _p(x_out), T,
            ctypes.byref(out), _p(topk_idx), _p(topk_w), _p(ws),
            ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes, _stream(stream)))
        return out

    def moe_combine_pending(self, p: "moe_pending", y, stream=None):
        """Completes a pending output into y with moe_combine."""
        self._check(self.lib.moe_combine(self.handle, p.rows, None, p.w, p.shared, p.residual,
                                         p.T, p.k, p.d, _p(y), _stream(stream)))

    def moe_tile_weights(self, src: "DeviceExperts", dst_gate_up, dst_down, stream=None):
        w = src.struct()
        self._check(self.lib.moe_tile_weights(self.handle, ctypes.byref(w), _p(dst_gate_up),
                                              _p(dst_down), _stream(stream)))

    def moe_probe_read(self, buf, nbytes: int, sink, blocks: int = 0, stream=None):
        self._check(self.lib.moe_probe_read(self.handle, _p(buf), nbytes, blocks, _p(sink),
                                            _stream(stream)))

    def moe_probe_mfma(self, shape: int, iters: int, sink, blocks: int = 0, stream=None):
        self._check(self.lib.moe_probe_mfma(self.handle, shape, iters, blocks, _p(sink),
                                            _stream(stream)))

    def moe_timing(self, capacity: int):
        self._check(self.lib.moe_timing(self.handle, capacity))

    def moe_timing_read(self) -> dict:
        """{kernel name: (launches, total ms)} since the last read."""
        buf = (moe_kernel_time * 32)()
        n = ctypes.c_int()
        self._check(self.lib.moe_timing_read(self.handle, buf, 32, ctypes.byref(n)))
        return {buf[i].name.decode(): (buf[i].launches, buf[i].total_ms)
                for i in range(min(n.value, 32))}

    def moe_combine(self, rows, token_row, topk_w, shared, residual, T, k, d, y, stream=None):
        self._check(self.lib.moe_combine(self.handle, _p(rows), _p(token_row), _p(topk_w),
                                         _p(shared), _p(residual), T, k, d, _p(y),
                                         _stream(stream)))


@dataclass
class DeviceExperts:
    """Expert weights resident on the GPU in one of the moe_wfmt formats."""
    fmt: int
    n_experts: int
    d: int
    inter: int
    w_gate_up: torch.Tensor
    w_down: torch.Tensor
    s_gate_up: Optional[torch.Tensor] = None
    s_down: Optional[torch.Tensor] = None
    layout: int = MOE_LAYOUT_ROWS

    def struct(self) -> moe_weights:
        return moe_weights(self.fmt, self.layout, self.n_experts, self.d, self.inter,
                           _p(self.w_gate_up), _p(self.s_gate_up), _p(self.w_down),
                           _p(self.s_down))

    def tiled(self, ctx: "Context") -> "DeviceExperts":
        """A copy of the codes in MOE_LAYOUT_TILED order (scales shared)."""
        if self.fmt == MOE_W_FP32 or self.layout == MOE_LAYOUT_TILED:
            return self
        gu = torch.empty_like(self.w_gate_up)
        dn = torch.empty_like(self.w_down)
        ctx.moe_tile_weights(self, gu, dn)
        return DeviceExperts(self.fmt, self.n_experts, self.d, self.inter, gu, dn,
                             self.s_gate_up, self.s_down, MOE_LAYOUT_TILED)

    @property
    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size()
                   for t in (self.w_gate_up, self.w_down, self.s_gate_up, self.s_down)
                   if t is not None)

    @staticmethod
    def upload(w, device) -> "DeviceExperts":
        """From a synth.ExpertWeights (host numpy)."""
        fmt = FMT[w.fmt]
        if w.fmt in ("int4_b32", "int4_b128"):
            gu, dn = w.gu_packed, w.dn_packed
        else:
            gu, dn = w.gu, w.dn
        t = lambda a: None if a is None else torch.from_numpy(a).to(device)
        return DeviceExperts(fmt, w.E, w.d, w.inter, t(gu), t(dn), t(w.gu_s), t(w.dn_s))

    def select(self, ids) -> "DeviceExperts":
        """Experts `ids` (in that order) as a new dense set, gathered whole on
        the device; both code layouts keep each expert's bytes contiguous, so
        format and layout carry over."""
        dev = self.w_gate_up.device
        ix = torch.as_tensor([int(i) for i in ids], dtype=torch.long, device=dev)
        if ix.numel() == 0 or int(ix.min()) < 0 or int(ix.max()) >= self.n_experts:
            raise ValueError(f"expert ids must be in [0, {self.n_experts})")
        g = lambda a: None if a is None else a.index_select(0, ix)
        return DeviceExperts(self.fmt, int(ix.numel()), self.d, self.inter, g(self.w_gate_up),
                             g(self.w_down), g(self.s_gate_up), g(self.s_down), self.layout)

    def clone(self) -> "DeviceExperts":
        c = lambda a: None if a is None else a.clone()
        return DeviceExperts(self.fmt, self.n_experts, self.d, self.inter, c(self.w_gate_up),
                             c(self.w_down), c(self.s_gate_up), c(self.s_down), self.layout)
