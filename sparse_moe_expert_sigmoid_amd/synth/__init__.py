"""Seeded synthetic inputs for the routed-MoE layer (host side).

This module draws numbers only; it holds none of the layer's arithmetic.
The tests feed the same arrays to the CPU oracle and to the HIP path, and the
benchmark uses them as its workload.  The generator itself is the C file
beside this one (counter-based SplitMix64, documented there).

The layer shapes and value distributions follow the workloads of the two
models the pages convert:

* Kimi-Linear-48B-A3B (DETAILS.md of the LiteRT-LM conversion, "Conversion
  notes", bullet on the mixture of experts): 256 routed experts, top 8,
  sigmoid scores with a selection bias, weights renormalised and scaled by
  2.446, int8 experts with one scale per output row and expert; the APEX-GGUF
  model card ("Method") gives the expert intermediate size 2048.
* Qwen3-30B-A3B (litert-community model card, "Available Artifacts" and
  "Conversion Notes"): 128 experts, top 8, softmax router renormalised over
  the 8, int4 experts in blocks of 32 with fp32 scales raised to 2^-14.

The hidden sizes (2304, 2048), the Qwen3 intermediate size (768) and all
value distributions are not on the pages; they are this workload's synthetic
choices (stated in the layer specs below).
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmoe_synth.so")
_lib = None


_DEV_LIB_PATH = os.path.join(_HERE, "libmoe_synth_dev.so")
_dev_lib = None
_HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build(verbose: bool = False, device: bool = True) -> str:
    """Compile the host generator with gcc and its device twin with hipcc for
    gfx950 (always recompiles both; device=False skips the twin)."""
    import subprocess
    src = os.path.join(_HERE, "synth.c")
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-shared",
           "-fPIC", "-std=c11", "-Wall", "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    if device:
        dsrc = os.path.join(_HERE, "synth_dev.hip")
        dtmp = _DEV_LIB_PATH + ".tmp"
        cmd = [_HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
               "-ffp-contract=off", "-Wall", "-Xclang", "-target-feature", "-Xclang",
               "-packed-fp32-ops", "-o", dtmp, dsrc]
        if verbose:
            print(" ".join(cmd))
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {dsrc}:\n{r.stderr}")
        os.replace(dtmp, _DEV_LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    u64, i64, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_void_p
    lib.synth_key.argtypes = [u64, u64]
    lib.synth_key.restype = u64
    lib.synth_hash.argtypes = [u64, u64, u64, i64, vp]
    lib.synth_splitmix64.argtypes = [u64, i64, vp]
    lib.synth_uniform.argtypes = [u64, u64, i64, ctypes.c_float, ctypes.c_float, vp]
    lib.synth_normal.argtypes = [u64, u64, i64, ctypes.c_double, vp]
    lib.synth_randint8.argtypes = [u64, u64, i64, ctypes.c_int, ctypes.c_int, vp]
    lib.synth_randint8_at.argtypes = [u64, u64, u64, i64, ctypes.c_int, ctypes.c_int, vp]
    lib.synth_scale_at.argtypes = [u64, u64, u64, i64, ctypes.c_float, u64, vp, ctypes.c_int,
                                   ctypes.c_float, vp]
    lib.synth_scale.argtypes = [u64, u64, i64, ctypes.c_float, u64, vp, ctypes.c_int,
                                ctypes.c_float, vp]
    lib.synth_pack_int4.argtypes = [vp, i64, vp]
    for f in ("synth_splitmix64", "synth_hash", "synth_uniform", "synth_normal", "synth_randint8",
              "synth_scale", "synth_pack_int4", "synth_randint8_at", "synth_scale_at"):
        getattr(lib, f).restype = None
    _lib = lib
    return lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


# --------------------------------------------------------------------------
# primitive draws
# --------------------------------------------------------------------------

def splitmix64(state: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.uint64)
    _load().synth_splitmix64(state, n, _ptr(out))
    return out


def hashes(seed: int, tid: int, n: int, start: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint64)
    _load().synth_hash(seed, tid, start, n, _ptr(out))
    return out


def uniform(seed: int, tid: int, shape, lo: float, hi: float) -> np.ndarray:
    out = np.empty(shape, dtype=np.float32)
    _load().synth_uniform(seed, tid, out.size, lo, hi, _ptr(out))
    return out


def normal(seed: int, tid: int, shape, std: float) -> np.ndarray:
    out = np.empty(shape, dtype=np.float32)
    _load().synth_normal(seed, tid, out.size, float(std), _ptr(out))
    return out


def randint8(seed: int, tid: int, shape, lo: int, hi: int, start: int = 0) -> np.ndarray:
    """Elements start .. start+size-1 of the int8 tensor (seed, tid)."""
    out = np.empty(shape, dtype=np.int8)
    _load().synth_randint8_at(seed, tid, start, out.size, lo, hi, _ptr(out))
    return out


# int4 scale values that exercise the 2^-14 clamp: zero, an fp32 subnormal,
# 2^-20 and just below 2^-14; about 1 in 1024 blocks draws one of them and
# about 1 in 1024 others sits exactly at 2^-14.
CLAMP_SPECIALS = np.array([0.0, 1e-40, 2.0 ** -20, 0.999 * 2.0 ** -14], dtype=np.float32)
TWO_M14 = np.float32(2.0 ** -14)


def scales(seed: int, tid: int, shape, c: float, special_tid: int = 0,
           start: int = 0) -> np.ndarray:
    """Elements start .. start+size-1 of the scale tensor (seed, tid)."""
    out = np.empty(shape, dtype=np.float32)
    sp = CLAMP_SPECIALS
    _load().synth_scale_at(seed, tid, start, out.size, float(np.float32(c)), special_tid,
                           _ptr(sp), len(sp), float(TWO_M14), _ptr(out))
    return out


# --------------------------------------------------------------------------
# device twin (libmoe_synth_dev.so): the same draws written straight into HBM
# --------------------------------------------------------------------------

def _load_dev():
    global _dev_lib
    if _dev_lib is not None:
        return _dev_lib
    if not os.path.exists(_DEV_LIB_PATH):
        raise RuntimeError(f"{_DEV_LIB_PATH} is not built; run build() first")
    lib = ctypes.CDLL(_DEV_LIB_PATH)
    u64, i64, vp, ci = ctypes.c_uint64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    lib.synth_dev_randint8.argtypes = [u64, u64, u64, i64, ci, ci, vp, vp]
    lib.synth_dev_scale.argtypes = [u64, u64, u64, i64, ctypes.c_float, u64, vp, ci,
                                    ctypes.c_float, vp, vp]
    lib.synth_dev_randint8.restype = ci
    lib.synth_dev_scale.restype = ci
    _dev_lib = lib
    return lib


def _stream_handle(stream):
    import torch
    st = torch.cuda.current_stream() if stream is None else stream
    return st.cuda_stream


def dev_randint8(seed: int, tid: int, out, lo: int, hi: int, start: int = 0, stream=None):
    """Fill the int8 torch tensor `out` (contiguous, on the GPU) with elements
    start .. start+numel-1 of the tensor (seed, tid)."""
    assert out.is_contiguous() and out.dtype.itemsize == 1
    rc = _load_dev().synth_dev_randint8(seed, tid, start, out.numel(), lo, hi, out.data_ptr(),
                                        _stream_handle(stream))
    if rc != 0:
        raise RuntimeError(f"synth_dev_randint8 failed (hip error {rc})")
    return out


def dev_scales(seed: int, tid: int, out, c: float, special_tid: int = 0, start: int = 0,
               stream=None):
    """Fill the fp32 torch tensor `out` on the GPU with scale elements
    start .. start+numel-1 of (seed, tid), as scales() draws them."""
    assert out.is_contiguous() and out.dtype.itemsize == 4
    sp = CLAMP_SPECIALS
    rc = _load_dev().synth_dev_scale(seed, tid, start, out.numel(), float(np.float32(c)),
                                     special_tid, _ptr(sp), len(sp), float(TWO_M14),
                                     out.data_ptr(), _stream_handle(stream))
    if rc != 0:
        raise RuntimeError(f"synth_dev_scale failed (hip error {rc})")
    return out


def pack_int4(codes: np.ndarray) -> np.ndarray:
    """Two int4 codes per byte along the last axis (element 2i in the low nibble)."""
    assert codes.dtype == np.int8 and codes.shape[-1] % 2 == 0
    codes = np.ascontiguousarray(codes)
    out = np.empty(codes.shape[:-1] + (codes.shape[-1] // 2,), dtype=np.uint8)
    _load().synth_pack_int4(_ptr(codes), out.size, _ptr(out))
    return out


# --------------------------------------------------------------------------
# layer specs
# --------------------------------------------------------------------------

ROUTER_SIGMOID_BIAS = "sigmoid_bias"
ROUTER_SOFTMAX = "softmax"
FMT_FP32 = "fp32"
FMT_INT8_ROW = "int8_row"
FMT_INT4_B32 = "int4_b32"
FMT_INT4_B128 = "int4_b128"
INT4_BLOCK = {FMT_INT4_B32: 32, FMT_INT4_B128: 128}

KIMI_ROUTED_SCALE = float(np.float32(2.446))


@dataclass(frozen=True)
class LayerSpec:
    name: str
    T: int
    d: int
    E: int
    k: int
    inter: int
    router: str
    scale: float
    fmt: str
    shared: Optional[str]        # None, FMT_FP32 or FMT_INT8_ROW
    shared_inter: int
    wseed: int                   # weights (router, bias, experts, shared)
    xseed: int                   # activations
    dn_gain: float = 1.0         # factor on the down-projection scales

    @property
    def R(self) -> int:          # routed rows: every token picks k experts
        return self.T * self.k


def _seed(i: int) -> int:
    return 0x4D6F4500 + i


SPECS = {
    # Tiny single layer: T=32, d=512, 32 experts, top 8, I=256, fp32 shared.
    "tiny": LayerSpec("tiny", 32, 512, 32, 8, 256, ROUTER_SIGMOID_BIAS, KIMI_ROUTED_SCALE,
                      FMT_INT8_ROW, FMT_FP32, 256, _seed(0), _seed(0)),
    # Kimi-shaped decode step: T=8, d=2304, 256 experts, top 8, I=2048, int8 shared.
    "kimi_decode": LayerSpec("kimi_decode", 8, 2304, 256, 8, 2048, ROUTER_SIGMOID_BIAS,
                             KIMI_ROUTED_SCALE, FMT_INT8_ROW, FMT_INT8_ROW, 2048,
                             _seed(1), _seed(1)),
    # The same layer at prefill, T=1024 (same weights, new activations).
    "kimi_prefill": LayerSpec("kimi_prefill", 1024, 2304, 256, 8, 2048, ROUTER_SIGMOID_BIAS,
                              KIMI_ROUTED_SCALE, FMT_INT8_ROW, FMT_INT8_ROW, 2048,
                              _seed(1), _seed(2)),
    # Qwen3-shaped layer: d=2048, 128 experts, softmax top 8, I=768, int4 b32, no shared.
    "qwen_decode": LayerSpec("qwen_decode", 1, 2048, 128, 8, 768, ROUTER_SOFTMAX, 1.0,
                             FMT_INT4_B32, None, 0, _seed(3), _seed(3)),
    "qwen_prefill": LayerSpec("qwen_prefill", 128, 2048, 128, 8, 768, ROUTER_SOFTMAX, 1.0,
                              FMT_INT4_B32, None, 0, _seed(3), _seed(13)),
}


def spec(name: str, **kw) -> LayerSpec:
    s = SPECS[name]
    return replace(s, **kw) if kw else s


# tensor ids inside one seed
TID_X, TID_WR, TID_BIAS = 1, 2, 3
TID_GU, TID_GU_S, TID_DN, TID_DN_S = 4, 5, 6, 7
TID_SH_GU, TID_SH_GU_S, TID_SH_DN, TID_SH_DN_S = 8, 9, 10, 11
TID_GU_SPECIAL, TID_DN_SPECIAL, TID_SH_GU_SPECIAL, TID_SH_DN_SPECIAL = 12, 13, 14, 15


@dataclass
class ExpertWeights:
    """Weights of a set of SwiGLU experts in one storage format.

    fmt == int8_row: gu [E, 2I, d] int8, gu_s [E, 2I] fp32, dn [E, d, I] int8, dn_s [E, d]
    fmt == int4_b32: gu [E, 2I, d] int8 codes in [-8, 7], gu_s [E, 2I, d/32]
                     dn [E, d, I] int8 codes,               dn_s [E, d, I/32]
                     (gu_packed / dn_packed hold the nibble-packed copies)
    fmt == int4_b128: as int4_b32 with scales [E, 2I, d/128] and [E, d, I/128]
    fmt == fp32:     gu [E, 2I, d] fp32, dn [E, d, I] fp32, no scales
    Rows 0..I-1 of gu are the gate projection, rows I..2I-1 the up projection.
    """
    fmt: str
    E: int
    d: int
    inter: int
    gu: np.ndarray
    dn: np.ndarray
    gu_s: Optional[np.ndarray] = None
    dn_s: Optional[np.ndarray] = None
    gu_packed: Optional[np.ndarray] = None
    dn_packed: Optional[np.ndarray] = None


@dataclass
class LayerInputs:
    spec: LayerSpec
    x: np.ndarray
    wr: np.ndarray
    bias: Optional[np.ndarray]
    experts: ExpertWeights
    shared: Optional[ExpertWeights] = None
    extra: dict = field(default_factory=dict)


def make_experts(fmt: str, E: int, d: int, inter: int, seed: int, tids,
                 dn_gain: float = 1.0) -> ExpertWeights:
    t_gu, t_gu_s, t_dn, t_dn_s, t_gu_sp, t_dn_sp = tids
    if fmt == FMT_FP32:
        gu = normal(seed, t_gu, (E, 2 * inter, d), 1.0 / math.sqrt(d))
        dn = normal(seed, t_dn, (E, d, inter), 1.0 / math.sqrt(inter))
        return ExpertWeights(fmt, E, d, inter, gu, dn)
    if fmt == FMT_INT8_ROW:
        gu = randint8(seed, t_gu, (E, 2 * inter, d), -127, 127)
        dn = randint8(seed, t_dn, (E, d, inter), -127, 127)
        gu_s = scales(seed, t_gu_s, (E, 2 * inter), 1.0 / (127.0 * math.sqrt(d)))
        dn_s = scales(seed, t_dn_s, (E, d), dn_gain / (127.0 * math.sqrt(inter)))
        return ExpertWeights(fmt, E, d, inter, gu, dn, gu_s, dn_s)
    if fmt in INT4_BLOCK:
        B = INT4_BLOCK[fmt]
        assert d % B == 0 and inter % B == 0
        gu = randint8(seed, t_gu, (E, 2 * inter, d), -8, 7)
        dn = randint8(seed, t_dn, (E, d, inter), -8, 7)
        gu_s = scales(seed, t_gu_s, (E, 2 * inter, d // B), 1.0 / (8.0 * math.sqrt(d)),
                      special_tid=t_gu_sp)
        dn_s = scales(seed, t_dn_s, (E, d, inter // B), dn_gain / (8.0 * math.sqrt(inter)),
                      special_tid=t_dn_sp)
        return ExpertWeights(fmt, E, d, inter, gu, dn, gu_s, dn_s,
                             pack_int4(gu), pack_int4(dn))
    raise ValueError(fmt)


def make_x(s: LayerSpec, T: Optional[int] = None) -> np.ndarray:
    return normal(s.xseed, TID_X, (s.T if T is None else T, s.d), 1.0)


def make_layer(s: LayerSpec, with_x: bool = True) -> LayerInputs:
    wr = normal(s.wseed, TID_WR, (s.E, s.d), 1.0 / math.sqrt(s.d))
    bias = (uniform(s.wseed, TID_BIAS, (s.E,), -0.1, 0.1)
            if s.router == ROUTER_SIGMOID_BIAS else None)
    experts = make_experts(s.fmt, s.E, s.d, s.inter, s.wseed,
                           (TID_GU, TID_GU_S, TID_DN, TID_DN_S, TID_GU_SPECIAL, TID_DN_SPECIAL),
                           s.dn_gain)
    shared = None
    if s.shared is not None:
        shared = make_experts(s.shared, 1, s.d, s.shared_inter, s.wseed,
                              (TID_SH_GU, TID_SH_GU_S, TID_SH_DN, TID_SH_DN_S,
                               TID_SH_GU_SPECIAL, TID_SH_DN_SPECIAL), s.dn_gain)
    x = make_x(s) if with_x else None
    return LayerInputs(s, x, wr, bias, experts, shared)


# --------------------------------------------------------------------------
# slices of one layer's experts (host), and whole layers drawn on the device
# --------------------------------------------------------------------------

_ROUTED_TIDS = (TID_GU, TID_GU_S, TID_DN, TID_DN_S, TID_GU_SPECIAL, TID_DN_SPECIAL)
_SHARED_TIDS = (TID_SH_GU, TID_SH_GU_S, TID_SH_DN, TID_SH_DN_S, TID_SH_GU_SPECIAL,
                TID_SH_DN_SPECIAL)


def expert_slice(s: LayerSpec, experts, shared: bool = False) -> ExpertWeights:
    """The listed experts of the layer (routed, or the shared one with
    experts=[0]) as an ExpertWeights with E = len(experts), in list order;
    equal to indexing the arrays make_layer() draws, without drawing the rest."""
    fmt = s.shared if shared else s.fmt
    inter = s.shared_inter if shared else s.inter
    d = s.d
    t_gu, t_gu_s, t_dn, t_dn_s, t_gu_sp, t_dn_sp = _SHARED_TIDS if shared else _ROUTED_TIDS
    if fmt not in (FMT_INT8_ROW, FMT_INT4_B32, FMT_INT4_B128):
        raise ValueError(f"expert_slice: format {fmt} is drawn whole only")
    n = len(experts)
    lo, hi = (-127, 127) if fmt == FMT_INT8_ROW else (-8, 7)
    gu = np.empty((n, 2 * inter, d), np.int8)
    dn = np.empty((n, d, inter), np.int8)
    if fmt == FMT_INT8_ROW:
        gu_s = np.empty((n, 2 * inter), np.float32)
        dn_s = np.empty((n, d), np.float32)
    else:
        B = INT4_BLOCK[fmt]
        gu_s = np.empty((n, 2 * inter, d // B), np.float32)
        dn_s = np.empty((n, d, inter // B), np.float32)
    c_gu = 1.0 / ((127.0 if fmt == FMT_INT8_ROW else 8.0) * math.sqrt(d))
    c_dn = s.dn_gain / ((127.0 if fmt == FMT_INT8_ROW else 8.0) * math.sqrt(inter))
    sp_gu, sp_dn = (0, 0) if fmt == FMT_INT8_ROW else (t_gu_sp, t_dn_sp)
    for q, e in enumerate(experts):
        e = int(e)
        gu[q] = randint8(s.wseed, t_gu, gu[q].shape, lo, hi, start=e * gu[q].size)
        dn[q] = randint8(s.wseed, t_dn, dn[q].shape, lo, hi, start=e * dn[q].size)
        gu_s[q] = scales(s.wseed, t_gu_s, gu_s[q].shape, c_gu, sp_gu, start=e * gu_s[q].size)
        dn_s[q] = scales(s.wseed, t_dn_s, dn_s[q].shape, c_dn, sp_dn, start=e * dn_s[q].size)
    w = ExpertWeights(fmt, n, d, inter, gu, dn, gu_s, dn_s)
    if fmt in INT4_BLOCK:
        w.gu_packed, w.dn_packed = pack_int4(gu), pack_int4(dn)
    return w


def dev_int4_experts(s: LayerSpec, device, stream=None):
    """Packed codes and block scales of the layer's routed int4 experts drawn on
    the GPU, row-major, bit-identical to make_experts()' packed arrays:
    (gu [E,2I,d/2] uint8, gu_s [E,2I,d/B] fp32, dn [E,d,I/2] uint8,
    dn_s [E,d,I/B] fp32), B the format's block."""
    import torch
    if s.fmt not in INT4_BLOCK:
        raise ValueError("dev_int4_experts draws int4 experts only")
    B = INT4_BLOCK[s.fmt]
    E, d, inter = s.E, s.d, s.inter
    t_gu, t_gu_s, t_dn, t_dn_s, t_gu_sp, t_dn_sp = _ROUTED_TIDS

    def packed(tid, shape):
        c = torch.empty(shape, dtype=torch.int8, device=device)
        dev_randint8(s.wseed, tid, c, -8, 7, stream=stream)
        c16 = c.to(torch.int16)
        del c
        out = ((c16[..., 0::2] & 0xF) | ((c16[..., 1::2] & 0xF) << 4)).to(torch.uint8)
        return out.contiguous()

    gu = packed(t_gu, (E, 2 * inter, d))
    dn = packed(t_dn, (E, d, inter))
    gu_s = torch.empty((E, 2 * inter, d // B), dtype=torch.float32, device=device)
    dn_s = torch.empty((E, d, inter // B), dtype=torch.float32, device=device)
    dev_scales(s.wseed, t_gu_s, gu_s, 1.0 / (8.0 * math.sqrt(d)), special_tid=t_gu_sp,
               stream=stream)
    dev_scales(s.wseed, t_dn_s, dn_s, s.dn_gain / (8.0 * math.sqrt(inter)), special_tid=t_dn_sp,
               stream=stream)
    return gu, gu_s, dn, dn_s


def dev_int8_experts(s: LayerSpec, device, shared: bool = False, stream=None):
    """Codes and scales of the layer's routed experts (or its shared expert)
    drawn on the GPU, row-major, bit-identical to make_experts():
    (gu [E,2I,d] int8, gu_s [E,2I] fp32, dn [E,d,I] int8, dn_s [E,d] fp32)."""
    import torch
    fmt = s.shared if shared else s.fmt
    if fmt != FMT_INT8_ROW:
        raise ValueError("dev_int8_experts draws int8 per-row experts only")
    E = 1 if shared else s.E
    inter = s.shared_inter if shared else s.inter
    d = s.d
    t_gu, t_gu_s, t_dn, t_dn_s, _, _ = _SHARED_TIDS if shared else _ROUTED_TIDS
    gu = torch.empty((E, 2 * inter, d), dtype=torch.int8, device=device)
    dn = torch.empty((E, d, inter), dtype=torch.int8, device=device)
    gu_s = torch.empty((E, 2 * inter), dtype=torch.float32, device=device)
    dn_s = torch.empty((E, d), dtype=torch.float32, device=device)
    dev_randint8(s.wseed, t_gu, gu, -127, 127, stream=stream)
    dev_randint8(s.wseed, t_dn, dn, -127, 127, stream=stream)
    dev_scales(s.wseed, t_gu_s, gu_s, 1.0 / (127.0 * math.sqrt(d)), stream=stream)
    dev_scales(s.wseed, t_dn_s, dn_s, s.dn_gain / (127.0 * math.sqrt(inter)), stream=stream)
    return gu, gu_s, dn, dn_s


# --------------------------------------------------------------------------
# the 26-layer Kimi-shaped stack with Zipf-skewed routing
# --------------------------------------------------------------------------
#
# Layer l has its own weights (seed 0x4D6F4400 + l) and a selection bias
#     b_l[e] = fp32( u_l[e] + alpha * r_l(e)^-1.1 ),   u_l ~ U(-0.1, 0.1)
# where r_l is a seeded permutation of the ranks 1..E.  alpha is chosen once
# (tests/golden/make_stack_zipf.py, by bisection with the oracle's router on
# layer 0 at T=4096) so that the 64 most-selected experts take about 73% of
# the selections, the concentration the code-corpus routing statistics of
# the Kimi-Linear-48B-A3B-Code-CMF listing ("How it was made") report.  The
# stack is x_{l+1} = x_l + MoE_l(x_l): the residual sits outside the layer
# (Qwen3-30B-A3B model card, "Conversion Notes") and no norm is given.

STACK_LAYERS = 26
ZIPF_S = 1.1
TID_ZIPF_RANK = 16
STACK_X_SEED = _seed(4)
ZIPF_FILE = os.path.join(os.path.dirname(os.path.dirname(_HERE)), "tests", "golden",
                         "kimi_stack_zipf.json")


def stack_wseed(l: int) -> int:
    return 0x4D6F4400 + l


def zipf_ranks(seed: int, E: int) -> np.ndarray:
    """A seeded permutation of 1..E: expert e gets rank r[e] (1 = most favoured)."""
    order = np.argsort(hashes(seed, TID_ZIPF_RANK, E), kind="stable")
    r = np.empty(E, np.int64)
    r[order] = np.arange(1, E + 1)
    return r


def zipf_bias(seed: int, E: int, alpha: float) -> np.ndarray:
    u = uniform(seed, TID_BIAS, (E,), -0.1, 0.1).astype(np.float64)
    r = zipf_ranks(seed, E).astype(np.float64)
    return (u + alpha * r ** -ZIPF_S).astype(np.float32)


def stack_alpha() -> float:
    import json
    with open(ZIPF_FILE) as f:
        return float(json.load(f)["alpha"])


@dataclass(frozen=True)
class StackSpec:
    name: str
    layers: int
    T: int
    alpha: float                 # Zipf strength of the selection bias (sigmoid router)
    base: LayerSpec
    wseed0: int = 0x4D6F4400     # layer l draws its weights from seed wseed0 + l

    def layer(self, l: int) -> LayerSpec:
        return replace(self.base, name=f"{self.name}[{l}]", T=self.T, wseed=self.wseed0 + l,
                       xseed=STACK_X_SEED)


def stack_spec(T: int, layers: int = STACK_LAYERS, alpha: Optional[float] = None,
               name: Optional[str] = None) -> StackSpec:
    a = stack_alpha() if alpha is None else float(alpha)
    return StackSpec(name or f"kimi_stack_T{T}", layers, T, a, SPECS["kimi_decode"])


def stack_router(st: StackSpec, l: int):
    """(w_router [E,d] fp32, bias [E] fp32 or None) of layer l: the Zipf-skewed
    selection bias for a sigmoid router, none for a softmax router."""
    s = st.layer(l)
    wr = normal(s.wseed, TID_WR, (s.E, s.d), 1.0 / math.sqrt(s.d))
    if s.router != ROUTER_SIGMOID_BIAS:
        return wr, None
    return wr, zipf_bias(s.wseed, s.E, st.alpha)


# The 48-layer Qwen3-shaped stack (Qwen3-30B-A3B model card: 48 layers of 128
# experts, 8 per token; the int4 block-32 file): every layer as the
# qwen_decode layer (d=2048, softmax top 8 of 128, I=768, no shared expert)
# with its own weights (seed 0x51573300 + l).  A softmax router has no
# selection bias, so the routing is what random router rows give.  Without a
# norm between layers a random SwiGLU residual stream is unstable: the FFN is
# roughly quadratic in x, and with the single layer's scales some tokens grow
# about threefold per layer from layer 6 on and overflow by layer 12 (with
# 1/8 of them, one token in 16 still overflows by layer 27).  The down
# projections of this stack carry 1/QWEN_STACK_DN_GAIN_INV of the single
# layer's scales: with it the first 64 tokens of the stack input stay bounded
# through all 48 layers (max per-layer rms of y 0.006 against rms(x) ~ 1;
# checked with the oracle).
QWEN_STACK_LAYERS = 48
QWEN_STACK_DN_GAIN_INV = 64


def qwen_stack_spec(T: int, layers: int = QWEN_STACK_LAYERS,
                    name: Optional[str] = None) -> StackSpec:
    base = replace(SPECS["qwen_decode"], dn_gain=1.0 / QWEN_STACK_DN_GAIN_INV)
    return StackSpec(name or f"qwen_stack_T{T}", layers, T, 0.0, base, wseed0=0x51573300)


def stack_x(st: StackSpec) -> np.ndarray:
    """x_0 [T, d]: the first T rows of one N(0,1) tensor (T=1 is row 0 of T=4096)."""
    return normal(STACK_X_SEED, TID_X, (st.T, st.base.d), 1.0)


# ------------------------------------------------------------ float weights for the quantizer
# Expert e's float gate/up [2I, d] and down [d, I] matrices, N(0, QUANT_STD^2)
# (the spread of trained projection weights), one tensor id per (expert, part)
# so that any expert can be drawn alone.
TID_FLOAT_BASE = 0x100
QUANT_STD = 0.02


def float_expert(s: LayerSpec, e: int, part: str) -> np.ndarray:
    if part not in ("gu", "dn"):
        raise ValueError(part)
    shape = (2 * s.inter, s.d) if part == "gu" else (s.d, s.inter)
    return normal(s.wseed, TID_FLOAT_BASE + 2 * e + (part == "dn"), shape, QUANT_STD)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 (round to nearest even), as uint16 bit patterns."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)
