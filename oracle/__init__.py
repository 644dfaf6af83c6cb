"""CPU oracle for the routed mixture-of-experts layer — TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline
leg may import this package.  The product path (the HIP library and its
binding) never calls it and shares no code with it.

The arithmetic lives in ``oracle.c`` (plain C, fp64, sums in index order);
this module is argument marshalling over ctypes.  See oracle.c for the
passages of the pages each function follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

ROUTER = {"sigmoid_bias": 0, "softmax": 1}
FMT = {"fp32": 0, "int8_row": 1, "int4_b32": 2, "int4_b128": 3}
ACT = {"silu": 0, "gelu_tanh": 1}
INT4_BLOCK = {"int4_b32": 32, "int4_b128": 128}


def build(verbose: bool = False) -> str:
    """Compile the oracle with gcc (always recompiles)."""
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-std=c11",
           "-Wall", "-Wextra", "-shared", "-fPIC", "-o", tmp,
           os.path.join(_HERE, "oracle.c"), "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Experts(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int), ("E", ctypes.c_int), ("d", ctypes.c_int),
                ("inter", ctypes.c_int), ("gu", ctypes.c_void_p), ("gu_s", ctypes.c_void_p),
                ("dn", ctypes.c_void_p), ("dn_s", ctypes.c_void_p), ("act", ctypes.c_int)]


class _Layer(ctypes.Structure):
    _fields_ = [("router", ctypes.c_int), ("k", ctypes.c_int), ("scale", ctypes.c_float),
                ("wr", ctypes.c_void_p), ("bias", ctypes.c_void_p), ("experts", _Experts),
                ("has_shared", ctypes.c_int), ("shared", _Experts)]


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.oracle_sigmoid.argtypes = [ctypes.c_double]
    lib.oracle_sigmoid.restype = ctypes.c_double
    lib.oracle_silu.argtypes = [ctypes.c_double]
    lib.oracle_silu.restype = ctypes.c_double
    lib.oracle_gelu_tanh.argtypes = [ctypes.c_double]
    lib.oracle_gelu_tanh.restype = ctypes.c_double
    lib.oracle_route.argtypes = [ci, vp, vp, vp, i64, ci, ci, ci, ctypes.c_float, vp, vp, vp, vp]
    lib.oracle_route.restype = ci
    lib.oracle_permute.argtypes = [vp, i64, ci, ci, vp, vp, vp]
    lib.oracle_permute.restype = ci
    lib.oracle_ffn.argtypes = [ctypes.POINTER(_Experts), ci, vp, vp, vp]
    lib.oracle_ffn.restype = None
    lib.oracle_expert_rows.argtypes = [ctypes.POINTER(_Experts), vp, vp, vp, vp]
    lib.oracle_expert_rows.restype = ci
    lib.oracle_combine.argtypes = [vp, vp, vp, vp, vp, i64, ci, ci, vp]
    lib.oracle_combine.restype = None
    lib.oracle_layer.argtypes = [ctypes.POINTER(_Layer), vp, i64, vp, vp, vp, vp]
    lib.oracle_layer.restype = ci
    lib.oracle_coverage_set.argtypes = [vp, ci, ctypes.c_double, ci, vp]
    lib.oracle_coverage_set.restype = ci
    lib.oracle_quantize_int8_rows.argtypes = [vp, i64, ci, vp, vp]
    lib.oracle_quantize_int8_rows.restype = ci
    lib.oracle_quantize_int4_blocks.argtypes = [vp, i64, ci, ci, vp, vp]
    lib.oracle_quantize_int4_blocks.restype = ci
    _lib = lib
    return lib


def set_threads(n: int) -> None:
    """OpenMP threads of the oracle's parallel loops from now on (for timing it
    on one thread); the OpenMP runtime is the one the oracle library loaded."""
    _load()
    ctypes.CDLL("libgomp.so.1").omp_set_num_threads(int(n))


def _p(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data


def _f32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float32)


@dataclass
class Experts:
    """Expert weights as the oracle reads them (int4 codes unpacked, one int8 each)."""
    fmt: str
    gu: np.ndarray
    dn: np.ndarray
    gu_s: Optional[np.ndarray] = None
    dn_s: Optional[np.ndarray] = None
    act: str = "silu"

    def _struct(self):
        E, n2, d = self.gu.shape
        inter = n2 // 2
        assert self.dn.shape == (E, d, inter)
        if self.fmt == "fp32":
            assert self.gu.dtype == np.float32 and self.dn.dtype == np.float32
        else:
            assert self.gu.dtype == np.int8 and self.dn.dtype == np.int8
            if self.fmt == "int8_row":
                assert self.gu_s.shape == (E, n2) and self.dn_s.shape == (E, d)
            else:
                B = INT4_BLOCK[self.fmt]
                assert d % B == 0 and inter % B == 0
                assert self.gu_s.shape == (E, n2, d // B)
                assert self.dn_s.shape == (E, d, inter // B)
        keep = [np.ascontiguousarray(self.gu), np.ascontiguousarray(self.dn),
                _f32(self.gu_s), _f32(self.dn_s)]
        s = _Experts(FMT[self.fmt], E, d, inter, _p(keep[0]), _p(keep[2]), _p(keep[1]),
                     _p(keep[3]), ACT[self.act])
        return s, keep

    @staticmethod
    def of(w, act: str = "silu") -> "Experts":
        """From a synth.ExpertWeights."""
        return Experts(w.fmt, w.gu, w.dn, w.gu_s, w.dn_s, act)


def sigmoid(z: float) -> float:
    return _load().oracle_sigmoid(z)


def silu(z: float) -> float:
    return _load().oracle_silu(z)


def gelu_tanh(z: float) -> float:
    return _load().oracle_gelu_tanh(z)


def route(router: str, x, wr, bias, k: int, scale: float, want_logits: bool = False):
    """Returns idx [T,k] int32, w [T,k] float64, gap [T] float64 (and logits [T,E])."""
    x, wr, bias = _f32(x), _f32(wr), _f32(bias)
    T, d = x.shape
    E = wr.shape[0]
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    gap = np.empty(T, np.float64)
    logits = np.empty((T, E), np.float64) if want_logits else None
    rc = _load().oracle_route(ROUTER[router], _p(x), _p(wr), _p(bias), T, d, E, k, scale,
                              _p(idx), _p(w), _p(gap), _p(logits))
    if rc != 0:
        raise ValueError(f"oracle_route failed ({rc})")
    return (idx, w, gap, logits) if want_logits else (idx, w, gap)


def permute(idx, E: int):
    """Returns offsets [E+1], row_token [T*k], token_row [T*k] (all int32)."""
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    T, k = idx.shape
    offsets = np.empty(E + 1, np.int32)
    row_token = np.empty(T * k, np.int32)
    token_row = np.empty(T * k, np.int32)
    rc = _load().oracle_permute(_p(idx), T, k, E, _p(offsets), _p(row_token), _p(token_row))
    if rc != 0:
        raise ValueError(f"oracle_permute failed ({rc})")
    return offsets, row_token, token_row


def ffn(experts: Experts, e: int, x) -> np.ndarray:
    """FFN_e(x) for one fp32 vector x [d]; float64 [d]."""
    s, keep = experts._struct()
    x = _f32(x)
    out = np.empty(s.d, np.float64)
    h = np.empty(s.inter, np.float64)
    _load().oracle_ffn(ctypes.byref(s), e, _p(x), _p(out), _p(h))
    return out


def expert_rows(experts: Experts, x, row_token, offsets) -> np.ndarray:
    """rows[r] = FFN_{expert(r)}(x[row_token[r]]); row_token None = identity."""
    s, keep = experts._struct()
    x = _f32(x)
    offsets = np.ascontiguousarray(offsets, dtype=np.int32)
    assert offsets.shape == (s.E + 1,)
    rt = None if row_token is None else np.ascontiguousarray(row_token, dtype=np.int32)
    R = int(offsets[-1])
    rows = np.empty((R, s.d), np.float64)
    rc = _load().oracle_expert_rows(ctypes.byref(s), _p(x), _p(rt), _p(offsets), _p(rows))
    if rc != 0:
        raise ValueError(f"oracle_expert_rows failed ({rc})")
    return rows


def combine(rows, token_row, w, shared=None, residual=None) -> np.ndarray:
    rows, w = _f32(rows), _f32(w)
    shared, residual = _f32(shared), _f32(residual)
    token_row = np.ascontiguousarray(token_row, dtype=np.int32)
    T, k = w.shape
    d = rows.shape[1]
    y = np.empty((T, d), np.float64)
    _load().oracle_combine(_p(rows), _p(token_row), _p(w), _p(shared), _p(residual), T, k,
                           d, _p(y))
    return y


def layer(router: str, k: int, scale: float, x, wr, bias, experts: Experts,
          shared: Optional[Experts] = None, tokens=None):
    """Whole layer.  Returns (y [T,d] float64, idx [T,k], w [T,k] float64, gap [T]).

    `tokens` (optional) restricts the computation to those token rows of x
    (tokens are independent, so this equals slicing the full result)."""
    x = _f32(x)
    if tokens is not None:
        x = np.ascontiguousarray(x[np.asarray(tokens)])
    wr, bias = _f32(wr), _f32(bias)
    es, keep_e = experts._struct()
    L = _Layer()
    L.router, L.k, L.scale = ROUTER[router], k, scale
    L.wr, L.bias = _p(wr), _p(bias)
    L.experts = es
    keep_s = None
    if shared is not None:
        ss, keep_s = shared._struct()
        L.has_shared, L.shared = 1, ss
    else:
        L.has_shared = 0
    T, d = x.shape
    y = np.empty((T, d), np.float64)
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    gap = np.empty(T, np.float64)
    rc = _load().oracle_layer(ctypes.byref(L), _p(x), T, _p(idx), _p(w), _p(gap), _p(y))
    if rc != 0:
        raise ValueError(f"oracle_layer failed ({rc})")
    del keep_e, keep_s
    return y, idx, w, gap


def layer_of(inputs, tokens=None):
    """Whole layer for a synth.LayerInputs."""
    s = inputs.spec
    return layer(s.router, s.k, s.scale, inputs.x, inputs.wr, inputs.bias,
                 Experts.of(inputs.experts),
                 Experts.of(inputs.shared) if inputs.shared is not None else None,
                 tokens=tokens)


def coverage_set(counts, cover: float, k: int) -> np.ndarray:
    """Experts kept by the restriction: the smallest set reaching `cover` of
    the selection counts, padded to k; ascending ids (int32)."""
    counts = np.ascontiguousarray(counts, dtype=np.uint64)
    E = counts.shape[0]
    keep = np.empty(E, np.int32)
    n = _load().oracle_coverage_set(_p(counts), E, float(cover), k, _p(keep))
    if n < 0:
        raise ValueError(f"oracle_coverage_set failed ({n})")
    return keep[:n].copy()


def bf16_to_f32(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) as the fp32 values they denote (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def quantize(fmt: str, w) -> tuple:
    """Float weights [rows, K] -> (codes int8 [rows, K], scales fp32).
    fmt "int8_row": scales [rows]; "int4_b32" / "int4_b128": scales
    [rows, K/32] / [rows, K/128], codes unpacked (one int8 per code, in
    [-8, 7])."""
    w = _f32(w)
    rows, K = w.shape
    q = np.empty((rows, K), np.int8)
    if fmt == "int8_row":
        s = np.empty(rows, np.float32)
        rc = _load().oracle_quantize_int8_rows(_p(w), rows, K, _p(q), _p(s))
    elif fmt in INT4_BLOCK:
        B = INT4_BLOCK[fmt]
        s = np.empty((rows, K // B), np.float32)
        rc = _load().oracle_quantize_int4_blocks(_p(w), rows, K, B, _p(q), _p(s))
    else:
        raise ValueError(f"no quantizer for {fmt}")
    if rc != 0:
        raise ValueError(f"oracle quantizer failed ({rc})")
    return q, s
