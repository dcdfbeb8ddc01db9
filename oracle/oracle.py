"""ctypes wrapper around the C oracle (nvfp4_oracle.c).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module; the HIP library and its Python
binding never do.  The C source is the definition; this file only marshals
numpy arrays.  ``build()`` compiles the C file with gcc.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "nvfp4_oracle.c")
LIB = os.path.join(HERE, "libnvfp4_oracle.so")

BF16 = 0
FP32 = 1

_lib = None


def build() -> str:
    """Compile the oracle: plain C, no fast-math, no FMA contraction."""
    cmd = ["gcc", "-std=c11", "-O2", "-fno-fast-math", "-ffp-contract=off",
           "-fopenmp", "-fPIC", "-shared", SRC, "-o", LIB + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        build()
    lib = ctypes.CDLL(LIB)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.oracle_e2m1_value.restype = ctypes.c_double
    lib.oracle_e2m1_value.argtypes = [ctypes.c_uint]
    lib.oracle_e2m1_nearest.restype = ctypes.c_uint
    lib.oracle_e2m1_nearest.argtypes = [ctypes.c_float]
    lib.oracle_e4m3_value.restype = ctypes.c_double
    lib.oracle_e4m3_value.argtypes = [ctypes.c_uint]
    lib.oracle_e4m3_encode.restype = ctypes.c_uint
    lib.oracle_e4m3_encode.argtypes = [ctypes.c_float]
    lib.oracle_amax.restype = ctypes.c_float
    lib.oracle_amax.argtypes = [P, ctypes.c_int, I64]
    lib.oracle_gsa.restype = ctypes.c_float
    lib.oracle_gsa.argtypes = [ctypes.c_float]
    lib.oracle_quantize.restype = None
    lib.oracle_quantize.argtypes = [P, ctypes.c_int, I64, I64, ctypes.c_float, P, P]
    lib.oracle_dequantize.restype = None
    lib.oracle_dequantize.argtypes = [P, P, ctypes.c_float, I64, I64, P]
    lib.oracle_linear.restype = None
    lib.oracle_linear.argtypes = [P, P, ctypes.c_float, P, P, ctypes.c_float, I64, I64, I64, P]
    lib.oracle_linear_at.restype = None
    lib.oracle_linear_at.argtypes = [P, P, ctypes.c_float, P, P, ctypes.c_float, I64, I64, P, P, P]
    lib.oracle_grouped_linear.restype = None
    lib.oracle_grouped_linear.argtypes = [P, P, ctypes.c_float, P, P, ctypes.c_int,
                                          P, P, P, I64, I64, P]
    lib.oracle_rmsnorm.restype = None
    lib.oracle_rmsnorm.argtypes = [P, ctypes.c_int, P, ctypes.c_int, ctypes.c_double, I64, I64,
                                   P, P]
    lib.oracle_router_scores.restype = None
    lib.oracle_router_scores.argtypes = [P, I64, P]
    lib.oracle_router_topk.restype = None
    lib.oracle_router_topk.argtypes = [P, P, I64, I64, ctypes.c_int, P, P]
    lib.oracle_swiglu_deinterleave.restype = None
    lib.oracle_swiglu_deinterleave.argtypes = [P, I64, I64, ctypes.c_int, ctypes.c_double, P]
    lib.oracle_set_threads.restype = None
    lib.oracle_set_threads.argtypes = [ctypes.c_int]
    lib.oracle_max_threads.restype = ctypes.c_int
    lib.oracle_max_threads.argtypes = []
    _lib = lib
    return lib


def set_threads(n: int) -> int:
    """Threads the oracle's parallel loops use from now on; returns the
    count in effect."""
    lib = _load()
    lib.oracle_set_threads(int(n))
    return lib.oracle_max_threads()


def _ptr(a: np.ndarray) -> ctypes.c_void_p:
    assert a.flags["C_CONTIGUOUS"]
    return ctypes.c_void_p(a.ctypes.data)


def _dtype_of(x: np.ndarray) -> int:
    if x.dtype == np.uint16:
        return BF16
    if x.dtype == np.float32:
        return FP32
    raise TypeError("x must be bf16 bits (uint16) or float32, got %s" % x.dtype)


# --- element codecs -------------------------------------------------------
def e2m1_value(code: int) -> float:
    return _load().oracle_e2m1_value(code)


def e2m1_nearest(q: float) -> int:
    return _load().oracle_e2m1_nearest(q)


def e4m3_value(byte: int) -> float:
    return _load().oracle_e4m3_value(byte)


def e4m3_encode(v: float) -> int:
    return _load().oracle_e4m3_encode(v)


# --- the method -------------------------------------------------------------
def amax(x: np.ndarray) -> np.float32:
    x = np.ascontiguousarray(x)
    return np.float32(_load().oracle_amax(_ptr(x), _dtype_of(x), x.size))


def gsa_from_amax(a: float) -> np.float32:
    return np.float32(_load().oracle_gsa(np.float32(a)))


def amax_gsa(x: np.ndarray) -> np.float32:
    return gsa_from_amax(amax(x))


def quantize(x: np.ndarray, gsa: float):
    """x: (M, K) bf16 bits (uint16) or float32.  Returns (codes, scales)."""
    x = np.ascontiguousarray(x)
    M, K = x.shape
    assert K % 16 == 0
    codes = np.zeros((M, K // 2), np.uint8)
    scales = np.zeros((M, K // 16), np.uint8)
    _load().oracle_quantize(_ptr(x), _dtype_of(x), M, K, np.float32(gsa),
                            _ptr(codes), _ptr(scales))
    return codes, scales


def dequantize(codes: np.ndarray, scales: np.ndarray, gsa: float) -> np.ndarray:
    codes = np.ascontiguousarray(codes)
    scales = np.ascontiguousarray(scales)
    M = codes.shape[0]
    K = codes.shape[1] * 2
    out = np.empty((M, K), np.float64)
    _load().oracle_dequantize(_ptr(codes), _ptr(scales), np.float32(gsa), M, K, _ptr(out))
    return out


def linear(a_codes, a_scales, gsa, w_codes, w_scales, ws2) -> np.ndarray:
    a_codes = np.ascontiguousarray(a_codes)
    a_scales = np.ascontiguousarray(a_scales)
    w_codes = np.ascontiguousarray(w_codes)
    w_scales = np.ascontiguousarray(w_scales)
    M, K = a_codes.shape[0], a_codes.shape[1] * 2
    N = w_codes.shape[0]
    assert w_codes.shape[1] * 2 == K
    y = np.empty((M, N), np.float64)
    _load().oracle_linear(_ptr(a_codes), _ptr(a_scales), np.float32(gsa), _ptr(w_codes),
                          _ptr(w_scales), np.float32(ws2), M, N, K, _ptr(y))
    return y


def linear_at(a_codes, a_scales, gsa, w_codes, w_scales, ws2, ms, ns) -> np.ndarray:
    a_codes = np.ascontiguousarray(a_codes)
    a_scales = np.ascontiguousarray(a_scales)
    w_codes = np.ascontiguousarray(w_codes)
    w_scales = np.ascontiguousarray(w_scales)
    ms = np.ascontiguousarray(ms, dtype=np.int64)
    ns = np.ascontiguousarray(ns, dtype=np.int64)
    K = a_codes.shape[1] * 2
    y = np.empty(ms.shape[0], np.float64)
    _load().oracle_linear_at(_ptr(a_codes), _ptr(a_scales), np.float32(gsa), _ptr(w_codes),
                             _ptr(w_scales), np.float32(ws2), K, ms.shape[0], _ptr(ms),
                             _ptr(ns), _ptr(y))
    return y


def grouped_linear(a_codes, a_scales, gsa, row_index, offsets, w_codes, w_scales, ws2,
                   M_total: int) -> np.ndarray:
    """w_codes: (G, N, K/2); w_scales: (G, N, K/16); ws2: (G,) float32.
    Returns y (M_total, N) float64; rows outside every group are NaN."""
    a_codes = np.ascontiguousarray(a_codes)
    a_scales = np.ascontiguousarray(a_scales)
    w_codes = np.ascontiguousarray(w_codes)
    w_scales = np.ascontiguousarray(w_scales)
    ws2 = np.ascontiguousarray(ws2, dtype=np.float32)
    offsets = np.ascontiguousarray(offsets, dtype=np.int32)
    G, N = w_codes.shape[0], w_codes.shape[1]
    K = w_codes.shape[2] * 2
    y = np.full((M_total, N), np.nan, np.float64)
    if row_index is not None:
        row_index = np.ascontiguousarray(row_index, dtype=np.int32)
        rp = _ptr(row_index)
    else:
        rp = None
    _load().oracle_grouped_linear(_ptr(a_codes), _ptr(a_scales), np.float32(gsa), rp,
                                  _ptr(offsets), G, _ptr(w_codes), _ptr(w_scales),
                                  _ptr(ws2), N, K, _ptr(y))
    return y


def rmsnorm(x: np.ndarray, w: np.ndarray, eps: float = 1e-6):
    """RMSNorm of each row of x (M, K) (bf16 bits or float32) with weight w
    (K,) (bf16 bits or float32): inv_rms (M,) and y (M, K), both float64
    (nvfp4_oracle.c, oracle_rmsnorm)."""
    x = np.ascontiguousarray(x)
    w = np.ascontiguousarray(w)
    M, K = x.shape
    assert w.shape == (K,)
    inv = np.empty(M, np.float64)
    y = np.empty((M, K), np.float64)
    _load().oracle_rmsnorm(_ptr(x), _dtype_of(x), _ptr(w), _dtype_of(w), ctypes.c_double(eps),
                           M, K, _ptr(inv), _ptr(y))
    return inv, y


def quantize_rows(y: np.ndarray):
    """Quantize each row of y (M, K) float32 with its own global scale
    gsa[m] = max(max|y[m]|, 1e-8) / 2688: codes, scales, gsa (M,)."""
    y = np.ascontiguousarray(y, dtype=np.float32)
    M, K = y.shape
    codes = np.zeros((M, K // 2), np.uint8)
    scales = np.zeros((M, K // 16), np.uint8)
    gsa = np.zeros(M, np.float32)
    for m in range(M):
        gsa[m] = amax_gsa(y[m:m + 1])
        codes[m:m + 1], scales[m:m + 1] = quantize(y[m:m + 1], gsa[m])
    return codes, scales, gsa


def linear_rows(a_codes, a_scales, gsa_rows, w_codes, w_scales, ws2) -> np.ndarray:
    """The linear with one activation global scale per row: row m is the
    linear of row m alone with gsa_rows[m] (y (M, N) float64)."""
    a_codes = np.ascontiguousarray(a_codes)
    a_scales = np.ascontiguousarray(a_scales)
    gsa_rows = np.asarray(gsa_rows, dtype=np.float32)
    M = a_codes.shape[0]
    y = np.empty((M, w_codes.shape[0]), np.float64)
    for m in range(M):
        y[m:m + 1] = linear(a_codes[m:m + 1], a_scales[m:m + 1], gsa_rows[m], w_codes, w_scales,
                            ws2)
    return y


def swiglu_deinterleave(l1: np.ndarray, granularity: int = 8, limit: float = 0.0) -> np.ndarray:
    """h = silu(gate) * up, de-interleaved (nvfp4_oracle.c,
    oracle_swiglu_deinterleave); limit > 0 clamps as documented there."""
    l1 = np.ascontiguousarray(l1, dtype=np.float32)
    M, NI = l1.shape
    assert NI % (2 * granularity) == 0
    h = np.empty((M, NI // 2), np.float64)
    _load().oracle_swiglu_deinterleave(_ptr(l1), M, NI, granularity, float(limit), _ptr(h))
    return h


def router_scores(logits: np.ndarray) -> np.ndarray:
    """sqrt(softplus(z)) of every logit, float64 (nvfp4_oracle.c,
    oracle_router_scores)."""
    z = np.ascontiguousarray(logits, dtype=np.float64)
    s = np.empty_like(z)
    _load().oracle_router_scores(_ptr(z), z.size, _ptr(s))
    return s


def router_topk(logits: np.ndarray, bias, k: int):
    """Top-k experts of each row of logits (M, N) by sqrt(softplus(z)) + bias:
    idx (M, k) int32 best first (lower index on ties) and their scores
    sqrt(softplus(z)) (M, k) float64, bias excluded (nvfp4_oracle.c,
    oracle_router_topk)."""
    z = np.ascontiguousarray(logits, dtype=np.float64)
    M, N = z.shape
    assert 1 <= k <= N
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float64)
    idx = np.zeros((M, k), np.int32)
    sc = np.zeros((M, k), np.float64)
    _load().oracle_router_topk(_ptr(z), None if b is None else _ptr(b), M, N, k, _ptr(idx),
                               _ptr(sc))
    return idx, sc
