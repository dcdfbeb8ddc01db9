"""Python binding of the NVFP4 C ABI (include/nvfp4.h) -- marshalling only.

Each function has the name of the C entry point it calls and takes torch
tensors that already live on the GPU; it passes their data pointers, sizes
and the current HIP stream, and raises on a negative status.  Every step of
the computation runs in the HIP library; there is no fallback.  Importing
this module loads libnvfp4.so and fails loudly when it has not been built
(``python -m moe_amax_gsa_amd.build``).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch  # loaded first: the library binds to torch's HIP runtime

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnvfp4.so")

OK = 0
DTYPE_BF16 = 0
DTYPE_FP32 = 1
OP_AMAX_GSA = 0
OP_QUANTIZE = 1
OP_LINEAR = 2
OP_GROUPED_LINEAR = 3
OP_LINEAR_RUN = 4
OP_GROUPED_SWIGLU = 5
OP_QUANTIZE_WEIGHT = 6
OP_RMSNORM_QUANTIZE = 7
OP_ROUTER_TOPK = 8
OP_GROUPED_RUN = 9
OP_MOE_RUN = 10
ERR_SCRATCH = -7
NOALLOC_SCRATCH_BYTES = 16 << 20

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m moe_amax_gsa_amd.build`")

lib = ctypes.CDLL(LIB_PATH)

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I = ctypes.c_int
_SZ = ctypes.c_size_t

lib.nvfp4_abi_version.restype = _I
lib.nvfp4_abi_version.argtypes = []
lib.nvfp4_status_string.restype = ctypes.c_char_p
lib.nvfp4_status_string.argtypes = [_I]
lib.nvfp4_workspace_bytes.restype = _SZ
lib.nvfp4_workspace_bytes.argtypes = [_I, _I64, _I64, _I64, _I]
lib.nvfp4_amax_gsa.restype = _I
lib.nvfp4_amax_gsa.argtypes = [_P, _I, _I64, _P, _P, _SZ, _P]
lib.nvfp4_quantize_from_buffer.restype = _I
lib.nvfp4_quantize_from_buffer.argtypes = [_P, _I, _I64, _I64, _P, _P, _P, _P]
lib.nvfp4_linear.restype = _I
lib.nvfp4_linear.argtypes = [_P, _P, _P, _P, _P, _P, _P, _I, _I64, _I64, _I64, _P, _SZ, _P]
lib.nvfp4_linear_rows.restype = _I
lib.nvfp4_linear_rows.argtypes = [_P, _P, _P, _P, _P, _P, _P, _I, _I64, _I64, _I64, _P, _SZ, _P]
lib.nvfp4_router_topk.restype = _I
lib.nvfp4_router_topk.argtypes = [_P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I, _P, _P, _P,
                                  _SZ, _P]
lib.nvfp4_linear_run.restype = _I
lib.nvfp4_linear_run.argtypes = [_P, _I, _P, _P, _P, _P, _P, _P, _P, _I, _I64, _I64, _I64, _P, _SZ,
                                 _P]
lib.nvfp4_linear_run_noalloc.restype = _I
lib.nvfp4_linear_run_noalloc.argtypes = [_P, _I, _P, _P, _P, _P, _P, _P, _P, _I, _I64, _I64, _I64,
                                         _P]
lib.nvfp4_grouped_linear.restype = _I
lib.nvfp4_grouped_linear.argtypes = [_P, _P, _P, _I64, _P, _P, _I, _I64, _P, _P, _P, _P, _I,
                                     _I64, _I64, _P]
lib.nvfp4_amax_quantize.restype = _I
lib.nvfp4_amax_quantize.argtypes = [_P, _I, _I64, _I64, _P, _P, _P, _P, _SZ, _P]
lib.nvfp4_rmsnorm_quantize.restype = _I
lib.nvfp4_rmsnorm_quantize.argtypes = [_P, _I, _P, _I, ctypes.c_float, _I64, _I64, _I, _P, _P,
                                       _P, _P, _P, _SZ, _P]
lib.nvfp4_quantize_weight.restype = _I
lib.nvfp4_quantize_weight.argtypes = [_P, _I, _I64, _I64, _P, _P, _P, _P, _SZ, _P]
lib.nvfp4_grouped_linear_swiglu.restype = _I
lib.nvfp4_grouped_linear_swiglu.argtypes = [_P, _P, _P, _I64, _P, _P, _I, _I64, _P, _P, _P, _P,
                                            _P, _P, _P, _I64, _I64, _I, ctypes.c_float, _P, _SZ,
                                            _P]
lib.nvfp4_grouped_linear_run.restype = _I
lib.nvfp4_grouped_linear_run.argtypes = [_P, _I, _I64, _P, _P, _P, _P, _P, _I, _I64, _P, _P, _P,
                                         _P, _I, _I64, _I64, _P, _SZ, _P]
lib.nvfp4_moe_run.restype = _I
lib.nvfp4_moe_run.argtypes = [_P, _I, _I64, _P, _P, _P, _P, _P, _I, _I64, _P, _P, _P, _I64, _I64,
                              _I, ctypes.c_float, _P, _P, _P, _P, _P, _P, _P, _I64, _P, _I, _P,
                              _SZ, _P]
lib.nvfp4_swiglu_deinterleave.restype = _I
lib.nvfp4_swiglu_deinterleave.argtypes = [_P, _P, _I64, _I64, _I, ctypes.c_float, _P]


class Nvfp4Error(RuntimeError):
    pass


def _check(status: int, what: str) -> None:
    if status != OK:
        raise Nvfp4Error(f"{what}: {lib.nvfp4_status_string(status).decode()} ({status})")


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype == torch.float32:
        return DTYPE_FP32
    raise ValueError(f"unsupported dtype {t.dtype}")


def _nbytes(t: Optional[torch.Tensor]) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def _room(t: Optional[torch.Tensor], nbytes: int, what: str, dtype=None,
          optional: bool = False) -> None:
    """The kernels address raw device pointers: refuse a buffer smaller than
    what the call reads or writes (or of the wrong element type) before any
    pointer reaches the library."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{what} is required")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{what} must be {dtype}, got {t.dtype}")
    if _nbytes(t) < nbytes:
        raise ValueError(f"{what} holds {_nbytes(t)} bytes, the call needs {nbytes}")


def _out(t: torch.Tensor, n: int, what: str) -> None:
    """An output of n elements in bf16 or fp32."""
    _dtype(t)
    _room(t, n * t.element_size(), what)


_U8, _F32, _I32 = torch.uint8, torch.float32, torch.int32


def _linear_operands(a_codes, a_scales, gsa, n_gsa, w_codes, w_scales, ws2, n_ws2, M, N, K):
    _room(a_codes, M * (K // 2), "activation codes", _U8)
    _room(a_scales, M * (K // 16), "activation scales", _U8)
    _room(gsa, 4 * n_gsa, "gsa", _F32)
    _room(w_codes, N * (K // 2), "w_codes", _U8)
    _room(w_scales, N * (K // 16), "w_scales", _U8)
    _room(ws2, 4 * n_ws2, "ws2", _F32)


def _grouped_operands(a_codes, a_scales, a_rows, gsa, row_index, offsets, G, M_total, w_codes,
                      w_scales, ws2, N, K):
    _room(a_codes, a_rows * (K // 2), "activation codes", _U8)
    _room(a_scales, a_rows * (K // 16), "activation scales", _U8)
    _room(gsa, 4, "gsa", _F32)
    _room(row_index, 4 * M_total, "row_index", _I32, optional=True)
    _room(offsets, 4 * (G + 1), "group_offsets", _I32)
    _room(w_codes, G * N * (K // 2), "w_codes", _U8)
    _room(w_scales, G * N * (K // 16), "w_scales", _U8)
    _room(ws2, 4 * G, "ws2", _F32)


def nvfp4_abi_version() -> int:
    return lib.nvfp4_abi_version()


def nvfp4_workspace_bytes(op: int, M: int, N: int = 0, K: int = 0, G: int = 0) -> int:
    return lib.nvfp4_workspace_bytes(op, M, N, K, G)


def nvfp4_amax_gsa(x: torch.Tensor, gsa: torch.Tensor, ws: Optional[torch.Tensor] = None,
                   stream=None) -> None:
    """gsa[0] = max(max|x|, 1e-8) / 2688 on the device (x bf16 or fp32)."""
    _room(gsa, 4, "gsa", _F32)
    _check(lib.nvfp4_amax_gsa(_ptr(x), _dtype(x), x.numel(), _ptr(gsa), _ptr(ws),
                              0 if ws is None else ws.numel() * ws.element_size(),
                              _stream(stream)), "nvfp4_amax_gsa")


def nvfp4_quantize_from_buffer(x: torch.Tensor, gsa: torch.Tensor, codes: torch.Tensor,
                               scales: torch.Tensor, stream=None) -> None:
    """x (M, K) -> codes (M, K/2) uint8, scales (M, K/16) uint8 with device gsa."""
    M, K = x.shape
    _room(gsa, 4, "gsa", _F32)
    _room(codes, M * (K // 2), "codes", _U8)
    _room(scales, M * (K // 16), "scales", _U8)
    _check(lib.nvfp4_quantize_from_buffer(_ptr(x), _dtype(x), M, K, _ptr(gsa), _ptr(codes),
                                          _ptr(scales), _stream(stream)),
           "nvfp4_quantize_from_buffer")


def nvfp4_linear(a_codes: torch.Tensor, a_scales: torch.Tensor, gsa: torch.Tensor,
                 w_codes: torch.Tensor, w_scales: torch.Tensor, ws2: torch.Tensor,
                 y: torch.Tensor, ws: Optional[torch.Tensor] = None, stream=None) -> None:
    """y (M, N) = gsa * ws2 * dequant(A) @ dequant(W)^T."""
    M = a_codes.shape[0]
    K = a_codes.shape[1] * 2
    N = w_codes.shape[0]
    _linear_operands(a_codes, a_scales, gsa, 1, w_codes, w_scales, ws2, 1, M, N, K)
    _out(y, M * N, "y")
    _check(lib.nvfp4_linear(_ptr(a_codes), _ptr(a_scales), _ptr(gsa), _ptr(w_codes),
                            _ptr(w_scales), _ptr(ws2), _ptr(y), _dtype(y), M, N, K, _ptr(ws),
                            0 if ws is None else ws.numel() * ws.element_size(),
                            _stream(stream)), "nvfp4_linear")


def nvfp4_linear_rows(a_codes: torch.Tensor, a_scales: torch.Tensor, gsa_rows: torch.Tensor,
                      w_codes: torch.Tensor, w_scales: torch.Tensor, ws2: torch.Tensor,
                      y: torch.Tensor, ws: Optional[torch.Tensor] = None, stream=None) -> None:
    """y[m] = gsa_rows[m] * ws2 * dequant(A[m]) @ dequant(W)^T; gsa_rows (M,)."""
    M = a_codes.shape[0]
    K = a_codes.shape[1] * 2
    N = w_codes.shape[0]
    _linear_operands(a_codes, a_scales, gsa_rows, M, w_codes, w_scales, ws2, 1, M, N, K)
    _out(y, M * N, "y")
    _check(lib.nvfp4_linear_rows(_ptr(a_codes), _ptr(a_scales), _ptr(gsa_rows), _ptr(w_codes),
                                 _ptr(w_scales), _ptr(ws2), _ptr(y), _dtype(y), M, N, K,
                                 _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                                 _stream(stream)), "nvfp4_linear_rows")


def nvfp4_router_topk(a_codes: torch.Tensor, a_scales: torch.Tensor, gsa: torch.Tensor,
                      w_codes: torch.Tensor, w_scales: torch.Tensor, ws2: torch.Tensor,
                      bias: Optional[torch.Tensor], topk_idx: torch.Tensor,
                      topk_score: torch.Tensor, ws: torch.Tensor, stream=None) -> None:
    """Gate logits of A (M, K) against W (N, K), then the top k experts of
    sqrt(softplus(logit)) + bias: topk_idx (M, k) int32, topk_score (M, k)."""
    M = a_codes.shape[0]
    K = a_codes.shape[1] * 2
    N = w_codes.shape[0]
    k = topk_idx.shape[1]
    _linear_operands(a_codes, a_scales, gsa, 1, w_codes, w_scales, ws2, 1, M, N, K)
    _room(bias, 4 * N, "bias", _F32, optional=True)
    _room(topk_idx, 4 * M * k, "topk_idx", _I32)
    _room(topk_score, 4 * M * k, "topk_score", _F32)
    _check(lib.nvfp4_router_topk(_ptr(a_codes), _ptr(a_scales), _ptr(gsa), _ptr(w_codes),
                                 _ptr(w_scales), _ptr(ws2), _ptr(bias), M, N, K, k,
                                 _ptr(topk_idx), _ptr(topk_score), _ptr(ws),
                                 ws.numel() * ws.element_size(), _stream(stream)),
           "nvfp4_router_topk")


def nvfp4_linear_run(x: torch.Tensor, gsa: torch.Tensor, codes: torch.Tensor,
                     scales: torch.Tensor, w_codes: torch.Tensor, w_scales: torch.Tensor,
                     ws2: torch.Tensor, y: torch.Tensor, ws: Optional[torch.Tensor] = None,
                     stream=None) -> None:
    """amax -> gsa -> quantize -> linear on x (M, K); writes gsa, codes, scales, y."""
    M, K = x.shape
    N = w_codes.shape[0]
    _linear_operands(codes, scales, gsa, 1, w_codes, w_scales, ws2, 1, M, N, K)
    _out(y, M * N, "y")
    _check(lib.nvfp4_linear_run(_ptr(x), _dtype(x), _ptr(gsa), _ptr(codes), _ptr(scales),
                                _ptr(w_codes), _ptr(w_scales), _ptr(ws2), _ptr(y), _dtype(y),
                                M, N, K, _ptr(ws),
                                0 if ws is None else ws.numel() * ws.element_size(),
                                _stream(stream)), "nvfp4_linear_run")


def nvfp4_linear_run_noalloc(x: torch.Tensor, gsa: torch.Tensor, codes: torch.Tensor,
                             scales: torch.Tensor, w_codes: torch.Tensor,
                             w_scales: torch.Tensor, ws2: torch.Tensor, y: torch.Tensor,
                             stream=None) -> None:
    """nvfp4_linear_run without a workspace: the library's static scratch."""
    M, K = x.shape
    N = w_codes.shape[0]
    _linear_operands(codes, scales, gsa, 1, w_codes, w_scales, ws2, 1, M, N, K)
    _out(y, M * N, "y")
    _check(lib.nvfp4_linear_run_noalloc(_ptr(x), _dtype(x), _ptr(gsa), _ptr(codes), _ptr(scales),
                                        _ptr(w_codes), _ptr(w_scales), _ptr(ws2), _ptr(y),
                                        _dtype(y), M, N, K, _stream(stream)),
           "nvfp4_linear_run_noalloc")


def nvfp4_grouped_linear(a_codes: torch.Tensor, a_scales: torch.Tensor, gsa: torch.Tensor,
                         row_index: Optional[torch.Tensor], group_offsets: torch.Tensor,
                         w_codes: torch.Tensor, w_scales: torch.Tensor, ws2: torch.Tensor,
                         y: torch.Tensor, stream=None) -> None:
    """w_codes (G, N, K/2), w_scales (G, N, K/16), ws2 (G,), y (M_total, N)."""
    G, N = w_codes.shape[0], w_codes.shape[1]
    K = w_codes.shape[2] * 2
    _grouped_operands(a_codes, a_scales, a_codes.shape[0], gsa, row_index, group_offsets, G,
                      y.shape[0], w_codes, w_scales, ws2, N, K)
    _out(y, y.shape[0] * N, "y")
    _check(lib.nvfp4_grouped_linear(_ptr(a_codes), _ptr(a_scales), _ptr(gsa), a_codes.shape[0],
                                    _ptr(row_index), _ptr(group_offsets), G, y.shape[0],
                                    _ptr(w_codes), _ptr(w_scales), _ptr(ws2), _ptr(y),
                                    _dtype(y), N, K, _stream(stream)), "nvfp4_grouped_linear")


def nvfp4_amax_quantize(x: torch.Tensor, gsa: torch.Tensor, codes: torch.Tensor,
                        scales: torch.Tensor, ws: Optional[torch.Tensor] = None,
                        stream=None) -> None:
    """Steps 1 and 2: gsa, codes (M, K/2), scales (M, K/16) of x (M, K)."""
    M, K = x.shape
    _room(gsa, 4, "gsa", _F32)
    _room(codes, M * (K // 2), "codes", _U8)
    _room(scales, M * (K // 16), "scales", _U8)
    _check(lib.nvfp4_amax_quantize(_ptr(x), _dtype(x), M, K, _ptr(gsa), _ptr(codes),
                                   _ptr(scales), _ptr(ws),
                                   0 if ws is None else ws.numel() * ws.element_size(),
                                   _stream(stream)), "nvfp4_amax_quantize")


def nvfp4_rmsnorm_quantize(x: torch.Tensor, norm_weight: torch.Tensor, gsa: torch.Tensor,
                           inv_rms: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor,
                           eps: float = 1e-6, per_row: bool = False,
                           ws: Optional[torch.Tensor] = None, stream=None) -> None:
    """RMSNorm of x (M, K) with norm_weight (K,), quantized: codes (M, K/2),
    scales (M, K/16), inv_rms (M,), gsa (1,) or, per_row, (M,)."""
    M, K = x.shape
    _room(norm_weight, K * norm_weight.element_size(), "norm_weight")
    _room(gsa, 4 * (M if per_row else 1), "gsa", _F32)
    _room(inv_rms, 4 * M, "inv_rms", _F32)
    _room(codes, M * (K // 2), "codes", _U8)
    _room(scales, M * (K // 16), "scales", _U8)
    _check(lib.nvfp4_rmsnorm_quantize(_ptr(x), _dtype(x), _ptr(norm_weight), _dtype(norm_weight),
                                      eps, M, K, 1 if per_row else 0, _ptr(gsa), _ptr(inv_rms),
                                      _ptr(codes), _ptr(scales), _ptr(ws),
                                      0 if ws is None else ws.numel() * ws.element_size(),
                                      _stream(stream)), "nvfp4_rmsnorm_quantize")


def nvfp4_quantize_weight(w: torch.Tensor, ws2: torch.Tensor, codes: torch.Tensor,
                          scales: torch.Tensor, ws: Optional[torch.Tensor] = None,
                          stream=None) -> None:
    """w (N, K) bf16/fp32 -> codes (N, K/2), scales (N, K/16), ws2 (1,) fp32."""
    N, K = w.shape
    _room(ws2, 4, "ws2", _F32)
    _room(codes, N * (K // 2), "codes", _U8)
    _room(scales, N * (K // 16), "scales", _U8)
    _check(lib.nvfp4_quantize_weight(_ptr(w), _dtype(w), N, K, _ptr(ws2), _ptr(codes),
                                     _ptr(scales), _ptr(ws),
                                     0 if ws is None else ws.numel() * ws.element_size(),
                                     _stream(stream)), "nvfp4_quantize_weight")


def nvfp4_grouped_linear_swiglu(a_codes: torch.Tensor, a_scales: torch.Tensor, gsa: torch.Tensor,
                                row_index: Optional[torch.Tensor], group_offsets: torch.Tensor,
                                w_codes: torch.Tensor, w_scales: torch.Tensor, ws2: torch.Tensor,
                                h: torch.Tensor, gsa_h: torch.Tensor, granularity: int,
                                ws: torch.Tensor, stream=None,
                                h_codes: Optional[torch.Tensor] = None,
                                h_scales: Optional[torch.Tensor] = None,
                                limit: float = 0.0) -> None:
    """w_codes (G, N_inter, K/2), w_scales (G, N_inter, K/16), ws2 (G,);
    h (M_total, N_inter/2) fp32 and gsa_h (1,) fp32 are written, and with
    h_codes / h_scales also h's codes and scales.  limit: the SwiGLU limit
    (<= 0: none)."""
    G, NI = w_codes.shape[0], w_codes.shape[1]
    K = w_codes.shape[2] * 2
    P = h.shape[0]
    _grouped_operands(a_codes, a_scales, a_codes.shape[0], gsa, row_index, group_offsets, G, P,
                      w_codes, w_scales, ws2, NI, K)
    _room(h, 4 * P * (NI // 2), "h", _F32)
    _room(gsa_h, 4, "gsa_h", _F32)
    _room(h_codes, P * (NI // 4), "h_codes", _U8, optional=True)
    _room(h_scales, P * (NI // 32), "h_scales", _U8, optional=True)
    _check(lib.nvfp4_grouped_linear_swiglu(
        _ptr(a_codes), _ptr(a_scales), _ptr(gsa), a_codes.shape[0], _ptr(row_index),
        _ptr(group_offsets), G, h.shape[0], _ptr(w_codes), _ptr(w_scales), _ptr(ws2), _ptr(h),
        _ptr(gsa_h), _ptr(h_codes), _ptr(h_scales), NI, K, granularity, limit, _ptr(ws),
        ws.numel() * ws.element_size(), _stream(stream)), "nvfp4_grouped_linear_swiglu")


def nvfp4_swiglu_deinterleave(l1: torch.Tensor, h: torch.Tensor, granularity: int = 8,
                              stream=None, limit: float = 0.0) -> None:
    """h (M, N/2) = silu(gate) * up from granularity-interleaved l1 (M, N),
    fp32; limit > 0 caps the gate at limit and clamps up to [-limit, limit]."""
    M, NI = l1.shape
    _room(l1, 4 * M * NI, "l1", _F32)
    _room(h, 4 * M * (NI // 2), "h", _F32)
    _check(lib.nvfp4_swiglu_deinterleave(_ptr(l1), _ptr(h), M, NI, granularity, limit,
                                         _stream(stream)), "nvfp4_swiglu_deinterleave")


def nvfp4_grouped_linear_run(x: torch.Tensor, gsa: torch.Tensor, x_codes: torch.Tensor,
                             x_scales: torch.Tensor, row_index: Optional[torch.Tensor],
                             group_offsets: torch.Tensor, w_codes: torch.Tensor,
                             w_scales: torch.Tensor, ws2: torch.Tensor, y: torch.Tensor,
                             ws: Optional[torch.Tensor] = None, stream=None) -> None:
    """Steps 1-3 of the grouped linear on x (x_rows, K): w_codes (G, N, K/2),
    w_scales (G, N, K/16), ws2 (G,), y (M_total, N); gsa, x_codes and
    x_scales receive x's quantization."""
    G, N = w_codes.shape[0], w_codes.shape[1]
    K = w_codes.shape[2] * 2
    R = x.shape[0]
    _grouped_operands(x_codes, x_scales, R, gsa, row_index, group_offsets, G, y.shape[0],
                      w_codes, w_scales, ws2, N, K)
    _out(y, y.shape[0] * N, "y")
    _check(lib.nvfp4_grouped_linear_run(_ptr(x), _dtype(x), x.shape[0], _ptr(gsa), _ptr(x_codes),
                                        _ptr(x_scales), _ptr(row_index), _ptr(group_offsets), G,
                                        y.shape[0], _ptr(w_codes), _ptr(w_scales), _ptr(ws2),
                                        _ptr(y), _dtype(y), N, K, _ptr(ws), _nbytes(ws),
                                        _stream(stream)), "nvfp4_grouped_linear_run")


def nvfp4_moe_run(x: torch.Tensor, gsa_x: torch.Tensor, x_codes: torch.Tensor,
                  x_scales: torch.Tensor, row_index: torch.Tensor, group_offsets: torch.Tensor,
                  w1_codes: torch.Tensor, w1_scales: torch.Tensor, w1_ws2: torch.Tensor,
                  granularity: int, h: torch.Tensor, gsa_h: torch.Tensor, h_codes: torch.Tensor,
                  h_scales: torch.Tensor, w2_codes: torch.Tensor, w2_scales: torch.Tensor,
                  w2_ws2: torch.Tensor, y: torch.Tensor, ws: torch.Tensor, limit: float = 0.0,
                  stream=None) -> None:
    """The routed-expert pair on x (T, K1): w1 (E, N1, K1/2 | K1/16), w2 (E,
    N2, N1/4 | N1/32), h (P, N1/2), y (P, N2) for the P pairs."""
    E, N1 = w1_codes.shape[0], w1_codes.shape[1]
    K1 = w1_codes.shape[2] * 2
    N2 = w2_codes.shape[1]
    T, P = x.shape[0], row_index.shape[0]
    _grouped_operands(x_codes, x_scales, T, gsa_x, row_index, group_offsets, E, P, w1_codes,
                      w1_scales, w1_ws2, N1, K1)
    _room(h, 4 * P * (N1 // 2), "h", _F32)
    _room(gsa_h, 4, "gsa_h", _F32)
    _room(h_codes, P * (N1 // 4), "h_codes", _U8)
    _room(h_scales, P * (N1 // 32), "h_scales", _U8)
    _room(w2_codes, E * N2 * (N1 // 4), "w2_codes", _U8)
    _room(w2_scales, E * N2 * (N1 // 32), "w2_scales", _U8)
    _room(w2_ws2, 4 * E, "w2_ws2", _F32)
    _out(y, P * N2, "y")
    _check(lib.nvfp4_moe_run(_ptr(x), _dtype(x), x.shape[0], _ptr(gsa_x), _ptr(x_codes),
                             _ptr(x_scales), _ptr(row_index), _ptr(group_offsets), E,
                             row_index.shape[0], _ptr(w1_codes), _ptr(w1_scales), _ptr(w1_ws2),
                             N1, K1, granularity, limit, _ptr(h), _ptr(gsa_h), _ptr(h_codes),
                             _ptr(h_scales), _ptr(w2_codes), _ptr(w2_scales), _ptr(w2_ws2), N2,
                             _ptr(y), _dtype(y), _ptr(ws), _nbytes(ws), _stream(stream)),
           "nvfp4_moe_run")
