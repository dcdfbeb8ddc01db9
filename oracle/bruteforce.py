"""Exact rational brute force for tiny NVFP4 GEMMs -- test infrastructure only.

An independent second definition of the linear layer's output, used to pin
the C oracle: E2M1 magnitudes come from the table printed in the commit
message of nvfp4-megamoe-kernel commit 0d1cd1e (dsv4/kernels/indexer, the
E2M1 decode fix), E4M3 scale bytes are decoded by torch's float8_e4m3fn
conversion, and every product and sum is a Python Fraction (no rounding).

    y[m, n] = gsa * ws2 * sum_k (lut[a]*sfa) * (lut[w]*sfw)

(dequant rule from commit db07d17's message on weight_scale_2, GEMM form
from dsv4/_archive/layers/linear.py finalize_weights).  Pure-Python loops:
small shapes only.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import torch

# Magnitudes in code order 0b000 .. 0b111 as printed on the page.
E2M1_TABLE = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2),
              Fraction(2), Fraction(3), Fraction(4), Fraction(6)]


def e2m1(code: int) -> Fraction:
    mag = E2M1_TABLE[code & 7]
    return -mag if code & 8 else mag


def e4m3(byte: int) -> Fraction:
    v = torch.tensor([byte], dtype=torch.uint8).view(torch.float8_e4m3fn).float().item()
    return Fraction(v)


def unpack(codes: np.ndarray) -> np.ndarray:
    """(R, K/2) bytes -> (R, K) codes, element 2j in the low nibble of byte j."""
    R, KB = codes.shape
    out = np.empty((R, 2 * KB), np.int64)
    out[:, 0::2] = codes & 0x0F
    out[:, 1::2] = codes >> 4
    return out


def linear_exact(a_codes, a_scales, gsa, w_codes, w_scales, ws2):
    a = unpack(np.asarray(a_codes))
    w = unpack(np.asarray(w_codes))
    M, K = a.shape
    N = w.shape[0]
    g = Fraction(float(np.float32(gsa))) * Fraction(float(np.float32(ws2)))
    y = [[Fraction(0)] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                acc += (e2m1(int(a[m, k])) * e4m3(int(a_scales[m, k // 16])) *
                        e2m1(int(w[n, k])) * e4m3(int(w_scales[n, k // 16])))
            y[m][n] = g * acc
    return y
