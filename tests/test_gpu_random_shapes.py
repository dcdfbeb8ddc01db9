"""Seeded random shapes through the C ABI against the CPU oracle: many small
problems whose sizes fall on and between the dispatch boundaries (activation
rows around 1, 4, 16 and one tile; K multiples of 16 that are or are not
multiples of 256 and 512; N with partial tiles; groups empty, small and
large, gathered rows with invalid indices).  Same bar as the parity tests:
gsa, codes and scales bit-exact, outputs within 1e-3 of the oracle's FP64
sum, rows no group writes left untouched."""
import sys

import numpy as np
import pytest
import torch

from oracle import oracle
from moe_amax_gsa_amd import workloads as W

pytestmark = pytest.mark.gpu
REL_TOL = 1e-3
DEV = "cuda"
M_CHOICES = [1, 2, 3, 4, 5, 8, 13, 16, 17, 31, 64, 100, 128, 129, 300]


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def C():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    from moe_amax_gsa_amd import nvfp4
    return nvfp4


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def rel_err(y, ref):
    return float(np.max(np.abs(y - ref)) / max(np.max(np.abs(ref)), 1e-300))


def random_k(rng, kmax_blocks):
    """K: a multiple of 512, of 256, or of 16 only, in turn."""
    kind = rng.integers(0, 3)
    if kind == 0:
        return 512 * int(rng.integers(1, max(2, kmax_blocks // 32)))
    if kind == 1:
        return 256 * int(rng.integers(1, max(2, kmax_blocks // 16)))
    return 16 * int(rng.integers(1, kmax_blocks))


def operands(rng, rows, K):
    codes = rng.integers(0, 256, (rows, K // 2), dtype=np.uint8)
    scales = rng.integers(0x20, 0x48, (rows, K // 16), dtype=np.uint8)
    return codes, scales


@pytest.mark.parametrize("case", range(30))
def test_random_linear(C, case):
    """nvfp4_linear on random (M, N, K), fp32 output, with the workspace the
    library asks for (split K where it takes it)."""
    rng = np.random.default_rng(1000 + case)
    M = int(rng.choice(M_CHOICES))
    N = int(rng.integers(1, 520))
    K = random_k(rng, 96)
    say("random linear", case, M, N, K)
    ac, asf = operands(rng, M, K)
    wc, wsf = operands(rng, N, K)
    gsa, ws2 = np.float32(rng.uniform(0.01, 1.0)), np.float32(rng.uniform(0.002, 0.01))
    nws = C.nvfp4_workspace_bytes(C.OP_LINEAR, M, N, K)
    ws = torch.empty(max(nws, 16), dtype=torch.uint8, device=DEV)
    y = torch.full((M, N), -7.0, dtype=torch.float32, device=DEV)
    C.nvfp4_linear(to_dev(ac), to_dev(asf), to_dev(np.array([gsa])), to_dev(wc), to_dev(wsf),
                   to_dev(np.array([ws2])), y, ws)
    ref = oracle.linear(ac, asf, gsa, wc, wsf, ws2)
    yh = y.cpu().numpy().astype(np.float64)
    assert not np.any(np.isnan(yh))
    assert rel_err(yh, ref) <= REL_TOL, (M, N, K)


@pytest.mark.parametrize("case", range(20))
def test_random_linear_run(C, case):
    """nvfp4_linear_run on random (M, N, K) with a bf16 or fp32 activation
    (0.1% outliers): gsa, codes and scales bit-exact with the oracle's amax
    and quantize, y within 1e-3 of the oracle's linear on those codes."""
    rng = np.random.default_rng(2000 + case)
    M = int(rng.choice(M_CHOICES[:12]))
    N = int(rng.integers(1, 1100))
    K = random_k(rng, 128)
    dtype = "bf16" if rng.integers(0, 2) == 0 else "fp32"
    say("random linear run", case, M, N, K, dtype)
    inp = W.make_linear(M, K, N, seed=3000 + case, x="outliers")
    xh = inp.x if dtype == "bf16" else np.ascontiguousarray(W.bf16_bits_to_f32(inp.x))
    x = W.bf16_to_torch(inp.x, DEV) if dtype == "bf16" else to_dev(xh)
    gsa = torch.zeros(1, dtype=torch.float32, device=DEV)
    codes = torch.full((M, K // 2), 0x5A, dtype=torch.uint8, device=DEV)
    scales = torch.full((M, K // 16), 0x5A, dtype=torch.uint8, device=DEV)
    nws = C.nvfp4_workspace_bytes(C.OP_LINEAR_RUN, M, N, K)
    ws = torch.empty(max(nws, 16), dtype=torch.uint8, device=DEV)
    y = torch.full((M, N), -7.0, dtype=torch.float32, device=DEV)
    C.nvfp4_linear_run(x, gsa, codes, scales, to_dev(inp.w_codes), to_dev(inp.w_scales),
                       to_dev(np.array([inp.ws2], np.float32)), y, ws)
    g = np.float32(gsa.cpu().numpy()[0])
    assert g == oracle.amax_gsa(xh)
    oc, os_ = oracle.quantize(xh, g)
    assert np.array_equal(codes.cpu().numpy(), oc) and np.array_equal(scales.cpu().numpy(), os_)
    ref = oracle.linear(oc, os_, g, inp.w_codes, inp.w_scales, inp.ws2)
    assert rel_err(y.cpu().numpy().astype(np.float64), ref) <= REL_TOL, (M, N, K)


def random_groups(rng):
    G = int(rng.integers(1, 13))
    big = rng.integers(0, 3) == 0  # a third of the cases: groups for the tiles
    sizes = rng.integers(0, 90 if big else 6, G)
    sizes[rng.random(G) < 0.25] = 0
    return G, [int(v) for v in sizes]


@pytest.mark.parametrize("case", range(24))
def test_random_grouped_linear(C, case):
    """nvfp4_grouped_linear on random groups (empty, a few rows, tens of
    rows), rows before and after the groups, gathered rows with a few
    invalid indices: written rows against the oracle, the others untouched."""
    rng = np.random.default_rng(4000 + case)
    G, sizes = random_groups(rng)
    N = int(rng.integers(1, 300))
    K = random_k(rng, 64)
    start, tail = int(rng.integers(0, 4)), int(rng.integers(0, 4))
    offsets = (start + np.concatenate([[0], np.cumsum(sizes)])).astype(np.int32)
    M_total = int(offsets[-1]) + tail
    a_rows = int(rng.integers(1, 40))
    row_index = rng.integers(0, a_rows, M_total).astype(np.int32)
    for r in rng.integers(0, max(M_total, 1), 2):
        if M_total:
            row_index[r] = rng.choice([-1, a_rows, 1 << 20])
    say("random grouped", case, G, sizes, N, K, M_total)
    ac, asf = operands(rng, a_rows, K)
    wc = rng.integers(0, 256, (G, N, K // 2), dtype=np.uint8)
    wsf = rng.integers(0x20, 0x48, (G, N, K // 16), dtype=np.uint8)
    ws2 = rng.uniform(0.002, 0.01, G).astype(np.float32)
    gsa = np.float32(0.37)
    y = torch.full((M_total, N), -7.0, dtype=torch.float32, device=DEV)
    C.nvfp4_grouped_linear(to_dev(ac), to_dev(asf), to_dev(np.array([gsa])), to_dev(row_index),
                           to_dev(offsets), to_dev(wc), to_dev(wsf), to_dev(ws2), y)
    yh = y.cpu().numpy().astype(np.float64)
    live = np.zeros(M_total, bool)
    live[offsets[0]:offsets[-1]] = True
    live &= (row_index >= 0) & (row_index < a_rows)
    assert np.all(yh[~live] == -7.0)
    if live.any():
        ri = np.where(live, row_index, 0).astype(np.int32)
        ref = oracle.grouped_linear(ac, asf, gsa, ri, offsets, wc, wsf, ws2, M_total)
        assert not np.any(np.isnan(yh[live]))
        assert rel_err(yh[live], ref[live]) <= REL_TOL


@pytest.mark.parametrize("case", range(16))
def test_random_grouped_linear_run(C, case):
    """nvfp4_grouped_linear_run on random groups over a small activation
    (bf16 or fp32): x's gsa, codes and scales bit-exact, written rows within
    1e-3 of the oracle's grouped linear on those codes."""
    rng = np.random.default_rng(5000 + case)
    G, sizes = random_groups(rng)
    N = int(rng.integers(1, 300))
    K = random_k(rng, 64)
    x_rows = int(rng.integers(1, 24))
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    M_total = int(offsets[-1])
    row_index = rng.integers(0, x_rows, M_total).astype(np.int32)
    dtype = "bf16" if rng.integers(0, 2) == 0 else "fp32"
    say("random grouped run", case, G, sizes, N, K, x_rows, dtype)
    inp = W.make_linear(x_rows, K, 1, seed=6000 + case, x="normal")
    xh = inp.x if dtype == "bf16" else np.ascontiguousarray(W.bf16_bits_to_f32(inp.x))
    x = W.bf16_to_torch(inp.x, DEV) if dtype == "bf16" else to_dev(xh)
    wc = rng.integers(0, 256, (G, N, K // 2), dtype=np.uint8)
    wsf = rng.integers(0x20, 0x48, (G, N, K // 16), dtype=np.uint8)
    ws2 = rng.uniform(0.002, 0.01, G).astype(np.float32)
    gsa = torch.zeros(1, dtype=torch.float32, device=DEV)
    codes = torch.full((x_rows, K // 2), 0x5A, dtype=torch.uint8, device=DEV)
    scales = torch.full((x_rows, K // 16), 0x5A, dtype=torch.uint8, device=DEV)
    nws = C.nvfp4_workspace_bytes(C.OP_GROUPED_RUN, x_rows, N, K, G)
    ws = torch.empty(max(nws, 16), dtype=torch.uint8, device=DEV)
    y = torch.full((max(M_total, 1), N), -7.0, dtype=torch.float32, device=DEV)
    C.nvfp4_grouped_linear_run(x, gsa, codes, scales, to_dev(row_index), to_dev(offsets),
                               to_dev(wc), to_dev(wsf), to_dev(ws2), y[:M_total], ws)
    g = np.float32(gsa.cpu().numpy()[0])
    assert g == oracle.amax_gsa(xh)
    oc, os_ = oracle.quantize(xh, g)
    assert np.array_equal(codes.cpu().numpy(), oc) and np.array_equal(scales.cpu().numpy(), os_)
    if M_total:
        ref = oracle.grouped_linear(oc, os_, g, row_index, offsets, wc, wsf, ws2, M_total)
        assert rel_err(y[:M_total].cpu().numpy().astype(np.float64), ref) <= REL_TOL
