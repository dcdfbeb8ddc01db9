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


@pytest.mark.parametrize("case", range(40))
def test_random_few_rows_many_columns(C, case):
    """Up to 16 rows against 2000 to 20000 weight rows, K any multiple of 16
    (the weight ring, the tiles and the few-row kernels meet here):
    nvfp4_linear_run's gsa, codes and scales bit-exact with the oracle, y of
    linear_run, linear and linear_rows (gsa per row) within 1e-3 of the
    oracle on sampled columns (both ends and a random spread), and the bf16
    output the float32 one rounded."""
    rng = np.random.default_rng(6000 + case)
    M = int(rng.integers(1, 17))
    N = int(rng.integers(2000, 20001))
    K = int(rng.choice([256, 1024, 2048, 7168])) if rng.integers(0, 2) else random_k(rng, 256)
    say("random few rows, many columns", case, M, N, K)
    inp = W.make_linear(M, K, N, seed=7000 + case, x="outliers", sf=(0.125, 8.0), ws2=0.004)
    x = W.bf16_to_torch(inp.x, DEV)
    gsa = torch.zeros(1, dtype=torch.float32, device=DEV)
    codes = torch.full((M, K // 2), 0x5A, dtype=torch.uint8, device=DEV)
    scales = torch.full((M, K // 16), 0x5A, dtype=torch.uint8, device=DEV)
    ws = torch.empty(max(16, C.nvfp4_workspace_bytes(C.OP_LINEAR_RUN, M, N, K)),
                     dtype=torch.uint8, device=DEV)
    wc, wsf = to_dev(inp.w_codes), to_dev(inp.w_scales)
    ws2 = to_dev(np.array([inp.ws2], np.float32))
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    C.nvfp4_linear_run(x, gsa, codes, scales, wc, wsf, ws2, y, ws)
    g = np.float32(gsa.cpu().numpy()[0])
    assert g == oracle.amax_gsa(inp.x)
    oc, os_ = oracle.quantize(inp.x, g)
    assert np.array_equal(codes.cpu().numpy(), oc) and np.array_equal(scales.cpu().numpy(), os_)
    cols = np.unique(np.concatenate([np.arange(16), np.arange(N - 40, N),
                                     rng.choice(N, 96, replace=False)]))
    ref = oracle.linear(oc, os_, g, inp.w_codes[cols], inp.w_scales[cols], inp.ws2)
    assert rel_err(y.cpu().numpy().astype(np.float64)[:, cols], ref) <= REL_TOL, (M, N, K)
    y2 = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    C.nvfp4_linear(codes, scales, gsa, wc, wsf, ws2, y2)
    assert rel_err(y2.cpu().numpy().astype(np.float64)[:, cols], ref) <= REL_TOL, (M, N, K)
    y16 = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)
    C.nvfp4_linear(codes, scales, gsa, wc, wsf, ws2, y16)
    assert torch.equal(y16.cpu(), y2.cpu().to(torch.bfloat16))
    grow = torch.full((M,), float(g), dtype=torch.float32, device=DEV)
    grow[::2] *= 4.0
    y3 = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    C.nvfp4_linear_rows(codes, scales, grow, wc, wsf, ws2, y3)
    sc = np.ones(M)
    sc[::2] = 4.0
    assert rel_err(y3.cpu().numpy().astype(np.float64)[:, cols], ref * sc[:, None]) <= REL_TOL


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


# ---------------------------------------------------------------- more entry points
import test_gpu_parity as P  # noqa: E402  (shared GPU helpers of the parity tests)


@pytest.mark.parametrize("case", range(16))
def test_random_amax_quantize(C, case):
    """nvfp4_amax_quantize across the one-workgroup size (65 536 elements)
    and the inline-partials size: gsa, codes and scales bit-exact."""
    rng = np.random.default_rng(7000 + case)
    band = case % 3
    numel_hi = [65536, 4 << 20, 16 << 20][band]
    K = 16 * int(rng.integers(1, 600))
    M = max(1, int(rng.integers(numel_hi // 8, numel_hi)) // K)
    dtype = "bf16" if rng.integers(0, 2) == 0 else "fp32"
    say("random amax quantize", case, M, K, dtype)
    inp = W.make_linear(M, K, 1, seed=7100 + case, x="outliers")
    xh = inp.x if dtype == "bf16" else np.ascontiguousarray(W.bf16_bits_to_f32(inp.x))
    x = W.bf16_to_torch(inp.x, DEV) if dtype == "bf16" else to_dev(xh)
    gsa = torch.zeros(1, dtype=torch.float32, device=DEV)
    codes = torch.full((M, K // 2), 0x5A, dtype=torch.uint8, device=DEV)
    scales = torch.full((M, K // 16), 0x5A, dtype=torch.uint8, device=DEV)
    nws = C.nvfp4_workspace_bytes(C.OP_AMAX_GSA, M * K)
    ws = torch.full((max(nws, 16),), 0xAB, dtype=torch.uint8, device=DEV)
    C.nvfp4_amax_quantize(x, gsa, codes, scales, ws)
    g = np.float32(gsa.cpu().numpy()[0])
    assert g == oracle.amax_gsa(xh)
    oc, os_ = oracle.quantize(xh, g)
    assert np.array_equal(codes.cpu().numpy(), oc) and np.array_equal(scales.cpu().numpy(), os_)


@pytest.mark.parametrize("case", range(12))
def test_random_rmsnorm_quantize(C, case):
    """nvfp4_rmsnorm_quantize on random (M, K), one scale or one per row:
    inv_rms within 1e-5 of the binary64 oracle, codes, scales and gsa
    bit-exact with the oracle's quantize of the rows rebuilt from the GPU's
    inv_rms (as the parity test does)."""
    rng = np.random.default_rng(8000 + case)
    M = int(rng.choice(M_CHOICES))
    K = 16 * int(rng.integers(1, 520))
    per_row = bool(rng.integers(0, 2))
    xd = "bf16" if rng.integers(0, 2) == 0 else "fp32"
    say("random rmsnorm", case, M, K, per_row, xd)
    r = W.make_rmsnorm(M, K, 8100 + case)
    xh = r.x if xd == "bf16" else np.ascontiguousarray(W.bf16_bits_to_f32(r.x))
    x = W.bf16_to_torch(r.x, DEV) if xd == "bf16" else to_dev(xh)
    w = W.bf16_to_torch(r.w, DEV)
    gsa, inv, codes, scales = P.gpu_rmsnorm_quantize(C, x, w, per_row)
    inv_g = inv.cpu().numpy()
    inv_o, _ = oracle.rmsnorm(xh, r.w, 1e-6)
    assert np.max(np.abs(inv_g / inv_o - 1.0)) <= P.INV_RMS_TOL
    y32 = (W.bf16_bits_to_f32(r.x) * inv_g[:, None]).astype(np.float32) * \
        W.bf16_bits_to_f32(r.w)[None, :]
    if per_row:
        oc, os_, og = oracle.quantize_rows(y32)
        assert np.array_equal(gsa.cpu().numpy(), og)
    else:
        og = oracle.amax_gsa(y32)
        assert np.float32(gsa.cpu().numpy()[0]) == og
        oc, os_ = oracle.quantize(y32, og)
    assert np.array_equal(codes.cpu().numpy(), oc) and np.array_equal(scales.cpu().numpy(), os_)


@pytest.mark.parametrize("case", range(12))
def test_random_router_topk(C, case):
    """nvfp4_router_topk on random (M, N, K, k): logits within 1e-3 of the
    oracle's linear, the choice equal to the oracle's on the GPU's own
    logits up to fp32 near-ties (as the parity test checks)."""
    rng = np.random.default_rng(9000 + case)
    M = int(rng.choice([1, 2, 3, 7, 16, 17, 40]))
    N = int(rng.integers(8, 1025))
    k = int(rng.integers(1, min(N, 16) + 1))
    K = 16 * int(rng.integers(1, 200))
    say("random router", case, M, N, K, k)
    r, ga, ac, as_, gw, wc, wsf = P.router_inputs(M, K, N, k, seed=9100 + case)
    idx_g, sc_g, z = P.gpu_router(C, ac, as_, ga, wc, wsf, gw, r.bias, k)
    zo = oracle.linear(ac, as_, ga, wc, wsf, gw)
    assert np.max(np.abs(z - zo)) <= REL_TOL * np.max(np.abs(zo))
    vmax = np.max(np.abs(oracle.router_scores(z))) + np.max(np.abs(r.bias))
    P.check_choice(idx_g, sc_g, z, r.bias, k, eps=1e-6 * vmax)


@pytest.mark.parametrize("case", range(12))
def test_random_grouped_swiglu(C, case):
    """nvfp4_grouped_linear_swiglu on random groups, granularities and
    limits against the separate calls: h bit-identical, the same gsa_h, h's
    codes and scales identical, rows outside the groups or with an invalid
    row_index unwritten; h against the oracle's SwiGLU of the GPU's l1."""
    rng = np.random.default_rng(10000 + case)
    G, sizes = random_groups(rng)
    gran = int(rng.choice([1, 2, 4, 8]))
    N = 32 * int(rng.integers(1, 12))
    K = 256 * int(rng.integers(1, 5))
    start, tail = int(rng.integers(0, 3)), int(rng.integers(0, 3))
    offsets = (start + np.concatenate([[0], np.cumsum(sizes)])).astype(np.int32)
    P_rows = int(offsets[-1]) + tail
    a_rows = int(rng.integers(1, 30))
    row_index = rng.integers(0, a_rows, max(P_rows, 1)).astype(np.int32)[:P_rows]
    if P_rows:
        row_index[int(rng.integers(0, P_rows))] = -1
    say("random grouped swiglu", case, G, sizes, N, K, gran)
    ac, asf = operands(rng, a_rows, K)
    wc = rng.integers(0, 256, (G, N, K // 2), dtype=np.uint8)
    wsf = rng.integers(0x20, 0x48, (G, N, K // 16), dtype=np.uint8)
    ws2 = rng.uniform(0.002, 0.01, G).astype(np.float32)
    d = dict(ac=to_dev(ac), asf=to_dev(asf), gsa=to_dev(np.array([np.float32(0.37)])),
             ri=to_dev(row_index), off=to_dev(offsets), wc=to_dev(wc), wsf=to_dev(wsf),
             ws2=to_dev(ws2))
    l1 = torch.zeros(P_rows, N, dtype=torch.float32, device=DEV)
    C.nvfp4_grouped_linear(d["ac"], d["asf"], d["gsa"], d["ri"], d["off"], d["wc"], d["wsf"],
                           d["ws2"], l1)
    nz = l1[l1 != 0]
    limit = float(torch.median(torch.abs(nz))) if (case % 2 and nz.numel()) else 0.0
    h1 = torch.zeros(P_rows, N // 2, dtype=torch.float32, device=DEV)
    g1 = torch.zeros(1, dtype=torch.float32, device=DEV)
    nws = C.nvfp4_workspace_bytes(C.OP_GROUPED_SWIGLU, P_rows, N, 0, G)
    ws = torch.full((max(nws, 16),), 0xAB, dtype=torch.uint8, device=DEV)
    hc1 = torch.full((P_rows, N // 4), 0x5A, dtype=torch.uint8, device=DEV)
    hs1 = torch.full((P_rows, N // 32), 0x5A, dtype=torch.uint8, device=DEV)
    C.nvfp4_grouped_linear_swiglu(d["ac"], d["asf"], d["gsa"], d["ri"], d["off"], d["wc"],
                                  d["wsf"], d["ws2"], h1, g1, gran, ws, h_codes=hc1,
                                  h_scales=hs1, limit=limit)
    h2 = torch.zeros(P_rows, N // 2, dtype=torch.float32, device=DEV)
    g2 = torch.zeros(1, dtype=torch.float32, device=DEV)
    C.nvfp4_swiglu_deinterleave(l1, h2, gran, limit=limit)
    C.nvfp4_amax_gsa(h2, g2, torch.empty(max(C.nvfp4_workspace_bytes(C.OP_AMAX_GSA,
                                                                      P_rows * N // 2), 16),
                                         dtype=torch.uint8, device=DEV))
    hc2, hs2 = P.gpu_quantize(C, h2, g2)
    torch.cuda.synchronize()
    a, b = h1.cpu().numpy(), h2.cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    assert np.float32(g1.cpu().numpy()[0]) == np.float32(g2.cpu().numpy()[0])
    assert torch.equal(hc1, hc2) and torch.equal(hs1, hs2)
    if P_rows:
        href = oracle.swiglu_deinterleave(l1.cpu().numpy(), gran, limit)
        assert np.max(np.abs(a - href)) <= 1e-6 * max(np.max(np.abs(href)), 1e-30)


@pytest.mark.parametrize("case", range(10))
def test_random_moe_run(C, case):
    """nvfp4_moe_run on random token counts, expert counts, top-k, sizes and
    routing: every step against the oracle on the GPU's own input to it,
    every output bit-equal to the separate calls (as the parity test
    checks)."""
    rng = np.random.default_rng(11000 + case)
    experts = int(rng.integers(2, 33))
    topk = int(rng.integers(1, min(8, experts) + 1))
    tokens = int(rng.choice([1, 2, 3, 5, 9, 17, 40, 80]))
    K1 = 256 * int(rng.integers(1, 9))
    N1 = 512 * int(rng.integers(1, 3))
    N2 = int(rng.integers(1, 300))
    routing = "zipf" if rng.integers(0, 2) else "uniform"
    say("random moe run", case, tokens, experts, topk, K1, N1, N2, routing)
    moe = W.make_moe(tokens=tokens, experts=experts, topk=topk, K1=K1, N1=N1, K2=N1 // 2,
                     N2=N2, granularity=8, seed=11100 + case, routing=routing)
    P.moe_run_matches_separate_calls(C, moe)


def rne_bf16(a: np.ndarray) -> np.ndarray:
    return torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).float().numpy()


@pytest.mark.parametrize("case", range(16))
def test_random_bf16_outputs_are_rounded_fp32(C, case):
    """The bf16 output of nvfp4_linear, nvfp4_linear_rows and
    nvfp4_grouped_linear on random shapes is the same call's fp32 output
    rounded to nearest even, bit for bit (the output type changes the store
    only); the per-row-gsa linear with every row's gsa equal matches the
    one-gsa linear, and it is within 1e-3 of the oracle row by row."""
    rng = np.random.default_rng(12000 + case)
    M = int(rng.choice(M_CHOICES))
    N = int(rng.integers(1, 400))
    K = random_k(rng, 80)
    say("random bf16 outputs", case, M, N, K)
    ac, asf = operands(rng, M, K)
    wc, wsf = operands(rng, N, K)
    gsa_rows = rng.uniform(0.01, 1.0, M).astype(np.float32)
    ws2 = np.float32(0.004)
    nws = C.nvfp4_workspace_bytes(C.OP_LINEAR, M, N, K)
    ws = torch.empty(max(nws, 16), dtype=torch.uint8, device=DEV)
    d = [to_dev(v) for v in (ac, asf)] + [to_dev(gsa_rows)] + [to_dev(v) for v in (wc, wsf)] + \
        [to_dev(np.array([ws2]))]
    outs = {}
    for name, fn in [("rows", C.nvfp4_linear_rows), ("one", C.nvfp4_linear)]:
        for dt in (torch.float32, torch.bfloat16):
            y = torch.full((M, N), -7.0, dtype=dt, device=DEV)
            args = list(d)
            if name == "one":
                args[2] = to_dev(np.full(1, gsa_rows[0], np.float32))
            fn(*args, y, ws)
            outs[name, dt] = y.float().cpu().numpy()
        assert np.array_equal(rne_bf16(outs[name, torch.float32]), outs[name, torch.bfloat16])
    ref = np.stack([oracle.linear(ac[m:m + 1], asf[m:m + 1], gsa_rows[m], wc, wsf, ws2)[0]
                    for m in range(M)])
    assert rel_err(outs["rows", torch.float32].astype(np.float64), ref) <= REL_TOL
    # the first row's scale for every row: the one-gsa linear's result
    args = list(d)
    args[2] = to_dev(np.full(M, gsa_rows[0], np.float32))
    y = torch.full((M, N), -7.0, dtype=torch.float32, device=DEV)
    C.nvfp4_linear_rows(*args, y, ws)
    assert np.array_equal(y.cpu().numpy(), outs["one", torch.float32])
    # grouped, bf16 against fp32 of the same call
    G = int(rng.integers(1, 5))
    cut = np.sort(rng.integers(0, M + 1, G - 1))
    offsets = np.concatenate([[0], cut, [M]]).astype(np.int32)
    wg = rng.integers(0, 256, (G, N, K // 2), dtype=np.uint8)
    sg = rng.integers(0x20, 0x48, (G, N, K // 16), dtype=np.uint8)
    w2 = rng.uniform(0.002, 0.01, G).astype(np.float32)
    g_out = {}
    for dt in (torch.float32, torch.bfloat16):
        y = torch.full((M, N), -7.0, dtype=dt, device=DEV)
        C.nvfp4_grouped_linear(d[0], d[1], to_dev(np.array([np.float32(0.3)])), None,
                               to_dev(offsets), to_dev(wg), to_dev(sg), to_dev(w2), y)
        g_out[dt] = y.float().cpu().numpy()
    assert np.array_equal(rne_bf16(g_out[torch.float32]), g_out[torch.bfloat16])


@pytest.mark.parametrize("case", range(12))
def test_random_noalloc_matches_linear_run(C, case):
    """nvfp4_linear_run_noalloc on random shapes that fit its static
    scratch: gsa, codes, scales and y bit-equal to nvfp4_linear_run's."""
    rng = np.random.default_rng(13000 + case)
    M = int(rng.choice(M_CHOICES))
    N = int(rng.integers(1, 1500))
    K = random_k(rng, 128)
    need = max(C.nvfp4_workspace_bytes(C.OP_LINEAR_RUN, M, N, K), 0)
    if need > C.NOALLOC_SCRATCH_BYTES:
        pytest.skip("larger than the static scratch")
    say("random noalloc", case, M, N, K)
    inp = W.make_linear(M, K, N, seed=13100 + case, x="outliers")
    x = W.bf16_to_torch(inp.x, DEV)
    wc, wsf = to_dev(inp.w_codes), to_dev(inp.w_scales)
    w2 = to_dev(np.array([inp.ws2], np.float32))
    res = []
    for noalloc in (False, True):
        gsa = torch.zeros(1, dtype=torch.float32, device=DEV)
        codes = torch.full((M, K // 2), 0x5A, dtype=torch.uint8, device=DEV)
        scales = torch.full((M, K // 16), 0x5A, dtype=torch.uint8, device=DEV)
        y = torch.full((M, N), -7.0, dtype=torch.float32, device=DEV)
        if noalloc:
            C.nvfp4_linear_run_noalloc(x, gsa, codes, scales, wc, wsf, w2, y)
        else:
            ws = torch.empty(max(need, 16), dtype=torch.uint8, device=DEV)
            C.nvfp4_linear_run(x, gsa, codes, scales, wc, wsf, w2, y, ws)
        res.append([t.cpu().numpy() for t in (gsa, codes, scales, y)])
    for a, b in zip(*res):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))


def _random_graph_step(C, kind, rng):
    """(step, outputs) for one entry point on random sizes: step() enqueues
    the call on the current stream, outputs() lists what it writes."""
    if kind == "linear_run":
        M = int(rng.choice([1, 3, 16, 17, 100]))
        N, K = int(rng.integers(1, 600)), random_k(rng, 64)
        inp = W.make_linear(M, K, N, seed=int(rng.integers(1 << 30)), x="outliers")
        x = W.bf16_to_torch(inp.x, DEV)
        wc, wsf = to_dev(inp.w_codes), to_dev(inp.w_scales)
        w2 = to_dev(np.array([inp.ws2], np.float32))
        gsa = torch.zeros(1, device=DEV)
        codes = torch.zeros(M, K // 2, dtype=torch.uint8, device=DEV)
        scales = torch.zeros(M, K // 16, dtype=torch.uint8, device=DEV)
        y = torch.zeros(M, N, device=DEV)
        ws = torch.empty(max(C.nvfp4_workspace_bytes(C.OP_LINEAR_RUN, M, N, K), 16),
                         dtype=torch.uint8, device=DEV)
        return (lambda: C.nvfp4_linear_run(x, gsa, codes, scales, wc, wsf, w2, y, ws),
                lambda: [gsa, codes, scales, y])
    if kind == "grouped_run":
        G, sizes = random_groups(rng)
        N, K = int(rng.integers(1, 300)), random_k(rng, 64)
        x_rows = int(rng.integers(1, 20))
        offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
        P_rows = int(offsets[-1])
        inp = W.make_linear(x_rows, K, 1, seed=int(rng.integers(1 << 30)))
        x = W.bf16_to_torch(inp.x, DEV)
        ri = to_dev(rng.integers(0, x_rows, max(P_rows, 1)).astype(np.int32))
        off = to_dev(offsets)
        wc = to_dev(rng.integers(0, 256, (G, N, K // 2), dtype=np.uint8))
        wsf = to_dev(rng.integers(0x20, 0x48, (G, N, K // 16), dtype=np.uint8))
        w2 = to_dev(rng.uniform(0.002, 0.01, G).astype(np.float32))
        gsa = torch.zeros(1, device=DEV)
        codes = torch.zeros(x_rows, K // 2, dtype=torch.uint8, device=DEV)
        scales = torch.zeros(x_rows, K // 16, dtype=torch.uint8, device=DEV)
        y = torch.zeros(max(P_rows, 1), N, device=DEV)
        ws = torch.empty(max(C.nvfp4_workspace_bytes(C.OP_GROUPED_RUN, x_rows, N, K, G), 16),
                         dtype=torch.uint8, device=DEV)
        return (lambda: C.nvfp4_grouped_linear_run(x, gsa, codes, scales, ri[:P_rows], off, wc,
                                                   wsf, w2, y[:P_rows], ws),
                lambda: [gsa, codes, scales, y[:P_rows]])
    if kind == "router":
        M = int(rng.choice([1, 5, 16, 17, 40]))
        N = int(rng.integers(8, 513))
        k = int(rng.integers(1, min(N, 8) + 1))
        K = 16 * int(rng.integers(1, 100))
        r, ga, ac, as_, gw, wc, wsf = P.router_inputs(M, K, N, k, seed=int(rng.integers(1 << 30)))
        idx = torch.zeros(M, k, dtype=torch.int32, device=DEV)
        sc = torch.zeros(M, k, device=DEV)
        ws = torch.zeros(max(C.nvfp4_workspace_bytes(C.OP_ROUTER_TOPK, M, N, K), 16),
                         dtype=torch.uint8, device=DEV)  # the ticket counter starts at zero
        args = (to_dev(ac), to_dev(as_), torch.tensor([ga], device=DEV), to_dev(wc), to_dev(wsf),
                torch.tensor([gw], device=DEV), to_dev(r.bias), idx, sc, ws)
        return (lambda: C.nvfp4_router_topk(*args), lambda: [idx, sc])
    from moe_amax_gsa_amd.layer import Nvfp4MoE
    tokens = int(rng.choice([1, 3, 40]))
    experts = int(rng.integers(2, 17))
    topk = int(rng.integers(1, min(4, experts) + 1))
    moe = W.make_moe(tokens=tokens, experts=experts, topk=topk, K1=256 * int(rng.integers(1, 4)),
                     N1=512, K2=256, N2=int(rng.integers(1, 200)), granularity=8,
                     seed=int(rng.integers(1 << 30)))
    Pn = int(moe.offsets[-1])
    layer = Nvfp4MoE(*W.moe_weights_to(moe, DEV), max_pairs=Pn, max_tokens=moe.T)
    x = W.bf16_to_torch(moe.x, DEV)
    ri, off = to_dev(moe.pair_token), to_dev(moe.offsets)
    return (lambda: layer(x, ri, off),
            lambda: [layer.y2[:Pn], layer.h[:Pn], layer.gsa1, layer.gsa2])


@pytest.mark.parametrize("case", range(12))
def test_random_graph_replays(C, case):
    """A random entry point on random sizes captured in a HIP graph and
    replayed three times, its outputs overwritten and eager work in
    between: every replay equal to the eager call bit for bit."""
    rng = np.random.default_rng(14000 + case)
    kind = ["linear_run", "grouped_run", "router", "moe_run"][case % 4]
    say("random graph replay", case, kind)
    step, outs = _random_graph_step(C, kind, rng)
    step()
    torch.cuda.synchronize()
    eager = [t.clone() for t in outs()]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(3):
        for t in outs():
            t.fill_(float("nan") if t.dtype.is_floating_point else 0x5A)
        _ = torch.randn(1000, device=DEV).sum()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs(), eager):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))


@pytest.mark.parametrize("case", range(10))
def test_random_quantize_weight_and_amax(C, case):
    """nvfp4_quantize_weight on a random bf16 weight (N, K): weight_scale_2,
    codes and scales bit-exact with the oracle's amax, gsa and quantize; and
    nvfp4_amax_gsa on a random-length tensor equal to the oracle's gsa."""
    rng = np.random.default_rng(15000 + case)
    N = int(rng.integers(1, 3000))
    K = 16 * int(rng.integers(1, 700))
    say("random quantize weight", case, N, K)
    w = W.to_bf16_bits(rng.standard_normal((N, K)) * rng.uniform(0.001, 1.0))
    ws2 = torch.zeros(1, device=DEV)
    codes = torch.full((N, K // 2), 0x5A, dtype=torch.uint8, device=DEV)
    scales = torch.full((N, K // 16), 0x5A, dtype=torch.uint8, device=DEV)
    nws = C.nvfp4_workspace_bytes(C.OP_QUANTIZE_WEIGHT, 0, N, K)
    ws = torch.full((max(nws, 16),), 0xAB, dtype=torch.uint8, device=DEV)
    C.nvfp4_quantize_weight(W.bf16_to_torch(w, DEV), ws2, codes, scales, ws)
    g = oracle.amax_gsa(w)
    assert np.float32(ws2.cpu().numpy()[0]) == g
    oc, os_ = oracle.quantize(w, g)
    assert np.array_equal(codes.cpu().numpy(), oc) and np.array_equal(scales.cpu().numpy(), os_)
    n = int(rng.integers(1, 3_000_000))
    x = rng.standard_normal(n).astype(np.float32) * np.float32(rng.uniform(0.1, 100.0))
    x[int(rng.integers(0, n))] = -np.float32(rng.uniform(100.0, 1e4))
    gsa = torch.zeros(1, device=DEV)
    nws = C.nvfp4_workspace_bytes(C.OP_AMAX_GSA, n)
    C.nvfp4_amax_gsa(to_dev(x), gsa, torch.full((max(nws, 16),), 0xAB, dtype=torch.uint8,
                                                device=DEV))
    assert np.float32(gsa.cpu().numpy()[0]) == oracle.amax_gsa(x.reshape(1, -1)[:, :n])


@pytest.mark.parametrize("case", range(10))
def test_random_swiglu_deinterleave(C, case):
    """nvfp4_swiglu_deinterleave on random (M, N) and granularity, with and
    without a limit: within 1e-6 of the oracle's binary64 SwiGLU."""
    rng = np.random.default_rng(16000 + case)
    gran = int(rng.choice([1, 2, 4, 8, 16]))
    M = int(rng.integers(0, 400))
    N = 2 * gran * int(rng.integers(1, 200))
    limit = float(rng.choice([0.0, 0.5, 3.0]))
    say("random swiglu", case, M, N, gran, limit)
    l1 = (rng.standard_normal((M, N)) * 3.0).astype(np.float32)
    h = torch.full((M, N // 2), -7.0, device=DEV)
    C.nvfp4_swiglu_deinterleave(to_dev(l1), h, gran, limit=limit)
    if M:
        ref = oracle.swiglu_deinterleave(l1, gran, limit)
        hh = h.cpu().numpy()
        assert np.max(np.abs(hh - ref)) <= 1e-6 * max(np.max(np.abs(ref)), 1e-30)
