"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Bar: gsa, codes and scales bit-exact; linear outputs within
max|y - y_ref| / max|y_ref| <= 1e-3 of the oracle's FP64 accumulation of the
same dequantized operands (stepwise: the oracle consumes the GPU's own
quantized activations, checked bit-exact first); integer-valued special
cases bit-exact.  Full-size workloads are checked on sampled outputs.
"""
import sys

import numpy as np
import pytest
import torch

from oracle import oracle
from moe_amax_gsa_amd import workloads as W

pytestmark = pytest.mark.gpu
REL_TOL = 1e-3
DEV = "cuda"


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


def x_dev(bits: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return W.bf16_to_torch(bits, DEV)
    return to_dev(W.bf16_bits_to_f32(bits))


def x_host(bits: np.ndarray, dtype: str) -> np.ndarray:
    return bits if dtype == "bf16" else np.ascontiguousarray(W.bf16_bits_to_f32(bits))


def gpu_gsa(C, x):
    gsa = torch.zeros(1, dtype=torch.float32, device=DEV)
    nws = max(16, C.nvfp4_workspace_bytes(C.OP_AMAX_GSA, x.numel()))
    ws = torch.full((nws,), 0xAB, dtype=torch.uint8, device=DEV)  # garbage: no init needed
    C.nvfp4_amax_gsa(x, gsa, ws)
    return gsa


def gpu_quantize(C, x, gsa):
    M, K = x.shape
    codes = torch.full((M, K // 2), 0x5A, dtype=torch.uint8, device=DEV)
    scales = torch.full((M, K // 16), 0x5A, dtype=torch.uint8, device=DEV)
    C.nvfp4_quantize_from_buffer(x, gsa, codes, scales)
    return codes, scales


def rel_err(y, ref):
    return float(np.max(np.abs(y - ref)) / max(np.max(np.abs(ref)), 1e-300))


def f32(t: torch.Tensor) -> np.float32:
    return np.float32(t.cpu().numpy()[0])


# ---------------------------------------------------------------- amax / gsa
AMAX_CASES = [
    (1, "bf16", "last"), (7, "bf16", "first"), (1000, "fp32", "last"), (65536, "bf16", "mid"),
    (65537, "bf16", "last"), (100003, "fp32", "last"), (2 ** 20 + 5, "bf16", "last"),
    (2048 * 7168, "bf16", "last"), (3 * 2 ** 20 + 3, "fp32", "first"), (4096, "bf16", "zero"),
    (70000, "bf16", "negzero"),
]


@pytest.mark.parametrize("n,dtype,plant", AMAX_CASES)
def test_amax_gsa_bitexact(C, n, dtype, plant):
    say("amax", n, dtype, plant)
    rng = np.random.default_rng(n)
    x = rng.standard_normal(n)
    if plant == "zero":
        x[:] = 0.0
    elif plant == "negzero":
        x[:] = -0.0
    else:
        pos = {"last": n - 1, "first": 0, "mid": n // 2}[plant]
        x[pos] = -50.0  # a negative maximum
    bits = W.to_bf16_bits(x)
    g = gpu_gsa(C, x_dev(bits, dtype))
    want = oracle.amax_gsa(x_host(bits, dtype))
    assert f32(g) == want


def test_amax_race_repeat(C):
    """Large grid, maximum planted in the last workgroup's range, many runs."""
    n = 2 ** 24 + 3
    say("amax race", n)
    rng = np.random.default_rng(1)
    x = rng.standard_normal(n)
    x[-2] = 123.0
    bits = W.to_bf16_bits(x)
    xd = x_dev(bits, "bf16")
    want = oracle.amax_gsa(bits)
    for _ in range(20):
        assert f32(gpu_gsa(C, xd)) == want


# ---------------------------------------------------------------- quantize
QUANT_CASES = [
    (1, 16, "normal", "bf16"), (3, 48, "normal", "fp32"), (7, 256, "outliers", "bf16"),
    (33, 1040, "zero_blocks", "fp32"), (16, 7168, "student_t", "bf16"), (300, 512, "normal", "bf16"),
    (5, 2048, "student_t", "fp32"),
    (1171, 7200, "outliers", "bf16"), (1100, 7632, "zero_blocks", "fp32"),  # ragged, ~1M halves
]


@pytest.mark.parametrize("M,K,dist,dtype", QUANT_CASES)
def test_quantize_bitexact(C, M, K, dist, dtype):
    say("quantize", M, K, dist, dtype)
    rng = np.random.default_rng(M * 7 + K)
    bits = W.to_bf16_bits(W.draw_activation(rng, M, K, dist))
    xd = x_dev(bits, dtype)
    g = gpu_gsa(C, xd)
    assert f32(g) == oracle.amax_gsa(x_host(bits, dtype))
    codes, scales = gpu_quantize(C, xd, g)
    oc, os_ = oracle.quantize(x_host(bits, dtype), f32(g))
    assert np.array_equal(scales.cpu().numpy(), os_)
    assert np.array_equal(codes.cpu().numpy(), oc)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_amax_quantize_past_inline_limit(C, dtype):
    """nvfp4_amax_quantize well past 2^20 half-blocks (2341 x 7184: the amax
    partials, a finalize launch, then the quantize reading gsa, its last
    workgroup ragged): gsa, codes and scales of the whole tensor bit-exact
    with the oracle."""
    M, K = 2341, 7184
    assert M * K // 8 >= 1 << 21 and (M * K // 8) % 256 != 0
    say("amax quantize past the inline limit", M, K, dtype)
    rng = np.random.default_rng(2341)
    bits = W.to_bf16_bits(W.draw_activation(rng, M, K, "outliers"))
    xd = x_dev(bits, dtype)
    gsa = torch.zeros(1, dtype=torch.float32, device=DEV)
    codes = torch.full((M, K // 2), 0x5A, dtype=torch.uint8, device=DEV)
    scales = torch.full((M, K // 16), 0x5A, dtype=torch.uint8, device=DEV)
    nws = max(16, C.nvfp4_workspace_bytes(C.OP_LINEAR_RUN, M, 0, K))
    C.nvfp4_amax_quantize(xd, gsa, codes, scales,
                          torch.full((nws,), 0xAB, dtype=torch.uint8, device=DEV))
    g = oracle.amax_gsa(x_host(bits, dtype))
    assert f32(gsa) == g
    oc, os_ = oracle.quantize(x_host(bits, dtype), g)
    assert np.array_equal(scales.cpu().numpy(), os_)
    assert np.array_equal(codes.cpu().numpy(), oc)


EXTREME = ["tiny", "huge", "block_range", "elem_range"]


@pytest.mark.parametrize("kind", EXTREME)
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("M,K", [(3, 512), (40, 2048)])
def test_quantize_extreme_magnitudes_bitexact(C, M, K, dtype, kind):
    """Activations at the edges of the formats' ranges (bf16 subnormals under
    the gsa floor, values near 1e30, blocks spread over eight decades so
    that zero, subnormal and normal E4M3 scales sit side by side, elements
    spread over forty decades): gsa, codes and scales bit-exact with the
    oracle through nvfp4_amax_gsa + nvfp4_quantize_from_buffer and through
    nvfp4_amax_quantize (one workgroup at 3 x 512, two phases at 40 x 2048)."""
    say("quantize extreme", M, K, dtype, kind)
    rng = np.random.default_rng(M * 11 + K + len(kind))
    bits = W.to_bf16_bits(W.draw_activation(rng, M, K, kind))
    xd = x_dev(bits, dtype)
    want = oracle.amax_gsa(x_host(bits, dtype))
    oc, os_ = oracle.quantize(x_host(bits, dtype), want)
    g = gpu_gsa(C, xd)
    assert f32(g) == want
    codes, scales = gpu_quantize(C, xd, g)
    assert np.array_equal(scales.cpu().numpy(), os_)
    assert np.array_equal(codes.cpu().numpy(), oc)
    g2 = torch.zeros(1, dtype=torch.float32, device=DEV)
    c2 = torch.full((M, K // 2), 0x5A, dtype=torch.uint8, device=DEV)
    s2 = torch.full((M, K // 16), 0x5A, dtype=torch.uint8, device=DEV)
    nws = max(16, C.nvfp4_workspace_bytes(C.OP_LINEAR_RUN, M, 0, K))
    C.nvfp4_amax_quantize(xd, g2, c2, s2, torch.full((nws,), 0xAB, dtype=torch.uint8, device=DEV))
    assert f32(g2) == want
    assert np.array_equal(s2.cpu().numpy(), os_) and np.array_equal(c2.cpu().numpy(), oc)


@pytest.mark.parametrize("kind", EXTREME)
@pytest.mark.parametrize("M,K,N", [(1, 7168, 256), (3, 1024, 96), (64, 1024, 256)])
def test_linear_run_extreme_magnitudes(C, M, K, N, kind):
    """nvfp4_linear_run (the one-row kernel quantizing in LDS, the few-row
    kernel, the amax + quantize + tiled linear) on those activations: gsa,
    codes and scales bit-exact with the oracle, y within 1e-3 of the
    oracle's (all zero where every activation scale rounds to zero)."""
    say("linear run extreme", M, K, N, kind)
    inp = W.make_linear(M, K, N, seed=500 + M + len(kind), x=kind)
    x = W.bf16_to_torch(inp.x, DEV)
    gsa = torch.zeros(1, dtype=torch.float32, device=DEV)
    codes = torch.full((M, K // 2), 0x5A, dtype=torch.uint8, device=DEV)
    scales = torch.full((M, K // 16), 0x5A, dtype=torch.uint8, device=DEV)
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    nws = max(16, C.nvfp4_workspace_bytes(C.OP_LINEAR_RUN, M, N, K))
    ws = torch.full((nws,), 0xAB, dtype=torch.uint8, device=DEV)
    C.nvfp4_linear_run(x, gsa, codes, scales, to_dev(inp.w_codes), to_dev(inp.w_scales),
                       torch.tensor([inp.ws2], dtype=torch.float32, device=DEV), y, ws)
    g = f32(gsa)
    assert g == oracle.amax_gsa(inp.x)
    oc, os_ = oracle.quantize(inp.x, g)
    assert np.array_equal(scales.cpu().numpy(), os_) and np.array_equal(codes.cpu().numpy(), oc)
    ref = oracle.linear(oc, os_, g, inp.w_codes, inp.w_scales, inp.ws2)
    yg = y.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(yg))
    if not np.any(ref):
        assert not np.any(yg)
    else:
        assert rel_err(yg, ref) <= REL_TOL


@pytest.mark.parametrize("M,K,dtype", [(18003, 7504, "bf16"), (18003, 7504, "fp32")])
def test_quantize_large_tensor_rows(C, M, K, dtype):
    """Tensors of more than 2^24 half-blocks (the quantize then gives each
    thread four, and the last workgroup is ragged): gsa from the oracle's
    amax of the whole tensor, codes and scales of sampled rows (first, last,
    and 60 more) bit-exact with the oracle's quantize of those rows.  The
    input is drawn on the device by torch's seeded generator: N(0, 1) with
    every 97th row scaled by 50."""
    say("quantize large", M, K, dtype)
    assert M * K // 8 >= 1 << 24 and (M * K // 8) % 1024 != 0
    g = torch.Generator(device=DEV)
    g.manual_seed(M + K)
    xf = torch.randn(M, K, generator=g, device=DEV, dtype=torch.float32)
    xf[::97] *= 50.0
    xb = xf.to(torch.bfloat16)
    xd = xb if dtype == "bf16" else xb.to(torch.float32)
    del xf
    gsa = gpu_gsa(C, xd)
    codes, scales = gpu_quantize(C, xd, gsa)
    # the oracle's gsa: its amax over the whole tensor (rows in slices)
    bits = xb.view(torch.int16)
    amax_bits = 0
    for r0 in range(0, M, 2048):
        part = bits[r0:r0 + 2048].cpu().numpy().view(np.uint16)
        amax_bits = max(amax_bits, int(np.max(part & 0x7FFF)))
    row_max = np.zeros((1, 8), np.uint16)
    row_max[0, 0] = amax_bits
    assert f32(gsa) == oracle.amax_gsa(row_max)
    rows = np.unique(np.concatenate([[0, 1, M - 2, M - 1], np.arange(0, M, 97)[:8],
                                     np.random.default_rng(M).integers(0, M, 50)]))
    rows_t = torch.from_numpy(rows).to(DEV)
    sub = bits[rows_t].cpu().numpy().view(np.uint16)
    oc, os_ = oracle.quantize(x_host(sub, dtype), f32(gsa))
    assert np.array_equal(codes[rows_t].cpu().numpy(), oc)
    assert np.array_equal(scales[rows_t].cpu().numpy(), os_)


AMAXQ_CASES = [
    (1, 256, "bf16"), (1, 7168, "bf16"), (2, 8192, "fp32"),  # one workgroup, 1 or 2
    (1, 16384, "bf16"),                                     # half-blocks a thread
    (3, 4096, "fp32"), (9, 3072, "bf16"), (1, 16400, "bf16"),  # one-workgroup amax, then
    (8, 7168, "bf16"), (16, 4096, "bf16"),                   # the quantize
    (17, 4096, "bf16"), (512, 7168, "fp32"),  # two-phase amax, the quantize reducing the
    (512, 7168, "bf16"), (499, 7184, "bf16"),  # partials itself (9 to 448 of them)
    (600, 7168, "bf16"), (1000, 7168, "fp32"),  # 512 partials, each a larger slice
    (1200, 7168, "fp32"),                      # 2^20 half-blocks and more: a finalize launch
]


@pytest.mark.parametrize("M,K,dtype", AMAXQ_CASES)
def test_amax_quantize_bitexact(C, M, K, dtype):
    """nvfp4_amax_quantize: gsa, codes and scales bit-exact with the oracle's
    amax -> gsa -> quantize, on both of its paths."""
    say("amax_quantize", M, K, dtype)
    inp = W.make_linear(M, K, 16, seed=M * 3 + K, x="outliers")
    xd = x_dev(inp.x, dtype)
    gsa = torch.full((1,), -1.0, dtype=torch.float32, device=DEV)
    codes = torch.full((M, K // 2), 0x5A, dtype=torch.uint8, device=DEV)
    scales = torch.full((M, K // 16), 0x5A, dtype=torch.uint8, device=DEV)
    ws = torch.full((max(16, C.nvfp4_workspace_bytes(C.OP_AMAX_GSA, M * K)),), 0xAB,
                    dtype=torch.uint8, device=DEV)
    C.nvfp4_amax_quantize(xd, gsa, codes, scales, ws)
    g = oracle.amax_gsa(x_host(inp.x, dtype))
    assert f32(gsa) == g
    oc, os_ = oracle.quantize(x_host(inp.x, dtype), g)
    assert np.array_equal(codes.cpu().numpy(), oc) and np.array_equal(scales.cpu().numpy(), os_)
    if M * K <= 65536:  # no workspace up to 65536 elements
        assert C.nvfp4_workspace_bytes(C.OP_AMAX_GSA, M * K) == 0
        codes.fill_(0x5A)
        scales.fill_(0x5A)
        gsa.fill_(-1.0)
        C.nvfp4_amax_quantize(xd, gsa, codes, scales)
        assert f32(gsa) == g
        assert np.array_equal(codes.cpu().numpy(), oc) and np.array_equal(scales.cpu().numpy(), os_)


def test_amax_quantize_empty(C):
    gsa = torch.full((1,), -1.0, dtype=torch.float32, device=DEV)
    x = torch.empty(0, 64, dtype=torch.bfloat16, device=DEV)
    e = torch.empty(0, 32, dtype=torch.uint8, device=DEV)
    C.nvfp4_amax_quantize(x, gsa, e, e[:, :4])
    assert f32(gsa) == oracle.gsa_from_amax(0.0)


def test_quantize_small_gsa_saturates(C):
    """A caller gsa far too small (the pages' input_scale bug) saturates
    block scales at 448 on both sides."""
    say("quantize saturation")
    rng = np.random.default_rng(3)
    bits = W.to_bf16_bits(rng.standard_normal((8, 256)) * 7956.0)
    xd = x_dev(bits, "bf16")
    g = torch.tensor([0.000251], dtype=torch.float32, device=DEV)
    codes, scales = gpu_quantize(C, xd, g)
    oc, os_ = oracle.quantize(bits, f32(g))
    assert np.array_equal(scales.cpu().numpy(), os_) and np.any(os_ == 0x7E)
    assert np.array_equal(codes.cpu().numpy(), oc)


def test_quantize_signed_zero_and_underflow(C):
    say("quantize zeros")
    x = np.zeros((2, 64))
    x[0, :16] = 1e-4 * np.linspace(-1, 1, 16)
    x[0, 20] = 1000.0
    bits = W.to_bf16_bits(x)
    bits[1, 5] = 0x8000
    xd = x_dev(bits, "bf16")
    g = gpu_gsa(C, xd)
    codes, scales = gpu_quantize(C, xd, g)
    oc, os_ = oracle.quantize(bits, f32(g))
    assert np.array_equal(scales.cpu().numpy(), os_)
    assert np.array_equal(codes.cpu().numpy(), oc)


def near_tie_activation(M=4, K=4096, seed=11):
    """fp32 activation whose quantize decisions sit at rounding ties.

    gsa is 2^-8 (one element is 10.5 = 2688 * 2^-8).  Even blocks have an
    exact scale (block max 6 gsa dec(c)) and elements within 40 ulp of every
    E2M1 decision point t * s, t in {.25, .75, 1.25, 1.75, 2.5, 3.5, 5};
    odd blocks have a block max within 40 ulp of 6 gsa times the midpoint of
    two neighbouring E4M3 values.  The oracle decides every code."""
    rng = np.random.default_rng(seed)
    gsa = 2.0 ** -8
    ties = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    x = np.zeros((M * K // 16, 16), np.float32)
    for b in range(x.shape[0]):
        c = 1 + b % 126
        sc = oracle.e4m3_value(c) * gsa
        if b % 2 == 0:
            x[b, 0] = np.float32(6.0 * sc)
            for i in range(1, 16):
                t = ties[(b + i) % len(ties)]
                k = int(rng.integers(-40, 41))
                x[b, i] = np.float32(t * sc * (1.0 + k * 2.0 ** -23))
        else:
            mid = 0.5 * (oracle.e4m3_value(c - 1) + oracle.e4m3_value(c))
            bm = np.float32(6.0 * gsa * mid)
            bm = (bm.view(np.uint32) + np.uint32(int(rng.integers(0, 41)))).view(np.float32) \
                if b % 4 == 1 else (bm.view(np.uint32) - np.uint32(int(rng.integers(0, 41)))).view(np.float32)
            x[b, 0] = bm
            x[b, 1:] = (rng.uniform(-0.9, 0.9, 15) * bm).astype(np.float32)
        x[b] *= np.where(rng.random(16) < 0.5, -1.0, 1.0).astype(np.float32)
    x = x.reshape(M, K)
    x[0, 0] = np.float32(10.5)
    assert np.max(np.abs(x)) == np.float32(10.5)
    return np.ascontiguousarray(x)


@pytest.mark.parametrize("M,K", [(4, 4096), (1, 7168), (2, 2048)])
def test_quantize_near_rounding_ties(C, M, K):
    """Codes and scales at and around every rounding tie, through
    quantize_from_buffer and through the one-launch decode path (one row
    with K = 7168 is the decode kernel's two half-blocks a lane)."""
    say("quantize near ties", M, K)
    x = near_tie_activation(M, K)
    M, K = x.shape
    xd = to_dev(x)
    g = gpu_gsa(C, xd)
    assert f32(g) == np.float32(2.0 ** -8) == oracle.amax_gsa(x)
    oc, os_ = oracle.quantize(x, np.float32(2.0 ** -8))
    codes, scales = gpu_quantize(C, xd, g)
    assert np.array_equal(scales.cpu().numpy(), os_)
    assert np.array_equal(codes.cpu().numpy(), oc)
    # the fused path quantizes inside every workgroup: same bits
    N = 64
    inp = W.make_linear(1, K, N, seed=5)
    wc, ws = to_dev(inp.w_codes), to_dev(inp.w_scales)
    ws2 = torch.tensor([inp.ws2], dtype=torch.float32, device=DEV)
    gsa2 = torch.zeros(1, dtype=torch.float32, device=DEV)
    codes2 = torch.full((M, K // 2), 0x5A, dtype=torch.uint8, device=DEV)
    scales2 = torch.full((M, K // 16), 0x5A, dtype=torch.uint8, device=DEV)
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    C.nvfp4_linear_run(xd, gsa2, codes2, scales2, wc, ws, ws2, y)
    assert f32(gsa2) == np.float32(2.0 ** -8)
    assert np.array_equal(scales2.cpu().numpy(), os_)
    assert np.array_equal(codes2.cpu().numpy(), oc)
    ref = oracle.linear(oc, os_, np.float32(2.0 ** -8), inp.w_codes, inp.w_scales, inp.ws2)
    assert rel_err(y.cpu().numpy().astype(np.float64), ref) <= REL_TOL


# ---------------------------------------------------------------- linear
def run_linear(C, inp: W.LinearInputs, y_dtype=torch.float32, dtype="bf16"):
    xd = x_dev(inp.x, dtype)
    g = gpu_gsa(C, xd)
    codes, scales = gpu_quantize(C, xd, g)
    wc, ws = to_dev(inp.w_codes), to_dev(inp.w_scales)
    ws2 = torch.tensor([inp.ws2], dtype=torch.float32, device=DEV)
    y = torch.full((inp.M, inp.N), float("nan"), dtype=y_dtype, device=DEV)
    C.nvfp4_linear(codes, scales, g, wc, ws, ws2, y)
    return g, codes, scales, y


LINEAR_CASES = [
    (1, 16, 16), (1, 17, 48), (2, 40, 256), (3, 33, 272), (5, 130, 1024), (16, 64, 512),
    (17, 40, 256), (33, 130, 1040), (130, 300, 512), (129, 257, 2064), (256, 256, 7168),
    (1, 7, 128), (2, 33, 384), (4, 130, 1152),                 # 16-row kernel, ragged K
    (1, 7, 512), (2, 33, 1024), (4, 130, 2048), (3, 64, 7168),  # 4-row kernel
    (128, 64, 256), (200, 100, 768), (129, 65, 1280), (600, 333, 1536),  # LDS-staged tiles
    (64, 96, 1024),                                            # eight-wave tiles, two chunks
]


@pytest.mark.parametrize("M,N,K", LINEAR_CASES)
def test_linear_parity(C, M, N, K):
    say("linear", M, N, K)
    inp = W.make_linear(M, K, N, seed=M + N + K, x="outliers", sf=(0.125, 8.0), ws2=0.0037)
    g, codes, scales, y = run_linear(C, inp)
    oc, os_ = oracle.quantize(inp.x, f32(g))
    assert np.array_equal(codes.cpu().numpy(), oc) and np.array_equal(scales.cpu().numpy(), os_)
    ref = oracle.linear(oc, os_, f32(g), inp.w_codes, inp.w_scales, inp.ws2)
    yg = y.cpu().numpy().astype(np.float64)
    assert not np.any(np.isnan(yg))
    assert rel_err(yg, ref) <= REL_TOL


SPLIT_CASES = [(17, 64, 512), (64, 96, 1024), (130, 300, 768), (256, 256, 7168),
               (100, 40, 2304), (129, 65, 1280)]


@pytest.mark.parametrize("M,N,K", SPLIT_CASES)
def test_linear_split_k(C, M, N, K):
    """Few output tiles: with the workspace the tiled kernel splits K and a
    second kernel adds the partials in split order.  Against the oracle,
    and against the unsplit kernel (the same sums in another fp32 order)."""
    say("linear split K", M, N, K)
    need = C.nvfp4_workspace_bytes(C.OP_LINEAR, M, N, K)
    assert need > 0
    inp = W.make_linear(M, K, N, seed=M + 2 * N + K, x="outliers", sf=(0.125, 8.0), ws2=0.0037)
    xd = x_dev(inp.x, "bf16")
    g = gpu_gsa(C, xd)
    codes, scales = gpu_quantize(C, xd, g)
    wc, wsf = to_dev(inp.w_codes), to_dev(inp.w_scales)
    ws2 = torch.tensor([inp.ws2], dtype=torch.float32, device=DEV)
    ws = torch.full((need,), 0xAB, dtype=torch.uint8, device=DEV)
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    C.nvfp4_linear(codes, scales, g, wc, wsf, ws2, y, ws)
    y1 = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    C.nvfp4_linear(codes, scales, g, wc, wsf, ws2, y1)          # no workspace: unsplit
    oc, os_ = oracle.quantize(inp.x, f32(g))
    ref = oracle.linear(oc, os_, f32(g), inp.w_codes, inp.w_scales, inp.ws2)
    yg, y1g = y.cpu().numpy().astype(np.float64), y1.cpu().numpy().astype(np.float64)
    assert not np.any(np.isnan(yg))
    assert rel_err(yg, ref) <= REL_TOL
    assert rel_err(yg, y1g) <= 1e-5
    # deterministic: a second call gives the same bits
    y2 = torch.empty_like(y)
    C.nvfp4_linear(codes, scales, g, wc, wsf, ws2, y2, ws)
    assert torch.equal(y2, y)
    # bf16 output and per-row gsa through the same split
    y16 = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)
    C.nvfp4_linear(codes, scales, g, wc, wsf, ws2, y16, ws)
    assert torch.equal(y16.cpu(), y.cpu().to(torch.bfloat16))
    grow = torch.full((M,), float(f32(g)), dtype=torch.float32, device=DEV)
    grow[::3] *= 2.0
    yr = torch.empty_like(y)
    C.nvfp4_linear_rows(codes, scales, grow, wc, wsf, ws2, yr, ws)
    scale = np.ones(M)
    scale[::3] = 2.0
    assert torch.equal(yr.cpu(), torch.from_numpy((yg * scale[:, None]).astype(np.float32)))


@pytest.mark.parametrize("M,N,K", [(1, 64, 7168), (3, 100, 256), (40, 96, 1024), (200, 160, 7168)])
def test_linear_integer_case_bitexact(C, M, N, K):
    """All block scales 1.0, gsa = ws2 = 1: outputs are multiples of 1/4 below
    2^22, exact in FP32 on any summation order -- catches nibble order,
    scale indexing and tail bugs that a tolerance would hide."""
    say("linear integer", M, N, K)
    rng = np.random.default_rng(K + M)
    ac = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    wc = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    asf = np.full((M, K // 16), 0x38, np.uint8)
    wsf = np.full((N, K // 16), 0x38, np.uint8)
    one = torch.ones(1, dtype=torch.float32, device=DEV)
    ref = oracle.linear(ac, asf, 1.0, wc, wsf, 1.0)
    need = C.nvfp4_workspace_bytes(C.OP_LINEAR, M, N, K)
    for ws in [None] + ([torch.empty(need, dtype=torch.uint8, device=DEV)] if need else []):
        y = torch.empty(M, N, dtype=torch.float32, device=DEV)
        C.nvfp4_linear(to_dev(ac), to_dev(asf), one, to_dev(wc), to_dev(wsf), one, y, ws)
        assert np.array_equal(y.cpu().numpy().astype(np.float64), ref)


FEW_ROWS_WIDE = [(1, 8192 + 40), (2, 8192), (3, 12288 + 8), (4, 16384 + 24), (4, 10240),
                 (3, 4096 + 40), (4, 8192 + 8), (4, 3072), (5, 8192 + 40),
                 (7, 12288 + 8), (8, 12288 + 72), (12, 16384 + 8), (16, 12288), (6, 16384 + 40),
                 (16, 6144 + 8), (14, 6144), (8, 10240), (12, 10240 + 40), (7, 10240)]


def linear_by_column_chunks(ac, asf, g, wc, wsf, ws2, cols, chunk=2048):
    """The oracle's linear on the weight rows `cols`, a chunk at a time."""
    return np.concatenate([oracle.linear(ac, asf, g, wc[cols[i:i + chunk]], wsf[cols[i:i + chunk]],
                                         ws2) for i in range(0, len(cols), chunk)], axis=1)


@pytest.mark.parametrize("M,N", FEW_ROWS_WIDE)
def test_linear_few_rows_many_columns_integer_exact(C, M, N):
    """Up to 16 rows against thousands of weight rows (the weight ring for up
    to 4 rows, the tiled kernels from 8 rows and 10240 weight rows, 15 rows
    and 6144 or 5 rows and 16384, the 16-row kernel for 3 or 4 rows below the ring's range, the
    few-row kernels between): the integer case of the linear, exact on any
    summation order, on every output, ragged N included."""
    K = 2048
    say("linear few rows, many columns, integer", M, N, K)
    rng = np.random.default_rng(M * 7 + N)
    ac = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    wc = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    asf = np.full((M, K // 16), 0x38, np.uint8)
    wsf = np.full((N, K // 16), 0x38, np.uint8)
    one = torch.ones(1, dtype=torch.float32, device=DEV)
    ref = linear_by_column_chunks(ac, asf, 1.0, wc, wsf, 1.0, np.arange(N))
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    C.nvfp4_linear(to_dev(ac), to_dev(asf), one, to_dev(wc), to_dev(wsf), one, y)
    assert np.array_equal(y.cpu().numpy().astype(np.float64), ref)


@pytest.mark.parametrize("M,N", FEW_ROWS_WIDE)
def test_linear_few_rows_many_columns_parity(C, M, N):
    """The same shapes at K = 7168 with random codes and scales: sampled
    columns (both ends and the ragged tail, and a random spread) against the
    oracle, the bf16 output as the float32 one rounded, and one gsa per row
    (nvfp4_linear_rows) as the one-gsa output scaled per row."""
    K = 7168
    say("linear few rows, many columns", M, N, K)
    inp = W.make_linear(M, K, N, seed=M + N, x="outliers", sf=(0.125, 8.0), ws2=0.0037)
    g, codes, scales, y = run_linear(C, inp)
    oc, os_ = codes.cpu().numpy(), scales.cpu().numpy()
    rng = np.random.default_rng(N)
    cols = np.unique(np.concatenate([np.arange(64), np.arange(N - 80, N),
                                     rng.choice(N, 256, replace=False)]))
    ref = linear_by_column_chunks(oc, os_, f32(g), inp.w_codes, inp.w_scales, inp.ws2, cols)
    yg = y.cpu().numpy().astype(np.float64)
    assert not np.any(np.isnan(yg))
    assert rel_err(yg[:, cols], ref) <= REL_TOL
    wc, wsc = to_dev(inp.w_codes), to_dev(inp.w_scales)
    ws2 = torch.tensor([inp.ws2], dtype=torch.float32, device=DEV)
    y16 = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)
    C.nvfp4_linear(codes, scales, g, wc, wsc, ws2, y16)
    assert torch.equal(y16.cpu(), y.cpu().to(torch.bfloat16))
    grow = torch.full((M,), float(f32(g)), dtype=torch.float32, device=DEV)
    grow[::3] *= 2.0
    yr = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    C.nvfp4_linear_rows(codes, scales, grow, wc, wsc, ws2, yr)
    scale = np.ones(M)
    scale[::3] = 2.0
    ry = yr.cpu().numpy().astype(np.float64)
    assert rel_err(ry[:, cols], ref * scale[:, None]) <= REL_TOL
    err = np.max(np.abs(ry - yg * scale[:, None]), axis=1) / np.max(np.abs(yg * scale[:, None]), axis=1)
    assert np.max(err) <= 1e-4
    yr16 = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)
    C.nvfp4_linear_rows(codes, scales, grow, wc, wsc, ws2, yr16)
    assert torch.equal(yr16.cpu(), yr.cpu().to(torch.bfloat16))


E4M3_FINITE = np.array([b for b in range(256) if (b & 0x7F) != 0x7F], np.uint8)  # 254 bytes


def every_scale_byte_operands(M, N, K, side, seed):
    """Operands on which every finite E4M3 byte (both signs, subnormals,
    zero) is a block scale of `side` ('a' or 'w') and every output is exact
    in FP32 on any summation order.  That side's scale of block b in row r
    is E4M3_FINITE[(r + b) % 254]; the other side has unit scales and
    nonzero codes in a single block per row, so an output is one decoded
    scale times a 16-term sum of E2M1 products (a multiple of 1/4 of
    magnitude <= 576): at most 16 significant bits."""
    rng = np.random.default_rng(seed)
    nb = K // 16
    ac = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    wc = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    asf = np.full((M, nb), 0x38, np.uint8)
    wsf = np.full((N, nb), 0x38, np.uint8)
    block_of_byte = np.arange(K // 2)[None, :] // 8
    if side == "a":
        asf = E4M3_FINITE[(np.arange(M)[:, None] + np.arange(nb)[None, :]) % 254]
        wc = np.where(block_of_byte == (np.arange(N) % nb)[:, None], wc, 0).astype(np.uint8)
    else:
        wsf = E4M3_FINITE[(np.arange(N)[:, None] + np.arange(nb)[None, :]) % 254]
        ac = np.where(block_of_byte == ((7 * np.arange(M)) % nb)[:, None], ac, 0).astype(np.uint8)
    return ac, asf, wc, wsf


@pytest.mark.parametrize("side", ["a", "w"])
@pytest.mark.parametrize("M", [1, 3, 16, 200])
def test_linear_every_scale_byte_exact(C, M, side):
    """Every finite E4M3 scale byte on either operand, through each linear
    kernel (one row, a few rows, many rows) and the grouped form: outputs
    bit-identical to the oracle.  Pins the kernels' scale decoding over its
    whole domain (E4M3FN as the pages define the scale format)."""
    say("linear every scale byte", M, side)
    N, K = 256, 4096
    ac, asf, wc, wsf = every_scale_byte_operands(M, N, K, side, seed=M + (side == "w"))
    ref = oracle.linear(ac, asf, 1.0, wc, wsf, 1.0)
    one = torch.ones(2, dtype=torch.float32, device=DEV)
    need = C.nvfp4_workspace_bytes(C.OP_LINEAR, M, N, K)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV) if need else None
    y = torch.empty(M, N, dtype=torch.float32, device=DEV)
    C.nvfp4_linear(to_dev(ac), to_dev(asf), one[:1], to_dev(wc), to_dev(wsf), one[:1], y, ws)
    assert np.array_equal(y.cpu().numpy().astype(np.float64), ref)
    # grouped: two experts with the same weights, the rows split between them
    wc2, wsf2 = np.stack([wc, wc]), np.stack([wsf, wsf])
    offsets = np.array([0, M // 2, M], np.int32)
    yg = torch.empty(M, N, dtype=torch.float32, device=DEV)
    C.nvfp4_grouped_linear(to_dev(ac), to_dev(asf), one[:1], None, to_dev(offsets),
                           to_dev(wc2), to_dev(wsf2), one, yg)
    assert np.array_equal(yg.cpu().numpy().astype(np.float64), ref)


WIDE_SHAPES = [(2000, 6600, 512), (2048, 7168, 256), (1800, 7000, 768)]


@pytest.mark.parametrize("M,N,K", WIDE_SHAPES)
def test_linear_wide_tiles_integer_exact(C, M, N, K):
    """Shapes with enough 256 x 256 tiles to fill the chip (ragged in both
    dimensions, one to three 256-element chunks): all block scales 1.0 and
    gsa = ws2 = 1, so every output is a multiple of 1/4 below 2^15 and exact
    on any summation order.  The whole output is compared bit for bit with
    the FP64 product of the oracle's dequantized operands; bf16 output is
    that value rounded to nearest even."""
    say("linear wide integer", M, N, K)
    rng = np.random.default_rng(M + N + K)
    ac = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    wc = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    asf = np.full((M, K // 16), 0x38, np.uint8)
    wsf = np.full((N, K // 16), 0x38, np.uint8)
    ref = oracle.dequantize(ac, asf, 1.0) @ oracle.dequantize(wc, wsf, 1.0).T
    one = torch.ones(1, dtype=torch.float32, device=DEV)
    y = torch.empty(M, N, dtype=torch.float32, device=DEV)
    C.nvfp4_linear(to_dev(ac), to_dev(asf), one, to_dev(wc), to_dev(wsf), one, y)
    assert np.array_equal(y.cpu().numpy().astype(np.float64), ref)
    y16 = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)
    C.nvfp4_linear(to_dev(ac), to_dev(asf), one, to_dev(wc), to_dev(wsf), one, y16)
    assert torch.equal(y16.cpu(), torch.from_numpy(ref.astype(np.float32)).to(torch.bfloat16))


@pytest.mark.parametrize("side", ["a", "w"])
def test_linear_wide_tiles_every_scale_byte_exact(C, side):
    """Every finite E4M3 scale byte on either operand through the 256 x 256
    tiles (3072 x 4096: 192 tiles, K = 256: both step pairs of a chunk's
    scale layout): the whole output bit-identical to the FP64 product of the
    oracle's dequantized operands (exact on any summation order here)."""
    say("linear wide every scale byte", side)
    M, N, K = 3072, 4096, 256
    ac, asf, wc, wsf = every_scale_byte_operands(M, N, K, side, seed=5 + (side == "w"))
    ref = oracle.dequantize(ac, asf, 1.0) @ oracle.dequantize(wc, wsf, 1.0).T
    one = torch.ones(1, dtype=torch.float32, device=DEV)
    y = torch.empty(M, N, dtype=torch.float32, device=DEV)
    C.nvfp4_linear(to_dev(ac), to_dev(asf), one, to_dev(wc), to_dev(wsf), one, y)
    assert np.array_equal(y.cpu().numpy().astype(np.float64), ref)


@pytest.mark.parametrize("M,N,K", WIDE_SHAPES[:2])
def test_linear_wide_tiles_parity(C, M, N, K):
    """The same shapes with scales over the E4M3 range and a quantized
    activation: sampled outputs (tile corners and edges included) within
    1e-3 of the oracle, also with one gsa per row."""
    say("linear wide parity", M, N, K)
    inp = W.make_linear(M, K, N, seed=K, x="outliers", sf=(0.125, 8.0), ws2=0.003)
    g, codes, scales, y = run_linear(C, inp)
    oc, os_ = oracle.quantize(inp.x, f32(g))
    assert np.array_equal(codes.cpu().numpy(), oc) and np.array_equal(scales.cpu().numpy(), os_)
    ms, ns = sample_positions(M, N, 4096, 3)
    edge = np.array([255, 256, 511, 512, M - 1, M - 2] * 2)[:12] % M
    ms = np.concatenate([ms, edge, np.full(6, M // 2)])
    ns = np.concatenate([ns, np.array([0, 255, 256, N - 1, N - 2, 4095] * 2)[:12] % N,
                         np.array([63, 64, 127, 128, 191, 192]) % N])
    ref = oracle.linear_at(oc, os_, f32(g), inp.w_codes, inp.w_scales, inp.ws2, ms, ns)
    yg = y.cpu().numpy().astype(np.float64)
    assert rel_err(yg[ms, ns], ref) <= REL_TOL
    # one gsa per row: row m scaled by 2^(m % 3) exactly
    grow = torch.full((M,), float(f32(g)), dtype=torch.float32, device=DEV)
    grow *= torch.tensor([1.0, 2.0, 4.0], device=DEV).repeat(M // 3 + 1)[:M]
    yr = torch.empty_like(y)
    ws2 = torch.tensor([inp.ws2], dtype=torch.float32, device=DEV)
    C.nvfp4_linear_rows(codes, scales, grow, to_dev(inp.w_codes), to_dev(inp.w_scales), ws2, yr)
    mult = np.array([1.0, 2.0, 4.0])[np.arange(M) % 3]
    assert np.array_equal(yr.cpu().numpy(), (yg * mult[:, None]).astype(np.float32))


@pytest.mark.parametrize("M", [1, 64])
def test_linear_bf16_output_is_rounded_fp32(C, M):
    say("linear bf16 out", M)
    inp = W.make_linear(M, 512, 96, seed=5)
    _, codes, scales, y32 = run_linear(C, inp)
    wc, ws = to_dev(inp.w_codes), to_dev(inp.w_scales)
    ws2 = torch.tensor([inp.ws2], dtype=torch.float32, device=DEV)
    g = gpu_gsa(C, x_dev(inp.x, "bf16"))
    y16 = torch.empty(M, 96, dtype=torch.bfloat16, device=DEV)
    C.nvfp4_linear(codes, scales, g, wc, ws, ws2, y16)
    assert torch.equal(y16.cpu(), y32.cpu().to(torch.bfloat16))


def test_linear_deterministic(C):
    say("linear determinism")
    inp = W.make_linear(300, 2048, 200, seed=9)
    outs = [run_linear(C, inp)[3].cpu() for _ in range(3)]
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])


RUN_CASES = [
    (1, 256, 64, "bf16"), (1, 7168, 1536, "bf16"), (1, 7168, 100, "fp32"), (2, 2048, 48, "bf16"),
    (3, 4096, 40, "fp32"), (5, 512, 33, "bf16"), (16, 1024, 64, "bf16"),  # one kernel
    (1, 272, 40, "bf16"), (4, 7168, 40, "bf16"), (20, 512, 64, "fp32"),    # separate kernels
    (100, 7168, 96, "bf16"),  # amax partials, then the same workspace for a 14-way split K
    (700, 7168, 64, "bf16"),  # more than 512 amax partials: a separate finalize
    (1, 7168, 32768, "bf16"), (2, 2048, 24576, "fp32"),  # long weight streams: the ring
    (2, 4096, 12288 + 8, "bf16"), (4, 2048, 16384 + 24, "fp32"),  # quantize, then the ring
    (1, 7168, 12288, "bf16"),
    (6, 2048, 16384 + 40, "bf16"), (8, 1024, 12288, "fp32"),      # quantize, then the tiles
    (16, 1024, 6144 + 8, "bf16"),
    (1, 2048, 8192 + 40, "bf16"),                                 # one kernel
]


@pytest.mark.parametrize("M,K,N,dtype", RUN_CASES)
def test_linear_run_matches_the_three_steps(C, M, K, N, dtype):
    """nvfp4_linear_run writes what amax_gsa + quantize_from_buffer + linear
    write: gsa/codes/scales bit-exact with the oracle, y within 1e-3."""
    say("linear_run", M, K, N, dtype)
    inp = W.make_linear(M, K, N, seed=3 * M + K + N, x="outliers", sf=(0.125, 8.0), ws2=0.004)
    xd = x_dev(inp.x, dtype)
    gsa = torch.zeros(1, dtype=torch.float32, device=DEV)
    codes = torch.full((M, K // 2), 0x5A, dtype=torch.uint8, device=DEV)
    scales = torch.full((M, K // 16), 0x5A, dtype=torch.uint8, device=DEV)
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    nws = max(16, C.nvfp4_workspace_bytes(C.OP_LINEAR_RUN, M, N, K))
    ws = torch.empty(nws, dtype=torch.uint8, device=DEV)
    C.nvfp4_linear_run(xd, gsa, codes, scales, to_dev(inp.w_codes), to_dev(inp.w_scales),
                       torch.tensor([inp.ws2], dtype=torch.float32, device=DEV), y, ws)
    g = f32(gsa)
    assert g == oracle.amax_gsa(x_host(inp.x, dtype))
    oc, os_ = oracle.quantize(x_host(inp.x, dtype), g)
    assert np.array_equal(codes.cpu().numpy(), oc) and np.array_equal(scales.cpu().numpy(), os_)
    ref = oracle.linear(oc, os_, g, inp.w_codes, inp.w_scales, inp.ws2)
    yg = y.cpu().numpy().astype(np.float64)
    assert not np.any(np.isnan(yg))
    assert rel_err(yg, ref) <= REL_TOL


# ---------------------------------------------------------------- grouped / MoE
def moe_small(**kw):
    base = dict(tokens=9, experts=6, topk=2, K1=256, N1=64, K2=32, N2=40, granularity=8,
                seed=17)
    base.update(kw)
    base["K2"] = base["N1"] // 2
    return W.make_moe(**base)


def run_moe_stepwise(C, moe, sample=None, fused=True):
    """Run the layer; check every step against the oracle on the GPU's own
    input to that step.  sample: number of sampled outputs per GEMM (None =
    all).  fused: SwiGLU in the L1 epilogue (then L1 is checked through h,
    the SwiGLU of the oracle's L1 output), else the separate calls."""
    from moe_amax_gsa_amd.layer import Nvfp4MoE
    P = int(moe.offsets[-1])
    w = W.moe_weights_to(moe, DEV, keep_host=True)
    layer = Nvfp4MoE(*w, max_pairs=P, max_tokens=moe.T, granularity=moe.granularity, fused=fused)
    assert layer.fused == fused
    xd = W.bf16_to_torch(moe.x, DEV)
    ri = to_dev(moe.pair_token)
    off = to_dev(moe.offsets)
    y2 = layer(xd, ri, off).cpu().numpy().astype(np.float64)
    torch.cuda.synchronize()
    g1 = f32(layer.gsa1)
    assert g1 == oracle.amax_gsa(moe.x)
    oc1, os1 = oracle.quantize(moe.x, g1)
    assert np.array_equal(layer.x_codes[:moe.T].cpu().numpy(), oc1)
    assert np.array_equal(layer.x_scales[:moe.T].cpu().numpy(), os1)
    y1 = None if fused else layer.y1[:P].cpu().numpy().astype(np.float64)
    h = layer.h[:P].cpu().numpy()
    hc = layer.h_codes[:P].cpu().numpy()
    hs = layer.h_scales[:P].cpu().numpy()
    g2 = f32(layer.gsa2)
    gran = moe.granularity
    rng = np.random.default_rng(0)

    def silu_mul(g, u):
        return g / (1.0 + np.exp(-g)) * u

    for layer_id, Ncols in [(0, moe.N1), (1, moe.N2)]:
        ref_max = 0.0
        err_max = 0.0
        for e in moe.active_experts:
            r0, r1 = int(moe.offsets[e]), int(moe.offsets[e + 1])
            wc, wsf, w2 = moe.weight(layer_id, int(e))
            rows = np.arange(r0, r1)
            if layer_id == 0:
                ac, asf, g = oc1[moe.pair_token[rows]], os1[moe.pair_token[rows]], g1
            else:
                ac, asf, g = hc[rows], hs[rows], g2
            if layer_id == 0 and fused:
                # h against the SwiGLU of the oracle's L1 output (fp32 as the
                # GPU holds it, SwiGLU in double)
                if sample is None:
                    l1 = oracle.linear(ac, asf, g, wc, wsf, w2).astype(np.float32)
                    ref = oracle.swiglu_deinterleave(l1, gran)
                    got = h[rows].astype(np.float64)
                else:
                    ms = rng.integers(0, len(rows), sample)
                    cs = rng.integers(0, Ncols // 2, sample)
                    cs[:2] = [0, Ncols // 2 - 1]
                    gcol = (cs // gran) * 2 * gran + cs % gran
                    lg = oracle.linear_at(ac, asf, g, wc, wsf, w2, ms, gcol).astype(np.float32)
                    lu = oracle.linear_at(ac, asf, g, wc, wsf, w2, ms, gcol + gran).astype(np.float32)
                    ref = silu_mul(lg.astype(np.float64), lu.astype(np.float64))
                    got = h[rows[ms], cs].astype(np.float64)
            elif sample is None:
                ref = oracle.linear(ac, asf, g, wc, wsf, w2)
                got = (y1 if layer_id == 0 else y2)[rows]
            else:
                ms = rng.integers(0, len(rows), sample)
                ns = rng.integers(0, Ncols, sample)
                ns[:2] = [0, Ncols - 1]
                ref = oracle.linear_at(ac, asf, g, wc, wsf, w2, ms, ns)
                got = (y1 if layer_id == 0 else y2)[rows[ms], ns]
            ref_max = max(ref_max, float(np.max(np.abs(ref))))
            err_max = max(err_max, float(np.max(np.abs(got - ref))))
        assert err_max / ref_max <= REL_TOL, (layer_id, err_max / ref_max)
        if layer_id == 0:
            if not fused:
                # SwiGLU on the GPU's own L1 output (tolerance only: exp rounding)
                href = oracle.swiglu_deinterleave(layer.y1[:P].cpu().numpy(), gran)
                assert np.max(np.abs(h - href)) <= 1e-6 * np.max(np.abs(href))
            # re-quantize of the GPU's own h: bit-exact
            assert g2 == oracle.amax_gsa(h)
            oc2, os2 = oracle.quantize(h, g2)
            assert np.array_equal(hc, oc2) and np.array_equal(hs, os2)


@pytest.mark.parametrize("N,K", [(48, 256), (130, 1024), (1024, 7168)])
def test_quantize_weight(C, N, K):
    """Weight-side quantize at load time: codes, scales and weight_scale_2
    bit-exact with the oracle's amax -> gsa -> quantize of the bf16 weight,
    and the layer built from it gives the oracle's linear of those codes."""
    from moe_amax_gsa_amd.layer import Nvfp4Linear
    say(f"quantize weight N={N} K={K}")
    rng = np.random.default_rng(N + K)
    w = W.to_bf16_bits(rng.standard_normal((N, K)) * 0.02)
    w[rng.integers(0, N), rng.integers(0, K)] = W.to_bf16_bits(np.array([0.75]))[0]
    wd = W.bf16_to_torch(w, DEV)
    lin = Nvfp4Linear.from_weight(wd, max_tokens=8)
    torch.cuda.synchronize()
    g = oracle.amax_gsa(w)
    assert f32(lin.ws2) == g
    oc, os_ = oracle.quantize(w, g)
    assert np.array_equal(lin.w_codes.cpu().numpy(), oc)
    assert np.array_equal(lin.w_scales.cpu().numpy(), os_)
    x = W.to_bf16_bits(rng.standard_normal((5, K)))
    y = lin(W.bf16_to_torch(x, DEV)).cpu().numpy().astype(np.float64)
    gx = oracle.amax_gsa(x)
    xc, xs = oracle.quantize(x, gx)
    ref = oracle.linear(xc, xs, gx, oc, os_, g)
    assert rel_err(y, ref) <= REL_TOL


def test_moe_forward_quantized_matches_forward(C):
    """Nvfp4MoE.forward_quantized on the codes that forward itself made
    gives the same output bits."""
    from moe_amax_gsa_amd.layer import Nvfp4MoE
    say("moe forward_quantized")
    moe = moe_small()
    w = W.moe_weights_to(moe, DEV)
    P = int(moe.offsets[-1])
    layer = Nvfp4MoE(*w, max_pairs=P, max_tokens=moe.T, granularity=moe.granularity)
    x = W.bf16_to_torch(moe.x, DEV)
    ri = torch.from_numpy(moe.pair_token).to(DEV)
    off = torch.from_numpy(moe.offsets).to(DEV)
    y1 = layer(x, ri, off).clone()
    xc, xs = layer.x_codes[:moe.T].clone(), layer.x_scales[:moe.T].clone()
    g = layer.gsa1.clone()
    y2 = layer.forward_quantized(xc, xs, g, ri, off)
    assert torch.equal(y1, y2)


def test_moe_fused_and_unfused_agree_with_rows_outside_groups(C):
    """The last three pairs belong to no expert (offsets[E] < P) and the
    intermediate buffers hold large garbage: the grouped linear leaves those
    rows unwritten, yet both paths keep them out of h's amax, so gsa_h and
    every grouped row's output agree bit for bit, and gsa_h is the oracle's
    amax over the grouped rows of h only."""
    from moe_amax_gsa_amd.layer import Nvfp4MoE
    say("moe rows outside groups")
    moe = moe_small()
    P = int(moe.offsets[-1])
    off_h = np.minimum(moe.offsets, P - 3).astype(np.int32)
    w = W.moe_weights_to(moe, DEV)
    xd = W.bf16_to_torch(moe.x, DEV)
    ri, off = to_dev(moe.pair_token), to_dev(off_h)
    outs = []
    for fused in (True, False):
        layer = Nvfp4MoE(*w, max_pairs=P, max_tokens=moe.T, granularity=moe.granularity,
                         fused=fused)
        assert layer.fused == fused
        layer.h.fill_(1.0e6)
        layer.y2.fill_(7.0)
        if layer.y1 is not None:
            layer.y1.fill_(-3.0e5)
        y2 = layer(xd, ri, off).clone()
        torch.cuda.synchronize()
        outs.append((f32(layer.gsa2), y2[:P - 3].cpu().numpy(), layer.h[:P - 3].cpu().numpy()))
    (gf, yf, hf), (gu, yu, hu) = outs
    assert np.array_equal(hf, hu)
    assert gf == gu == oracle.amax_gsa(np.ascontiguousarray(hf))
    assert np.array_equal(yf, yu)


@pytest.mark.parametrize("fused", [True, False], ids=["fused", "unfused"])
def test_moe_small_stepwise(C, fused):
    say("moe small", fused)
    run_moe_stepwise(C, moe_small(), fused=fused)


@pytest.mark.parametrize("fused", [True, False], ids=["fused", "unfused"])
def test_moe_small_skewed_groups(C, fused):
    """One expert takes many rows (more than one pass of the grouped kernel),
    several experts are empty."""
    say("moe skewed", fused)
    run_moe_stepwise(C, moe_small(tokens=40, experts=3, topk=2, K1=512, N1=64, N2=24, seed=4),
                     fused=fused)


@pytest.mark.parametrize("lim", ["off", "median"])
@pytest.mark.parametrize("gran", [8, 4, 2, 1])
@pytest.mark.parametrize("K,N", [(256, 64), (768, 160), (2048, 96)])
def test_grouped_swiglu_matches_unfused(C, K, N, gran, lim):
    """nvfp4_grouped_linear_swiglu against the three separate calls on the
    same inputs: h bit-identical and the same gsa_h.  Group sizes 0 .. 19,
    invalid row indices (rows left unwritten in both, and out of the amax:
    both h buffers start at zero), partial column tiles; without a SwiGLU
    limit and with one at the median |l1| (so both clamps act)."""
    say(f"grouped swiglu K={K} N={N} gran={gran} limit={lim}")
    rng = np.random.default_rng(K + N + gran)
    sizes = [3, 0, 1, 19, 2, 0, 5, 9]
    G = len(sizes)
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    P = int(offsets[-1])
    a_rows = 11
    row_index = rng.integers(0, a_rows, P).astype(np.int32)
    row_index[[4, 10, 20]] = [-1, a_rows, 1 << 20]
    ac = to_dev(rng.integers(0, 256, (a_rows, K // 2), dtype=np.uint8))
    asf = to_dev(rng.integers(0x20, 0x48, (a_rows, K // 16), dtype=np.uint8))
    wc = to_dev(rng.integers(0, 256, (G, N, K // 2), dtype=np.uint8))
    wsf = to_dev(rng.integers(0x20, 0x48, (G, N, K // 16), dtype=np.uint8))
    ws2 = to_dev(rng.uniform(0.002, 0.01, G).astype(np.float32))
    gsa = to_dev(np.array([0.37], np.float32))
    ri, off = to_dev(row_index), to_dev(offsets)
    l1 = torch.zeros(P, N, dtype=torch.float32, device=DEV)
    C.nvfp4_grouped_linear(ac, asf, gsa, ri, off, wc, wsf, ws2, l1)
    limit = 0.0 if lim == "off" else float(torch.median(torch.abs(l1[l1 != 0])))
    # fused
    h1 = torch.zeros(P, N // 2, dtype=torch.float32, device=DEV)
    g1 = torch.zeros(1, dtype=torch.float32, device=DEV)
    ws = torch.empty(max(C.nvfp4_workspace_bytes(C.OP_GROUPED_SWIGLU, 0, N, 0, G), 16),
                     dtype=torch.uint8, device=DEV)
    hc1 = torch.full((P, N // 4), 0x5A, dtype=torch.uint8, device=DEV)
    hs1 = torch.full((P, N // 32), 0x5A, dtype=torch.uint8, device=DEV)
    C.nvfp4_grouped_linear_swiglu(ac, asf, gsa, ri, off, wc, wsf, ws2, h1, g1, gran, ws,
                                  h_codes=hc1, h_scales=hs1, limit=limit)
    # unfused
    h2 = torch.zeros(P, N // 2, dtype=torch.float32, device=DEV)
    g2 = torch.zeros(1, dtype=torch.float32, device=DEV)
    C.nvfp4_swiglu_deinterleave(l1, h2, gran, limit=limit)
    aws = torch.empty(max(C.nvfp4_workspace_bytes(C.OP_AMAX_GSA, P * N // 2), 16),
                      dtype=torch.uint8, device=DEV)
    C.nvfp4_amax_gsa(h2, g2, aws)
    hc2, hs2 = gpu_quantize(C, h2, g2)
    torch.cuda.synchronize()
    a, b = h1.cpu().numpy(), h2.cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    assert f32(g1) == f32(g2)
    assert np.all(a[[4, 10]] == 0.0)  # invalid row indices: unwritten
    # h's quantize in the same call (the partials reduced by the quantize)
    assert torch.equal(hc1, hc2) and torch.equal(hs1, hs2)
    # and h against the oracle's SwiGLU of the same l1 (written rows)
    href = oracle.swiglu_deinterleave(l1.cpu().numpy(), gran, limit)
    keep = np.ones(P, bool)
    keep[[4, 10, 20]] = False
    assert np.max(np.abs(a[keep] - href[keep])) <= 1e-6 * max(np.max(np.abs(href[keep])), 1e-30)


@pytest.mark.parametrize("G,rows", [(64, {0: 1, 17: 2, 63: 1}), (100, {5: 3, 6: 1, 99: 2}),
                                    (700, {3: 1, 511: 2, 512: 1, 699: 1})])
def test_grouped_sparse_groups(C, G, rows):
    """Fewer rows than groups (one decoded token over many experts): the
    ring launches one row of workgroups per possible group with rows and
    each finds its group on the device (700 groups: a scan over more
    groups than threads).  Linear against the oracle; fused SwiGLU
    bit-identical with the unfused calls."""
    K, N, gran = 512, 64, 8
    say(f"grouped sparse G={G} rows={rows}")
    rng = np.random.default_rng(G)
    sizes = np.zeros(G, np.int64)
    for g, n in rows.items():
        sizes[g] = n
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    P = int(offsets[-1])
    assert P < G
    a_rows = 3
    row_index = rng.integers(0, a_rows, P).astype(np.int32)
    ac = rng.integers(0, 256, (a_rows, K // 2), dtype=np.uint8)
    asf = rng.integers(0x20, 0x48, (a_rows, K // 16), dtype=np.uint8)
    wc = rng.integers(0, 256, (G, N, K // 2), dtype=np.uint8)
    wsf = rng.integers(0x20, 0x48, (G, N, K // 16), dtype=np.uint8)
    ws2 = rng.uniform(0.002, 0.01, G).astype(np.float32)
    gsa = np.float32(0.37)
    d = dict(ac=to_dev(ac), asf=to_dev(asf), gsa=to_dev(np.array([gsa], np.float32)),
             ri=to_dev(row_index), off=to_dev(offsets), wc=to_dev(wc), wsf=to_dev(wsf),
             ws2=to_dev(ws2))
    y = torch.full((P, N), -7.0, dtype=torch.float32, device=DEV)
    C.nvfp4_grouped_linear(d["ac"], d["asf"], d["gsa"], d["ri"], d["off"], d["wc"], d["wsf"],
                           d["ws2"], y)
    ref = oracle.grouped_linear(ac, asf, gsa, row_index, offsets, wc, wsf, ws2, P)
    assert rel_err(y.cpu().numpy().astype(np.float64), ref) <= REL_TOL
    h1 = torch.zeros(P, N // 2, dtype=torch.float32, device=DEV)
    g1 = torch.zeros(1, dtype=torch.float32, device=DEV)
    ws = torch.full((max(C.nvfp4_workspace_bytes(C.OP_GROUPED_SWIGLU, 0, N, 0, G), 16),), 0xAB,
                    dtype=torch.uint8, device=DEV)
    hc1 = torch.full((P, N // 4), 0x5A, dtype=torch.uint8, device=DEV)
    hs1 = torch.full((P, N // 32), 0x5A, dtype=torch.uint8, device=DEV)
    C.nvfp4_grouped_linear_swiglu(d["ac"], d["asf"], d["gsa"], d["ri"], d["off"], d["wc"],
                                  d["wsf"], d["ws2"], h1, g1, gran, ws, h_codes=hc1, h_scales=hs1)
    h2 = torch.zeros(P, N // 2, dtype=torch.float32, device=DEV)
    g2 = torch.zeros(1, dtype=torch.float32, device=DEV)
    C.nvfp4_swiglu_deinterleave(y, h2, gran)
    C.nvfp4_amax_gsa(h2, g2, None)
    hc2, hs2 = gpu_quantize(C, h2, g2)
    torch.cuda.synchronize()
    assert np.array_equal(h1.cpu().numpy().view(np.uint32), h2.cpu().numpy().view(np.uint32))
    assert f32(g1) == f32(g2)
    assert torch.equal(hc1, hc2) and torch.equal(hs1, hs2)


def test_grouped_swiglu_quantize_many_partials(C):
    """More amax partials than one quantize workgroup reduces (128 groups x
    17 workgroups of 128 columns = 2176): the finalize runs as its own kernel
    before h's quantize.  h's codes and scales against the oracle's quantize
    of the GPU's h."""
    K, N, gran, G = 256, 2112, 8, 128
    say("grouped swiglu quantize, 2176 partials")
    rng = np.random.default_rng(5)
    sizes = rng.integers(1, 4, G)
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    P = int(offsets[-1])
    a_rows = 5
    row_index = rng.integers(0, a_rows, P).astype(np.int32)
    ac = to_dev(rng.integers(0, 256, (a_rows, K // 2), dtype=np.uint8))
    asf = to_dev(rng.integers(0x20, 0x48, (a_rows, K // 16), dtype=np.uint8))
    wc = to_dev(rng.integers(0, 256, (G, N, K // 2), dtype=np.uint8))
    wsf = to_dev(rng.integers(0x20, 0x48, (G, N, K // 16), dtype=np.uint8))
    ws2 = to_dev(rng.uniform(0.002, 0.01, G).astype(np.float32))
    gsa = to_dev(np.array([0.37], np.float32))
    nws = C.nvfp4_workspace_bytes(C.OP_GROUPED_SWIGLU, 0, N, 0, G)
    assert nws >= 2176 * 4
    ws = torch.full((nws,), 0xAB, dtype=torch.uint8, device=DEV)
    h = torch.zeros(P, N // 2, dtype=torch.float32, device=DEV)
    gh = torch.zeros(1, dtype=torch.float32, device=DEV)
    hc = torch.full((P, N // 4), 0x5A, dtype=torch.uint8, device=DEV)
    hs = torch.full((P, N // 32), 0x5A, dtype=torch.uint8, device=DEV)
    C.nvfp4_grouped_linear_swiglu(ac, asf, gsa, to_dev(row_index), to_dev(offsets), wc, wsf, ws2,
                                  h, gh, gran, ws, h_codes=hc, h_scales=hs)
    hh = h.cpu().numpy()
    assert f32(gh) == oracle.amax_gsa(hh)
    oc, os_ = oracle.quantize(hh, f32(gh))
    assert np.array_equal(hc.cpu().numpy(), oc) and np.array_equal(hs.cpu().numpy(), os_)


def test_grouped_row_index_bounds(C):
    """Row indices outside the activation rows and rows past the last group
    are left unwritten."""
    say("grouped bounds")
    rng = np.random.default_rng(2)
    K, N, G = 64, 32, 2
    ac = rng.integers(0, 256, (3, K // 2), dtype=np.uint8)
    asf = np.full((3, K // 16), 0x38, np.uint8)
    wc = rng.integers(0, 256, (G, N, K // 2), dtype=np.uint8)
    wsf = np.full((G, N, K // 16), 0x38, np.uint8)
    offsets = np.array([0, 2, 4], np.int32)
    row_index = np.array([0, 7, 2, -1, 1, 1], np.int32)  # rows 1, 3 invalid; rows 4, 5 ungrouped
    one = torch.ones(G, dtype=torch.float32, device=DEV)
    y = torch.full((6, N), -7.0, dtype=torch.float32, device=DEV)
    C.nvfp4_grouped_linear(to_dev(ac), to_dev(asf), one[:1], to_dev(row_index), to_dev(offsets),
                           to_dev(wc), to_dev(wsf), one, y)
    yh = y.cpu().numpy().astype(np.float64)
    assert np.all(yh[[1, 3, 4, 5]] == -7.0)
    for r, g in [(0, 0), (2, 1)]:
        ref = oracle.linear(ac[row_index[r]:row_index[r] + 1], asf[:1], 1.0, wc[g], wsf[g], 1.0)
        assert np.array_equal(yh[r], ref[0])


@pytest.mark.parametrize("sizes", [[3, 0, 1, 19, 2, 0, 5, 9], [3, 0, 1, 4, 2, 0, 7, 1],
                                   [1, 0, 2, 1, 2, 0, 1, 1], [1, 0, 5, 0, 0, 1, 0, 1]],
                         ids=["large-groups", "small-groups", "decode-groups", "decode-uneven"])
@pytest.mark.parametrize("K,N", [(256, 72), (768, 64), (1280, 40), (2048, 136), (1024, 200),
                                 (512, 273)])
def test_grouped_ring_shapes(C, K, N, sizes):
    """Grouped linear on 16-byte aligned operands with K % 256 == 0: group
    sizes 0 .. 19 (a mean above 4 rows takes 16 rows per pass, else 8, so
    the 19-row group makes two passes; a mean of 2 rows or fewer splits
    each tile's K range between two waves where the super-chunk count is
    even, and passes two rows at a time, so the 5-row group makes three),
    invalid row indices, K of 1, 3, 4, 5 and 8 super-chunks against
    a 3- or 4-slot ring, N with partial tiles and whole idle waves (N = 273:
    one valid column in the last tile, so an invalid row's mask comes from
    lanes whose own column is past N).  Every written row against the
    oracle; invalid rows and rows past the last group stay unwritten."""
    say(f"grouped ring K={K} N={N} sizes={sizes}")
    rng = np.random.default_rng(K + N + sum(sizes))
    G = len(sizes)
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    P = int(offsets[-1])
    a_rows = 11
    row_index = rng.integers(0, a_rows, P + 3).astype(np.int32)
    bad = [i for i in (4, 10, 20) if i < P]
    row_index[bad] = [-1, a_rows, 1 << 20][:len(bad)]  # invalid: not written
    ac = rng.integers(0, 256, (a_rows, K // 2), dtype=np.uint8)
    asf = rng.integers(0x20, 0x48, (a_rows, K // 16), dtype=np.uint8)
    wc = rng.integers(0, 256, (G, N, K // 2), dtype=np.uint8)
    wsf = rng.integers(0x20, 0x48, (G, N, K // 16), dtype=np.uint8)
    ws2 = rng.uniform(0.002, 0.01, G).astype(np.float32)
    gsa = np.float32(0.37)
    y = torch.full((P + 3, N), -7.0, dtype=torch.float32, device=DEV)
    C.nvfp4_grouped_linear(to_dev(ac), to_dev(asf), to_dev(np.array([gsa], np.float32)),
                           to_dev(row_index), to_dev(offsets), to_dev(wc), to_dev(wsf),
                           to_dev(ws2), y)
    yh = y.cpu().numpy().astype(np.float64)
    assert np.all(yh[P:] == -7.0)
    for g in range(G):
        for r in range(offsets[g], offsets[g + 1]):
            src = int(row_index[r])
            if src < 0 or src >= a_rows:
                assert np.all(yh[r] == -7.0), r
                continue
            ref = oracle.linear(ac[src:src + 1], asf[src:src + 1], float(gsa), wc[g], wsf[g],
                                float(ws2[g]))[0]
            err = np.max(np.abs(yh[r] - ref)) / max(np.max(np.abs(ref)), 1e-30)
            assert err <= REL_TOL, (g, r, err)


# ---------------------------------------------------------------- RMSNorm -> quantize
# inv_rms: the kernel sums K squares in float32 (per-thread runs of K/2048
# terms, then a 256-way tree) and takes a correctly rounded divide and
# square root: relative error below (K/2048 + 12) * 2^-24 + 2 ulp, under
# 4e-6 for K <= 32768.  1e-5 leaves room.
INV_RMS_TOL = 1e-5


def rms_case(M, K, seed, zero_row=False):
    r = W.make_rmsnorm(M, K, seed, zero_row=zero_row)
    return r.x, r.w


def gpu_rmsnorm_quantize(C, x, w, per_row, eps=1e-6):
    M, K = x.shape
    gsa = torch.full((M if per_row else 1,), -1.0, dtype=torch.float32, device=DEV)
    inv = torch.full((M,), -1.0, dtype=torch.float32, device=DEV)
    codes = torch.full((M, K // 2), 0x5A, dtype=torch.uint8, device=DEV)
    scales = torch.full((M, K // 16), 0x5A, dtype=torch.uint8, device=DEV)
    nws = max(4, C.nvfp4_workspace_bytes(C.OP_RMSNORM_QUANTIZE, M, 0, K))
    ws = torch.full((nws,), 0xAB, dtype=torch.uint8, device=DEV)
    C.nvfp4_rmsnorm_quantize(x, w, gsa, inv, codes, scales, eps=eps, per_row=per_row, ws=ws)
    return gsa, inv, codes, scales


RMS_CASES = [
    (1, 16, "bf16", "bf16"), (1, 7168, "bf16", "bf16"), (3, 272, "fp32", "bf16"),
    (5, 1040, "bf16", "fp32"), (64, 2048, "fp32", "fp32"), (130, 7168, "bf16", "bf16"),
    (257, 4096, "bf16", "fp32"),
    (1, 32768, "bf16", "fp32"), (3, 12288, "fp32", "bf16"),   # four, two half-blocks a thread
    (2, 33024, "fp32", "bf16"),                               # too long for one row kernel
    (4100, 32, "bf16", "bf16"),           # one scale over > 4096 rows: separate finalize
]


@pytest.mark.parametrize("per_row", [False, True], ids=["one_gsa", "gsa_per_row"])
@pytest.mark.parametrize("M,K,xd,wd", RMS_CASES)
def test_rmsnorm_quantize(C, M, K, xd, wd, per_row):
    """inv_rms against the oracle's binary64 RMSNorm; the normalized rows
    rebuilt on the host from the GPU's inv_rms with the kernel's two float32
    products, (x * inv_rms) * w, so that the quantize decisions are taken in
    one precision on both sides: gsa, codes and scales bit-exact with the
    oracle's quantize of those rows."""
    say(f"rmsnorm quantize M={M} K={K} x={xd} w={wd} per_row={per_row}")
    xb, wb = rms_case(M, K, seed=M * 7 + K, zero_row=M >= 3)
    xh, wh = x_host(xb, xd), x_host(wb, wd)
    gsa, inv, codes, scales = gpu_rmsnorm_quantize(C, x_dev(xb, xd), x_dev(wb, wd), per_row)
    inv_g = inv.cpu().numpy()
    inv_o, y_o = oracle.rmsnorm(xh, wh, 1e-6)
    assert np.max(np.abs(inv_g / inv_o - 1.0)) <= INV_RMS_TOL
    x32 = W.bf16_bits_to_f32(xb)
    w32 = W.bf16_bits_to_f32(wb)
    y32 = (x32 * inv_g[:, None]).astype(np.float32) * w32[None, :]
    assert y32.dtype == np.float32
    assert np.max(np.abs(y32 - y_o)) <= 4 * INV_RMS_TOL * np.max(np.abs(y_o))
    if per_row:
        oc, os_, og = oracle.quantize_rows(y32)
        assert np.array_equal(gsa.cpu().numpy(), og)
    else:
        og = oracle.amax_gsa(y32)
        assert f32(gsa) == og
        oc, os_ = oracle.quantize(y32, og)
    assert np.array_equal(codes.cpu().numpy(), oc)
    assert np.array_equal(scales.cpu().numpy(), os_)
    if M >= 3:  # the zero row: inv_rms = 1/sqrt(eps), codes and scales 0
        assert np.all(codes.cpu().numpy()[M // 2] == 0) and np.all(scales.cpu().numpy()[M // 2] == 0)


def test_rmsnorm_quantize_empty(C):
    say("rmsnorm quantize M=0")
    x = torch.empty(0, 256, dtype=torch.bfloat16, device=DEV)
    w = torch.ones(256, dtype=torch.bfloat16, device=DEV)
    gsa, _, _, _ = gpu_rmsnorm_quantize(C, x, w, per_row=False)
    assert f32(gsa) == oracle.gsa_from_amax(0.0)


LINEAR_ROWS_CASES = [
    (1, 96, 7168), (3, 130, 1024),            # one-pass kernel
    (9, 40, 2048), (5, 33, 272),              # 16-row kernel, staged and ragged K
    (64, 96, 1024), (130, 300, 768),          # LDS-staged tiles (eight / four waves)
    (40, 70, 320), (33, 50, 272),             # direct tiles, aligned and ragged K
]


@pytest.mark.parametrize("M,N,K", LINEAR_ROWS_CASES)
def test_linear_rows(C, M, N, K):
    """RMSNorm -> quantize with one gsa per row, then the linear that takes
    that gsa: y[m] against the oracle's linear of row m with gsa[m]; bf16
    output is the float32 output rounded."""
    say(f"linear rows M={M} N={N} K={K}")
    xb, wb = rms_case(M, K, seed=M + N + K)
    gsa, _, codes, scales = gpu_rmsnorm_quantize(C, x_dev(xb, "bf16"), x_dev(wb, "bf16"), True)
    inp = W.make_linear(1, K, N, seed=K + 1, sf=(0.125, 8.0), ws2=0.0037)
    wc, wsc = to_dev(inp.w_codes), to_dev(inp.w_scales)
    ws2 = torch.tensor([inp.ws2], dtype=torch.float32, device=DEV)
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    C.nvfp4_linear_rows(codes, scales, gsa, wc, wsc, ws2, y)
    ref = oracle.linear_rows(codes.cpu().numpy(), scales.cpu().numpy(), gsa.cpu().numpy(),
                             inp.w_codes, inp.w_scales, inp.ws2)
    yg = y.cpu().numpy().astype(np.float64)
    assert not np.any(np.isnan(yg))
    # each row against its own magnitude: the rows' scales differ by up to e^6
    err = np.max(np.abs(yg - ref), axis=1) / np.maximum(np.max(np.abs(ref), axis=1), 1e-300)
    assert np.max(err) <= REL_TOL
    y16 = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)
    C.nvfp4_linear_rows(codes, scales, gsa, wc, wsc, ws2, y16)
    assert torch.equal(y16.cpu(), y.cpu().to(torch.bfloat16))


@pytest.mark.parametrize("per_row", [False, True], ids=["one_gsa", "gsa_per_row"])
def test_layer_rmsnorm_forward(C, per_row):
    """Nvfp4Linear.rmsnorm_forward: the oracle's RMSNorm -> quantize ->
    linear, row by row against each row's magnitude."""
    from moe_amax_gsa_amd.layer import Nvfp4Linear
    M, K, N = 7, 1024, 80
    say(f"layer rmsnorm_forward per_row={per_row}")
    xb, wb = rms_case(M, K, seed=77)
    inp = W.make_linear(1, K, N, seed=78, ws2=0.0041)
    lin = Nvfp4Linear(to_dev(inp.w_codes), to_dev(inp.w_scales), inp.ws2, max_tokens=16)
    y = lin.rmsnorm_forward(x_dev(xb, "bf16"), x_dev(wb, "bf16"), gsa_per_row=per_row)
    yg = y.cpu().numpy().astype(np.float64)
    y32 = ((W.bf16_bits_to_f32(xb) * lin.inv_rms[:M].cpu().numpy()[:, None]).astype(np.float32)
           * W.bf16_bits_to_f32(wb)[None, :])
    if per_row:
        oc, os_, og = oracle.quantize_rows(y32)
        ref = oracle.linear_rows(oc, os_, og, inp.w_codes, inp.w_scales, inp.ws2)
    else:
        og = oracle.amax_gsa(y32)
        oc, os_ = oracle.quantize(y32, og)
        ref = oracle.linear(oc, os_, og, inp.w_codes, inp.w_scales, inp.ws2)
    assert np.array_equal(lin.codes[:M].cpu().numpy(), oc)
    err = np.max(np.abs(yg - ref), axis=1) / np.maximum(np.max(np.abs(ref), axis=1), 1e-300)
    assert np.max(err) <= REL_TOL


# ---------------------------------------------------------------- router
def router_inputs(M, K, N, k, seed):
    """Router operands quantized by the oracle: A from x, the gate weight
    with its own global scale (the load-time recipe)."""
    r = W.make_router(M, K, N, k, seed)
    ga = oracle.amax_gsa(r.x)
    ac, as_ = oracle.quantize(r.x, ga)
    gw = oracle.amax_gsa(r.w)
    wc, wsf = oracle.quantize(r.w, gw)
    return r, ga, ac, as_, gw, wc, wsf


def gpu_router(C, ac, as_, ga, wc, wsf, gw, bias, k):
    M, N = ac.shape[0], wc.shape[0]
    idx = torch.full((M, k), -7, dtype=torch.int32, device=DEV)
    sc = torch.full((M, k), float("nan"), dtype=torch.float32, device=DEV)
    K = ac.shape[1] * 2
    ws = torch.full((max(16, C.nvfp4_workspace_bytes(C.OP_ROUTER_TOPK, M, N, K)),), 0xAB,
                    dtype=torch.uint8, device=DEV)
    cnt = (M * N * 4 + 15) // 16 * 16  # the one-launch path's ticket counter (M <= 16)
    if M <= 16:
        ws[cnt:cnt + 4].zero_()  # zero before the first call, as the ABI asks
    args = (to_dev(ac), to_dev(as_), torch.tensor([ga], device=DEV), to_dev(wc), to_dev(wsf),
            torch.tensor([gw], device=DEV), None if bias is None else to_dev(bias), idx, sc, ws)
    C.nvfp4_router_topk(*args)
    logits = ws[:M * N * 4].view(torch.float32).view(M, N).cpu().numpy()
    idx1, sc1 = idx.cpu().numpy(), sc.cpu().numpy()
    if M <= 16:
        # the counter is left zero, and a second call (garbage logits area)
        # chooses the same experts
        assert int(ws[cnt:cnt + 4].view(torch.int32).item()) == 0
        ws[:M * N * 4].fill_(0xAB)
        idx.fill_(-7)
        C.nvfp4_router_topk(*args)
        assert np.array_equal(idx.cpu().numpy(), idx1)
        assert int(ws[cnt:cnt + 4].view(torch.int32).item()) == 0
    return idx1, sc1, logits


def check_choice(idx_g, sc_g, z, bias, k, eps):
    """The GPU's choice on its own logits z, against the oracle's choice on
    the same logits: identical, or different only among values within eps
    of each other (fp32 scores on the GPU, binary64 in the oracle)."""
    idx_o, sc_o = oracle.router_topk(z, bias, k)
    v = oracle.router_scores(z) + (0.0 if bias is None else bias.astype(np.float64))
    for m in range(z.shape[0]):
        assert len(set(idx_g[m])) == k and np.all((idx_g[m] >= 0) & (idx_g[m] < z.shape[1]))
        if not np.array_equal(idx_g[m], idx_o[m]):
            assert np.all(np.abs(v[m, idx_g[m]] - v[m, idx_o[m]]) <= eps), m
    # the scores: sqrt(softplus) of the chosen logits, to a few fp32 ulp
    ref = oracle.router_scores(np.take_along_axis(z.astype(np.float64), idx_g.astype(np.int64),
                                                  axis=1))
    assert np.allclose(sc_g, ref, rtol=2e-6, atol=0)
    return idx_o


ROUTER_CASES = [
    (1, 384, 7168, 6), (1, 256, 7168, 8), (3, 256, 1024, 8),   # weight-streaming kernels
    (16, 384, 2048, 6), (5, 33, 272, 1),
    (17, 256, 512, 8), (64, 384, 7168, 6), (130, 96, 768, 4),   # tiled kernels
    (2, 1024, 256, 32), (4, 64, 256, 64),                       # 1024 experts; k = N
]


@pytest.mark.parametrize("M,N,K,k", ROUTER_CASES)
def test_router_topk(C, M, N, K, k):
    """Gate logits against the oracle's linear (1e-3 of the largest); the
    choice against the oracle's on the GPU's own logits (equal up to fp32
    near-ties); and, where the oracle's own logits leave a clear gap after
    the k-th expert, the same set of experts as the oracle end to end."""
    say(f"router M={M} N={N} K={K} k={k}")
    r, ga, ac, as_, gw, wc, wsf = router_inputs(M, K, N, k, seed=M * 31 + N + K + k)
    idx_g, sc_g, z = gpu_router(C, ac, as_, ga, wc, wsf, gw, r.bias, k)
    zo = oracle.linear(ac, as_, ga, wc, wsf, gw)
    dz = np.max(np.abs(z - zo))
    assert dz <= REL_TOL * np.max(np.abs(zo))
    vmax = np.max(np.abs(oracle.router_scores(z))) + np.max(np.abs(r.bias))
    check_choice(idx_g, sc_g, z, r.bias, k, eps=1e-6 * vmax)
    # end to end: |d s / d z| <= 0.6, so the GPU's values are within
    # 0.6 dz (+ fp32 rounding) of the oracle's
    vo = oracle.router_scores(zo) + r.bias.astype(np.float64)
    delta = 0.6 * dz + 1e-6 * vmax
    idx_e, _ = oracle.router_topk(zo, r.bias, k)
    checked = 0
    for m in range(M):
        srt = np.sort(vo[m])[::-1]
        if k < N and srt[k - 1] - srt[k] <= 2 * delta:
            continue
        assert set(idx_g[m]) == set(idx_e[m]), m
        checked += 1
    assert checked >= (M + 1) // 2


@pytest.mark.parametrize("M,N,K,k", [(1, 384, 1024, 6), (9, 256, 1024, 8), (40, 128, 1024, 8)])
def test_router_integer_case_exact(C, M, N, K, k):
    """Scales 1.0 and gsa = gsb = 2^-4: the logits are exact on both sides,
    so the choice (no bias) is the oracle's exactly, ties included."""
    say(f"router integer M={M} N={N} K={K}")
    rng = np.random.default_rng(M + N)
    ac = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    wc = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    asf = np.full((M, K // 16), 0x38, np.uint8)
    wsf = np.full((N, K // 16), 0x38, np.uint8)
    g = np.float32(2.0 ** -4)
    idx_g, sc_g, z = gpu_router(C, ac, asf, g, wc, wsf, g, None, k)
    zo = oracle.linear(ac, asf, g, wc, wsf, g)
    assert np.array_equal(z.astype(np.float64), zo)
    idx_o, sc_o = oracle.router_topk(zo, None, k)
    assert np.array_equal(idx_g, idx_o)
    assert np.allclose(sc_g, sc_o, rtol=2e-6, atol=0)


@pytest.mark.parametrize("M", [1, 64, 200])
def test_layer_linear_sizes_its_workspace(C, M):
    """Nvfp4Linear sized for 256 tokens: one token (weight-streaming
    kernel), 64 and 200 tokens (few tiles: split K through the layer's own
    workspace) -- against the oracle."""
    from moe_amax_gsa_amd.layer import Nvfp4Linear
    K, N = 2048, 96
    say(f"layer linear M={M}")
    inp = W.make_linear(M, K, N, seed=M + 5, ws2=0.006)
    lin = Nvfp4Linear(to_dev(inp.w_codes), to_dev(inp.w_scales), inp.ws2, max_tokens=256)
    y = lin(W.bf16_to_torch(inp.x, DEV)).cpu().numpy().astype(np.float64)
    g = f32(lin.gsa)
    oc, os_ = oracle.quantize(inp.x, g)
    ref = oracle.linear(oc, os_, g, inp.w_codes, inp.w_scales, inp.ws2)
    assert rel_err(y, ref) <= REL_TOL


def test_router_layer(C):
    """Nvfp4Router: gate weight quantized at load time, activation quantized
    per call, then the choice -- against the oracle's chain on the same
    bf16 inputs."""
    from moe_amax_gsa_amd.layer import Nvfp4Router
    say("router layer")
    for M in [3, 40]:  # 40 rows: the gate linear splits K inside the router's workspace
        r = W.make_router(M, 2048, 256, 8, seed=12 + M)
        router = Nvfp4Router.from_weight(W.bf16_to_torch(r.w, DEV), to_dev(r.bias), topk=8,
                                         max_tokens=64)
        check_router_layer(router, r, M)


def check_router_layer(router, r, M):
    idx, sc = router(W.bf16_to_torch(r.x, DEV))
    idx, sc = idx.cpu().numpy(), sc.cpu().numpy()
    gw = oracle.amax_gsa(r.w)
    assert f32(router.gate.ws2) == gw
    ga = oracle.amax_gsa(r.x)
    ac, as_ = oracle.quantize(r.x, ga)
    wc, wsf = oracle.quantize(r.w, gw)
    z = router.ws[:M * 256 * 4].view(torch.float32).view(M, 256).cpu().numpy()
    zo = oracle.linear(ac, as_, ga, wc, wsf, gw)
    assert np.max(np.abs(z - zo)) <= REL_TOL * np.max(np.abs(zo))
    vmax = np.max(np.abs(oracle.router_scores(z))) + np.max(np.abs(r.bias))
    check_choice(idx, sc, z, r.bias, 8, eps=1e-6 * vmax)


@pytest.mark.parametrize("limit", [0.0, 6.0, 1e30])
def test_swiglu_parity(C, limit):
    """The unfused SwiGLU against the oracle within 1e-6 relative, without a
    limit, with one that clamps gate and up values on both sides (|l1| up
    to ~25), and with one that clamps nothing."""
    say("swiglu", limit)
    rng = np.random.default_rng(1)
    l1 = (rng.standard_normal((37, 96)) * 5).astype(np.float32)
    h = torch.empty(37, 48, dtype=torch.float32, device=DEV)
    C.nvfp4_swiglu_deinterleave(to_dev(l1), h, 8, limit=limit)
    href = oracle.swiglu_deinterleave(l1, 8, limit)
    assert np.max(np.abs(h.cpu().numpy() - href)) <= 1e-6 * np.max(np.abs(href))


# ---------------------------------------------------------------- full workloads
def sample_positions(M, N, n, seed):
    rng = np.random.default_rng(seed)
    ms = rng.integers(0, M, n)
    ns = rng.integers(0, N, n)
    ms[:4] = [0, 0, M - 1, M - 1]
    ns[:4] = [0, N - 1, 0, N - 1]
    return ms, ns


@pytest.mark.parametrize("name", ["tiny_m1_k256_n256", "decode_m1_k7168_n1536",
                                  "prefill_m512_k7168_n4096", "stress_m2048_k7168_n7168"])
def test_workload_linear(C, name):
    say("workload", name)
    inp = W.make(name)
    g, codes, scales, y = run_linear(C, inp)
    assert f32(g) == oracle.amax_gsa(inp.x)
    oc, os_ = oracle.quantize(inp.x, f32(g))
    assert np.array_equal(scales.cpu().numpy(), os_)
    assert np.array_equal(codes.cpu().numpy(), oc)
    yg = y.cpu().numpy().astype(np.float64)
    assert not np.any(np.isnan(yg))
    if inp.M * inp.N <= 1 << 16:
        ref = oracle.linear(oc, os_, f32(g), inp.w_codes, inp.w_scales, inp.ws2)
        assert rel_err(yg, ref) <= REL_TOL
    else:
        ms, ns = sample_positions(inp.M, inp.N, 4096, 1)
        ref = oracle.linear_at(oc, os_, f32(g), inp.w_codes, inp.w_scales, inp.ws2, ms, ns)
        assert rel_err(yg[ms, ns], ref) <= REL_TOL


def test_workload_lm_head_decode(C):
    """A one-row decode with the lm_head's shape through nvfp4_linear_run (the
    ring, 128 weight rows a workgroup): gsa, codes and scales bit-exact, 4096
    sampled outputs within 1e-3."""
    say("workload lm_head decode")
    inp = W.make("lm_head_m1_k7168_n129280")
    xd = W.bf16_to_torch(inp.x, DEV)
    gsa = torch.zeros(1, dtype=torch.float32, device=DEV)
    codes = torch.full((1, inp.K // 2), 0x5A, dtype=torch.uint8, device=DEV)
    scales = torch.full((1, inp.K // 16), 0x5A, dtype=torch.uint8, device=DEV)
    y = torch.full((1, inp.N), float("nan"), dtype=torch.float32, device=DEV)
    C.nvfp4_linear_run(xd, gsa, codes, scales, to_dev(inp.w_codes), to_dev(inp.w_scales),
                       torch.tensor([inp.ws2], dtype=torch.float32, device=DEV), y)
    g = f32(gsa)
    assert g == oracle.amax_gsa(inp.x)
    oc, os_ = oracle.quantize(inp.x, g)
    assert np.array_equal(codes.cpu().numpy(), oc) and np.array_equal(scales.cpu().numpy(), os_)
    yg = y.cpu().numpy().astype(np.float64)
    assert not np.any(np.isnan(yg))
    ms, ns = sample_positions(1, inp.N, 4096, 2)
    ref = oracle.linear_at(oc, os_, g, inp.w_codes, inp.w_scales, inp.ws2, ms, ns)
    assert rel_err(yg[ms, ns], ref) <= REL_TOL


def test_workload_moe(C):
    say("workload moe_t64_e256_top8")
    run_moe_stepwise(C, W.make("moe_t64_e256_top8"), sample=64)



# ------------------------------------------------------- grouped, tiled
def grouped_case(seed, sizes, K, N, start=0, tail=0, a_rows=64, bad=()):
    """Random grouped operands: groups of the given sizes starting at output
    row `start` (rows before it and `tail` rows after the last group are in
    no group), row_index uniform over a_rows with the entries in `bad`
    pointing outside [0, a_rows)."""
    rng = np.random.default_rng(seed)
    G = len(sizes)
    offsets = (start + np.concatenate([[0], np.cumsum(sizes)])).astype(np.int32)
    M_total = int(offsets[-1]) + tail
    row_index = rng.integers(0, a_rows, M_total).astype(np.int32)
    for r, v in bad:
        row_index[r] = v
    ac = rng.integers(0, 256, (a_rows, K // 2), dtype=np.uint8)
    asf = rng.integers(0x20, 0x48, (a_rows, K // 16), dtype=np.uint8)
    wc = rng.integers(0, 256, (G, N, K // 2), dtype=np.uint8)
    wsf = rng.integers(0x20, 0x48, (G, N, K // 16), dtype=np.uint8)
    ws2 = rng.uniform(0.002, 0.01, G).astype(np.float32)
    return dict(G=G, offsets=offsets, M_total=M_total, row_index=row_index, ac=ac, asf=asf,
                wc=wc, wsf=wsf, ws2=ws2, gsa=np.float32(0.37), a_rows=a_rows)


def grouped_gpu(C, c, y_dtype=torch.float32):
    y = torch.full((c["M_total"], c["wc"].shape[1]), -7.0, dtype=y_dtype, device=DEV)
    C.nvfp4_grouped_linear(to_dev(c["ac"]), to_dev(c["asf"]),
                           to_dev(np.array([c["gsa"]], np.float32)), to_dev(c["row_index"]),
                           to_dev(c["offsets"]), to_dev(c["wc"]), to_dev(c["wsf"]),
                           to_dev(c["ws2"]), y)
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64)


def grouped_expected_rows(c):
    """Output rows the grouped linear writes: inside a group, with a valid
    row_index."""
    live = np.zeros(c["M_total"], bool)
    live[c["offsets"][0]:c["offsets"][-1]] = True
    ri = c["row_index"]
    return live & (ri >= 0) & (ri < c["a_rows"])


TILED_CASES = [
    # (sizes, K, N): mean rows per group >= 32 takes the tiled kernel.
    # 128 x 64 tiles: a 129-row group makes two row tiles (the second one
    # row), empty groups make none; N not a multiple of 64
    ([37, 0, 128, 129, 5, 203], 512, 200),    # few tiles: eight waves per tile
    ([37, 0, 128, 129, 5, 203], 768, 64),     # K % 512 != 0: four waves per tile
    ([37, 0, 128, 129, 5, 203], 7168, 136),   # long K, 14 chunks of 512
    ([300], 1024, 40),                        # one group (G = 1)
    ([33] * 40, 256, 72),                     # 40 groups of 33 rows: scan over 40 groups
    ([2, 0, 0, 90, 1, 1, 1, 1, 300], 512, 64),  # skewed: mean 44, most groups tiny
    # larger groups: ragged row tiles, partial column tiles
    ([130, 0, 128, 255, 97, 301], 512, 200),  # groups of 2 to 5 row tiles, one empty
    ([130, 0, 128, 255, 97, 301], 768, 520),  # K % 512 != 0; the last column tile 8 wide
    ([200, 200, 200], 7168, 256),             # long K, 14 chunks of 512
    ([96] * 20, 256, 64),                     # 20 groups of 96 rows, one chunk of 256
    ([1, 0, 0, 500, 3, 2, 1, 300], 512, 136),  # skewed: mean 101, most groups tiny
]


@pytest.mark.parametrize("sizes,K,N", TILED_CASES)
def test_grouped_tiled_shapes(C, sizes, K, N):
    """The grouped linear on the tiled kernel (mean rows per group >= 32):
    every written row against the oracle's grouped linear, rows before the
    first group, after the last and with an invalid row_index unwritten."""
    say(f"grouped tiled sizes={sizes[:9]} K={K} N={N}")
    c = grouped_case(K + N + len(sizes), sizes, K, N, start=3, tail=4,
                     bad=[(5, -1), (40, 64), (100, 1 << 20)])
    y = grouped_gpu(C, c)
    live = grouped_expected_rows(c)
    assert np.all(y[~live] == -7.0)
    ri = np.where(live, c["row_index"], 0).astype(np.int32)
    ref = oracle.grouped_linear(c["ac"], c["asf"], c["gsa"], ri, c["offsets"], c["wc"], c["wsf"],
                                c["ws2"], c["M_total"])
    assert not np.any(np.isnan(y[live]))
    assert rel_err(y[live], ref[live]) <= REL_TOL


def test_grouped_tiled_many_groups_and_identity_rows(C):
    """150 groups (the tile search scans the offsets 64 groups at a time,
    three passes), a third of them empty, 40 rows per group on average;
    once with a row gather and once with row_index NULL (output row r reads
    activation row r).  Every written row against the oracle."""
    say("grouped tiled 150 groups")
    rng = np.random.default_rng(150)
    sizes = rng.integers(0, 121, 150)
    sizes[rng.random(150) < 0.33] = 0
    K, N = 256, 136
    c = grouped_case(150, list(sizes), K, N, a_rows=int(sizes.sum()) + 8)
    assert c["M_total"] / c["G"] >= 32
    for gather in (True, False):
        if not gather:
            c["row_index"] = np.arange(c["M_total"], dtype=np.int32)
        y = torch.full((c["M_total"], N), -7.0, dtype=torch.float32, device=DEV)
        C.nvfp4_grouped_linear(to_dev(c["ac"]), to_dev(c["asf"]),
                               to_dev(np.array([c["gsa"]], np.float32)),
                               to_dev(c["row_index"]) if gather else None,
                               to_dev(c["offsets"]), to_dev(c["wc"]), to_dev(c["wsf"]),
                               to_dev(c["ws2"]), y)
        yh = y.cpu().numpy().astype(np.float64)
        ref = oracle.grouped_linear(c["ac"], c["asf"], c["gsa"], c["row_index"], c["offsets"],
                                    c["wc"], c["wsf"], c["ws2"], c["M_total"])
        assert not np.any(np.isnan(yh))
        assert rel_err(yh, ref) <= REL_TOL, gather


@pytest.mark.parametrize("sizes", [[64, 100, 3, 150], [100, 200, 3, 150]],
                         ids=["mean-80", "mean-114"])
def test_grouped_tiled_bf16_is_rounded_fp32(C, sizes):
    """bf16 output of the tiled grouped kernel: the fp32 output rounded to
    nearest even, bit for bit."""
    say("grouped tiled bf16", sizes)
    c = grouped_case(77, sizes, 512, 96, start=1, tail=2)
    y32 = grouped_gpu(C, c)
    y16 = grouped_gpu(C, c, torch.bfloat16)
    live = grouped_expected_rows(c)
    r = torch.from_numpy(y32[live].astype(np.float32)).to(torch.bfloat16).float().numpy()
    assert np.array_equal(r, y16[live].astype(np.float32))


def test_grouped_tiled_many_tiles(C):
    """More row x column tiles than CUs (four waves per tile, two workgroups
    per CU, the tiles spread over the XCDs in runs): 4096 rows over 32
    groups of skewed sizes; sampled outputs against the oracle, every row
    of every group sampled at least once."""
    say("grouped tiled many tiles")
    rng = np.random.default_rng(11)
    sizes = rng.multinomial(4096 - 32, np.linspace(3.0, 0.2, 32) / np.linspace(3.0, 0.2, 32).sum())
    sizes = sizes + 1
    K, N = 512, 1088
    c = grouped_case(11, list(sizes), K, N, a_rows=512)
    y = grouped_gpu(C, c)
    off = c["offsets"]
    errs, refmax = 0.0, 0.0
    for g in range(c["G"]):
        rows = np.arange(off[g], off[g + 1])
        ns = rng.integers(0, N, rows.size)
        if rows.size >= 2:
            ns[:2] = [0, N - 1]
        ms = c["row_index"][rows]
        ref = oracle.linear_at(c["ac"], c["asf"], c["gsa"], c["wc"][g], c["wsf"][g],
                               c["ws2"][g], ms, ns)
        errs = max(errs, float(np.max(np.abs(y[rows, ns] - ref))))
        refmax = max(refmax, float(np.max(np.abs(ref))))
    assert errs / refmax <= REL_TOL



@pytest.mark.parametrize("lim", ["off", "median"])
@pytest.mark.parametrize("gran", [8, 1])
@pytest.mark.parametrize("K,N", [(512, 256), (768, 416)])
def test_grouped_swiglu_tiled_matches_unfused(C, K, N, gran, lim):
    """The fused SwiGLU epilogue of the tiled grouped kernel (groups of 32
    or more rows on average) against the separate calls.  N = 416: a partial
    last column tile."""
    grouped_swiglu_fused_matches_unfused(C, [37, 0, 128, 129, 5, 203], K, N, gran, lim)


@pytest.mark.parametrize("lim", ["off", "median"])
@pytest.mark.parametrize("gran", [1, 2, 4, 8])
@pytest.mark.parametrize("K,N", [(512, 512), (768, 384)])
def test_grouped_swiglu_large_groups_match_unfused(C, K, N, gran, lim):
    """The same with groups of 2 to 5 row tiles and every granularity the
    entry point takes (gate and up columns 1 to 8 apart).  N = 384: a
    partial last column tile."""
    grouped_swiglu_fused_matches_unfused(C, [130, 0, 128, 255, 97, 301], K, N, gran, lim)


def test_grouped_swiglu_large_h_finalize_launch(C):
    """An h of 2^20 half-blocks and more (16 groups of 260 rows, N = 4096):
    its amax partials go through a finalize launch before the quantize;
    the same checks as the other fused SwiGLU cases."""
    grouped_swiglu_fused_matches_unfused(C, [260] * 16, 256, 4096, 8, "off")


def grouped_swiglu_fused_matches_unfused(C, sizes, K, N, gran, lim):
    """The fused SwiGLU epilogue of a tiled grouped kernel against the
    separate calls, which take the same tiled kernel for the linear: h
    bit-identical, the same gsa_h, h's codes and scales identical; rows
    outside every group and with an invalid row_index unwritten in both and
    outside the amax.  h against the oracle's SwiGLU of the GPU's l1, codes
    and scales against the oracle's quantize of the GPU's h."""
    say(f"grouped swiglu tiled sizes={sizes} K={K} N={N} gran={gran} limit={lim}")
    c = grouped_case(K + N + gran, sizes, K, N, start=3, tail=4,
                     bad=[(5, -1), (40, 64), (100, 1 << 20)])
    P = c["M_total"]
    live = grouped_expected_rows(c)
    d = {k: to_dev(c[k]) for k in ("ac", "asf", "row_index", "offsets", "wc", "wsf", "ws2")}
    gsa = to_dev(np.array([c["gsa"]], np.float32))
    l1 = torch.zeros(P, N, dtype=torch.float32, device=DEV)
    C.nvfp4_grouped_linear(d["ac"], d["asf"], gsa, d["row_index"], d["offsets"], d["wc"],
                           d["wsf"], d["ws2"], l1)
    limit = 0.0 if lim == "off" else float(torch.median(torch.abs(l1[l1 != 0])))
    h1 = torch.zeros(P, N // 2, dtype=torch.float32, device=DEV)
    g1 = torch.zeros(1, dtype=torch.float32, device=DEV)
    nws = C.nvfp4_workspace_bytes(C.OP_GROUPED_SWIGLU, P, N, 0, c["G"])
    ws = torch.full((nws,), 0xAB, dtype=torch.uint8, device=DEV)
    hc1 = torch.full((P, N // 4), 0x5A, dtype=torch.uint8, device=DEV)
    hs1 = torch.full((P, N // 32), 0x5A, dtype=torch.uint8, device=DEV)
    C.nvfp4_grouped_linear_swiglu(d["ac"], d["asf"], gsa, d["row_index"], d["offsets"], d["wc"],
                                  d["wsf"], d["ws2"], h1, g1, gran, ws, h_codes=hc1,
                                  h_scales=hs1, limit=limit)
    h2 = torch.zeros(P, N // 2, dtype=torch.float32, device=DEV)
    g2 = torch.zeros(1, dtype=torch.float32, device=DEV)
    C.nvfp4_swiglu_deinterleave(l1, h2, gran, limit=limit)
    C.nvfp4_amax_gsa(h2, g2, torch.empty(max(C.nvfp4_workspace_bytes(C.OP_AMAX_GSA,
                                                                      P * N // 2), 16),
                                         dtype=torch.uint8, device=DEV))
    hc2, hs2 = gpu_quantize(C, h2, g2)
    torch.cuda.synchronize()
    a, b = h1.cpu().numpy(), h2.cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    assert np.all(a[~live] == 0.0)
    assert f32(g1) == f32(g2)
    assert torch.equal(hc1, hc2) and torch.equal(hs1, hs2)
    href = oracle.swiglu_deinterleave(l1.cpu().numpy(), gran, limit)
    assert np.max(np.abs(a[live] - href[live])) <= 1e-6 * np.max(np.abs(href[live]))
    assert f32(g1) == oracle.amax_gsa(a)
    oc, os_ = oracle.quantize(a, f32(g1))
    assert np.array_equal(hc1.cpu().numpy(), oc) and np.array_equal(hs1.cpu().numpy(), os_)


@pytest.mark.parametrize("name", ["moe_l1_t512_e32_top8_k7168_n4096",
                                  "moe_l1_t512_e32_top8_k7168_n4096_zipf"])
def test_workload_routed_first_projection(C, name):
    """512 tokens, top 8 of 32 experts, the first expert projection through
    nvfp4_grouped_linear_run: gsa, codes and scales bit-exact with the
    oracle's quantize; 32 sampled outputs of every expert (its first and
    last rows, first and last columns among them) within 1e-3 of the
    oracle's linear of those codes."""
    say("workload", name)
    moe = W.make(name)
    P = int(moe.offsets[-1])
    w1c, w1s, w1w, _, _, _ = W.moe_weights_to(moe, DEV, first_only=True)
    xd = W.bf16_to_torch(moe.x, DEV)
    gsa = torch.full((1,), -1.0, dtype=torch.float32, device=DEV)
    codes = torch.full((moe.T, moe.K1 // 2), 0x5A, dtype=torch.uint8, device=DEV)
    scales = torch.full((moe.T, moe.K1 // 16), 0x5A, dtype=torch.uint8, device=DEV)
    y = torch.full((P, moe.N1), float("nan"), dtype=torch.float32, device=DEV)
    nws = max(16, C.nvfp4_workspace_bytes(C.OP_GROUPED_RUN, moe.T, moe.N1, moe.K1, moe.E))
    ws = torch.full((nws,), 0xAB, dtype=torch.uint8, device=DEV)
    C.nvfp4_grouped_linear_run(xd, gsa, codes, scales, to_dev(moe.pair_token),
                               to_dev(moe.offsets), w1c, w1s, w1w, y, ws)
    torch.cuda.synchronize()
    del w1c, w1s
    g = f32(gsa)
    assert g == oracle.amax_gsa(moe.x)
    oc, os_ = oracle.quantize(moe.x, g)
    assert np.array_equal(codes.cpu().numpy(), oc) and np.array_equal(scales.cpu().numpy(), os_)
    yh = y.cpu().numpy()
    assert not np.any(np.isnan(yh))
    rng = np.random.default_rng(0)
    errs, refmax = 0.0, 0.0
    for e in moe.active_experts:
        r0, r1 = int(moe.offsets[e]), int(moe.offsets[e + 1])
        wc, wsf, w2 = moe.weight(0, int(e))
        moe.drop_cache()
        rows = rng.integers(r0, r1, 32)
        rows[:2] = [r0, r1 - 1]
        ns = rng.integers(0, moe.N1, 32)
        ns[:2] = [0, moe.N1 - 1]
        ref = oracle.linear_at(oc, os_, g, wc, wsf, w2, moe.pair_token[rows], ns)
        got = yh[rows, ns].astype(np.float64)
        errs = max(errs, float(np.max(np.abs(got - ref))))
        refmax = max(refmax, float(np.max(np.abs(ref))))
    assert errs / refmax <= REL_TOL


# ---------------------------------------------------------------- grouped runs
def run_grouped(C, gi, dtype):
    """nvfp4_grouped_linear_run on a make_grouped input; the GPU's outputs."""
    rows = gi.T * gi.G
    xd = x_dev(gi.x, dtype)
    gsa = torch.full((1,), -1.0, dtype=torch.float32, device=DEV)
    codes = torch.full((rows, gi.K // 2), 0x5A, dtype=torch.uint8, device=DEV)
    scales = torch.full((rows, gi.K // 16), 0x5A, dtype=torch.uint8, device=DEV)
    y = torch.full((rows, gi.N), float("nan"), dtype=torch.float32, device=DEV)
    nws = max(16, C.nvfp4_workspace_bytes(C.OP_GROUPED_RUN, rows, gi.N, gi.K, gi.G))
    ws = torch.full((nws,), 0xAB, dtype=torch.uint8, device=DEV)
    C.nvfp4_grouped_linear_run(xd, gsa, codes, scales, to_dev(gi.row_index), to_dev(gi.offsets),
                               to_dev(gi.w_codes), to_dev(gi.w_scales), to_dev(gi.ws2), y, ws)
    torch.cuda.synchronize()
    return (f32(gsa), codes.cpu().numpy(), scales.cpu().numpy(),
            y.cpu().numpy().astype(np.float64))


GROUPED_RUN_CASES = [
    # (T, G, K, N, dtype); token t's slice g is row t*G + g of x
    (1, 8, 1024, 96, "bf16"),    # 8192 elements: one launch
    (2, 4, 2048, 40, "fp32"),    # 16384 elements, fp32: one launch
    (1, 8, 8192, 64, "bf16"),    # the pages' wo_a slices: amax partials, then one launch
    (3, 2, 7168, 130, "bf16"),   # 43008 elements, N not a multiple of 16
    (1, 2, 272, 32, "bf16"),     # K % 256 != 0: the two ABI calls
    (1, 1, 7168, 4096, "bf16"),  # one projection (G = 1)
    (64, 8, 512, 96, "bf16"),    # 64 tokens: quantize first, then the tiled kernel
    (40, 3, 1024, 130, "fp32"),  # 40 rows per group, fp32 activation, ragged N
]


@pytest.mark.parametrize("T,G,K,N,dtype", GROUPED_RUN_CASES)
def test_grouped_linear_run(C, T, G, K, N, dtype):
    """gsa and every row's codes and scales bit-exact with the oracle's
    quantize of the whole activation; outputs within 1e-3 of the oracle's
    grouped linear on those codes."""
    say("grouped run", T, G, K, N, dtype)
    gi = W.make_grouped(T, G, K, N, seed=T + G + K + N, x="outliers")
    g, codes, scales, y = run_grouped(C, gi, dtype)
    xh = x_host(gi.x, dtype)
    assert g == oracle.amax_gsa(xh)
    oc, os_ = oracle.quantize(xh, g)
    assert np.array_equal(codes, oc) and np.array_equal(scales, os_)
    ref = oracle.grouped_linear(oc, os_, g, gi.row_index, gi.offsets, gi.w_codes, gi.w_scales,
                                gi.ws2, T * G)
    assert not np.any(np.isnan(y))
    assert rel_err(y, ref) <= REL_TOL


@pytest.mark.parametrize("kind", EXTREME)
@pytest.mark.parametrize("T,G,K,N", [(1, 8, 1024, 96), (1, 8, 8192, 64), (64, 8, 512, 96)])
def test_grouped_linear_run_extreme_magnitudes(C, T, G, K, N, kind):
    """The grouped run's three paths (every workgroup reducing and
    quantizing x itself; amax partials, then the ring quantizing its rows;
    quantize, then the tiled kernel) on activations at the edges of the
    formats' ranges: gsa, codes and scales bit-exact, outputs within 1e-3
    of the oracle's (all zero where every activation scale is zero)."""
    say("grouped run extreme", T, G, K, N, kind)
    gi = W.make_grouped(T, G, K, N, seed=T + G + K + N + len(kind), x=kind)
    g, codes, scales, y = run_grouped(C, gi, "bf16")
    assert g == oracle.amax_gsa(gi.x)
    oc, os_ = oracle.quantize(gi.x, g)
    assert np.array_equal(codes, oc) and np.array_equal(scales, os_)
    ref = oracle.grouped_linear(oc, os_, g, gi.row_index, gi.offsets, gi.w_codes, gi.w_scales,
                                gi.ws2, T * G)
    assert np.all(np.isfinite(y))
    if not np.any(ref):
        assert not np.any(y)
    else:
        assert rel_err(y, ref) <= REL_TOL


def test_grouped_linear_run_routed_token(C):
    """One token routed to 6 of 16 experts (the decode of routed experts),
    plus two output rows past the last group (left unwritten)."""
    say("grouped run routed")
    moe = W.make_moe(tokens=1, experts=16, topk=6, K1=1024, N1=64, K2=32, N2=8, seed=7)
    w1c, w1s, w1w, _, _, _ = W.moe_weights_to(moe, DEV, keep_host=True)
    P = int(moe.offsets[-1])
    ri = np.concatenate([moe.pair_token, [0, 0]]).astype(np.int32)
    xd = W.bf16_to_torch(moe.x, DEV)
    gsa = torch.zeros(1, dtype=torch.float32, device=DEV)
    codes = torch.full((1, moe.K1 // 2), 0x5A, dtype=torch.uint8, device=DEV)
    scales = torch.full((1, moe.K1 // 16), 0x5A, dtype=torch.uint8, device=DEV)
    y = torch.full((P + 2, moe.N1), 7.0, dtype=torch.float32, device=DEV)
    C.nvfp4_grouped_linear_run(xd, gsa, codes, scales, to_dev(ri), to_dev(moe.offsets), w1c, w1s,
                               w1w, y)
    g = f32(gsa)
    assert g == oracle.amax_gsa(moe.x)
    oc, os_ = oracle.quantize(moe.x, g)
    assert np.array_equal(codes.cpu().numpy(), oc) and np.array_equal(scales.cpu().numpy(), os_)
    wc = np.stack([moe.weight(0, e)[0] for e in range(moe.E)])
    wsf = np.stack([moe.weight(0, e)[1] for e in range(moe.E)])
    w2 = np.array([moe.weight(0, e)[2] for e in range(moe.E)], np.float32)
    ref = oracle.grouped_linear(oc, os_, g, moe.pair_token, moe.offsets, wc, wsf, w2, P)
    yg = y.cpu().numpy().astype(np.float64)
    assert rel_err(yg[:P], ref) <= REL_TOL
    assert np.all(yg[P:] == 7.0)


@pytest.mark.parametrize("tokens,experts,topk,K1,N1,N2", [
    (1, 8, 4, 512, 512, 40),      # a decoded token: two launches
    (2, 16, 8, 1024, 512, 64),    # two tokens (2048 elements): two launches
    (40, 6, 2, 512, 512, 24),     # x past 16384 elements: x quantized first
    (1, 16, 12, 1024, 6144, 6144),  # 576 ring workgroups each: the split prologue
    (256, 8, 2, 512, 512, 64),    # 64 pairs per expert: both projections tiled
    (96, 3, 1, 1024, 512, 136),   # 32 pairs per expert, N2 a partial column tile
    (384, 8, 2, 512, 512, 136),   # 96 pairs per expert, both projections tiled
])
def test_moe_run(C, tokens, experts, topk, K1, N1, N2):
    """nvfp4_moe_run: every step against the oracle on the GPU's own input to
    it, and every output bit-equal to the separate calls'."""
    say("moe run", tokens, experts, topk, K1, N1, N2)
    moe = W.make_moe(tokens=tokens, experts=experts, topk=topk, K1=K1, N1=N1, K2=N1 // 2, N2=N2,
                     granularity=8, seed=tokens + experts)
    moe_run_matches_separate_calls(C, moe)


def test_moe_run_decode_skewed_groups(C):
    """Six tokens, 2 of 32 experts each with Zipf routing: one pair per
    expert on average (both projections split each weight tile's K range
    between two waves), while the first expert holds 5 pairs, so its tiles
    make three passes of two rows.  Every step against the oracle, every
    output bit-equal to the separate calls."""
    say("moe run decode zipf")
    moe = W.make_moe(tokens=6, experts=32, topk=2, K1=1024, N1=1024, K2=512, N2=64,
                     granularity=8, seed=5, routing="zipf")
    counts = np.diff(moe.offsets)
    assert counts.max() == 5 and -(-int(counts.sum()) // moe.E) == 1
    moe_run_matches_separate_calls(C, moe)


def moe_run_matches_separate_calls(C, moe):
    """The MoE pair stepwise against the oracle, then the layer through
    nvfp4_moe_run and through the separate calls: gsa, codes, scales, h and
    y bit-equal between the two."""
    from moe_amax_gsa_amd.layer import Nvfp4MoE
    run_moe_stepwise(C, moe, fused=True)
    P = int(moe.offsets[-1])
    w = W.moe_weights_to(moe, DEV)
    xd = W.bf16_to_torch(moe.x, DEV)
    ri, off = to_dev(moe.pair_token), to_dev(moe.offsets)
    outs = []
    for run_entry in (True, False):
        layer = Nvfp4MoE(*w, max_pairs=P, max_tokens=moe.T, granularity=8, run_entry=run_entry)
        assert layer.run_entry == run_entry
        y2 = layer(xd, ri, off).clone()
        torch.cuda.synchronize()
        outs.append([t.cpu().numpy() for t in (layer.gsa1, layer.x_codes[:moe.T],
                                               layer.x_scales[:moe.T], layer.h[:P], layer.gsa2,
                                               layer.h_codes[:P], layer.h_scales[:P], y2)])
    for a, b in zip(*outs):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))


@pytest.mark.parametrize("limit", [0.0, 2.0])
def test_moe_run_tiled_skewed_matches_separate_calls(C, limit):
    """nvfp4_moe_run with Zipf routing (128 tokens, 2 of 8 experts: the first
    experts take most pairs, the last few under 32), both projections on the
    tiled kernel, without and with a SwiGLU limit that clamps: every output
    bit-equal to the separate calls (which take the same kernels for the
    projections), and y against the oracle on the GPU's own h codes."""
    from moe_amax_gsa_amd.layer import Nvfp4MoE
    say("moe run tiled zipf", limit)
    moe = W.make_moe(tokens=128, experts=8, topk=2, K1=512, N1=512, K2=256, N2=136,
                     granularity=8, seed=21, routing="zipf")
    P = int(moe.offsets[-1])
    assert P / moe.E >= 32
    w = W.moe_weights_to(moe, DEV, keep_host=True)
    xd = W.bf16_to_torch(moe.x, DEV)
    ri, off = to_dev(moe.pair_token), to_dev(moe.offsets)
    outs = []
    for run_entry in (True, False):
        layer = Nvfp4MoE(*w, max_pairs=P, max_tokens=moe.T, granularity=8,
                         swiglu_limit=limit, run_entry=run_entry)
        assert layer.run_entry == run_entry
        y2 = layer(xd, ri, off).clone()
        torch.cuda.synchronize()
        outs.append([t.cpu().numpy() for t in (layer.gsa1, layer.h[:P], layer.gsa2,
                                               layer.h_codes[:P], layer.h_scales[:P], y2)])
    for a, b in zip(*outs):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
    g2, hc, hs, y = outs[0][2][0], outs[0][3], outs[0][4], outs[0][5].astype(np.float64)
    w2c = np.stack([moe.weight(1, e)[0] for e in range(moe.E)])
    w2s = np.stack([moe.weight(1, e)[1] for e in range(moe.E)])
    w2w = np.array([moe.weight(1, e)[2] for e in range(moe.E)], np.float32)
    ref = oracle.grouped_linear(hc, hs, g2, None, moe.offsets, w2c, w2s, w2w, P)
    assert rel_err(y, ref) <= REL_TOL


def test_workload_moe_prefill(C):
    """A prefill batch through the routed experts (512 tokens, top 8 of 32,
    about 128 pairs per expert, the MoE workload's projection sizes) through
    nvfp4_moe_run, both projections on the tiled kernel: every step against
    the oracle on the GPU's own input to it, 32 sampled outputs per expert
    and projection."""
    say("workload moe_t512_e32_top8")
    run_moe_stepwise(C, W.make("moe_t512_e32_top8"), sample=32)


def test_workload_moe_one_token(C):
    """One decoded token of the MoE workload's experts (K1 = 7168, N1 = 4096,
    K2 = 2048, N2 = 7168, 8 of 256 experts) through nvfp4_moe_run."""
    say("workload moe one token")
    c = W.WORKLOADS["moe_t64_e256_top8"]
    moe = W.make_moe(tokens=1, experts=c["experts"], topk=c["topk"], seed=c["seed"])
    run_moe_stepwise(C, moe, sample=64)


def test_workload_grouped_wo_a(C):
    """The dense grouped linear at the pages' wo_a size (one token, 8 slices
    of 8192 against 8 weights of 1536 rows): every output."""
    say("workload grouped wo_a")
    gi = W.make("grouped_wo_a_t1_g8_k8192_n1536")
    g, codes, scales, y = run_grouped(C, gi, "bf16")
    assert g == oracle.amax_gsa(gi.x)
    oc, os_ = oracle.quantize(gi.x, g)
    assert np.array_equal(codes, oc) and np.array_equal(scales, os_)
    ref = oracle.grouped_linear(oc, os_, g, gi.row_index, gi.offsets, gi.w_codes, gi.w_scales,
                                gi.ws2, gi.T * gi.G)
    assert rel_err(y, ref) <= REL_TOL


def _graph_scenario(name):
    """(step, outputs): step() enqueues one call of the named path on the
    current stream; outputs() are the tensors it writes."""
    from moe_amax_gsa_amd.layer import Nvfp4GroupedLinear, Nvfp4MoE, Nvfp4Router
    if name == "router_one_launch":
        r = W.make_router(1, 1024, 64, topk=6, seed=3)
        router = Nvfp4Router.from_weight(W.bf16_to_torch(r.w, DEV), to_dev(r.bias), r.topk,
                                         max_tokens=1)
        x = W.bf16_to_torch(r.x, DEV)
        return (lambda: router(x)), (lambda: [router.idx, router.score])
    if name in ("moe_run_one_token", "moe_run_tiled"):
        tokens, experts, topk = (1, 16, 4) if name == "moe_run_one_token" else (128, 4, 2)
        moe = W.make_moe(tokens=tokens, experts=experts, topk=topk, K1=512, N1=512, K2=256,
                         N2=136, granularity=8, seed=9)
        P = int(moe.offsets[-1])
        layer = Nvfp4MoE(*W.moe_weights_to(moe, DEV), max_pairs=P, max_tokens=moe.T)
        assert layer.run_entry
        x = W.bf16_to_torch(moe.x, DEV)
        ri, off = to_dev(moe.pair_token), to_dev(moe.offsets)
        return ((lambda: layer(x, ri, off)),
                (lambda: [layer.y2[:P], layer.h[:P], layer.gsa1, layer.gsa2]))
    T = 1 if name == "grouped_run_one_token" else 64
    gi = W.make_grouped(T, 4, 1024, 96, seed=5)
    g = Nvfp4GroupedLinear(to_dev(gi.w_codes), to_dev(gi.w_scales), to_dev(gi.ws2),
                           max_tokens=T)
    o = W.bf16_to_torch(gi.x, DEV).reshape(T, 4 * 1024)
    return (lambda: g(o)), (lambda: [g.y, g.gsa])


@pytest.mark.parametrize("name", ["router_one_launch", "moe_run_one_token", "moe_run_tiled",
                                  "grouped_run_one_token", "grouped_run_tiled"])
def test_graph_capture_replays_of_the_run_paths(C, name):
    """Each one-call path captured once in a HIP graph and replayed four
    times, with its outputs overwritten and eager work in between; every
    replay's outputs equal the eager call's bit for bit (the router's
    ticket counter is left at zero by every call, so replays keep
    working)."""
    say("graph replay", name)
    step, outs = _graph_scenario(name)
    step()
    torch.cuda.synchronize()
    eager = [t.clone() for t in outs()]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for i in range(4):
        for t in outs():
            if t.dtype.is_floating_point:
                t.fill_(float("nan"))
            else:
                t.fill_(-7)
        _ = torch.randn(1000, device=DEV).sum()  # eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs(), eager):
            assert torch.equal(a.view(torch.uint8) if a.dtype.is_floating_point else a,
                               b.view(torch.uint8) if b.dtype.is_floating_point else b), (name, i)


def test_graph_capture_replays_match_eager(C):
    """The whole step (amax, quantize, linear) captured once and replayed,
    with eager work in between; every replay equals the eager result."""
    say("graph capture")
    from moe_amax_gsa_amd.layer import Nvfp4Linear
    inp = W.make_linear(1, 7168, 1536, seed=1, x="outliers")
    layer = Nvfp4Linear(to_dev(inp.w_codes), to_dev(inp.w_scales), inp.ws2, max_tokens=1)
    x = W.bf16_to_torch(inp.x, DEV)
    eager = layer(x).clone()
    for fn in [layer.forward, layer.run]:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn(x)  # warm-up on the capture stream
        torch.cuda.current_stream().wait_stream(s)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            out = fn(x)
        for i in range(4):
            layer.y.fill_(float("nan"))
            layer.gsa.fill_(0.0)
            _ = torch.randn(1000, device=DEV).sum()  # eager work between replays
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, eager), (fn.__name__, i)
