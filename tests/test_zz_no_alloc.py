"""nvfp4_linear_run_noalloc against nvfp4_linear_run, through the C ABI.

The allocation-free variant runs the same kernels with the library's static
scratch in place of the caller's workspace, so gsa, codes, scales and y
must equal nvfp4_linear_run's bit for bit; y is also held to the oracle's
bar (max|y - y_ref| / max|y_ref| <= 1e-3) on sampled outputs.  Each case is
two calls in a row, the second with a smaller input, so the second runs on
scratch the first left behind.  Run alone in a fresh process and after the
other tests.
"""
import ctypes
import sys

import numpy as np
import pytest
import torch

from oracle import oracle
from moe_amax_gsa_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda"
REL_TOL = 1e-3


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def C():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    from moe_amax_gsa_amd import nvfp4
    return nvfp4


def one_call(C, M, K, N, seed, y_dtype):
    """Both entry points on the same seeded input; returns their outputs."""
    inp = W.make_linear(M, K, N, seed, "outliers", (0.25, 4.0), 0.005)
    x = W.bf16_to_torch(inp.x, DEV)
    wc = torch.from_numpy(inp.w_codes).to(DEV)
    wsf = torch.from_numpy(inp.w_scales).to(DEV)
    ws2 = torch.tensor([inp.ws2], dtype=torch.float32, device=DEV)
    outs = []
    for noalloc in (False, True):
        gsa = torch.full((1,), -1.0, dtype=torch.float32, device=DEV)
        codes = torch.full((M, K // 2), 0x5A, dtype=torch.uint8, device=DEV)
        scales = torch.full((M, K // 16), 0x5A, dtype=torch.uint8, device=DEV)
        y = torch.full((M, N), float("nan"), dtype=y_dtype, device=DEV)
        if noalloc:
            C.nvfp4_linear_run_noalloc(x, gsa, codes, scales, wc, wsf, ws2, y)
        else:
            nws = max(16, C.nvfp4_workspace_bytes(C.OP_LINEAR_RUN, M, N, K, 1))
            ws = torch.full((nws,), 0xAB, dtype=torch.uint8, device=DEV)
            C.nvfp4_linear_run(x, gsa, codes, scales, wc, wsf, ws2, y, ws)
        torch.cuda.synchronize()
        outs.append((gsa.cpu().numpy(), codes.cpu().numpy(), scales.cpu().numpy(),
                     y.float().cpu().numpy()))
    return inp, outs


# Two calls in a row per case, the second smaller:
#  - 128 x 7168 -> 2048 splits K 7 ways, its partials filling 7.3 MB of
#    the scratch; then 40 x 2048 -> 384, also split, on what that left;
#  - 512 x 7168 -> 1024 uses the amax partials; then one decode row, which
#    needs no scratch at all;
#  - 64 x 7168 -> 384 (the router gate's shape, split 14 ways), then
#    17 x 1024 -> 96 just past the weight-streaming kernel's row limit;
#  - 2048 x 7168 -> 7168 (224 tiles of 256 x 256, the amax partials of a
#    14.7 M-element activation), then 128 x 7168 -> 2048 (split K).
CASES = [((128, 7168, 2048), (40, 2048, 384)),
         ((512, 7168, 1024), (1, 7168, 1536)),
         ((64, 7168, 384), (17, 1024, 96)),
         ((2048, 7168, 7168), (128, 7168, 2048))]


@pytest.mark.parametrize("first,second", CASES,
                         ids=["split", "amax_then_decode", "router", "wide_then_split"])
def test_noalloc_matches_linear_run(C, first, second):
    for i, (M, K, N) in enumerate((first, second)):
        y_dtype = torch.float32 if i == 0 else torch.bfloat16
        say(f"noalloc call {i}: M={M} K={K} N={N} y={y_dtype}")
        need = C.nvfp4_workspace_bytes(C.OP_LINEAR_RUN, M, N, K, 1)
        assert need <= C.NOALLOC_SCRATCH_BYTES
        inp, ((g0, c0, s0, y0), (g1, c1, s1, y1)) = one_call(C, M, K, N, 100 + 10 * i + M,
                                                             y_dtype)
        assert np.array_equal(g0.view(np.uint32), g1.view(np.uint32))
        assert np.array_equal(c0, c1) and np.array_equal(s0, s1)
        assert np.array_equal(y0.view(np.uint32), y1.view(np.uint32))
        # the oracle's bar on sampled outputs (the GPU's own codes, checked
        # bit-exact against the oracle's quantize first)
        g = np.float32(g1[0])
        assert g == oracle.amax_gsa(inp.x)
        oc, os_ = oracle.quantize(inp.x, g)
        assert np.array_equal(c1, oc) and np.array_equal(s1, os_)
        rng = np.random.default_rng(M + N)
        ms = rng.integers(0, M, 256)
        ns = rng.integers(0, N, 256)
        ms[:2], ns[:2] = [0, M - 1], [0, N - 1]
        ref = oracle.linear_at(oc, os_, g, inp.w_codes, inp.w_scales, inp.ws2, ms, ns)
        got = y1[ms, ns].astype(np.float64)
        tol = REL_TOL if y_dtype == torch.float32 else 2.0 ** -8 + REL_TOL
        assert np.max(np.abs(got - ref)) / np.max(np.abs(ref)) <= tol


def test_noalloc_graph_replays(C):
    """Three calls captured in one HIP graph on one stream, sharing the
    static scratch: 512 x 7168 -> 1024 (amax partials, tiled linear), one
    decode row 1 x 7168 -> 1536 (one kernel) and 128 x 7168 -> 2048 (split K,
    its partials in the scratch).  Replayed three times with the outputs
    overwritten and eager work in between: every replay equal to the eager
    calls bit for bit."""
    say("noalloc graph replays")
    calls = []
    for i, (M, K, N) in enumerate([(512, 7168, 1024), (1, 7168, 1536), (128, 7168, 2048)]):
        inp = W.make_linear(M, K, N, 900 + i, "outliers", (0.25, 4.0), 0.005)
        t = dict(x=W.bf16_to_torch(inp.x, DEV),
                 gsa=torch.zeros(1, dtype=torch.float32, device=DEV),
                 codes=torch.empty(M, K // 2, dtype=torch.uint8, device=DEV),
                 scales=torch.empty(M, K // 16, dtype=torch.uint8, device=DEV),
                 wc=torch.from_numpy(inp.w_codes).to(DEV),
                 wsf=torch.from_numpy(inp.w_scales).to(DEV),
                 ws2=torch.tensor([inp.ws2], dtype=torch.float32, device=DEV),
                 y=torch.empty(M, N, dtype=torch.bfloat16 if i == 1 else torch.float32,
                               device=DEV))
        calls.append(t)

    def step():
        for t in calls:
            C.nvfp4_linear_run_noalloc(t["x"], t["gsa"], t["codes"], t["scales"], t["wc"],
                                       t["wsf"], t["ws2"], t["y"])

    def outs():
        return [t[k] for t in calls for k in ("gsa", "codes", "scales", "y")]

    step()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs()]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(3):
        for o in outs():
            o.fill_(float("nan") if o.dtype.is_floating_point else 0x5A)
        _ = torch.randn(1000, device=DEV).sum()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs(), eager):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))


def test_noalloc_rejects_bad_arguments_before_touching_the_device(C):
    L = C.lib
    fake = ctypes.c_void_p(4096)  # never dereferenced
    f = L.nvfp4_linear_run_noalloc
    # (x, x_dtype, gsa, codes, scales, w_codes, w_scales, ws2, y, y_dtype, M, N, K, stream)
    assert f(fake, 5, fake, fake, fake, fake, fake, fake, fake, 1, 2, 8, 32, None) == -3
    assert f(fake, 0, fake, fake, fake, fake, fake, fake, fake, 1, 2, 8, 40, None) == -2
    assert f(fake, 0, None, fake, fake, fake, fake, fake, fake, 1, 2, 8, 32, None) == -1
    assert f(fake, 0, fake, fake, fake, fake, fake, fake, fake, 1, 0, 8, 32, None) == 0
