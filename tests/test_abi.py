"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/nvfp4.h declares, and rejects bad arguments with a
negative status before touching the device."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4.h")
LIB = os.path.join(ROOT, "moe_amax_gsa_amd", "libnvfp4.so")


@pytest.fixture(scope="module")
def C():
    if not os.path.exists(LIB):
        from moe_amax_gsa_amd import build
        build.build(verbose=False)
    from moe_amax_gsa_amd import nvfp4
    return nvfp4


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nvfp4_\w+)\s*\(", text)))


def test_header_declares_the_four_entry_points():
    names = declared_functions()
    for n in ["nvfp4_amax_gsa", "nvfp4_quantize_from_buffer", "nvfp4_linear",
              "nvfp4_grouped_linear"]:
        assert n in names


def test_library_exports_every_declared_symbol(C):
    lib = ctypes.CDLL(C.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert C.nvfp4_abi_version() == 10


def test_status_strings(C):
    for st in [0, -1, -2, -3, -4, -5, -6]:
        assert C.lib.nvfp4_status_string(st)
    assert C.lib.nvfp4_status_string(-99) == b"unknown status"


def test_validation_errors_return_before_any_launch(C):
    L = C.lib
    fake = ctypes.c_void_p(4096)  # never dereferenced: every call below fails validation
    # bad dtype, negative size, K % 16, null pointers, workspace
    assert L.nvfp4_amax_gsa(fake, 7, 10, fake, None, 0, None) == -3
    assert L.nvfp4_amax_gsa(fake, 0, -1, fake, None, 0, None) == -2
    assert L.nvfp4_amax_gsa(fake, 0, 10, None, None, 0, None) == -1
    assert L.nvfp4_amax_gsa(ctypes.c_void_p(4097), 0, 10, fake, None, 0, None) == -5
    big = 10 ** 7
    need = C.nvfp4_workspace_bytes(C.OP_AMAX_GSA, big)
    assert need > 0
    assert L.nvfp4_amax_gsa(fake, 0, big, fake, None, 0, None) == -4
    assert L.nvfp4_amax_gsa(fake, 0, big, fake, fake, need - 4, None) == -4
    assert C.nvfp4_workspace_bytes(C.OP_AMAX_GSA, 1000) == 0
    assert L.nvfp4_quantize_from_buffer(fake, 0, 4, 15, fake, fake, fake, None) == -2
    assert L.nvfp4_quantize_from_buffer(fake, 0, 4, 0, fake, fake, fake, None) == -2
    assert L.nvfp4_quantize_from_buffer(fake, 2, 4, 16, fake, fake, fake, None) == -3
    assert L.nvfp4_quantize_from_buffer(fake, 0, 4, 16, None, fake, fake, None) == -1
    assert L.nvfp4_quantize_from_buffer(fake, 0, 0, 16, None, None, None, None) == 0  # no-op
    args = [fake] * 7
    assert L.nvfp4_linear(*args, 0, 2, 3, 24, None, 0, None) == -2
    assert L.nvfp4_linear(*args, 5, 2, 3, 32, None, 0, None) == -3
    assert L.nvfp4_linear(fake, fake, None, fake, fake, fake, fake, 1, 2, 3, 32, None, 0,
                          None) == -1
    assert L.nvfp4_linear(*args, 1, 0, 3, 32, None, 0, None) == 0  # M == 0: no-op
    # grouped: no row_index needs a_rows >= M_total; G must be positive
    assert L.nvfp4_grouped_linear(fake, fake, fake, 4, None, fake, 2, 8, fake, fake, fake, fake,
                                  1, 16, 32, None) == -2
    assert L.nvfp4_grouped_linear(fake, fake, fake, 8, None, fake, 0, 8, fake, fake, fake, fake,
                                  1, 16, 32, None) == -2
    assert L.nvfp4_swiglu_deinterleave(fake, fake, 2, 24, 8, 0.0, None) == -2
    assert L.nvfp4_swiglu_deinterleave(fake, fake, 2, 32, 0, 0.0, None) == -2
    assert L.nvfp4_swiglu_deinterleave(fake, fake, 2, 32, 8, float("nan"), None) == -2
    assert L.nvfp4_swiglu_deinterleave(fake, fake, 0, 32, 8, 10.0, None) == 0  # M == 0
    gs = L.nvfp4_grouped_linear_swiglu
    # (a_codes, a_scales, gsa, a_rows, row_index, offsets, G, M_total, w_codes, w_scales, ws2,
    #  h, gsa_h, h_codes, h_scales, N_inter, K, granularity, limit, ws, ws_bytes, stream)
    assert gs(fake, fake, fake, 4, None, fake, 1, 4, fake, fake, fake, fake, fake, None, None,
              32, 256, 8, float("nan"), fake, 1 << 20, None) == -2


def test_validation_of_the_fused_and_load_time_entries(C):
    L = C.lib
    fake = ctypes.c_void_p(4096)  # never dereferenced: every call below fails validation
    rq = L.nvfp4_rmsnorm_quantize
    # (x, x_dtype, w, w_dtype, eps, M, K, per_row, gsa, inv_rms, codes, scales, ws, ws_bytes, s)
    assert rq(fake, 0, fake, 0, 1e-6, 4, 24, 0, fake, fake, fake, fake, fake, 64, None) == -2
    assert rq(fake, 0, fake, 0, 0.0, 4, 32, 1, fake, fake, fake, fake, None, 0, None) == -2
    assert rq(fake, 0, fake, 0, -1.0, 4, 32, 1, fake, fake, fake, fake, None, 0, None) == -2
    assert rq(fake, 0, fake, 0, float("nan"), 4, 32, 1, fake, fake, fake, fake, None, 0,
              None) == -2
    assert rq(fake, 3, fake, 0, 1e-6, 4, 32, 1, fake, fake, fake, fake, None, 0, None) == -3
    assert rq(fake, 0, fake, 0, 1e-6, 4, 32, 1, None, fake, fake, fake, None, 0, None) == -1
    assert rq(fake, 0, None, 0, 1e-6, 4, 32, 1, fake, fake, fake, fake, None, 0, None) == -1
    assert rq(ctypes.c_void_p(4104), 0, fake, 0, 1e-6, 4, 32, 1, fake, fake, fake, fake, None,
              0, None) == -5
    # one global scale needs M * 4 bytes of workspace for the row maxima
    assert C.nvfp4_workspace_bytes(C.OP_RMSNORM_QUANTIZE, 4, 0, 32) == 16
    assert rq(fake, 0, fake, 0, 1e-6, 4, 32, 0, fake, fake, fake, fake, fake, 12, None) == -4
    assert rq(fake, 0, fake, 0, 1e-6, 4, 32, 0, fake, fake, fake, fake, None, 0, None) == -4
    assert rq(fake, 0, fake, 0, 1e-6, 0, 32, 1, fake, None, None, None, None, 0, None) == 0
    lr = L.nvfp4_linear_rows
    args = [fake] * 7
    assert lr(*args, 0, 2, 3, 24, None, 0, None) == -2
    assert lr(*args, 5, 2, 3, 32, None, 0, None) == -3
    assert lr(fake, fake, None, fake, fake, fake, fake, 1, 2, 3, 32, None, 0, None) == -1
    assert lr(*args, 1, 0, 3, 32, None, 0, None) == 0  # M == 0: no-op
    rt = L.nvfp4_router_topk
    # (a_codes, a_scales, gsa, w_codes, w_scales, ws2, bias, M, N, K, k, idx, score, ws, bytes, s)
    assert rt(*[fake] * 7, 2, 1025, 64, 8, fake, fake, fake, 1 << 20, None) == -2  # N > 1024
    assert rt(*[fake] * 7, 2, 64, 64, 0, fake, fake, fake, 1 << 20, None) == -2     # k < 1
    assert rt(*[fake] * 7, 2, 64, 64, 65, fake, fake, fake, 1 << 20, None) == -2    # k > N
    assert rt(*[fake] * 7, 2, 64, 40, 8, fake, fake, fake, 1 << 20, None) == -2     # K % 16
    assert rt(*[fake] * 6, None, 2, 64, 64, 8, None, fake, fake, 1 << 20, None) == -1
    assert rt(*[fake] * 6, None, 2, 64, 64, 8, fake, fake, fake, 2 * 64 * 4 - 4, None) == -4
    assert rt(*[fake] * 6, None, 2, 64, 64, 8, fake, fake, None, 0, None) == -4
    assert rt(*[fake] * 6, None, 0, 64, 64, 8, None, None, None, 0, None) == 0   # M == 0
    qw = L.nvfp4_quantize_weight
    assert qw(fake, 0, 0, 32, fake, fake, fake, None, 0, None) == -2
    assert qw(fake, 0, 4, 40, fake, fake, fake, None, 0, None) == -2
    assert qw(fake, 0, 4, 32, None, fake, fake, None, 0, None) == -1
    big = C.nvfp4_workspace_bytes(C.OP_QUANTIZE_WEIGHT, 0, 4096, 4096)
    assert big > 0
    assert qw(fake, 0, 4096, 4096, fake, fake, fake, None, 0, None) == -4


def test_linear_workspace_is_optional_and_sized_by_shape(C):
    # one output tile per device's worth of compute units: no split, no bytes
    assert C.nvfp4_workspace_bytes(C.OP_LINEAR, 4096, 4096, 7168) == 0
    assert C.nvfp4_workspace_bytes(C.OP_LINEAR, 8, 64, 7168) == 0      # weight-streaming kernel
    assert C.nvfp4_workspace_bytes(C.OP_LINEAR, 64, 96, 1000) == 0     # K not in 256-chunks
    n = C.nvfp4_workspace_bytes(C.OP_LINEAR, 64, 96, 1024)
    assert n > 0 and n % (64 * 96 * 4) == 0
    r = C.nvfp4_workspace_bytes(C.OP_ROUTER_TOPK, 64, 96, 1024)
    assert r == 64 * 96 * 4 + n


def test_validation_of_amax_quantize(C):
    L = C.lib
    fake = ctypes.c_void_p(4096)
    aq = L.nvfp4_amax_quantize
    assert aq(fake, 2, 4, 32, fake, fake, fake, None, 0, None) == -3     # dtype
    assert aq(fake, 0, 4, 40, fake, fake, fake, None, 0, None) == -2     # K % 16
    assert aq(fake, 0, -1, 32, fake, fake, fake, None, 0, None) == -2    # M < 0
    assert aq(fake, 0, 4, 32, None, fake, fake, None, 0, None) == -1     # gsa
    assert aq(None, 0, 4, 32, fake, fake, fake, None, 0, None) == -1     # x
    assert aq(ctypes.c_void_p(4104), 0, 4, 32, fake, fake, fake, None, 0, None) == -5
    # beyond one workgroup the two-phase amax needs its workspace
    assert aq(fake, 0, 1024, 1024, fake, fake, fake, None, 0, None) == -4


def test_validation_of_the_run_entries(C):
    L = C.lib
    fake = ctypes.c_void_p(4096)  # never dereferenced: every call below fails validation
    gr = L.nvfp4_grouped_linear_run
    # (x, x_dtype, x_rows, gsa, x_codes, x_scales, row_index, offsets, G, M_total, w_codes,
    #  w_scales, ws2, y, y_dtype, N, K, ws, ws_bytes, stream)
    assert gr(fake, 3, 2, fake, fake, fake, fake, fake, 2, 2, fake, fake, fake, fake, 1, 16, 256,
              None, 0, None) == -3                                           # dtype
    assert gr(fake, 0, 2, fake, fake, fake, fake, fake, 2, 2, fake, fake, fake, fake, 1, 16, 40,
              None, 0, None) == -2                                           # K % 16
    assert gr(fake, 0, 1, fake, fake, fake, None, fake, 2, 2, fake, fake, fake, fake, 1, 16, 256,
              None, 0, None) == -2                                           # rows without index
    assert gr(fake, 0, 2, None, fake, fake, fake, fake, 2, 2, fake, fake, fake, fake, 1, 16, 256,
              None, 0, None) == -1                                           # gsa
    assert gr(fake, 0, 2, fake, None, fake, fake, fake, 2, 2, fake, fake, fake, fake, 1, 16, 256,
              None, 0, None) == -1                                           # x_codes
    assert gr(fake, 0, 8, fake, fake, fake, fake, fake, 2, 8, fake, fake, fake, fake, 1, 16, 8192,
              None, 0, None) == -4                                           # 65536 elements: ws
    assert C.nvfp4_workspace_bytes(C.OP_GROUPED_RUN, 8, 16, 8192, 2) > 0
    assert C.nvfp4_workspace_bytes(C.OP_GROUPED_RUN, 1, 16, 8192, 2) == 0
    mr = L.nvfp4_moe_run
    # (x, x_dtype, T, gsa_x, x_codes, x_scales, row_index, offsets, E, P, w1_codes, w1_scales,
    #  w1_ws2, N1, K1, gran, limit, h, gsa_h, h_codes, h_scales, w2_codes, w2_scales, w2_ws2,
    #  N2, y, y_dtype, ws, ws_bytes, stream)
    f = [fake] * 3
    assert mr(fake, 0, 1, *f, fake, fake, 8, 8, *f, 512, 512, 8, float("nan"), *[fake] * 4, *f,
              40, fake, 1, fake, 1 << 20, None) == -2                        # NaN limit
    assert mr(fake, 0, 1, *f, None, fake, 8, 8, *f, 512, 512, 8, 0.0, *[fake] * 4, *f, 40, fake,
              1, fake, 1 << 20, None) == -1                                  # row_index
    assert mr(fake, 0, 1, *f, fake, fake, 8, 8, *f, 384, 512, 8, 0.0, *[fake] * 4, *f, 40, fake,
              1, fake, 1 << 20, None) == -2                                  # N1 / 2 % 256
    assert mr(fake, 0, 1, *f, fake, fake, 8, 8, *f, 512, 512, 8, 0.0, *[fake] * 4, *f, 40, fake,
              1, fake, 4, None) in (-4, -5)                                   # workspace
    assert C.nvfp4_workspace_bytes(C.OP_MOE_RUN, 1, 4096, 7168, 256) >= 4 * 128 * 256


def test_binding_refuses_undersized_buffers_before_the_library(C):
    """The kernels address raw pointers, so the binding checks every buffer's
    size and element type against what the call touches before any pointer
    reaches the library: an undersized or mistyped buffer raises ValueError
    naming it; well-sized host tensors get as far as the device check."""
    import torch
    M, N, K = 3, 32, 64
    ok = dict(a_codes=torch.zeros(M, K // 2, dtype=torch.uint8),
              a_scales=torch.zeros(M, K // 16, dtype=torch.uint8),
              gsa=torch.zeros(1), w_codes=torch.zeros(N, K // 2, dtype=torch.uint8),
              w_scales=torch.zeros(N, K // 16, dtype=torch.uint8), ws2=torch.zeros(1),
              y=torch.zeros(M, N))
    with pytest.raises(ValueError, match="on the GPU"):
        C.nvfp4_linear(**ok)
    for name, bad, msg in [("a_scales", torch.zeros(M, K // 16 - 1, dtype=torch.uint8), "holds"),
                           ("w_scales", torch.zeros(N - 1, K // 16, dtype=torch.uint8), "holds"),
                           ("gsa", torch.zeros(1, dtype=torch.float64), "must be"),
                           ("y", torch.zeros(M, N - 1), "holds")]:
        with pytest.raises(ValueError, match=msg):
            C.nvfp4_linear(**{**ok, name: bad})
    # grouped: offsets need G + 1 int32 entries, row_index one per output row
    G = 2
    g = dict(a_codes=ok["a_codes"], a_scales=ok["a_scales"], gsa=ok["gsa"],
             row_index=torch.zeros(4, dtype=torch.int32),
             group_offsets=torch.zeros(G + 1, dtype=torch.int32),
             w_codes=torch.zeros(G, N, K // 2, dtype=torch.uint8),
             w_scales=torch.zeros(G, N, K // 16, dtype=torch.uint8), ws2=torch.zeros(G),
             y=torch.zeros(4, N))
    with pytest.raises(ValueError, match="on the GPU"):
        C.nvfp4_grouped_linear(**g)
    for name, bad, msg in [("group_offsets", torch.zeros(G, dtype=torch.int32), "holds"),
                           ("group_offsets", torch.zeros(G + 1, dtype=torch.int64), "must be"),
                           ("row_index", torch.zeros(3, dtype=torch.int32), "holds"),
                           ("ws2", torch.zeros(G - 1), "holds")]:
        with pytest.raises(ValueError, match=msg):
            C.nvfp4_grouped_linear(**{**g, name: bad})
    with pytest.raises(ValueError, match="holds"):
        C.nvfp4_quantize_from_buffer(torch.zeros(M, K, dtype=torch.bfloat16), ok["gsa"],
                                     torch.zeros(M, K // 2 - 1, dtype=torch.uint8),
                                     ok["a_scales"])
