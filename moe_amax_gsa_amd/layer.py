"""NVFP4 linear layers over the C ABI: device buffers, allocated once.

``Nvfp4Linear`` runs the single-projection path (the pages' Nvfp4Linear:
amax -> gsa, quantize from the gsa buffer, block-scaled GEMM; see
dsv4/_archive/layers/linear.py, _run_impl).  ``Nvfp4MoE`` runs the routed
expert pair (L1 gate/up with granularity-8 interleave, SwiGLU, re-quantize,
L2), as README.md's MoE kernel section describes; where the shapes allow,
SwiGLU, the de-interleave and the first amax phase run in the L1 linear's
epilogue (nvfp4_grouped_linear_swiglu), else as separate calls.  Both keep gsa
on the device: no host synchronisation, no per-call host-to-device copy
(deleted PERFORMANCE_AUDIT.md, P0; docs/PERFORMANCE_AUDIT.md, P2).

Torch is used for memory and streams only; all arithmetic runs in
libnvfp4.so.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import nvfp4 as C


def _max_ws(op: int, max_rows: int, N: int, K: int) -> int:
    """Workspace for any row count up to max_rows: within a block of 128 rows
    the split-K partials grow with the rows, so the block ends bound it."""
    ms = sorted({min(128 * j, max_rows) for j in range(1, (max_rows + 127) // 128 + 1)})
    return max(C.nvfp4_workspace_bytes(op, m, N, K) for m in ms)


def _f32_scalar(v, device) -> torch.Tensor:
    if isinstance(v, torch.Tensor):
        return v.to(device=device, dtype=torch.float32).reshape(1).contiguous()
    return torch.tensor([float(v)], dtype=torch.float32, device=device)


class Nvfp4Linear:
    """y = Nvfp4Linear(x): x (M, K) bf16/fp32 -> y (M, N) fp32 (or bf16)."""

    def __init__(self, w_codes: torch.Tensor, w_scales: torch.Tensor, ws2, max_tokens: int,
                 out_dtype=torch.float32, x_dtype=torch.bfloat16):
        assert w_codes.dtype == torch.uint8 and w_scales.dtype == torch.uint8
        self.device = w_codes.device
        self.N, self.K = w_codes.shape[0], w_codes.shape[1] * 2
        self.w_codes = w_codes.contiguous()
        self.w_scales = w_scales.contiguous()
        self.ws2 = _f32_scalar(ws2, self.device)
        self.max_tokens = max_tokens
        dev = self.device
        self.gsa = torch.zeros(1, dtype=torch.float32, device=dev)
        # the largest row count needs the most split-K partials: size for it
        nws = max(C.nvfp4_workspace_bytes(C.OP_LINEAR_RUN, max_tokens, self.N, self.K),
                  C.nvfp4_workspace_bytes(C.OP_RMSNORM_QUANTIZE, max_tokens, 0, self.K))
        nws = max(nws, _max_ws(C.OP_LINEAR, max_tokens, self.N, self.K))
        self.ws = torch.empty(max(nws, 16), dtype=torch.uint8, device=dev)
        self.gsa_rows = torch.zeros(max_tokens, dtype=torch.float32, device=dev)
        self.inv_rms = torch.zeros(max_tokens, dtype=torch.float32, device=dev)
        self.codes = torch.empty(max_tokens, self.K // 2, dtype=torch.uint8, device=dev)
        self.scales = torch.empty(max_tokens, self.K // 16, dtype=torch.uint8, device=dev)
        self.y = torch.empty(max_tokens, self.N, dtype=out_dtype, device=dev)

    @classmethod
    def from_weight(cls, w: torch.Tensor, max_tokens: int, out_dtype=torch.float32,
                    x_dtype=torch.bfloat16, stream=None) -> "Nvfp4Linear":
        """Quantize a bf16/fp32 weight (N, K) at load time (nvfp4_quantize_weight:
        codes, scales and weight_scale_2 on the device) and build the layer."""
        w = w.contiguous()
        N, K = w.shape
        codes = torch.empty(N, K // 2, dtype=torch.uint8, device=w.device)
        scales = torch.empty(N, K // 16, dtype=torch.uint8, device=w.device)
        ws2 = torch.empty(1, dtype=torch.float32, device=w.device)
        ws = torch.empty(max(C.nvfp4_workspace_bytes(C.OP_QUANTIZE_WEIGHT, 0, N, K), 16),
                         dtype=torch.uint8, device=w.device)
        C.nvfp4_quantize_weight(w, ws2, codes, scales, ws, stream)
        return cls(codes, scales, ws2, max_tokens, out_dtype=out_dtype, x_dtype=x_dtype)

    def quantize(self, x: torch.Tensor, stream=None):
        M = x.shape[0]
        C.nvfp4_amax_quantize(x, self.gsa, self.codes[:M], self.scales[:M], self.ws, stream)
        return self.codes[:M], self.scales[:M], self.gsa

    def run_from_quantized(self, codes, scales, gsa, stream=None,
                           gsa_per_row: bool = False) -> torch.Tensor:
        """Step 3 on an already quantized activation; gsa is one scale, or
        with gsa_per_row one per row (M,)."""
        M = codes.shape[0]
        y = self.y[:M]
        if gsa_per_row:
            assert gsa.numel() >= M
            C.nvfp4_linear_rows(codes, scales, gsa, self.w_codes, self.w_scales, self.ws2, y,
                                self.ws, stream)
        else:
            C.nvfp4_linear(codes, scales, gsa, self.w_codes, self.w_scales, self.ws2, y, self.ws,
                           stream)
        return y

    def rmsnorm_forward(self, x: torch.Tensor, norm_weight: torch.Tensor, eps: float = 1e-6,
                        gsa_per_row: bool = False, stream=None) -> torch.Tensor:
        """RMSNorm of x fused into the quantize (nvfp4_rmsnorm_quantize), then
        step 3; with gsa_per_row every row keeps its own global scale."""
        M = x.shape[0]
        assert M <= self.max_tokens and x.shape[1] == self.K
        gsa = self.gsa_rows[:M] if gsa_per_row else self.gsa
        C.nvfp4_rmsnorm_quantize(x, norm_weight, gsa, self.inv_rms[:M], self.codes[:M],
                                 self.scales[:M], eps=eps, per_row=gsa_per_row, ws=self.ws,
                                 stream=stream)
        return self.run_from_quantized(self.codes[:M], self.scales[:M], gsa, stream, gsa_per_row)

    def forward(self, x: torch.Tensor, stream=None) -> torch.Tensor:
        """The three steps as three calls of the C ABI."""
        assert x.shape[0] <= self.max_tokens and x.shape[1] == self.K
        codes, scales, gsa = self.quantize(x, stream)
        return self.run_from_quantized(codes, scales, gsa, stream)

    def run(self, x: torch.Tensor, stream=None) -> torch.Tensor:
        """The same result through nvfp4_linear_run (one kernel for few rows)."""
        M = x.shape[0]
        assert M <= self.max_tokens and x.shape[1] == self.K
        y = self.y[:M]
        C.nvfp4_linear_run(x, self.gsa, self.codes[:M], self.scales[:M], self.w_codes,
                           self.w_scales, self.ws2, y, self.ws, stream)
        return y

    __call__ = forward


class Nvfp4Router:
    """The dense router: (idx, score) = Nvfp4Router(x) for x (M, K) bf16/fp32.

    The gate projection is an NVFP4 linear against the gate weight (N
    experts, quantized at load time when it comes as bf16); the expert
    choice is the top k of sqrt(softplus(logit)) + bias (nvfp4_router_topk).
    idx (M, k) int32, best first; score (M, k) fp32 = sqrt(softplus(logit)).
    """

    def __init__(self, gate: Nvfp4Linear, bias: Optional[torch.Tensor], topk: int):
        self.gate, self.topk = gate, topk
        dev = gate.device
        self.bias = None if bias is None else bias.to(device=dev, dtype=torch.float32).contiguous()
        M, N, K = gate.max_tokens, gate.N, gate.K
        nws = max(16, _max_ws(C.OP_ROUTER_TOPK, M, N, K),
                  *[C.nvfp4_workspace_bytes(C.OP_ROUTER_TOPK, m, N, K) for m in range(1, 17)])
        # zeroed: for up to 16 rows the call's ticket counter (the word after
        # the logits) must start at zero; every call leaves it zero
        self.ws = torch.zeros(nws, dtype=torch.uint8, device=dev)
        self.idx = torch.empty(M, topk, dtype=torch.int32, device=dev)
        self.score = torch.empty(M, topk, dtype=torch.float32, device=dev)

    @classmethod
    def from_weight(cls, w_gate: torch.Tensor, bias: Optional[torch.Tensor], topk: int,
                    max_tokens: int, stream=None) -> "Nvfp4Router":
        return cls(Nvfp4Linear.from_weight(w_gate, max_tokens, stream=stream), bias, topk)

    def route_quantized(self, codes, scales, gsa, stream=None):
        M = codes.shape[0]
        g = self.gate
        C.nvfp4_router_topk(codes, scales, gsa, g.w_codes, g.w_scales, g.ws2, self.bias,
                            self.idx[:M], self.score[:M], self.ws, stream)
        return self.idx[:M], self.score[:M]

    def forward(self, x: torch.Tensor, stream=None):
        assert x.shape[0] <= self.gate.max_tokens and x.shape[1] == self.gate.K
        codes, scales, gsa = self.gate.quantize(x, stream)
        return self.route_quantized(codes, scales, gsa, stream)

    __call__ = forward


class Nvfp4MoE:
    """Routed experts: y2 (P, N2) for the P (token, expert) pairs in expert order.

    x (T, K1) bf16; row_index (P,) int32 = token of each pair; offsets (E+1,)
    int32 = first pair of each expert.  L1 weights (E, N1, K1/2) hold
    gate/up column groups interleaved at ``granularity``; L2 weights
    (E, N2, N1/4) consume the SwiGLU output of width N1/2.  swiglu_limit > 0
    caps the gate at the limit and clamps up to [-limit, limit] before
    silu(gate) * up (0: no clamp).  forward runs the pair through
    nvfp4_moe_run where its conditions hold (run_entry), else as separate
    calls; forward_quantized always takes the separate calls.
    """

    def __init__(self, w1_codes, w1_scales, w1_ws2, w2_codes, w2_scales, w2_ws2, max_pairs: int,
                 max_tokens: int, granularity: int = 8, fused: bool = True,
                 swiglu_limit: float = 0.0, run_entry: bool = True):
        dev = w1_codes.device
        self.device = dev
        self.swiglu_limit = float(swiglu_limit)
        self.E, self.N1, self.K1 = w1_codes.shape[0], w1_codes.shape[1], w1_codes.shape[2] * 2
        self.N2, self.K2 = w2_codes.shape[1], w2_codes.shape[2] * 2
        assert self.K2 * 2 == self.N1, "L2 input width must be half the L1 output width"
        self.granularity = granularity
        self.w1_codes, self.w1_scales = w1_codes.contiguous(), w1_scales.contiguous()
        self.w2_codes, self.w2_scales = w2_codes.contiguous(), w2_scales.contiguous()
        self.w1_ws2 = w1_ws2.to(device=dev, dtype=torch.float32).contiguous()
        self.w2_ws2 = w2_ws2.to(device=dev, dtype=torch.float32).contiguous()
        self.gsa1 = torch.zeros(1, dtype=torch.float32, device=dev)
        self.gsa2 = torch.zeros(1, dtype=torch.float32, device=dev)
        nws = max(C.nvfp4_workspace_bytes(C.OP_AMAX_GSA, max_tokens * self.K1),
                  C.nvfp4_workspace_bytes(C.OP_AMAX_GSA, max_pairs * self.K2), 16)
        self.ws = torch.empty(nws, dtype=torch.uint8, device=dev)
        self.x_codes = torch.empty(max_tokens, self.K1 // 2, dtype=torch.uint8, device=dev)
        self.x_scales = torch.empty(max_tokens, self.K1 // 16, dtype=torch.uint8, device=dev)
        # SwiGLU in the L1 epilogue: the conditions nvfp4_grouped_linear_swiglu
        # states (the activation buffers below are allocated 16-byte aligned)
        self.fused = bool(fused and granularity in (1, 2, 4, 8) and self.K1 % 256 == 0
                          and self.K1 <= 48384 and self.N1 % (2 * granularity) == 0
                          and self.w1_codes.data_ptr() % 16 == 0
                          and self.w1_scales.data_ptr() % 16 == 0)
        self.ws_swiglu = torch.empty(
            max(C.nvfp4_workspace_bytes(C.OP_GROUPED_SWIGLU, max_pairs, self.N1, 0, self.E), 16),
            dtype=torch.uint8, device=dev)
        self.y1 = (None if self.fused else
                   torch.empty(max_pairs, self.N1, dtype=torch.float32, device=dev))
        self.h = torch.empty(max_pairs, self.K2, dtype=torch.float32, device=dev)
        self.h_codes = torch.empty(max_pairs, self.K2 // 2, dtype=torch.uint8, device=dev)
        self.h_scales = torch.empty(max_pairs, self.K2 // 16, dtype=torch.uint8, device=dev)
        self.y2 = torch.empty(max_pairs, self.N2, dtype=torch.float32, device=dev)
        # the whole pair through nvfp4_moe_run (two launches for a decoded
        # token): its conditions on top of the fused path's
        self.run_entry = bool(run_entry and self.fused and self.K2 % 256 == 0
                              and self.w2_codes.data_ptr() % 16 == 0
                              and self.w2_scales.data_ptr() % 16 == 0)
        self.ws_run = torch.empty(
            max(C.nvfp4_workspace_bytes(C.OP_MOE_RUN, max_tokens, self.N1, self.K1, self.E),
                C.nvfp4_workspace_bytes(C.OP_GROUPED_SWIGLU, max_pairs, self.N1, 0, self.E), 16),
            dtype=torch.uint8, device=dev)

    def forward(self, x, row_index, offsets, stream=None) -> torch.Tensor:
        T = x.shape[0]
        xc, xs = self.x_codes[:T], self.x_scales[:T]
        if self.run_entry and x.data_ptr() % 16 == 0:
            P = row_index.shape[0]
            y2 = self.y2[:P]
            C.nvfp4_moe_run(x, self.gsa1, xc, xs, row_index, offsets, self.w1_codes,
                            self.w1_scales, self.w1_ws2, self.granularity, self.h[:P], self.gsa2,
                            self.h_codes[:P], self.h_scales[:P], self.w2_codes, self.w2_scales,
                            self.w2_ws2, y2, self.ws_run, limit=self.swiglu_limit, stream=stream)
            return y2
        C.nvfp4_amax_quantize(x, self.gsa1, xc, xs, self.ws, stream)
        return self.forward_quantized(xc, xs, self.gsa1, row_index, offsets, stream)

    def forward_quantized(self, xc, xs, gsa, row_index, offsets, stream=None) -> torch.Tensor:
        """The expert pair on an already quantized activation (codes (T, K1/2),
        scales (T, K1/16), one device gsa) -- e.g. nvfp4_rmsnorm_quantize's
        output, which the router consumes too."""
        P = row_index.shape[0]
        h = self.h[:P]
        hc, hs = self.h_codes[:P], self.h_scales[:P]
        if self.fused:  # SwiGLU, amax and h's quantize with the gate/up projection
            C.nvfp4_grouped_linear_swiglu(xc, xs, gsa, row_index, offsets, self.w1_codes,
                                          self.w1_scales, self.w1_ws2, h, self.gsa2,
                                          self.granularity, self.ws_swiglu, stream,
                                          h_codes=hc, h_scales=hs, limit=self.swiglu_limit)
        else:
            y1 = self.y1[:P]
            # rows that belong to no group (or carry an out-of-range token) are
            # not written by the grouped linear: zero them first, so that they
            # give h = 0 and stay out of h's amax, as in the fused path
            y1.zero_()
            C.nvfp4_grouped_linear(xc, xs, gsa, row_index, offsets, self.w1_codes,
                                   self.w1_scales, self.w1_ws2, y1, stream)
            C.nvfp4_swiglu_deinterleave(y1, h, self.granularity, stream, limit=self.swiglu_limit)
            C.nvfp4_amax_gsa(h, self.gsa2, self.ws, stream)
            C.nvfp4_quantize_from_buffer(h, self.gsa2, hc, hs, stream)
        y2 = self.y2[:P]
        C.nvfp4_grouped_linear(hc, hs, self.gsa2, None, offsets, self.w2_codes, self.w2_scales,
                               self.w2_ws2, y2, stream)
        return y2

    __call__ = forward


class Nvfp4GroupedLinear:
    """The dense grouped linear (the pages' wo_a): z = Nvfp4GroupedLinear(o)
    for o (T, G * K) bf16/fp32 -> z (G, T, N), z[g, t] = token t's slice
    o[t, g*K:(g+1)*K] through group g's weight, with one gsa over all of o
    (dsv4/_archive/layers/grouped_linear.py, _run_impl).  Weights are stacked
    (G, N, K/2) and (G, N, K/16) with ws2 (G,).  One launch
    (nvfp4_grouped_linear_run) while o has at most 16384 elements, two
    beyond."""

    def __init__(self, w_codes: torch.Tensor, w_scales: torch.Tensor, ws2, max_tokens: int,
                 out_dtype=torch.float32):
        dev = w_codes.device
        self.device = dev
        self.G, self.N, self.K = w_codes.shape[0], w_codes.shape[1], w_codes.shape[2] * 2
        self.w_codes, self.w_scales = w_codes.contiguous(), w_scales.contiguous()
        self.ws2 = ws2.to(device=dev, dtype=torch.float32).contiguous()
        self.max_tokens = max_tokens
        rows = max_tokens * self.G
        self.gsa = torch.zeros(1, dtype=torch.float32, device=dev)
        self.codes = torch.empty(rows, self.K // 2, dtype=torch.uint8, device=dev)
        self.scales = torch.empty(rows, self.K // 16, dtype=torch.uint8, device=dev)
        self.y = torch.empty(rows, self.N, dtype=out_dtype, device=dev)
        self.ws = torch.empty(
            max(C.nvfp4_workspace_bytes(C.OP_GROUPED_RUN, rows, self.N, self.K, self.G), 16),
            dtype=torch.uint8, device=dev)
        self._routes = {}

    def routes(self, T: int):
        """(row_index, offsets) for T tokens: group g's rows g*T .. g*T+T-1
        read slices t*G + g (built once per T, on the device)."""
        if T not in self._routes:
            G = self.G
            ri = (torch.arange(T, device=self.device)[None, :] * G +
                  torch.arange(G, device=self.device)[:, None]).reshape(-1).to(torch.int32)
            off = (torch.arange(G + 1, device=self.device) * T).to(torch.int32)
            self._routes[T] = (ri.contiguous(), off.contiguous())
        return self._routes[T]

    def forward(self, o: torch.Tensor, stream=None) -> torch.Tensor:
        T = o.shape[0]
        assert T <= self.max_tokens and o.shape[1] == self.G * self.K
        x = o.reshape(T * self.G, self.K)
        ri, off = self.routes(T)
        rows = T * self.G
        y = self.y[:rows]
        C.nvfp4_grouped_linear_run(x, self.gsa, self.codes[:rows], self.scales[:rows], ri, off,
                                   self.w_codes, self.w_scales, self.ws2, y, self.ws, stream)
        return y.view(self.G, T, self.N)

    __call__ = forward
