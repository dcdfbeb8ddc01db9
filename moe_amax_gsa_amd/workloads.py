"""Seeded synthetic inputs for the NVFP4 linear layer.

This module draws random numbers and nothing else: it holds none of the
layer's arithmetic (no amax, no scale rule, no quantize, no GEMM).  Both the
HIP path and the CPU oracle consume what it returns.  Rounding of draws to
bf16 and to E4M3 is done by torch's own dtype conversions.

Recipe (numpy PCG64):
  * activations: ``default_rng(seed)``; X drawn in float64, then the
    workload's modifications (outliers, zero blocks, heavy tails), then the
    MoE routing, in that order; X is cast to float32 and rounded to bf16
    (round to nearest even) by torch.
  * weights: tensor ``layer`` of expert ``e`` uses ``default_rng([seed,
    1 + layer, e])``: packed E2M1 codes are uniform random bytes (two
    independent uniform nibbles), block scales are uniform float64 draws in
    [lo, hi] cast to float32 and rounded to E4M3 by torch, weight_scale_2 is
    a float32 constant or a uniform draw.
Weight layout: codes (N, K/2) uint8, scales (N, K/16) uint8 (E4M3 bits),
row n = output feature n, packed along K.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch


# ------------------------------------------------------------------ shapes
# The five workloads: a tiny case, a decode projection, a prefill
# projection, a routed-expert MoE pair of projections and a large-magnitude
# prefill stress case.
WORKLOADS = {
    "tiny_m1_k256_n256": dict(kind="linear", M=1, K=256, N=256, seed=0, x="normal",
                              sf=(0.5, 2.0), ws2=0.01),
    "decode_m1_k7168_n1536": dict(kind="linear", M=1, K=7168, N=1536, seed=1,
                                  x="outliers", sf=(0.25, 4.0), ws2=0.005),
    "prefill_m512_k7168_n4096": dict(kind="linear", M=512, K=7168, N=4096, seed=2,
                                     x="zero_blocks", sf=(0.25, 4.0), ws2=0.005),
    "moe_t64_e256_top8": dict(kind="moe", tokens=64, experts=256, topk=8, K1=7168,
                              N1=4096, K2=2048, N2=7168, granularity=8, seed=3,
                              sf=(0.25, 4.0), ws2=(0.002, 0.01)),
    # the MoE pair at prefill: 512 tokens, top 8 of 32 experts (128 pairs per
    # expert on average)
    "moe_t512_e32_top8": dict(kind="moe", tokens=512, experts=32, topk=8, K1=7168, N1=4096,
                              K2=2048, N2=7168, granularity=8, seed=14, sf=(0.25, 4.0),
                              ws2=(0.002, 0.01)),
    "stress_m2048_k7168_n7168": dict(kind="linear", M=2048, K=7168, N=7168, seed=4,
                                     x="student_t", sf=(0.125, 8.0), ws2=0.003),
    # the dense router: hidden 7168, 384 routed experts, 6 chosen per token
    "router_m1_k7168_e384_top6": dict(kind="router", M=1, K=7168, N=384, topk=6, seed=5),
    "router_m64_k7168_e384_top6": dict(kind="router", M=64, K=7168, N=384, topk=6, seed=6),
    # the dense grouped linear (wo_a): one decoded token's 8 slices of 8192
    # (heads_per_group * head_dim) against 8 weights of 1536 (o_lora_rank) rows
    "grouped_wo_a_t1_g8_k8192_n1536": dict(kind="grouped", T=1, G=8, K=8192, N=1536, seed=10,
                                           sf=(0.25, 4.0), ws2=(0.002, 0.01)),
    # a decode projection with the lm_head's shape (vocab 129280, hidden 7168)
    "lm_head_m1_k7168_n129280": dict(kind="linear", M=1, K=7168, N=129280, seed=11,
                                     x="normal", sf=(0.25, 4.0), ws2=0.005),
    # a prefill batch through the routed experts' first projection: 512
    # tokens, top 8 of 32 experts (128 rows per expert on average), routed
    # uniformly, or with expert e drawn with weight (e + 1)^-1.2 (a few
    # experts take most tokens)
    "moe_l1_t512_e32_top8_k7168_n4096": dict(kind="routed", tokens=512, experts=32, topk=8,
                                             K=7168, N=4096, seed=12, routing="uniform"),
    "moe_l1_t512_e32_top8_k7168_n4096_zipf": dict(kind="routed", tokens=512, experts=32,
                                                  topk=8, K=7168, N=4096, seed=13,
                                                  routing="zipf"),
    # RMSNorm -> quantize of the hidden state, one token and a prefill batch
    "rmsnorm_m1_k7168": dict(kind="rmsnorm", M=1, K=7168, seed=7),
    "rmsnorm_m512_k7168": dict(kind="rmsnorm", M=512, K=7168, seed=8),
}


def to_bf16_bits(x64: np.ndarray) -> np.ndarray:
    """float64 -> float32 -> bf16 (RNE, torch) -> raw uint16 bits."""
    t = torch.from_numpy(np.ascontiguousarray(x64, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def to_e4m3_bits(v64: np.ndarray) -> np.ndarray:
    """Positive float64 draws -> float32 -> E4M3 (torch RNE) -> uint8 bits."""
    t = torch.from_numpy(np.ascontiguousarray(v64, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().copy()


# ------------------------------------------------------------------ pieces
def draw_activation(rng: np.random.Generator, M: int, K: int, kind: str) -> np.ndarray:
    """float64 activations of the given kind (before bf16 rounding)."""
    if kind == "student_t":
        x = rng.standard_t(2.0, size=(M, K))
        x *= 1000.0 / np.max(np.abs(x))
        return x
    x = rng.standard_normal((M, K))
    if kind == "normal":
        pass
    elif kind == "outliers":
        # round(0.1%) of all entries, without replacement, multiplied by 100
        n_out = int(round(0.001 * M * K))
        idx = rng.choice(M * K, n_out, replace=False)
        x.reshape(-1)[idx] *= 100.0
    elif kind == "zero_blocks":
        # round(1%) of the 16-element blocks, without replacement, set to +0
        nblk = M * (K // 16)
        n_zero = int(round(0.01 * nblk))
        idx = rng.choice(nblk, n_zero, replace=False)
        x.reshape(-1, 16)[idx] = 0.0
    # the edges of the formats' ranges
    elif kind == "tiny":
        # bf16 subnormals (|x| < 2^-126): the amax floor sets gsa
        x *= 1e-39
    elif kind == "huge":
        x *= 1e30
    elif kind == "block_range":
        # each 16-element block its own magnitude, log-uniform over the
        # eight decades below 1 (zero, subnormal and normal E4M3 scales)
        mag = 10.0 ** rng.uniform(-8.0, 0.0, size=(M, K // 16))
        x *= np.repeat(mag, 16, axis=1)
    elif kind == "elem_range":
        # each element its own magnitude, log-uniform over 1e-20 .. 1e20
        x *= 10.0 ** rng.uniform(-20.0, 20.0, size=(M, K))
    else:
        raise ValueError(kind)
    return x


def draw_weight(seed: int, layer: int, expert: int, N: int, K: int, sf_lo: float,
                sf_hi: float, ws2=None):
    """Packed codes (N, K/2), E4M3 scale bits (N, K/16) and a float32 ws2."""
    rng = np.random.default_rng([seed, 1 + layer, expert])
    codes = np.frombuffer(rng.bytes(N * (K // 2)), dtype=np.uint8).reshape(N, K // 2).copy()
    scales = to_e4m3_bits(rng.uniform(sf_lo, sf_hi, size=(N, K // 16)))
    if isinstance(ws2, tuple):
        w2 = np.float32(rng.uniform(ws2[0], ws2[1]))
    else:
        w2 = np.float32(ws2)
    return codes, scales, w2


@dataclass
class LinearInputs:
    name: str
    x: np.ndarray          # (M, K) bf16 bits, uint16
    w_codes: np.ndarray    # (N, K/2) uint8
    w_scales: np.ndarray   # (N, K/16) uint8
    ws2: np.float32
    M: int
    K: int
    N: int


def make_linear(M: int, K: int, N: int, seed: int, x: str = "normal",
                sf=(0.25, 4.0), ws2: float = 0.005, name: str = "custom") -> LinearInputs:
    rng = np.random.default_rng(seed)
    xb = to_bf16_bits(draw_activation(rng, M, K, x))
    wc, wsc, w2 = draw_weight(seed, 0, 0, N, K, sf[0], sf[1], ws2)
    return LinearInputs(name, xb, wc, wsc, w2, M, K, N)


@dataclass
class MoEInputs:
    name: str
    x: np.ndarray              # (T, K1) bf16 bits
    pair_expert: np.ndarray    # (P,) int32, sorted by (expert, token)
    pair_token: np.ndarray     # (P,) int32 = row_index for L1
    offsets: np.ndarray        # (E+1,) int32
    T: int
    E: int
    topk: int
    K1: int
    N1: int
    K2: int
    N2: int
    granularity: int
    seed: int
    sf: tuple
    ws2_range: tuple
    _cache: dict = field(default_factory=dict, repr=False)

    @property
    def active_experts(self) -> np.ndarray:
        return np.nonzero(np.diff(self.offsets) > 0)[0]

    def weight(self, layer: int, e: int):
        """(codes, scales, ws2) of expert e; layer 0 = L1 (gate/up), 1 = L2."""
        key = (layer, e)
        if key not in self._cache:
            N, K = (self.N1, self.K1) if layer == 0 else (self.N2, self.K2)
            self._cache[key] = draw_weight(self.seed, layer, e, N, K, self.sf[0],
                                           self.sf[1], self.ws2_range)
        return self._cache[key]

    def drop_cache(self):
        self._cache.clear()


def make_moe(tokens=64, experts=256, topk=8, K1=7168, N1=4096, K2=2048, N2=7168,
             granularity=8, seed=3, sf=(0.25, 4.0), ws2=(0.002, 0.01),
             name="custom_moe", routing: str = "uniform") -> MoEInputs:
    """routing "uniform": each token's topk distinct experts uniformly at
    random; "zipf": drawn without replacement with weights (e + 1)^-1.2."""
    rng = np.random.default_rng(seed)
    xb = to_bf16_bits(draw_activation(rng, tokens, K1, "normal"))
    p = None
    if routing == "zipf":
        p = (np.arange(experts) + 1.0) ** -1.2
        p /= p.sum()
    elif routing != "uniform":
        raise ValueError(routing)
    tok, exp_ = [], []
    for t in range(tokens):
        chosen = rng.choice(experts, topk, replace=False, p=p)
        for e in chosen:
            tok.append(t)
            exp_.append(int(e))
    tok = np.asarray(tok, np.int64)
    exp_ = np.asarray(exp_, np.int64)
    order = np.lexsort((tok, exp_))       # sort by expert, then token
    pair_expert = exp_[order].astype(np.int32)
    pair_token = tok[order].astype(np.int32)
    counts = np.bincount(pair_expert, minlength=experts)
    offsets = np.zeros(experts + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    return MoEInputs(name, xb, pair_expert, pair_token, offsets, tokens, experts, topk,
                     K1, N1, K2, N2, granularity, seed, tuple(sf), tuple(ws2))


@dataclass
class GroupedInputs:
    """The dense grouped linear: x (T, G*K) bf16 bits, token t's slice g is
    row t*G + g of x viewed as (T*G, K); group g's output rows are
    g*T .. g*T + T - 1 (row_index maps them to their slices)."""
    name: str
    x: np.ndarray            # (T * G, K) bf16 bits
    row_index: np.ndarray    # (G * T,) int32
    offsets: np.ndarray      # (G + 1,) int32
    w_codes: np.ndarray      # (G, N, K/2) uint8
    w_scales: np.ndarray     # (G, N, K/16) uint8
    ws2: np.ndarray          # (G,) float32
    T: int
    G: int
    K: int
    N: int


def make_grouped(T: int, G: int, K: int, N: int, seed: int, sf=(0.25, 4.0),
                 ws2=(0.002, 0.01), x: str = "normal", name: str = "custom") -> GroupedInputs:
    rng = np.random.default_rng(seed)
    xb = to_bf16_bits(draw_activation(rng, T, G * K, x)).reshape(T * G, K)
    row_index = (np.arange(T)[None, :] * G + np.arange(G)[:, None]).reshape(-1).astype(np.int32)
    offsets = (np.arange(G + 1) * T).astype(np.int32)
    ws = [draw_weight(seed, 0, g, N, K, sf[0], sf[1], ws2) for g in range(G)]
    return GroupedInputs(name, np.ascontiguousarray(xb), row_index, offsets,
                         np.stack([w[0] for w in ws]), np.stack([w[1] for w in ws]),
                         np.array([w[2] for w in ws], np.float32), T, G, K, N)


@dataclass
class RouterInputs:
    name: str
    x: np.ndarray        # (M, K) bf16 bits
    w: np.ndarray        # (N, K) bf16 bits: the gate weight, one row per expert
    bias: np.ndarray     # (N,) float32 per-expert bias
    M: int
    K: int
    N: int
    topk: int


def make_router(M: int, K: int, N: int, topk: int, seed: int,
                name: str = "custom") -> RouterInputs:
    """x ~ N(0, 1); gate weight ~ N(0, (2 / sqrt(K))^2), so the logits spread
    about N(0, 4); bias ~ N(0, 0.05^2) in float32.  Draw order: x, w, bias."""
    rng = np.random.default_rng(seed)
    x = to_bf16_bits(rng.standard_normal((M, K)))
    w = to_bf16_bits(rng.standard_normal((N, K)) * (2.0 / np.sqrt(K)))
    bias = (rng.standard_normal(N) * 0.05).astype(np.float32)
    return RouterInputs(name, x, w, bias, M, K, N, topk)


@dataclass
class RMSNormInputs:
    name: str
    x: np.ndarray        # (M, K) bf16 bits
    w: np.ndarray        # (K,) bf16 bits: the norm weight
    M: int
    K: int


def make_rmsnorm(M: int, K: int, seed: int, zero_row: bool = False,
                 name: str = "custom") -> RMSNormInputs:
    """Rows of N(0, 1) times a per-row magnitude exp(U[-3, 3]) (hidden states
    of very different sizes), 0.2% of the entries times 40 (outliers), and
    optionally row M // 2 all zero; norm weight 1 + 0.25 N(0, 1).  Draw
    order: x, the row magnitudes, the outlier mask, w."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)) * np.exp(rng.uniform(-3, 3, (M, 1)))
    x[rng.random((M, K)) < 0.002] *= 40.0
    if zero_row:
        x[M // 2] = 0.0
    w = 1.0 + 0.25 * rng.standard_normal(K)
    return RMSNormInputs(name, to_bf16_bits(x), to_bf16_bits(w), M, K)


def make(name: str):
    """Build the named workload at its full size."""
    c = dict(WORKLOADS[name])
    kind = c.pop("kind")
    if kind == "linear":
        return make_linear(c["M"], c["K"], c["N"], c["seed"], c["x"], c["sf"], c["ws2"],
                           name=name)
    if kind == "router":
        return make_router(c["M"], c["K"], c["N"], c["topk"], c["seed"], name=name)
    if kind == "rmsnorm":
        return make_rmsnorm(c["M"], c["K"], c["seed"], name=name)
    if kind == "routed":  # the first projection only: K2, N2 are never drawn
        return make_moe(c["tokens"], c["experts"], c["topk"], c["K"], c["N"], 256, 16, 8,
                        c["seed"], name=name, routing=c["routing"])
    if kind == "grouped":
        return make_grouped(c["T"], c["G"], c["K"], c["N"], c["seed"], c["sf"], c["ws2"],
                            name=name)
    return make_moe(c["tokens"], c["experts"], c["topk"], c["K1"], c["N1"], c["K2"],
                    c["N2"], c["granularity"], c["seed"], c["sf"], c["ws2"], name=name)


# ------------------------------------------------------------------ upload
def bf16_to_torch(bits: np.ndarray, device) -> torch.Tensor:
    """uint16 bf16 bits -> torch bfloat16 tensor on device (bit copy)."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to(device)


def moe_weights_to(moe: MoEInputs, device, experts=None, keep_host: bool = False,
                   first_only: bool = False):
    """Stacked expert weights on the device: (w1_codes, w1_scales, w1_ws2,
    w2_codes, w2_scales, w2_ws2).  Experts outside ``experts`` (default:
    the experts that receive at least one token) are left zero -- the
    grouped kernels never read an empty group's weights.  first_only: the
    second projection's tensors are empty and never drawn."""
    E = moe.E
    if experts is None:
        experts = moe.active_experts
    N2, K2 = (0, 16) if first_only else (moe.N2, moe.K2)
    w1c = torch.zeros(E, moe.N1, moe.K1 // 2, dtype=torch.uint8, device=device)
    w1s = torch.zeros(E, moe.N1, moe.K1 // 16, dtype=torch.uint8, device=device)
    w2c = torch.zeros(E, N2, K2 // 2, dtype=torch.uint8, device=device)
    w2s = torch.zeros(E, N2, K2 // 16, dtype=torch.uint8, device=device)
    w1_ws2 = np.zeros(E, np.float32)
    w2_ws2 = np.zeros(E, np.float32)
    for e in experts:
        c, s, w = moe.weight(0, int(e))
        w1c[e].copy_(torch.from_numpy(c))
        w1s[e].copy_(torch.from_numpy(s))
        w1_ws2[e] = w
        if first_only:
            if not keep_host:
                moe.drop_cache()
            continue
        c, s, w = moe.weight(1, int(e))
        w2c[e].copy_(torch.from_numpy(c))
        w2s[e].copy_(torch.from_numpy(s))
        w2_ws2[e] = w
        if not keep_host:
            moe.drop_cache()
    return (w1c, w1s, torch.from_numpy(w1_ws2).to(device), w2c, w2s,
            torch.from_numpy(w2_ws2).to(device))
