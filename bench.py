"""Benchmark of the NVFP4 linear layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--only NAME] [--no-cpu]

A step is one pass of the layer's hot path over one batch of synthetic,
seeded input already resident in HBM: amax -> gsa, quantize from the gsa
buffer and the block-scaled linear (for the MoE workload also SwiGLU,
re-quantize and the second grouped linear).  Timing: W untimed eager steps,
then two HIP graphs of K steps each (launch cost off the critical path, as
a decode loop runs): the first covers steps 0..K-1 and is replayed once
untimed; then 512 MiB are copied to another buffer (1 GiB of other
traffic, so neither the 256 MB Infinity Cache nor any L2 holds a step's
weights), and the second graph, steps K..2K-1, is replayed once bracketed
by synchronisation and events: ms_per_step = that replay / K.  Step i reads
weight copy i mod C, where the C copies span at least 512 MB: within a
replay a copy is read again only after 512 MB of others, at any K.

Headline: the decode projection (M=1, K=7168, N=1536), step = one
nvfp4_linear_run call (amax, gsa, quantize and the weight-streaming linear
in one kernel for a one-row activation).  value = algorithmic bytes of the
step (weight codes + weight scales + bf16 activation + activation codes and
scales + fp32 output) / step time.  The same step as three ABI calls and the
other workloads are reported under "workloads".

roofline: the dominant kernel's average duration, from events around a
graph of K back-to-back launches of that kernel alone (at M=1 the whole step
is that one kernel).  Beside it, two measured floors of the same launch
shape: floor_us, an empty kernel with the same grid in a graph of K
launches, and stream_us, a read-only pass of the same weight bytes with the
same grid (libnvfp4_probe.so).  traffic: HBM bytes per launch from the
rocprofv3 FETCH_SIZE and WRITE_SIZE summary kept under profiles/, scaled by
what the same counters read for a copy of known size; reported only while
the kernel sources still hash to the value recorded there.

cpu_baseline: the oracle's step on every host core and on one, each for a
bounded time, with the CPU model.

    python bench.py --pmc-probe     (the program those counter runs profile;
                                     --pmc-probe-prefill, --pmc-probe-stress for
                                     the GEMM workloads)

Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2516.6  # dense f16/bf16 matrix cores: 256 CU * 4096 flop/clk * 2.4 GHz
ROTATE_BYTES = 512 << 20
HEAD = "decode_m1_k7168_n1536"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--only", default=None, help="extra workload to run (default: all)")
    p.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    p.add_argument("--no-extra", action="store_true", help="headline workload only")
    p.add_argument("--pmc-probe", action="store_true",
                   help="run only a 256 MiB copy and the headline kernel (for counter runs)")
    p.add_argument("--pmc-probe-prefill", action="store_true",
                   help="run only a 256 MiB copy, then the prefill quantize and linear "
                        "(for counter runs)")
    p.add_argument("--pmc-probe-stress", action="store_true",
                   help="run only a 256 MiB copy, then the stress quantize and linear, then "
                        "torch's bf16 matmul of the same shape (for counter runs)")
    return p.parse_args()


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


# ------------------------------------------------------------------ timing
FLUSH_BYTES = 512 << 20
_flush_bufs = []


def flush_caches() -> None:
    """Copy 512 MiB to another buffer on the current stream: 1 GiB of other
    traffic, after which the 256 MB Infinity Cache and the L2s hold none of
    a benchmark's inputs."""
    if not _flush_bufs:
        src = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda").fill_(3)
        _flush_bufs.extend([src, torch.empty_like(src)])
    _flush_bufs[1].copy_(_flush_bufs[0])


def graph_ms_per_step(step, steps: int, warmup: int) -> float:
    """step(i) enqueues step i.  W eager warmup steps; a graph of steps
    0..K-1 replayed once untimed; the caches flushed; a graph of steps
    K..2K-1 replayed once between events (ms per step)."""
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graphs = []
    for base in (0, steps):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            for i in range(steps):
                step(base + i)
        graphs.append(g)
    graphs[0].replay()
    torch.cuda.synchronize()
    flush_caches()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    graphs[1].replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def kernel_us(launch, iters: int, pre=None) -> float:
    """Average duration of launch(i) alone: `iters` launches captured back to
    back in a graph (after pre(0), which prepares the inputs), timed as
    graph_ms_per_step times a step."""
    if pre is not None:
        pre(0)
    return 1e3 * graph_ms_per_step(launch, iters, 2)


KERNEL_SOURCES = ["device.hpp", "launch.hpp", "router.hpp", "api.hip", "gemv.hip", "gemm.hip",
                  "quant.hip", "router.hip", "noalloc.hip"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "moe_amax_gsa_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(path: str):
    """Bytes per launch recorded by the counter runs, or None when the file
    is missing or the kernel sources changed since the counters were taken."""
    try:
        text = open(path).read()
    except OSError:
        return None
    m = re.search(r"```json\n(.*?)\n```", text, re.S)
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("source_hash") != kernel_source_hash():
        return None
    return rec.get("traffic_bytes_per_launch")


# ------------------------------------------------------------------ linear
class LinearBench:
    """One single-projection workload with rotated weight copies."""

    def __init__(self, C, inp, dev):
        from moe_amax_gsa_amd import workloads as W
        self.C, self.inp = C, inp
        M, K, N = inp.M, inp.K, inp.N
        wbytes = inp.w_codes.nbytes + inp.w_scales.nbytes
        self.ncopies = max(1, min(512, -(-ROTATE_BYTES // wbytes)))
        wc = torch.from_numpy(inp.w_codes).to(dev)
        wsf = torch.from_numpy(inp.w_scales).to(dev)
        self.w = [(wc, wsf)] + [(wc.clone(), wsf.clone()) for _ in range(self.ncopies - 1)]
        self.x = W.bf16_to_torch(inp.x, dev)
        self.ws2 = torch.tensor([inp.ws2], dtype=torch.float32, device=dev)
        self.gsa = torch.zeros(1, dtype=torch.float32, device=dev)
        nws = max(16, C.nvfp4_workspace_bytes(C.OP_LINEAR_RUN, M, N, K))
        self.ws = torch.empty(nws, dtype=torch.uint8, device=dev)
        self.codes = torch.empty(M, K // 2, dtype=torch.uint8, device=dev)
        self.scales = torch.empty(M, K // 16, dtype=torch.uint8, device=dev)
        self.y = torch.empty(M, N, dtype=torch.float32, device=dev)
        self.flops = 2.0 * M * N * K
        a_bytes = M * K // 2 + M * K // 16
        # nvfp4_linear: weights + quantized activation + fp32 output
        self.linear_bytes = wbytes + a_bytes + M * N * 4
        # a whole step: weights + bf16 activation + quantized activation written + output
        self.step_bytes = wbytes + M * K * 2 + a_bytes + M * N * 4
        self.quant_bytes = M * K * 2 + a_bytes

    def quantize(self, i=0):
        C = self.C
        C.nvfp4_amax_gsa(self.x, self.gsa, self.ws)
        C.nvfp4_quantize_from_buffer(self.x, self.gsa, self.codes, self.scales)

    def linear(self, i):
        wc, wsf = self.w[i % self.ncopies]
        self.C.nvfp4_linear(self.codes, self.scales, self.gsa, wc, wsf, self.ws2, self.y, self.ws)

    def step3(self, i):  # the three ABI calls
        self.quantize()
        self.linear(i)

    def run(self, i):  # nvfp4_linear_run
        wc, wsf = self.w[i % self.ncopies]
        self.C.nvfp4_linear_run(self.x, self.gsa, self.codes, self.scales, wc, wsf, self.ws2,
                                self.y, self.ws)


def bench_linear(C, name, dev, steps, warmup, kiters, settle=False):
    """settle: one untimed pass of the step graph before the timed ones (on
    the GEMM shapes the first timed pass of a workload ran 5-15% slower than
    the same pass repeated)."""
    from moe_amax_gsa_amd import workloads as W
    inp = W.make(name)
    b = LinearBench(C, inp, dev)
    r = {"rotated_weight_copies": b.ncopies}
    if settle:
        graph_ms_per_step(b.run, steps, warmup)
    r["step_us"] = 1e3 * graph_ms_per_step(b.run, steps, warmup)
    r["step3_us"] = 1e3 * graph_ms_per_step(b.step3, steps, warmup)
    r["linear_us"] = kernel_us(b.linear, kiters, pre=b.quantize)
    if inp.M > 16:
        # the same linear with bf16 output (the pages' layer returns bf16;
        # parity is checked on the fp32 output, whose RNE rounding the bf16
        # output equals bit for bit)
        y16 = torch.empty(inp.M, inp.N, dtype=torch.bfloat16, device=dev)

        def lin16(i):
            wc, wsf = b.w[i % b.ncopies]
            C.nvfp4_linear(b.codes, b.scales, b.gsa, wc, wsf, b.ws2, y16, b.ws)

        r["linear_bf16_out_us"] = kernel_us(lin16, kiters)
        del y16
    r["quant_us"] = kernel_us(lambda i: b.quantize(), kiters)
    r["step_GBps"] = b.step_bytes / (r["step_us"] * 1e-6) / 1e9
    r["step_TFLOPs"] = b.flops / (r["step_us"] * 1e-6) / 1e12
    r["linear_GBps"] = b.linear_bytes / (r["linear_us"] * 1e-6) / 1e9
    r["linear_TFLOPs"] = b.flops / (r["linear_us"] * 1e-6) / 1e12
    r["linear_frac_hbm"] = r["linear_GBps"] / HBM_PEAK_GBS
    r["linear_frac_mfma"] = r["linear_TFLOPs"] / MFMA_F16_PEAK_TFLOPS
    r["step_bytes"] = b.step_bytes
    r["linear_bytes"] = b.linear_bytes
    r["flops"] = b.flops
    return inp, b, r


def bench_moe(C, dev, steps, warmup):
    from moe_amax_gsa_amd import workloads as W
    from moe_amax_gsa_amd.layer import Nvfp4MoE
    moe = W.make("moe_t64_e256_top8")
    P = int(moe.offsets[-1])
    w = W.moe_weights_to(moe, dev)
    layer = Nvfp4MoE(*w, max_pairs=P, max_tokens=moe.T, granularity=moe.granularity)
    x = W.bf16_to_torch(moe.x, dev)
    ri = torch.from_numpy(moe.pair_token).to(dev)
    off = torch.from_numpy(moe.offsets).to(dev)
    nact = len(moe.active_experts)
    per_expert = (moe.N1 * moe.K1 // 2 + moe.N1 * moe.K1 // 16 +
                  moe.N2 * moe.K2 // 2 + moe.N2 * moe.K2 // 16)
    wbytes = nact * per_expert
    flops = 2.0 * P * (moe.N1 * moe.K1 + moe.N2 * moe.K2)
    us = 1e3 * graph_ms_per_step(lambda i: layer(x, ri, off), steps, warmup)
    res = {"step_us": us, "active_experts": nact, "weight_bytes": wbytes,
           "step_GBps": wbytes / (us * 1e-6) / 1e9,
           "step_frac_hbm": wbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
           "step_TFLOPs": flops / (us * 1e-6) / 1e12}
    # One decoded token routed to 8 experts.  Step i decodes token i mod 64
    # of the same workload with its own 8 experts, so consecutive steps read
    # different expert weights (one token's 198 MB would fit the Infinity
    # Cache).  nvfp4_moe_run: two launches; beside it the separate calls.
    ex = moe.pair_expert
    singles = []
    for t in range(moe.T):
        es = np.sort(ex[moe.pair_token == t])
        off1 = np.zeros(moe.E + 1, np.int32)
        off1[es + 1] = 1
        off1 = np.cumsum(off1).astype(np.int32)
        singles.append((W.bf16_to_torch(moe.x[t:t + 1], dev),
                        torch.zeros(len(es), dtype=torch.int32, device=dev),
                        torch.from_numpy(off1).to(dev)))
    b1 = moe.topk * per_expert
    layer1 = Nvfp4MoE(*w, max_pairs=moe.topk, max_tokens=1, granularity=moe.granularity)
    layer1s = Nvfp4MoE(*w, max_pairs=moe.topk, max_tokens=1, granularity=moe.granularity,
                       run_entry=False)
    assert layer1.run_entry
    us1 = 1e3 * graph_ms_per_step(lambda i: layer1(*singles[i % moe.T]), steps, warmup)
    us1s = 1e3 * graph_ms_per_step(lambda i: layer1s(*singles[i % moe.T]), steps, warmup)
    res.update({"one_token_step_us": us1, "one_token_weight_bytes": b1,
                "one_token_GBps": b1 / (us1 * 1e-6) / 1e9,
                "one_token_frac_hbm": b1 / (us1 * 1e-6) / 1e9 / HBM_PEAK_GBS,
                "one_token_launches": 2,
                "one_token_separate_calls_us": us1s,
                "one_token_rotation": "step i decodes token i mod 64 with its own 8 experts"})
    return res


def bench_moe_prefill(C, dev, steps, warmup, name="moe_t512_e32_top8"):
    """The MoE pair over a prefill batch (512 tokens, top 8 of 32 experts)
    through nvfp4_moe_run: x's amax and quantize, the gate/up projection
    with SwiGLU and h's amax in its epilogue, h's finalize and quantize, the
    second projection -- both projections on the tiled kernel.  All 32
    experts' weights (about 790 MB) are read every step."""
    from moe_amax_gsa_amd import workloads as W
    from moe_amax_gsa_amd.layer import Nvfp4MoE
    moe = W.make(name)
    P = int(moe.offsets[-1])
    w = W.moe_weights_to(moe, dev)
    layer = Nvfp4MoE(*w, max_pairs=P, max_tokens=moe.T, granularity=moe.granularity)
    assert layer.run_entry
    x = W.bf16_to_torch(moe.x, dev)
    ri = torch.from_numpy(moe.pair_token).to(dev)
    off = torch.from_numpy(moe.offsets).to(dev)
    flops = 2.0 * P * (moe.N1 * moe.K1 + moe.N2 * moe.K2)
    us = 1e3 * graph_ms_per_step(lambda i: layer(x, ri, off), steps, warmup)
    tf = flops / (us * 1e-6) / 1e12
    return {"pairs": P, "step_us": us, "flops": flops, "step_TFLOPs": tf,
            "step_frac_mfma": tf / MFMA_F16_PEAK_TFLOPS, "launches": 6,
            "steps_in_the_launches": "x amax partials, x quantize, gate/up + SwiGLU + h amax "
                                     "partials, h finalize, h quantize, second projection"}


def bench_grouped(C, name, dev, steps, warmup):
    """The dense grouped linear of one decoded token (nvfp4_grouped_linear_run
    through Nvfp4GroupedLinear), weight copies rotated over 512 MB."""
    from moe_amax_gsa_amd import workloads as W
    from moe_amax_gsa_amd.layer import Nvfp4GroupedLinear
    gi = W.make(name)
    wc = torch.from_numpy(gi.w_codes).to(dev)
    wsf = torch.from_numpy(gi.w_scales).to(dev)
    wbytes = gi.w_codes.nbytes + gi.w_scales.nbytes
    ncopies = max(1, min(64, -(-ROTATE_BYTES // wbytes)))
    layers = [Nvfp4GroupedLinear(wc if k == 0 else wc.clone(), wsf if k == 0 else wsf.clone(),
                                 torch.from_numpy(gi.ws2), max_tokens=gi.T)
              for k in range(ncopies)]
    o = W.bf16_to_torch(gi.x, dev).reshape(gi.T, gi.G * gi.K)
    us = 1e3 * graph_ms_per_step(lambda i: layers[i % ncopies](o), steps, warmup)
    nbytes = wbytes + gi.x.nbytes + gi.x.nbytes * 9 // 32 + gi.T * gi.G * gi.N * 4
    launches = 1 if gi.T * gi.G * gi.K <= 16384 else 2
    return {"step_us": us, "rotated_weight_copies": ncopies, "bytes_per_step": nbytes,
            "launches": launches, "step_GBps": nbytes / (us * 1e-6) / 1e9,
            "step_frac_hbm": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS}


def bench_routed(C, name, dev, steps, warmup):
    """The routed experts' first projection over a prefill batch (512 tokens,
    top 8 of 32 experts): the grouped linear on the tiled kernel from
    quantized codes (linear_us), and nvfp4_grouped_linear_run from the bf16
    activation (step_us: amax, quantize, grouped linear).  The stacked
    weights (about 530 MB) are one copy: a step reads them all, more than
    the Infinity Cache holds, before reading any again."""
    from moe_amax_gsa_amd import workloads as W
    moe = W.make(name)
    P = int(moe.offsets[-1])
    w1c, w1s, w1w, _, _, _ = W.moe_weights_to(moe, dev, first_only=True)
    x = W.bf16_to_torch(moe.x, dev)
    ri = torch.from_numpy(moe.pair_token).to(dev)
    off = torch.from_numpy(moe.offsets).to(dev)
    gsa = torch.zeros(1, dtype=torch.float32, device=dev)
    codes = torch.zeros(moe.T, moe.K1 // 2, dtype=torch.uint8, device=dev)
    scales = torch.zeros(moe.T, moe.K1 // 16, dtype=torch.uint8, device=dev)
    y = torch.empty(P, moe.N1, dtype=torch.float32, device=dev)
    nws = max(16, C.nvfp4_workspace_bytes(C.OP_GROUPED_RUN, moe.T, moe.N1, moe.K1, moe.E))
    ws = torch.zeros(nws, dtype=torch.uint8, device=dev)

    def run(i):
        C.nvfp4_grouped_linear_run(x, gsa, codes, scales, ri, off, w1c, w1s, w1w, y, ws)

    def linear(i):
        C.nvfp4_grouped_linear(codes, scales, gsa, ri, off, w1c, w1s, w1w, y)

    step_us = 1e3 * graph_ms_per_step(run, steps, warmup)
    lin_us = 1e3 * graph_ms_per_step(linear, steps, warmup)
    flops = 2.0 * P * moe.N1 * moe.K1
    sizes = np.diff(moe.offsets)
    wbytes = int(moe.E * moe.N1 * (moe.K1 // 2 + moe.K1 // 16))
    abytes = P * (moe.K1 // 2 + moe.K1 // 16) + P * moe.N1 * 4
    tf = flops / (lin_us * 1e-6) / 1e12
    return {"pairs": P, "rows_per_expert_min_mean_max": [int(sizes.min()), float(sizes.mean()),
                                                         int(sizes.max())],
            "step_us": step_us, "linear_us": lin_us, "flops": flops,
            "linear_TFLOPs": tf, "linear_frac_mfma": tf / MFMA_F16_PEAK_TFLOPS,
            "step_TFLOPs": flops / (step_us * 1e-6) / 1e12,
            "weight_bytes": wbytes,
            "linear_GBps_weights_and_rows": (wbytes + abytes) / (lin_us * 1e-6) / 1e9,
            "roofline_us": max(flops / (MFMA_F16_PEAK_TFLOPS * 1e12),
                               (wbytes + abytes) / (HBM_PEAK_GBS * 1e9)) * 1e6,
            "kernel": "gemm_lds_kernel, grouped (128 x 64 tiles over every group's rows)"}


def bench_big_decode(C, name, dev, steps, warmup):
    """A one-row decode with a long weight stream (the lm_head's shape):
    nvfp4_linear_run, and the grouped run with one group (G = 1)."""
    from moe_amax_gsa_amd import workloads as W
    inp = W.make(name)
    b = LinearBench(C, inp, dev)
    M, K, N = inp.M, inp.K, inp.N
    off = torch.tensor([0, M], dtype=torch.int32, device=dev)

    def grouped(i):
        wc, wsf = b.w[i % b.ncopies]
        C.nvfp4_grouped_linear_run(b.x, b.gsa, b.codes, b.scales, None, off, wc.view(1, N, K // 2),
                                   wsf.view(1, N, K // 16), b.ws2, b.y, b.ws)

    r = {"rotated_weight_copies": b.ncopies, "bytes_per_step": b.step_bytes}
    for key, fn in [("linear_run", b.run), ("grouped_run_g1", grouped)]:
        us = 1e3 * graph_ms_per_step(fn, steps, warmup)
        r[key + "_us"] = us
        r[key + "_GBps"] = b.step_bytes / (us * 1e-6) / 1e9
        r[key + "_frac_hbm"] = r[key + "_GBps"] / HBM_PEAK_GBS
    return r


def bench_router(C, name, dev, steps, warmup):
    """The dense router on an already quantized activation: gate linear and
    expert choice (nvfp4_router_topk), gate weights rotated."""
    from moe_amax_gsa_amd import workloads as W
    r = W.make(name)
    M, K, N, k = r.M, r.K, r.N, r.topk
    w = W.bf16_to_torch(r.w, dev)
    wc = torch.empty(N, K // 2, dtype=torch.uint8, device=dev)
    wsf = torch.empty(N, K // 16, dtype=torch.uint8, device=dev)
    ws2 = torch.empty(1, dtype=torch.float32, device=dev)
    qws = torch.empty(max(16, C.nvfp4_workspace_bytes(C.OP_QUANTIZE_WEIGHT, 0, N, K)),
                      dtype=torch.uint8, device=dev)
    C.nvfp4_quantize_weight(w, ws2, wc, wsf, qws)
    wbytes = N * K // 2 + N * K // 16
    ncopies = max(1, min(512, -(-ROTATE_BYTES // wbytes)))
    ws_ = [(wc, wsf)] + [(wc.clone(), wsf.clone()) for _ in range(ncopies - 1)]
    x = W.bf16_to_torch(r.x, dev)
    gsa = torch.empty(1, dtype=torch.float32, device=dev)
    aws = torch.empty(max(16, C.nvfp4_workspace_bytes(C.OP_AMAX_GSA, M * K)), dtype=torch.uint8,
                      device=dev)
    C.nvfp4_amax_gsa(x, gsa, aws)
    codes = torch.empty(M, K // 2, dtype=torch.uint8, device=dev)
    scales = torch.empty(M, K // 16, dtype=torch.uint8, device=dev)
    C.nvfp4_quantize_from_buffer(x, gsa, codes, scales)
    bias = torch.from_numpy(r.bias).to(dev)
    idx = torch.empty(M, k, dtype=torch.int32, device=dev)
    sc = torch.empty(M, k, dtype=torch.float32, device=dev)
    # zeroed: the one-launch path's ticket counter starts at zero
    rws = torch.zeros(max(16, C.nvfp4_workspace_bytes(C.OP_ROUTER_TOPK, M, N, K)),
                      dtype=torch.uint8, device=dev)

    def step(i):
        c, s_ = ws_[i % ncopies]
        C.nvfp4_router_topk(codes, scales, gsa, c, s_, ws2, bias, idx, sc, rws)

    us = 1e3 * graph_ms_per_step(step, steps, warmup)
    # weights + quantized activation + bias + logits written and read + choice
    nbytes = wbytes + M * K * 9 // 16 + N * 4 + M * N * 8 + M * k * 8
    return {"step_us": us, "rotated_weight_copies": ncopies, "bytes_per_step": nbytes,
            "step_GBps": nbytes / (us * 1e-6) / 1e9,
            "step_frac_hbm": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS}


def bench_rmsnorm(C, name, dev, steps, warmup):
    """RMSNorm fused into the quantize (nvfp4_rmsnorm_quantize), with one
    global scale and with one per row."""
    from moe_amax_gsa_amd import workloads as W
    r = W.make(name)
    M, K = r.M, r.K
    x, w = W.bf16_to_torch(r.x, dev), W.bf16_to_torch(r.w, dev)
    gsa = torch.empty(M, dtype=torch.float32, device=dev)
    inv = torch.empty(M, dtype=torch.float32, device=dev)
    codes = torch.empty(M, K // 2, dtype=torch.uint8, device=dev)
    scales = torch.empty(M, K // 16, dtype=torch.uint8, device=dev)
    ws = torch.empty(max(16, C.nvfp4_workspace_bytes(C.OP_RMSNORM_QUANTIZE, M, 0, K)),
                     dtype=torch.uint8, device=dev)
    res = {}
    for key, per_row in [("one_gsa", False), ("gsa_per_row", True)]:
        def step(i, per_row=per_row):
            C.nvfp4_rmsnorm_quantize(x, w, gsa, inv, codes, scales, per_row=per_row, ws=ws)
        res[key + "_us"] = 1e3 * graph_ms_per_step(step, steps, warmup)
    # x and the norm weight read once, codes + scales + inv_rms + gsa written
    nbytes = M * K * 2 + K * 2 + M * K * 9 // 16 + M * 8
    res["bytes_per_step"] = nbytes
    for key in ["one_gsa", "gsa_per_row"]:
        res[key + "_GBps"] = nbytes / (res[key + "_us"] * 1e-6) / 1e9
    return res


def bench_quantize_weight(C, dev, steps, warmup, N=129280, K=7168):
    """Load-time quantize of a bf16 weight the size of the lm_head (vocab
    129280 x hidden 7168): amax -> weight_scale_2 -> codes and scales.  The
    weight is drawn on the device (torch's seeded generator): a numpy draw
    of 0.9 G values would dominate the run."""
    g = torch.Generator(device=dev)
    g.manual_seed(9)
    w = (torch.randn(N, K, generator=g, device=dev, dtype=torch.float32) * 0.02).to(torch.bfloat16)
    ws2 = torch.empty(1, dtype=torch.float32, device=dev)
    codes = torch.empty(N, K // 2, dtype=torch.uint8, device=dev)
    scales = torch.empty(N, K // 16, dtype=torch.uint8, device=dev)
    ws = torch.empty(max(16, C.nvfp4_workspace_bytes(C.OP_QUANTIZE_WEIGHT, 0, N, K)),
                     dtype=torch.uint8, device=dev)
    us = 1e3 * graph_ms_per_step(lambda i: C.nvfp4_quantize_weight(w, ws2, codes, scales, ws),
                                 steps, warmup)
    # the two-phase amax reads w once, the quantize reads it again and writes
    nbytes = 2 * (N * K * 2) + N * K * 9 // 16
    del w
    return {"step_us": us, "N": N, "K": K, "bytes_per_step": nbytes,
            "step_GBps": nbytes / (us * 1e-6) / 1e9,
            "step_frac_hbm": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS}


# ------------------------------------------------------------------ oracle
def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(inp, budget_s=10.0):
    """The oracle's step (amax, quantize, FP64 linear) for the same workload
    on every host core this process may use, then on one core, each repeated
    within a time budget.  Returns [(seconds per step, steps, threads,
    seconds per step in amax + quantize, seconds per step in the linear)]."""
    from oracle import oracle
    legs = []
    for threads in (len(os.sched_getaffinity(0)), 1):
        used = oracle.set_threads(threads)
        n = 0
        tq = tl = 0.0
        t0 = time.perf_counter()
        while True:
            a = time.perf_counter()
            g = oracle.amax_gsa(inp.x)
            c, s = oracle.quantize(inp.x, g)
            b = time.perf_counter()
            oracle.linear(c, s, g, inp.w_codes, inp.w_scales, inp.ws2)
            tq += b - a
            tl += time.perf_counter() - b
            n += 1
            el = time.perf_counter() - t0
            if el >= budget_s or n >= 1000:
                break
        legs.append((el / n, n, used, tq / n, tl / n))
    return legs


# ------------------------------------------------------------------ probe
_probe_lib = None


def probe_lib():
    """libnvfp4_probe.so: an empty kernel and a read-only stream, for the
    measured floors of a launch shape."""
    global _probe_lib
    if _probe_lib is None:
        import ctypes
        from moe_amax_gsa_amd import build as B
        lib = ctypes.CDLL(B.PROBE_LIB)
        P, I, I64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
        lib.probe_empty.restype = I
        lib.probe_empty.argtypes = [I, I, P]
        lib.probe_stream.restype = I
        lib.probe_stream.argtypes = [P, I64, P, I64, I, I, P, P]
        _probe_lib = lib
    return _probe_lib


def launch_floors(b, grid: int, threads: int, steps: int):
    """floor_us: an empty kernel of the given grid; stream_us: a read-only
    pass of a step's weight codes and scales (rotated copies) with that grid;
    both as graph_ms_per_step times them."""
    import ctypes
    lib = probe_lib()
    out = torch.empty(grid * (threads // 64), dtype=torch.int32, device="cuda")

    def stream_of():
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def empty(i):
        assert lib.probe_empty(grid, threads, stream_of()) == 0

    def stream(i):
        wc, wsf = b.w[i % b.ncopies]
        assert lib.probe_stream(ctypes.c_void_p(wc.data_ptr()), wc.numel(),
                                ctypes.c_void_p(wsf.data_ptr()), wsf.numel(), grid, threads,
                                ctypes.c_void_p(out.data_ptr()), stream_of()) == 0

    return (1e3 * graph_ms_per_step(empty, steps, 2), 1e3 * graph_ms_per_step(stream, steps, 2))


def pmc_probe(C, dev, launches=20):
    """A 256 MiB device copy (three times, to calibrate the byte counters),
    then `launches` launches of the headline step on rotated weights."""
    from moe_amax_gsa_amd import workloads as W
    src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    b = LinearBench(C, W.make(HEAD), dev)
    for i in range(launches):
        b.run(i)
    torch.cuda.synchronize()
    print(json.dumps({"pmc_probe": HEAD, "copy_bytes": src.numel(), "copies": 3,
                      "launches": launches, "bytes_per_launch": b.step_bytes,
                      "source_hash": kernel_source_hash()}))


def pmc_probe_prefill(C, dev, launches=10, name="prefill_m512_k7168_n4096", matmul=False):
    """A 256 MiB device copy (three times), then `launches` rounds of the
    workload's amax + quantize and its linear, on rotated weights; with
    matmul, then `launches` of torch's bf16 matmul of the same shape (its
    counters as context)."""
    from moe_amax_gsa_amd import workloads as W
    src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    b = LinearBench(C, W.make(name), dev)
    for i in range(launches):
        b.quantize(i)
        b.linear(i)
    torch.cuda.synchronize()
    if matmul:
        inp = b.inp
        g = torch.Generator(device=dev)
        g.manual_seed(11)
        a = torch.randn(inp.M, inp.K, generator=g, device=dev).to(torch.bfloat16)
        bt = torch.randn(inp.K, inp.N, generator=g, device=dev).to(torch.bfloat16)
        for _ in range(launches):
            torch.matmul(a, bt)
        torch.cuda.synchronize()
    print(json.dumps({"pmc_probe": name, "copy_bytes": src.numel(), "copies": 3,
                      "launches": launches, "quant_bytes": b.quant_bytes, "flops": b.flops,
                      "torch_bf16_matmul": matmul, "source_hash": kernel_source_hash()}))


def torch_bf16_matmul_us(M, N, K, dev, iters=20):
    """Context only: torch's bf16 matmul (hipBLASLt) on random operands of
    the same shape, timed eagerly between events (not captured)."""
    g = torch.Generator(device=dev)
    g.manual_seed(11)
    a = torch.randn(M, K, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    bt = torch.randn(K, N, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, bt)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        torch.matmul(a, bt)
    e1.record()
    torch.cuda.synchronize()
    return 1e3 * e0.elapsed_time(e1) / iters


# ------------------------------------------------------------------ main
def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU (got --gpus {args.gpus}): the layer runs on one GPU "
              "and is not sharded across several", file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench needs a GPU"
    from moe_amax_gsa_amd import nvfp4 as C
    dev = torch.device("cuda:0")
    if args.pmc_probe:
        pmc_probe(C, dev)
        return
    if args.pmc_probe_prefill:
        pmc_probe_prefill(C, dev)
        return
    if args.pmc_probe_stress:
        pmc_probe_prefill(C, dev, name="stress_m2048_k7168_n7168", matmul=True)
        return
    kiters = 50

    log("headline", HEAD)
    inp, b, r = bench_linear(C, HEAD, dev, args.steps, args.warmup, kiters)
    workloads = {HEAD: r}
    if not args.no_extra:
        for name, steps in [("tiny_m1_k256_n256", args.steps),
                            ("prefill_m512_k7168_n4096", max(20, args.steps // 4)),
                            ("stress_m2048_k7168_n7168", max(10, args.steps // 10))]:
            if args.only and args.only != name:
                continue
            log("workload", name)
            workloads[name] = bench_linear(C, name, dev, steps, min(args.warmup, 10),
                                           min(kiters, steps), settle=name != "tiny_m1_k256_n256")[2]
            if name != "tiny_m1_k256_n256":
                c = __import__("moe_amax_gsa_amd.workloads", fromlist=["WORKLOADS"]).WORKLOADS[name]
                us = torch_bf16_matmul_us(c["M"], c["N"], c["K"], dev)
                workloads[name]["context_torch_bf16_matmul_us"] = us
                workloads[name]["context_torch_bf16_matmul_TFLOPs"] = (
                    workloads[name]["flops"] / (us * 1e-6) / 1e12)
        for name in ["router_m1_k7168_e384_top6", "router_m64_k7168_e384_top6"]:
            if args.only and args.only != name:
                continue
            log("workload", name)
            workloads[name] = bench_router(C, name, dev, args.steps, min(args.warmup, 10))
        for name in ["rmsnorm_m1_k7168", "rmsnorm_m512_k7168"]:
            if args.only and args.only != name:
                continue
            log("workload", name)
            workloads[name] = bench_rmsnorm(C, name, dev, args.steps, min(args.warmup, 10))
        if not args.only or args.only == "quantize_weight_n129280_k7168":
            log("workload quantize_weight_n129280_k7168")
            workloads["quantize_weight_n129280_k7168"] = bench_quantize_weight(
                C, dev, max(5, args.steps // 40), 2)
        for name in ["grouped_wo_a_t1_g8_k8192_n1536"]:
            if args.only and args.only != name:
                continue
            log("workload", name)
            workloads[name] = bench_grouped(C, name, dev, args.steps, min(args.warmup, 10))
        for name in ["lm_head_m1_k7168_n129280"]:
            if args.only and args.only != name:
                continue
            log("workload", name)
            workloads[name] = bench_big_decode(C, name, dev, max(10, args.steps // 4),
                                               min(args.warmup, 3))
        for name in ["moe_l1_t512_e32_top8_k7168_n4096", "moe_l1_t512_e32_top8_k7168_n4096_zipf"]:
            if args.only and args.only != name:
                continue
            log("workload", name)
            workloads[name] = bench_routed(C, name, dev, max(5, args.steps // 4),
                                           min(args.warmup, 3))
        if not args.only or args.only == "moe_t512_e32_top8":
            log("workload moe_t512_e32_top8")
            workloads["moe_t512_e32_top8"] = bench_moe_prefill(C, dev, max(5, args.steps // 4),
                                                              min(args.warmup, 3))
        if not args.only or args.only == "moe_t64_e256_top8":
            log("workload moe_t64_e256_top8")
            workloads["moe_t64_e256_top8"] = bench_moe(C, dev, max(10, args.steps // 10),
                                                      min(args.warmup, 3))

    cpu = None
    if not args.no_cpu:
        log("cpu baseline (oracle)")
        (t_all, n_all, c_all, q_all, l_all), (t_one, n_one, _, q_one, l_one) = cpu_baseline(inp)
        cpu = {"value": b.step_bytes / t_all / 1e9, "unit": "GB/s", "cores": c_all,
               "kind": "oracle", "cpu_model": cpu_model(),
               "sample": f"{n_all} whole oracle steps (amax, quantize, FP64 linear) of {HEAD} "
                         f"on {c_all} threads, {t_all * 1e3:.1f} ms each",
               "ms_amax_quantize": q_all * 1e3, "ms_linear": l_all * 1e3,
               "one_core": {"value": b.step_bytes / t_one / 1e9, "unit": "GB/s", "cores": 1,
                            "sample": f"{n_one} oracle steps of {HEAD} on 1 thread, "
                                      f"{t_one * 1e3:.1f} ms each",
                            "ms_amax_quantize": q_one * 1e3, "ms_linear": l_one * 1e3}}

    # at M=1 the step is one launch of the fused kernel: its average
    # duration is the step time of the graph of K launches
    kern_us = r["step_us"]
    run_gbps = b.step_bytes / (kern_us * 1e-6) / 1e9
    # the decode kernel's launch shape: 8 weight rows and K / 1024 waves
    # (two 512-element sets each) per workgroup
    grid, threads = -(-inp.N // 8), 64 * min(16, -(-inp.K // 1024))
    log("launch floors", grid, threads)
    floor_us, stream_us = launch_floors(b, grid, threads, args.steps)
    wbytes = inp.w_codes.nbytes + inp.w_scales.nbytes
    traffic = recorded_traffic(os.path.join(ROOT, "profiles", "traffic_gemv_narrow_run_decode_m1_k7168_n1536.md"))
    line = {
        "metric": "NVFP4 linear decode weight-stream GB/s (M=1, K=7168, N=1536)",
        "value": r["step_GBps"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["step_us"] * 1e-3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp4",
        "dtype_detail": "e2m1 x e2m1 block sums on the fp4 matrix cores, e4m3 block scales and "
                        "the global scales applied in f32, f32 accumulation",
        "data": "synthetic, seeded",
        "config": {"workload": HEAD, "M": 1, "K": 7168, "N": 1536,
                   "step": "nvfp4_linear_run (amax, gsa, quantize, linear)",
                   "bytes_per_step": b.step_bytes},
        "roofline": {"bound": "hbm", "achieved": run_gbps, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": run_gbps / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "gemv_narrow_kernel, run mode (amax, gsa, quantize and linear "
                               "for one activation row in one launch)",
                     "kernel_us": kern_us, "bytes_per_launch": b.step_bytes,
                     "floor_us": floor_us, "stream_us": stream_us,
                     "stream_GBps": wbytes / (stream_us * 1e-6) / 1e9,
                     "floors": f"floor_us: an empty kernel of the same grid ({grid} x {threads} "
                               f"threads); stream_us: a read-only pass of the {wbytes} weight "
                               "bytes with that grid; each in a graph of K launches"},
        "timing": {"graph_launches_per_replay": args.steps,
                   "weight_copies": b.ncopies,
                   "reuse_distance_bytes": b.ncopies * wbytes,
                   "distinct_weight_bytes_per_replay": min(args.steps, b.ncopies) * wbytes,
                   "flush_bytes_before_timed_replay": 2 * FLUSH_BYTES},
        "cpu_baseline": cpu,
        "workloads": workloads,
        "context": "the pages' whole-model decode on B200 took about 1.45 s per token "
                   "(61 layers; not comparable to one projection)",
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
