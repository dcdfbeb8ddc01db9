"""Benchmark of the NVFP4 linear layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--only NAME] [--no-cpu]

A step is one pass of the layer's hot path over one batch of synthetic,
seeded input already resident in HBM: amax -> gsa, quantize from the gsa
buffer, and the block-scaled linear (and, for the MoE workload, SwiGLU,
re-quantize and the second grouped linear).  The headline line is the
decode projection (M=1, K=7168, N=1536): decode weight-stream GB/s =
algorithmic bytes of the linear (weight codes + weight scales + activation
codes + scales + output) / step time.  Weight copies are rotated over more
than 512 MB so the 256 MB Infinity Cache cannot serve repeats.  The other
workloads are reported under "workloads" in the same JSON line.

Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2516.6  # dense f16/bf16 matrix cores: 256 CU * 4096 flop/clk * 2.4 GHz
ROTATE_BYTES = 512 << 20


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--only", default=None, help="run one workload")
    p.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    p.add_argument("--no-extra", action="store_true", help="headline workload only")
    return p.parse_args()


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


class Timer:
    """Events on the current (launch) stream."""

    def __init__(self):
        self.a = torch.cuda.Event(enable_timing=True)
        self.b = torch.cuda.Event(enable_timing=True)

    def start(self):
        self.a.record()

    def stop(self) -> float:
        self.b.record()
        self.b.synchronize()
        return self.a.elapsed_time(self.b)


# ------------------------------------------------------------------ linear
class LinearBench:
    """One workload of the single-projection path with rotated weight copies."""

    def __init__(self, C, inp, dev):
        from moe_amax_gsa_amd import workloads as W
        self.C, self.inp = C, inp
        M, K, N = inp.M, inp.K, inp.N
        wbytes = inp.w_codes.nbytes + inp.w_scales.nbytes
        self.ncopies = max(1, min(256, -(-ROTATE_BYTES // wbytes)))
        wc = torch.from_numpy(inp.w_codes).to(dev)
        wsf = torch.from_numpy(inp.w_scales).to(dev)
        self.w = [(wc, wsf)] + [(wc.clone(), wsf.clone()) for _ in range(self.ncopies - 1)]
        self.x = W.bf16_to_torch(inp.x, dev)
        self.ws2 = torch.tensor([inp.ws2], dtype=torch.float32, device=dev)
        self.gsa = torch.zeros(1, dtype=torch.float32, device=dev)
        nws = max(16, C.nvfp4_workspace_bytes(C.OP_AMAX_GSA, M * K))
        self.ws = torch.empty(nws, dtype=torch.uint8, device=dev)
        self.codes = torch.empty(M, K // 2, dtype=torch.uint8, device=dev)
        self.scales = torch.empty(M, K // 16, dtype=torch.uint8, device=dev)
        self.y = torch.empty(M, N, dtype=torch.float32, device=dev)
        self.flops = 2.0 * M * N * K
        # algorithmic bytes of the linear: W codes + W scales + A codes + A scales + y
        self.linear_bytes = wbytes + M * K // 2 + M * K // 16 + M * N * 4
        # quantize pass: read x, write codes + scales
        self.quant_bytes = M * K * 2 + M * K // 2 + M * K // 16

    def quantize(self):
        C = self.C
        C.nvfp4_amax_gsa(self.x, self.gsa, self.ws)
        C.nvfp4_quantize_from_buffer(self.x, self.gsa, self.codes, self.scales)

    def linear(self, i):
        wc, wsf = self.w[i % self.ncopies]
        self.C.nvfp4_linear(self.codes, self.scales, self.gsa, wc, wsf, self.ws2, self.y)

    def step(self, i):
        self.quantize()
        self.linear(i)


def time_steps(fn, steps, warmup) -> float:
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    t = Timer()
    t.start()
    for i in range(steps):
        fn(i)
    ms = t.stop()
    torch.cuda.synchronize()
    return ms / steps


def time_kernel(pre, kern, steps) -> float:
    """Average duration of kern(i) measured by events around each launch."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for i in range(steps):
        pre(i)
        evs[i][0].record()
        kern(i)
        evs[i][1].record()
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in evs) / steps


# ------------------------------------------------------------------ oracle
def cpu_baseline(inp, budget_s=12.0):
    """The oracle's step (amax, quantize, linear) on host cores for the same
    workload, repeated within a time budget."""
    from oracle import oracle
    threads = len(os.sched_getaffinity(0))
    os.environ.setdefault("OMP_NUM_THREADS", str(threads))
    oracle._load()
    n = 0
    t0 = time.perf_counter()
    while True:
        g = oracle.amax_gsa(inp.x)
        c, s = oracle.quantize(inp.x, g)
        oracle.linear(c, s, g, inp.w_codes, inp.w_scales, inp.ws2)
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s or n >= 1000:
            break
    return el / n, n, int(os.environ.get("OMP_NUM_THREADS", threads))


# ------------------------------------------------------------------ main
def bench_linear(C, name, dev, steps, warmup):
    from moe_amax_gsa_amd import workloads as W
    inp = W.make(name)
    b = LinearBench(C, inp, dev)
    ms = time_steps(b.step, steps, warmup)
    lin_ms = time_kernel(lambda i: b.quantize(), b.linear, steps)
    q_ms = time_kernel(lambda i: None, lambda i: b.quantize(), steps)
    r = {
        "ms_per_step": ms,
        "linear_us": lin_ms * 1e3,
        "quant_us": q_ms * 1e3,
        "rotated_weight_copies": b.ncopies,
        "linear_GBps": b.linear_bytes / (lin_ms * 1e-3) / 1e9,
        "linear_TFLOPs": b.flops / (lin_ms * 1e-3) / 1e12,
        "step_GBps": b.linear_bytes / (ms * 1e-3) / 1e9,
        "step_TFLOPs": b.flops / (ms * 1e-3) / 1e12,
    }
    r["linear_frac_hbm"] = r["linear_GBps"] / HBM_PEAK_GBS
    r["linear_frac_mfma"] = r["linear_TFLOPs"] / MFMA_F16_PEAK_TFLOPS
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
    ms = time_steps(lambda i: layer(x, ri, off), steps, warmup)
    return {"ms_per_step": ms, "active_experts": nact, "weight_bytes": wbytes,
            "step_GBps": wbytes / (ms * 1e-3) / 1e9,
            "step_frac_hbm": wbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "step_TFLOPs": flops / (ms * 1e-3) / 1e12}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the layer is not "
              "sharded across GPUs in this build", file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench needs a GPU"
    from moe_amax_gsa_amd import nvfp4 as C
    dev = torch.device("cuda:0")
    head = "decode_m1_k7168_n1536"

    log("headline", head)
    inp, b, r = bench_linear(C, head, dev, args.steps, args.warmup)
    workloads = {head: r}
    if not args.no_extra:
        for name, steps in [("tiny_m1_k256_n256", args.steps),
                            ("prefill_m512_k7168_n4096", max(20, args.steps // 4)),
                            ("stress_m2048_k7168_n7168", max(10, args.steps // 10))]:
            if args.only and args.only != name:
                continue
            log("workload", name)
            workloads[name] = bench_linear(C, name, dev, steps, min(args.warmup, 10))[2]
        if not args.only or args.only == "moe_t64_e256_top8":
            log("workload moe_t64_e256_top8")
            workloads["moe_t64_e256_top8"] = bench_moe(C, dev, max(10, args.steps // 10),
                                                      min(args.warmup, 5))

    cpu = None
    if not args.no_cpu:
        log("cpu baseline (oracle)")
        per_step_s, nrep, cores = cpu_baseline(inp)
        cpu = {"value": b.linear_bytes / per_step_s / 1e9, "unit": "GB/s", "cores": cores,
               "kind": "oracle",
               "sample": f"{nrep} full oracle steps (amax, quantize, FP64 linear) of {head}, "
                         f"{per_step_s * 1e3:.1f} ms each"}

    ms = r["ms_per_step"]
    line = {
        "metric": "NVFP4 linear decode weight-stream GB/s (M=1, K=7168, N=1536)",
        "value": r["step_GBps"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e2m1 x e2m1 (E4M3 block scales), fp32 accumulate",
        "data": "synthetic, seeded",
        "config": {"workload": head, "M": 1, "K": 7168, "N": 1536,
                   "step": "amax_gsa + quantize_from_buffer + linear",
                   "bytes_per_step": b.linear_bytes},
        "roofline": {"bound": "hbm", "achieved": r["linear_GBps"], "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": r["linear_GBps"] / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "gemv_fp4_kernel", "kernel_us": r["linear_us"]},
        "cpu_baseline": cpu,
        "workloads": workloads,
        "context": "pages' whole-model decode on B200: ~1.45 s/token (not comparable)",
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
