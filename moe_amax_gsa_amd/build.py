"""Ahead-of-time build of the HIP library (libnvfp4.so) for gfx950.

    python -m moe_amax_gsa_amd.build

Compiles every csrc/*.hip with hipcc into objects and links one shared
library next to this file, and the benchmark's measurement probes
(probe/probe.hip) into a second one.  No JIT at import time.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libnvfp4.so")
PROBE_SRC = os.path.join(HERE, "probe", "probe.hip")
PROBE_LIB = os.path.join(HERE, "libnvfp4_probe.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    # packed fp32 instructions are kept out of generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # IEEE fp32: correctly rounded division, denormals kept
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-flush-denormals-to-zero",
    "-fno-fast-math", "-Wall", "-Wno-unused-function",
]
PER_FILE = {
    "quant.hip": ["-ffp-contract=off"],
}


def sources():
    return sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    path = src if os.path.isabs(src) else os.path.join(CSRC, src)
    cmd = [HIPCC, *COMMON, *PER_FILE.get(src, []), "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    # the host pass does not know the gfx950 feature name; drop that noise
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs) + 1)) as ex:
        objs = list(ex.map(_compile, srcs + [PROBE_SRC]))
    _link(objs[:-1], LIB)
    _link(objs[-1:], PROBE_LIB)
    if verbose:
        print(f"built {LIB} from {', '.join(srcs)}; {PROBE_LIB} from probe/probe.hip")
    return LIB


if __name__ == "__main__":
    build()
