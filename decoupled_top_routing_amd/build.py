"""Build libmoe.so (HIP, gfx950) in-tree with hipcc.

Each source is compiled to an object under ``_build/`` in parallel, then
linked into ``decoupled_top_routing_amd/libmoe.so``.  Every build compiles
from scratch.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
OUT = PKG / "libmoe.so"
BUILD = ROOT / "_build"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-fno-gpu-rdc", "-Wall", "-Wno-unused-function",
    # no packed fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{ROOT / 'include'}", f"-I{CSRC}",
]

SOURCES = ["route.hip", "decode.hip", "decode_b1.hip", "prefill.hip",
           "channel_topk.hip", "util.hip", "noalloc.hip", "moe_abi.cpp"]


def _compile(src: str) -> Path:
    obj = BUILD / (Path(src).name + ".o")
    cmd = [HIPCC, *COMMON, "-x", "hip", "-c", str(CSRC / src), "-o", str(obj)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed on {src}")
    return obj


def build(verbose: bool = False) -> Path:
    BUILD.mkdir(exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT.with_suffix(".so.tmp")
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,-z,defs", *map(str, objs),
           "-o", str(tmp)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("link of libmoe.so failed")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    build(verbose=True)
