"""Builds the HIP library (libmoe_int4.so) in-tree for gfx950 with hipcc.

Each source is compiled to its own object in parallel (the kernel files take
most of the time), then the objects are linked into the shared library.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ_DIR = os.path.join(os.path.dirname(HERE), "_build")
LIB = os.path.join(HERE, "libmoe_int4.so")
SOURCES = ["moe_decode.hip", "moe_batch.hip", "moe_abi.cpp", "moe_cache.cpp", "moe_static.hip", "moe_probe.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # packed fp32 instructions are kept out of the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _clean(stderr: str) -> str:
    return "\n".join(l for l in (stderr or "").splitlines() if "packed-fp32-ops" not in l)


def _compile(src: str) -> tuple[str, str]:
    path = os.path.join(CSRC, src)
    obj = os.path.join(OBJ_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + FLAGS + ["-c", "-x", "hip", path, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n" + _clean(res.stderr))
    return obj, _clean(res.stderr)


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    if verbose:
        print(f"{HIPCC} {' '.join(FLAGS)} -c <{', '.join(srcs)}>", flush=True)
    with ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 1)) as pool:
        results = list(pool.map(_compile, srcs))
    objs = [o for o, _ in results]
    warnings = "\n".join(w for _, w in results if w.strip())
    if verbose and warnings:
        print(warnings, file=sys.stderr)
    tmp = LIB + ".tmp"
    res = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp],
                         capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc link failed:\n" + _clean(res.stderr))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
