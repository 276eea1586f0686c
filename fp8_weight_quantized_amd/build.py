"""Build libfp8q.so in-tree with hipcc for gfx950.

    python -m fp8_weight_quantized_amd.build [--jobs N] [--asm]

Every source is compiled to its own object (in parallel), then linked into
fp8_weight_quantized_amd/libfp8q.so.  Flags that matter:
  * --offload-arch=gfx950: CDNA4 only, no other targets;
  * no fast-math: the quantizers need correctly rounded fp32 division
    (hipcc's default); -ffast-math would turn it into a reciprocal;
  * packed fp32 instructions disabled (-packed-fp32-ops target feature).
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libfp8q.so")

SOURCES = [
    os.path.join(CSRC, "fp8q_api.cpp"),
    os.path.join(CSRC, "kernels", "quant.hip"),
    os.path.join(CSRC, "kernels", "w8a16.hip"),
    os.path.join(CSRC, "kernels", "w8a8.hip"),
    os.path.join(CSRC, "kernels", "kv_cache.hip"),
]

ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build fp8q)")


def common_flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-Wall",
        "-Wno-unused-result",
        "-I", os.path.join(ROOT, "include"),
        "-I", CSRC,
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    ]


def _compile(src: str, asm: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *common_flags(), "-c", src, "-o", obj]
    if asm:
        cmd += ["-save-temps=obj"]
    subprocess.check_call(cmd, cwd=BUILD)
    return obj


def build(jobs: int = 4, asm: bool = False, verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda s: _compile(s, asm), SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    subprocess.check_call([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB, file=sys.stderr)
    return LIB


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=4)
    ap.add_argument("--asm", action="store_true", help="keep the gfx950 assembly in _build/")
    args = ap.parse_args()
    build(args.jobs, args.asm)


if __name__ == "__main__":
    main()
