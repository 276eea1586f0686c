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
    os.path.join(CSRC, "kernels", "w8a16_gemm.hip"),
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


# Host-code sanitizers for the test suite's sanitizer build (AddressSanitizer
# and UndefinedBehaviorSanitizer on the host side only: each flag is scoped to
# the host compilation, the gfx950 code is built as usual).
SANITIZE_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-g"]
SANITIZE_DIR = os.path.join(BUILD, "sanitize")
SANITIZE_LIB = os.path.join(SANITIZE_DIR, "libfp8q_sanitize.so")


def _compile(src: str, asm: bool, outdir: str = BUILD, extra=()) -> str:
    obj = os.path.join(outdir, os.path.basename(src) + ".o")
    cmd = [hipcc(), *common_flags(), *extra, "-c", src, "-o", obj]
    if asm:
        cmd += ["-save-temps=obj"]
    subprocess.check_call(cmd, cwd=outdir)
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


def sources_digest() -> str:
    import hashlib
    h = hashlib.sha256()
    for root in (CSRC, os.path.join(ROOT, "include")):
        for dirpath, _, files in sorted(os.walk(root)):
            for f in sorted(files):
                if f.endswith((".cpp", ".hip", ".hpp", ".h")):
                    with open(os.path.join(dirpath, f), "rb") as fh:
                        h.update(f.encode() + fh.read())
    h.update(" ".join(SANITIZE_HOST).encode())
    return h.hexdigest()[:16]


def build_sanitize(jobs: int = 4) -> str:
    """The library with host-side AddressSanitizer + UndefinedBehaviorSanitizer
    (for CPU tests of the argument validation, loaded through FP8Q_LIBRARY
    with the sanitizer runtime preloaded).  Rebuilt only when a source changes."""
    os.makedirs(SANITIZE_DIR, exist_ok=True)
    stamp = os.path.join(SANITIZE_DIR, "digest")
    digest = sources_digest()
    if os.path.exists(SANITIZE_LIB) and os.path.exists(stamp) and open(stamp).read() == digest:
        return SANITIZE_LIB
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda s: _compile(s, False, SANITIZE_DIR, SANITIZE_HOST), SOURCES))
    tmp = SANITIZE_LIB + ".tmp%d" % os.getpid()
    subprocess.check_call([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *SANITIZE_HOST,
                           *objs, "-o", tmp])
    os.replace(tmp, SANITIZE_LIB)
    with open(stamp, "w") as f:
        f.write(digest)
    return SANITIZE_LIB


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=4)
    ap.add_argument("--asm", action="store_true", help="keep the gfx950 assembly in _build/")
    args = ap.parse_args()
    build(args.jobs, args.asm)


if __name__ == "__main__":
    main()
