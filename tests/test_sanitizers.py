"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

- The C ABI's argument validation, workspace queries, planners and describe
  calls: tests/test_abi.py rerun against a build of the library whose host
  code is instrumented (the gfx950 code is built as usual and never runs
  here), with the sanitizer runtime preloaded.
- The oracle: its pin tests rerun against an instrumented build of
  fp8q_oracle.c (the exhaustive 2^32 cast sweep is left out for time).

A test passes only if the rerun passes and no sanitizer report appears.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
REPORTS = ("ERROR: AddressSanitizer", "runtime error:", "ERROR: LeakSanitizer",
           "SUMMARY: UndefinedBehaviorSanitizer")


def _run(args, env_extra):
    env = dict(os.environ)
    env.update(env_extra)
    env["PYTHONDONTWRITEBYTECODE"] = "1"
    p = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu", *args], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=900)
    out = p.stdout + p.stderr
    for marker in REPORTS:
        assert marker not in out, out[-6000:]
    assert p.returncode == 0, out[-6000:]
    return out


def _clang_asan_runtime():
    libs = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not libs:
        pytest.skip("clang AddressSanitizer runtime not found")
    return libs[-1]


def test_abi_host_code_under_sanitizers():
    from fp8_weight_quantized_amd import build
    lib = build.build_sanitize()
    out = _run(["tests/test_abi.py"], {
        "LD_PRELOAD": _clang_asan_runtime(),
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "FP8Q_LIBRARY": lib,
    })
    assert " passed" in out


def test_oracle_under_sanitizers():
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    if not asan or not os.path.isabs(asan):
        pytest.skip("gcc AddressSanitizer runtime not found")
    pins = sorted(glob.glob(os.path.join(ROOT, "tests", "test_oracle_*.py")))
    out = _run([*[os.path.relpath(p, ROOT) for p in pins], "-k", "not every_fp32_pattern"], {
        "LD_PRELOAD": asan,
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "ORACLE_SANITIZE": "1",
    })
    assert " passed" in out
