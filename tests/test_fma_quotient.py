"""The FMA-corrected reciprocal product the kernels use for x / s is the
correctly rounded quotient (host-side check of the arithmetic, every bf16 x
against every dynamic scale and sampled others; see native/fma_quotient_check.c).
It does not run the kernels: their codes are compared with the oracle's by
the GPU tests."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def _has_fma() -> bool:
    try:
        with open("/proc/cpuinfo") as f:
            return " fma " in f.read()
    except OSError:
        return False


@pytest.mark.skipif(shutil.which("gcc") is None or not _has_fma(), reason="needs gcc and a host FMA")
def test_fma_corrected_quotient_is_correctly_rounded(tmp_path):
    exe = tmp_path / "fma_quotient_check"
    subprocess.run(["gcc", "-O2", "-mfma", "-ffp-contract=off", "-o", str(exe),
                    os.path.join(HERE, "native", "fma_quotient_check.c"), "-lm"], check=True)
    r = subprocess.run([str(exe), "500"], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert " 0 differences" in r.stdout, r.stdout
