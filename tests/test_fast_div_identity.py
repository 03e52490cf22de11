"""The GPU quantisers divide by the per-tensor Q scale as one multiply by
the rounded reciprocal and one fused-multiply-add correction; the codes
must equal those of IEEE division bit for bit (they are compared with the
oracle's codes on the GPU). This host test proves the identity the kernels
rely on over every pair of mantissas and every bf16 value
(`tests/host/fast_div_identity.c`)."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "host", "fast_div_identity.c")


def _has_fma():
    try:
        with open("/proc/cpuinfo") as f:
            return " fma " in f.read()
    except OSError:
        return False


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_fast_division_equals_ieee_division(tmp_path):
    exe = tmp_path / "fast_div_identity"
    flags = ["-O2", "-ffp-contract=off"] + (["-mfma"] if _has_fma() else [])
    subprocess.run(["gcc", *flags, "-o", str(exe), SRC, "-lm"], check=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    print(res.stdout)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "1073741824 checked, 0 differ" in res.stdout
