"""The Q quantizer's short quotient path against the IEEE division it replaces: an exhaustive
CPU check over every bf16 and fp16 input value and every block maximum (tests/
quant_division_check.c). The quantizer's codes are defined by y = x / s (IEEE division); the
kernel computes y from a once-per-block reciprocal and two FMAs where 2^-96 <= s < inf, and this
check shows that every code that path can produce equals the division's (about 2 * 10^9
(type, x, amax) cases; fp16 quotients are bit-identical too). GPU parity of the kernel's codes
with the oracle is in test_quant_gpu.py."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def _has_fma() -> bool:
    try:
        return " fma " in open("/proc/cpuinfo").read().replace("\n", " ")
    except OSError:
        return False


@pytest.mark.timeout(600)
def test_quotient_short_path_gives_the_division_codes(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "quant_division_check")
    cmd = [gcc, "-O2", "-ffp-contract=off", "-fopenmp", os.path.join(HERE, "quant_division_check.c"), "-o", exe, "-lm"]
    if _has_fma():
        cmd.insert(1, "-mfma")
    subprocess.run(cmd, check=True, capture_output=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=580,
                       env=dict(os.environ, OMP_NUM_THREADS=str(min(8, os.cpu_count() or 1))))
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    lines = r.stdout.strip().splitlines()
    assert len(lines) == 2 and all("E4M3 codes differing 0;" in l for l in lines)
    assert "fp32 quotients differing 0," in lines[1]   # fp16
