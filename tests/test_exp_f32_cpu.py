"""The tests' correctly rounded fp32 exponential (tests/exp_f32_rn.h, the
yardstick the GPU test holds the kernels' SiLU to), built for the host and run
against the C library: every input of a strided sweep of all 2^32 fp32 bit
patterns must give the fp32 rounding of the extended-precision exponential,
and so must (float)exp((double)x), the oracle's SiLU exponential.  W8A8_EXP_EXHAUSTIVE=1 runs all 2^32 inputs (about two minutes on 8
cores).  The 2^(j/64) table is pinned to a recomputation in 80-digit decimal
arithmetic."""
import os
import re
import shutil
import subprocess
import tempfile
from decimal import Decimal, getcontext

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.join(ROOT, "tests")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.fixture(scope="module")
def checker():
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not found")
    d = tempfile.mkdtemp(prefix="w8a8_exp_")
    exe = os.path.join(d, "exp_f32_check")
    subprocess.run([HIPCC, "-x", "hip", "--cuda-host-only", "-O2", "-mfma", "-std=c++17", "-ffp-contract=off",
                    "-I", TESTS, os.path.join(TESTS, "exp_f32_check.cpp"), "-o", exe, "-lpthread"],
                   check=True)
    yield exe
    shutil.rmtree(d, ignore_errors=True)


def _run(exe, step):
    out = subprocess.run([exe, str(step), str(min(8, os.cpu_count() or 1))], check=True,
                         capture_output=True, text=True).stdout.split()
    n, bad, diff_exp = map(int, out[:3])
    return n, bad, diff_exp, out[3:]


def test_exp_matches_libm_on_a_sweep(checker):
    step = 1 if os.environ.get("W8A8_EXP_EXHAUSTIVE") == "1" else 101
    n, bad, diff_exp, ex = _run(checker, step)
    assert n == (1 << 32) // step + (1 if (1 << 32) % step else 0)
    assert bad == 0, f"{bad} inputs differ from the extended-precision exponential, e.g. {ex}"
    assert diff_exp == 0  # the oracle's double exponential rounds the same way


def test_exp_table_is_two_to_the_j_over_64():
    getcontext().prec = 80
    text = open(os.path.join(TESTS, "exp_f32_rn.h")).read()

    def table(name):
        body = re.search(name + r"\[64\]\s*=\s*\{(.*?)\};", text, re.S).group(1)
        vals = [float.fromhex(v) for v in re.findall(r"-?0x[0-9a-fA-F.]+p[+-]?\d+", body)]
        assert len(vals) == 64
        return vals

    hi, lo = table("EXP2_J64_HI"), table("EXP2_J64_LO")
    for j in range(64):
        v = Decimal(2) ** (Decimal(j) / Decimal(64))
        assert hi[j] == float(v), j
        assert lo[j] == float(v - Decimal(hi[j])), j
