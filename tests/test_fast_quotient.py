"""The fp8 store kernels replace x / scale by x * (1/scale) plus one fused
multiply-add correction when the group maximum is a finite bf16 value
>= 2^-4.  This checks, exhaustively over every such (amax, x) bf16 pair, that
the fp8 code (e4m3 and e5m2) is the one the oracle gives for the IEEE
quotient (CPU only)."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("fq") / "fast_quotient_check")
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fopenmp",
                    "-I", os.path.join(ROOT, "oracle"),
                    "-o", exe, os.path.join(ROOT, "tests", "fast_quotient_check.c"),
                    os.path.join(ROOT, "oracle", "kv_oracle.c"), "-lm"], check=True)
    return exe


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_fast_quotient_matches_ieee_division(checker, fmt):
    r = subprocess.run([checker, fmt], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    checked, bad = [int(t) for t in r.stdout.split() if t.isdigit()]
    assert checked == 817512960 and bad == 0


def test_cachegen_unit_matches_ieee_division(tmp_path):
    # the CacheGen dequantiser's (q - MAX) / MAX: reciprocal product plus one
    # Markstein correction equals the IEEE quotient for every MAX and symbol
    exe = str(tmp_path / "cachegen_unit_check")
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-o", exe,
                    os.path.join(ROOT, "tests", "cachegen_unit_check.c"), "-lm"], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    checked, bad = [int(t) for t in r.stdout.split() if t.isdigit()]
    assert checked == sum(2 * m + 1 for m in range(1, 64)) and bad == 0
