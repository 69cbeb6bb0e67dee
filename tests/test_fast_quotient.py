"""The fp8 store kernels replace x / scale by x * (1/scale) plus one fused
multiply-add correction when the group maximum is a finite bf16 value
>= 2^-4.  This checks, exhaustively over every such (amax, x) bf16 pair, that
the e4m3 code is the one the oracle gives for the IEEE quotient (CPU only)."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_fast_quotient_matches_ieee_division_in_e4m3(tmp_path):
    exe = str(tmp_path / "fast_quotient_check")
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fopenmp",
                    "-I", os.path.join(ROOT, "oracle"),
                    "-o", exe, os.path.join(ROOT, "tests", "fast_quotient_check.c"),
                    os.path.join(ROOT, "oracle", "kv_oracle.c"), "-lm"], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    checked, bad = [int(t) for t in r.stdout.split() if t.isdigit()]
    assert checked == 817512960 and bad == 0
