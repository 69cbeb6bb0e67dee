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


def test_cachegen_fast_symbol_domain_and_rounding():
    # The CacheGen store takes a shortcut for rows whose max1 and factor are
    # finite: no clamp and no NaN test, and round-half-to-even by adding
    # 1.5 * 2^23.  (1) Over every MAX in [1, 63] and every finite positive
    # bf16 max1 with a finite factor, the extreme elements x = +-max1 give
    # y = x * factor + MAX (two float32 roundings) inside (-0.5, 2 * MAX + 0.5),
    # so every symbol of the row already lies in [0, 2 * MAX]; y is monotonic
    # in x, so the extremes bound the row.  (2) The low byte of
    # bits(y + 1.5 * 2^23) equals numpy's round-half-to-even of y for every
    # float32 y in [2^-3, 128) and for sampled y in (-0.5, 2^-3).
    import numpy as np
    m = np.arange(1, 0x7F80, dtype=np.uint32)
    max1 = (m << 16).view(np.float32)
    for MAX in range(1, 64):
        q = np.float32(MAX)
        with np.errstate(over="ignore"):
            factor = q / max1
        ok = np.isfinite(factor)
        f, x = factor[ok], max1[ok]
        y_hi = (x * f).astype(np.float32) + q
        y_lo = (-x * f).astype(np.float32) + q
        assert y_hi.dtype == np.float32 and y_lo.dtype == np.float32
        assert (y_lo > -0.5).all() and (y_hi < 2 * MAX + 0.5).all(), MAX
    magic = np.float32(12582912.0)
    for e in range(-3, 7):                                   # binades [2^e, 2^(e+1)) up to 128
        lo = np.float32(2.0 ** e).view(np.uint32)
        y = np.arange(lo, lo + (1 << 23), dtype=np.uint32).view(np.float32)
        got = ((y + magic).view(np.uint32) & 0xFF).astype(np.int64)
        assert np.array_equal(got, np.rint(y).astype(np.int64) & 0xFF), e
    rng = np.random.default_rng(5)
    y = rng.uniform(-0.5, 0.125, 4_000_000).astype(np.float32)
    y = y[y > -0.5]
    got = ((y + magic).view(np.uint32) & 0xFF).astype(np.int64)
    assert np.array_equal(got, np.rint(y).astype(np.int64) & 0xFF)
