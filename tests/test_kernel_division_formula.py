"""The quantizer kernels replace the per-element IEEE division x / s by a
reciprocal and one residual correction (Markstein's step).  This test replays
that formulation on the host over every pair of bf16 values (x, amax) the
kernels can see with the fast path enabled, and checks that the resulting
e4m3 code always equals the one of the IEEE quotient (see
tests/csrc/quotient_check.c).  Host logic only: no GPU, no oracle code."""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.slow
def test_reciprocal_division_gives_ieee_quotient_codes(tmp_path):
    exe = str(tmp_path / "quotient_check")
    subprocess.run(["gcc", "-std=c99", "-O2", "-fopenmp", "-ffp-contract=off",
                    os.path.join(HERE, "csrc", "quotient_check.c"), "-o", exe, "-lm"], check=True)
    out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout.split()
    pairs, bad = int(out[0]), int(out[1])
    assert pairs > 1_000_000_000
    assert bad == 0


@pytest.mark.slow
def test_requantizer_division_is_the_ieee_quotient(tmp_path):
    """The requantizer divides arbitrary fp32 values (dequantized codes) by a
    column scale with a two-word reciprocal and one residual correction; see
    tests/csrc/requant_quotient_check.c for the argument and what is replayed."""
    exe = str(tmp_path / "requant_quotient_check")
    subprocess.run(["gcc", "-std=c99", "-O2", "-fopenmp", "-ffp-contract=off",
                    os.path.join(HERE, "csrc", "requant_quotient_check.c"), "-o", exe, "-lm"], check=True)
    out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout.split()
    pairs, bad = int(out[0]), int(out[1])
    assert pairs > 4_000_000_000
    assert bad == 0
