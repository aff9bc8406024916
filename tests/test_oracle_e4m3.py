"""Pins of the oracle's e4m3 codec against things other than itself.

- PyTorch's CPU float8_e4m3fn cast is an independent implementation of OCP
  E4M3FN with round-to-nearest-even; inside [-448, 448] saturation never
  triggers, so it must agree with the oracle on every fp32 bit pattern there.
- The OCP OFP8 specification's E4M3 table (tests/golden/e4m3_ocp_facts.txt).
- Round trips, midpoint ties, monotonicity and saturation, which follow from
  the definition of a saturating RNE cast.
"""
import math
import os

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def torch_e4m3(f: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(f, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_encode_matches_torch_on_every_fp32_in_range(orc):
    """All 2 x 1,138,753,537 fp32 bit patterns with |f| <= 448 (both signs)."""
    hi = int(np.float32(448.0).view(np.uint32))
    chunk = 1 << 26
    for sign in (0, 0x80000000):
        start = 0
        while start <= hi:
            stop = min(start + chunk, hi + 1)
            bits = np.arange(start, stop, dtype=np.uint32) | np.uint32(sign)
            f = bits.view(np.float32)
            q = orc.e4m3_encode_array(f)
            ref = torch_e4m3(f)
            bad = np.nonzero(q != ref)[0]
            assert bad.size == 0, "first mismatch at fp32 bits 0x%08x: oracle 0x%02x torch 0x%02x" % (
                bits[bad[0]], q[bad[0]], ref[bad[0]])
            start = stop


def test_decode_matches_ocp_table(orc):
    with open(os.path.join(GOLDEN, "e4m3_ocp_facts.txt")) as fh:
        rows = [ln.split()[:2] for ln in fh if ln.strip() and not ln.startswith("#")]
    assert len(rows) == 10
    for code, val in rows:
        got = orc.e4m3_decode(int(code, 16))
        if val == "nan":
            assert math.isnan(got)
        else:
            assert got == float(val), code
            assert math.copysign(1.0, got) == math.copysign(1.0, float(val)), code


def test_decode_table_matches_torch(orc):
    table = orc.e4m3_decode_table()
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(table), nan)
    assert np.array_equal(table[~nan], ref[~nan])
    assert np.array_equal(np.signbit(table[~nan]), np.signbit(ref[~nan]))


def test_roundtrip_every_finite_code(orc):
    for c in range(256):
        if c & 0x7F == 0x7F:
            continue
        assert orc.e4m3_encode(orc.e4m3_decode(c)) == c, hex(c)


def test_midpoints_round_to_even(orc):
    vals = [orc.e4m3_decode(c) for c in range(0x7F)]          # 0 .. 448, increasing
    for c in range(0x7E):
        lo, hi = vals[c], vals[c + 1]
        mid = (lo + hi) / 2                                     # exact in fp32 (one more bit)
        assert np.float32(mid) == mid
        even = c if c % 2 == 0 else c + 1
        assert orc.e4m3_encode(mid) == even, (c, mid)
        assert orc.e4m3_encode(-mid) == even | 0x80
        below = float(np.nextafter(np.float32(mid), np.float32(0)))
        above = float(np.nextafter(np.float32(mid), np.float32(np.inf)))
        assert orc.e4m3_encode(below) == c
        assert orc.e4m3_encode(above) == c + 1


def test_monotonic_nondecreasing(orc):
    rng = np.random.default_rng(1)
    f = np.sort(rng.uniform(0, 460, 200000).astype(np.float32))
    q = orc.e4m3_encode_array(f).astype(np.int32)
    assert np.all(np.diff(q) >= 0)


def test_saturation_and_special_values(orc):
    for v in (448.0, 448.00003, 460.0, 463.99997, 464.0, 465.0, 480.0, 1e6, 3.4e38, math.inf):
        assert orc.e4m3_encode(v) == 0x7E, v
        assert orc.e4m3_encode(-v) == 0xFE, v
    assert orc.e4m3_encode(math.nan) == 0x7F
    assert orc.e4m3_encode(0.0) == 0x00
    assert orc.e4m3_encode(-0.0) == 0x80
    assert orc.e4m3_encode(-1e-5) == 0x80          # rounds to zero, keeps the sign
    assert orc.e4m3_encode(2.0 ** -10) == 0x00      # half the smallest subnormal: tie to even (0)
    assert orc.e4m3_encode(1.5 * 2.0 ** -9) == 0x02  # tie between 1 and 2: even
    assert orc.e4m3_encode(2.5 * 2.0 ** -9) == 0x02
    assert orc.e4m3_encode(3.5 * 2.0 ** -9) == 0x04
    assert orc.e4m3_encode(7.5 * 2.0 ** -9) == 0x08  # rounds up into the smallest normal
    assert orc.e4m3_encode(300.0) == 0x79           # 300 * 2^-5 = 9.375 -> 9 -> 288


def test_bf16_widening(orc):
    for h in (0x0000, 0x8000, 0x3F80, 0xBF80, 0x7F7F, 0x0001, 0x807F):
        assert orc.bf16_to_f32(h) == float(torch.tensor([h], dtype=torch.int32).to(torch.int16).view(torch.bfloat16).float())
