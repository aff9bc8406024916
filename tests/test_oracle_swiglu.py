"""Pins of the oracle's SwiGLU (the down projection's input, rounded to bf16).

The definition: h = bf16(fp64(g / (1 + exp(-g)) * u)), one rounding.
Independent references used here:
- 50-digit arithmetic (mpmath): h must be the correctly rounded bf16 of the
  exact value, for every finite bf16 gate value (u = 1, which makes h the
  bf16 rounding of silu itself) and for random and hand-picked (g, u) pairs
  spanning normal, subnormal and underflowing results -- except where the
  exact value lies within 2^-50 of a bf16 rounding midpoint, which fp64
  cannot resolve; every such exception must then be the rounding of the fp64
  value and sit that close to a midpoint;
- closed forms: silu(0) = 0 (the zero takes the sign of g * u), silu(g) = g
  to within 2^-1000 for g >= 1000, silu(g) * u rounds to a zero of u's
  negated sign for g <= -1000;
- PyTorch's fp32 silu (a different precision: it may differ only in the
  last bf16 place, and only rarely) and its chunk convention for the
  gate/up halves.
"""
import mpmath
import numpy as np
import pytest
import torch

from workloads import bits

mpmath.mp.dps = 50


def bf16_to_mpf(b: int):
    return mpmath.mpf(float(np.uint32(b << 16).view(np.float32)))


def mp_to_bf16(v) -> int:
    """Round-to-nearest-even bf16 bits of an mpf value (ties cannot occur for these values)."""
    if v == 0:
        return 0x8000 if mpmath.sign(v) < 0 else 0
    sign = 0x8000 if v < 0 else 0
    a = abs(v)
    e = int(mpmath.floor(mpmath.log(a, 2)))
    if a >= mpmath.ldexp(1, e + 1):            # guard the log against rounding
        e += 1
    elif a < mpmath.ldexp(1, e):
        e -= 1
    if e < -126:
        n = int(mpmath.nint(a * mpmath.ldexp(1, 133)))
        return sign | n                           # 128 = the smallest normal, encoded the same way
    n = int(mpmath.nint(a * mpmath.ldexp(1, 7 - e)))
    if n == 256:
        e, n = e + 1, 128
    if e > 127:
        return sign | 0x7F80
    return sign | ((e + 127) << 7) | (n - 128)


def mp_value(g: int, u: int):
    gm, um = bf16_to_mpf(g), bf16_to_mpf(u)
    return gm / (1 + mpmath.exp(-gm)) * um


def mp_swiglu(g: int, u: int) -> int:
    gm, um = bf16_to_mpf(g), bf16_to_mpf(u)
    if gm == 0 or um == 0:
        neg = (g >> 15) ^ (u >> 15)
        return 0x8000 if neg else 0
    return mp_to_bf16(mp_value(g, u))


def midpoint_distance(v) -> float:
    """Relative distance of an mpf value to the nearest bf16 rounding midpoint."""
    a = abs(v)
    e = int(mpmath.floor(mpmath.log(a, 2)))
    grid = mpmath.ldexp(1, max(e, -126) - 7)
    frac = a / grid - mpmath.floor(a / grid)
    return float(abs(frac - mpmath.mpf(0.5)) * grid / a)


def fp64_swiglu(g: int, u: int) -> float:
    gd = float(np.uint32(g << 16).view(np.float32))
    ud = float(np.uint32(u << 16).view(np.float32))
    return gd / (1.0 + np.exp(-gd)) * ud


def check_against_exact(orc, g, u, h):
    """Every disagreement with exact arithmetic must be the fp64 rounding of a value within
    2^-50 of a midpoint, with a gate where fp64 sees silu(g) as exactly g/2 (|g| < 2^-50)
    or exactly g (g > 36, where exp(-g) < 2^-52): the systematic classes."""
    want = np.array([mp_swiglu(int(a), int(b)) for a, b in zip(g, u)], dtype=np.uint16)
    bad = np.flatnonzero(h != want)
    for i in bad:
        v = mp_value(int(g[i]), int(u[i]))
        assert midpoint_distance(v) < 2.0 ** -50, (hex(g[i]), hex(u[i]), hex(h[i]), hex(want[i]))
        assert h[i] == orc.f64_to_bf16(fp64_swiglu(int(g[i]), int(u[i])))
        gv = float(np.uint32(int(g[i]) << 16).view(np.float32))
        assert abs(gv) < 2.0 ** -50 or gv > 36.0, gv
    return len(bad)


def finite_bf16():
    b = np.arange(0x10000, dtype=np.uint32)
    return b[((b >> 7) & 0xFF) != 0xFF]


def test_every_bf16_gate_gives_the_correctly_rounded_silu(orc):
    g = finite_bf16()
    gu = np.stack([g.astype(np.uint16), np.full(len(g), 0x3F80, dtype=np.uint16)], axis=1)   # u = 1
    h = orc.swiglu(gu.reshape(len(g), 2))[:, 0]
    n_bad = check_against_exact(orc, g, np.full(len(g), 0x3F80), h)
    # the only exceptions: the smallest gates, where g/2 falls on a subnormal bf16 midpoint
    assert n_bad == 128


def test_random_and_edge_pairs_against_50_digit_arithmetic(orc):
    rng = np.random.default_rng(7)
    # random normal-ish activations and a spread of magnitudes
    g = bits(torch.from_numpy(rng.standard_normal(6000).astype(np.float32) * 3).to(torch.bfloat16)).ravel()
    u = bits(torch.from_numpy(rng.standard_normal(6000).astype(np.float32)).to(torch.bfloat16)).ravel()
    # edge pairs: large |g|, tiny u (subnormal results), tiny g, huge u
    edge_g = np.array([0x42C8, 0xC2C8, 0xC2B4, 0xC2A0, 0x4480, 0xC480, 0x0001, 0x8001, 0x0080, 0x1F00, 0x5F00, 0xDF00,
                       0xC2B0, 0xC2AC, 0xC2A8, 0xC1F0, 0x41F0], dtype=np.uint16)
    edge_u = np.array([0x3C23, 0x3C23, 0x2000, 0x0010, 0x3F80, 0x3F80, 0x3F80, 0xBF80, 0x4000, 0x5F00, 0x1F00, 0x3F80,
                       0x3A83, 0xBA83, 0x0100, 0x3F80, 0xBF80], dtype=np.uint16)
    g = np.concatenate([g, edge_g, rng.integers(0, 0x7F80, 3000).astype(np.uint16)])
    u = np.concatenate([u, edge_u, rng.integers(0, 0x7F80, 3000).astype(np.uint16) | (rng.integers(0, 2, 3000) << 15).astype(np.uint16)])
    gu = np.stack([g, u], axis=1).astype(np.uint16)
    h = orc.swiglu(gu)[:, 0]
    assert check_against_exact(orc, g, u, h) < 20


def test_closed_forms(orc):
    # zero gate: the zero's sign is that of g * u
    assert orc.swiglu_value(0x0000, 0x3F80) == 0x0000
    assert orc.swiglu_value(0x8000, 0x3F80) == 0x8000
    assert orc.swiglu_value(0x0000, 0xBF80) == 0x8000
    assert orc.swiglu_value(0x8000, 0xBF80) == 0x0000
    # large positive gate: silu(g) = g, so h = bf16(g * u)
    rng = np.random.default_rng(3)
    for _ in range(200):
        gv = float(rng.uniform(1000, 1e5))
        uv = float(rng.standard_normal())
        gb = int(bits(torch.tensor([gv]).to(torch.bfloat16))[0])
        ub = int(bits(torch.tensor([uv]).to(torch.bfloat16))[0])
        exact = float(np.uint32(gb << 16).view(np.float32)) * float(np.uint32(ub << 16).view(np.float32))
        assert orc.swiglu_value(gb, ub) == orc.f64_to_bf16(exact)
    # large negative gate: silu(g) * u underflows to a zero of sign -sign(u)
    assert orc.swiglu_value(0xC47A, 0x3F80) == 0x8000        # g = -1000
    assert orc.swiglu_value(0xC47A, 0xBF80) == 0x0000


def test_gate_is_the_first_half_and_torch_fp32_agrees(orc):
    rng = np.random.default_rng(11)
    R, I = 64, 384
    gu32 = torch.from_numpy(rng.standard_normal((R, 2 * I)).astype(np.float32) * 2)
    gub = gu32.to(torch.bfloat16)
    h = orc.swiglu(bits(gub))
    g, u = torch.chunk(gub.float(), 2, dim=-1)
    ref = bits((torch.nn.functional.silu(g) * u).to(torch.bfloat16))
    diff = h.astype(np.int32) - ref.astype(np.int32)
    assert np.abs(diff).max() <= 1                           # fp32 torch may differ in the last place
    assert np.mean(diff != 0) < 2e-3
    hs = orc.swiglu(bits(torch.cat([torch.chunk(gub, 2, -1)[1], torch.chunk(gub, 2, -1)[0]], dim=-1)))
    assert not np.array_equal(hs, h)                         # swapping the halves changes the result


def test_swiglu_quant_composes_the_pinned_quantizers(orc):
    rng = np.random.default_rng(5)
    gub = torch.from_numpy(rng.standard_normal((256, 2 * 272)).astype(np.float32)).to(torch.bfloat16)
    h, q, s, qt, st = orc.swiglu_quant(bits(gub), dual=True)
    q2, s2 = orc.quant_act_1x128(h)
    qt2, st2 = orc.quant_act_128x1_t(h)
    assert np.array_equal(q, q2) and np.array_equal(s, s2)
    assert np.array_equal(qt, qt2) and np.array_equal(st, st2)
