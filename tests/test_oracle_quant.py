"""Pins of the oracle's tile quantizers.

Independent references used here:
- a PyTorch implementation built from library primitives (amax via
  torch.amax, fp32 division, torch's float8_e4m3fn cast), which shares
  nothing with oracle.c; within a tile |x / s| <= 448 * (1 + 2^-23) < 464, so
  torch's non-saturating cast is the saturating RNE cast there;
- closed-form invariants of the rule s = amax/448, q = e4m3(x/s):
  exactly representable tiles round-trip, |q| <= 448, every nonzero tile
  reaches 448, an all-zero tile has s = 1, power-of-two equivariance;
- brute force over every finite bf16 value under a range of tile maxima;
- the transposed quantizers against the row quantizer of the materialized
  transpose.
"""
import numpy as np
import pytest
import torch

from workloads import bits, random_bf16

TILE = 128


def cdiv(a, b):
    return (a + b - 1) // b


def torch_quant_tiles(x32: torch.Tensor):
    """x32: [T][L] fp32 tiles (zero-padded rows of length <= 128) -> (codes, scales) via torch."""
    amax = x32.abs().amax(dim=1)
    s = torch.where(amax == 0, torch.ones_like(amax), amax / torch.tensor(448.0, dtype=torch.float32))
    q = (x32 / s[:, None]).to(torch.float8_e4m3fn).view(torch.uint8)
    return q, s


def torch_quant_act(xb: torch.Tensor):
    R, C = xb.shape
    x = xb.float()
    nj = cdiv(C, TILE)
    xp = torch.zeros((R, nj * TILE), dtype=torch.float32)
    xp[:, :C] = x
    q, s = torch_quant_tiles(xp.reshape(R * nj, TILE))
    return q.reshape(R, nj * TILE)[:, :C].numpy(), s.reshape(R, nj).T.contiguous().numpy()


def torch_quant_w(wb: torch.Tensor):
    R, C = wb.shape
    ni, nj = cdiv(R, TILE), cdiv(C, TILE)
    xp = torch.zeros((ni * TILE, nj * TILE), dtype=torch.float32)
    xp[:R, :C] = wb.float()
    blocks = xp.reshape(ni, TILE, nj, TILE).permute(0, 2, 1, 3).reshape(ni * nj, TILE * TILE)
    q, s = torch_quant_tiles(blocks)
    q = q.reshape(ni, nj, TILE, TILE).permute(0, 2, 1, 3).reshape(ni * TILE, nj * TILE)[:R, :C]
    return q.numpy(), s.reshape(ni, nj).numpy()


def outlier_input(R, C, seed, n_out=3):
    x = random_bf16((R, C), seed).float()
    g = torch.Generator().manual_seed(seed + 1)
    cols = torch.randperm(C, generator=g)[:n_out]
    x[:, cols] *= 20
    return x.to(torch.bfloat16)


@pytest.mark.parametrize("R,C", [(256, 256), (37, 400), (130, 16), (1, 128), (64, 1040)])
def test_act_1x128_matches_torch_composition(orc, R, C):
    xb = outlier_input(R, C, R * 1000 + C)
    q, s = orc.quant_act_1x128(bits(xb))
    tq, ts = torch_quant_act(xb)
    assert s.shape == (cdiv(C, TILE), R)
    assert np.array_equal(q, tq)
    assert np.array_equal(s.view(np.uint32), ts.view(np.uint32))


@pytest.mark.parametrize("R,C", [(512, 256), (200, 336), (128, 128), (17, 48)])
def test_w_128x128_matches_torch_composition(orc, R, C):
    wb = random_bf16((R, C), 7 + R, std=0.02)
    q, s = orc.quant_w_128x128(bits(wb))
    tq, ts = torch_quant_w(wb)
    assert s.shape == (cdiv(R, TILE), cdiv(C, TILE))
    assert np.array_equal(q, tq)
    assert np.array_equal(s.view(np.uint32), ts.view(np.uint32))


@pytest.mark.parametrize("R,C", [(256, 384), (144, 80), (16, 16)])
def test_transposed_act_is_row_quant_of_transpose(orc, R, C):
    xb = outlier_input(R, C, 5 + R)
    qt, st = orc.quant_act_128x1_t(bits(xb))
    q2, s2 = orc.quant_act_1x128(bits(xb.T.contiguous()))
    assert qt.shape == (C, R) and st.shape == (cdiv(R, TILE), C)
    assert np.array_equal(qt, q2)
    assert np.array_equal(st.view(np.uint32), s2.view(np.uint32))


@pytest.mark.parametrize("R,C", [(256, 384), (200, 144)])
def test_transposed_w_is_transpose_of_w(orc, R, C):
    wb = random_bf16((R, C), 11 + C, std=0.02)
    qt, st = orc.quant_w_128x128_t(bits(wb))
    q, s = orc.quant_w_128x128(bits(wb))
    assert np.array_equal(qt, q.T)
    assert np.array_equal(st, s.T)


def e4m3_values(orc):
    """All finite non-negative e4m3 values and their codes."""
    codes = np.arange(0x7F)
    return np.array([orc.e4m3_decode(int(c)) for c in codes]), codes


@pytest.mark.parametrize("j", [0, -3, 5, -40, -60])
def test_exactly_representable_tile_round_trips(orc, j):
    """x = v * 2^j, v e4m3-representable, max |v| = 448: s = 2^j exactly, dec(q) * s == x."""
    vals, codes = e4m3_values(orc)
    rng = np.random.default_rng(abs(j) + 3)
    idx = rng.integers(0, len(vals), size=(4, TILE))
    idx[:, 0] = 0x7E
    sign = rng.integers(0, 2, size=idx.shape)
    v = np.where(sign == 1, -vals[idx], vals[idx]) * 2.0 ** j
    xb = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16)
    assert np.array_equal(xb.double().numpy(), v)           # exact in bf16 (3 mantissa bits)
    q, s = orc.quant_act_1x128(bits(xb))
    assert np.all(s == np.float32(2.0 ** j))
    dq = orc.e4m3_decode_table()[q] * float(2.0 ** j)
    assert np.array_equal(dq, v)


def test_codes_bounded_and_tile_max_reaches_448(orc):
    xb = outlier_input(96, 1024, 42)
    q, s = orc.quant_act_1x128(bits(xb))
    mag = q & 0x7F
    assert mag.max() <= 0x7E
    assert np.all(mag.reshape(96, 8, TILE).max(axis=2) == 0x7E)
    wb = random_bf16((256, 384), 9, std=0.02)
    qw, _ = orc.quant_w_128x128(bits(wb))
    assert np.all((qw & 0x7F).reshape(2, TILE, 3, TILE).max(axis=(1, 3)) == 0x7E)


def test_all_zero_tile_has_scale_one_and_keeps_zero_signs(orc):
    x = np.zeros((2, 256), dtype=np.uint16)
    x[0, 1::2] = 0x8000                       # -0.0
    x[1, 128:] = 0x3F80                       # second tile of row 1 is all ones
    q, s = orc.quant_act_1x128(x)
    assert s[0, 0] == 1.0 and s[1, 0] == 1.0 and s[0, 1] == 1.0
    assert s[1, 1] == np.float32(1.0) / np.float32(448.0)
    assert np.all(q[0, 0::2] == 0x00) and np.all(q[0, 1::2] == 0x80)
    assert np.all(q[1, :128] == 0x00) and np.all(q[1, 128:] == 0x7E)
    qw, sw = orc.quant_w_128x128(np.zeros((128, 128), dtype=np.uint16))
    assert sw[0, 0] == 1.0 and np.all(qw == 0)


@pytest.mark.parametrize("j", [1, 7, -9, 30])
def test_power_of_two_equivariance(orc, j):
    xb = outlier_input(64, 512, 77)
    x2 = (xb.double() * 2.0 ** j).to(torch.bfloat16)
    assert np.array_equal(x2.double().numpy(), xb.double().numpy() * 2.0 ** j)   # exact
    q1, s1 = orc.quant_act_1x128(bits(xb))
    q2, s2 = orc.quant_act_1x128(bits(x2))
    assert np.array_equal(q1, q2)
    assert np.array_equal(s2, s1 * np.float32(2.0 ** j))


def test_brute_force_all_bf16_values_under_many_scales(orc):
    """Every finite bf16 magnitude <= amax, both signs, in tiles whose first element is amax."""
    all_bits = np.arange(0, 0x7F80, dtype=np.uint32)                 # finite non-negative bf16
    allf = (all_bits << 16).view(np.float32)
    rng = np.random.default_rng(5)
    amax_bits = np.unique(np.concatenate([rng.integers(1, 0x7F80, 40), [0x3F80, 0x43E0, 0x0001, 0x0080, 0x7F7F, 0x1F00]]))
    for ab in amax_bits:
        amax = np.float32((np.uint32(ab) << 16).view(np.float32))
        mags = all_bits[allf <= amax]
        vals = np.concatenate([mags, mags | 0x8000]).astype(np.uint16)
        ntiles = cdiv(len(vals), TILE - 1)
        pad = np.zeros(ntiles * (TILE - 1), dtype=np.uint16)
        pad[:len(vals)] = vals
        tiles = np.empty((ntiles, TILE), dtype=np.uint16)
        tiles[:, 0] = ab
        tiles[:, 1:] = pad.reshape(ntiles, TILE - 1)
        q, s = orc.quant_act_1x128(tiles)
        sref = np.float32(amax) / np.float32(448.0)
        assert np.all(s == sref)
        x32 = (tiles.astype(np.uint32) << 16).view(np.float32)
        ref = torch_e4m3(x32 / sref)
        assert np.array_equal(q, ref), hex(ab)


def torch_e4m3(f):
    return torch.from_numpy(np.ascontiguousarray(f, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
