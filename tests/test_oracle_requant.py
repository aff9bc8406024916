"""Pins of the oracle's requantizer (saved 1x128 codes -> transposed 128x1 tiles).

Independent references used here:
- a PyTorch composition from library primitives: torch's float8_e4m3fn view
  decodes the codes, an fp32 tensor product dequantizes, torch.amax and an
  fp32 division give the scales and torch's float8 cast encodes (within a tile
  |d / st| <= 448 * (1 + 2^-23) < 464, where torch's cast saturates like the
  rule);
- a special case that reduces to the already pinned bf16 quantizer: with
  power-of-two scales every dequantized value is exact in bf16, so the result
  must equal the transposed 128x1 quantization of those bf16 values;
- closed forms: unit scales with a +-448 code in every 128-row column tile
  give st = 1 and qt = q transposed; an all-zero tile has scale 1 and keeps
  zero signs; |qt| <= 448 and every nonzero tile reaches 448;
- a per-element Python loop on a tiny ragged case;
- the error bound of two successive quantizations of a bf16 activation.
"""
import numpy as np
import pytest
import torch

from workloads import bits, random_bf16, random_codes, random_scales

TILE = 128


def cdiv(a, b):
    return (a + b - 1) // b


def torch_requant(q: np.ndarray, s: np.ndarray):
    """Library-primitive composition: decode, dequantize in fp32, 128x1 tiles of the transpose."""
    R, C = q.shape
    dec = torch.from_numpy(q).view(torch.float8_e4m3fn).float()          # [R][C]
    sc = torch.from_numpy(s).T.repeat_interleave(TILE, dim=1)[:, :C]      # [R][C], s[c // 128][r]
    d = (dec * sc).T.contiguous()                                         # fp32 product, [C][R]
    ni = cdiv(R, TILE)
    dp = torch.zeros((C, ni * TILE), dtype=torch.float32)
    dp[:, :R] = d
    tiles = dp.reshape(C * ni, TILE)
    amax = tiles.abs().amax(dim=1)
    st = torch.where(amax == 0, torch.ones_like(amax), amax / torch.tensor(448.0, dtype=torch.float32))
    qt = (tiles / st[:, None]).to(torch.float8_e4m3fn).view(torch.uint8)
    qt = qt.reshape(C, ni * TILE)[:, :R].numpy()
    return qt, st.reshape(C, ni).T.contiguous().numpy()


def assert_same(got, want):
    qt, st = got
    tq, ts = want
    assert qt.shape == tq.shape and st.shape == ts.shape
    bad = np.argwhere(qt != tq)
    assert bad.size == 0, "%d code mismatches, first at %s" % (len(bad), tuple(bad[0]))
    assert np.array_equal(st.view(np.uint32), ts.view(np.uint32))


@pytest.mark.parametrize("R,C", [(256, 256), (300, 400), (128, 16), (1, 128), (1040, 48)])
def test_random_codes_and_scales_match_torch_composition(orc, R, C):
    q = random_codes((R, C), 100 + R)
    s = random_scales((cdiv(C, TILE), R), 200 + C)
    got = orc.requant_act_t(q, s)
    assert got[0].shape == (C, R) and got[1].shape == (cdiv(R, TILE), C)
    assert_same(got, torch_requant(q, s))


@pytest.mark.parametrize("R,C", [(512, 384), (200, 272)])
def test_saved_activation_codes_match_torch_composition(orc, R, C):
    """The use: codes and scales as the 1x128 quantizer saved them."""
    x = random_bf16((R, C), 3 + R).float()
    x[:, torch.randperm(C, generator=torch.Generator().manual_seed(R))[:3]] *= 20
    q, s = orc.quant_act_1x128(bits(x.to(torch.bfloat16)))
    assert_same(orc.requant_act_t(q, s), torch_requant(q, s))


def test_tiny_scales_and_subnormal_products(orc):
    """Scales near and below the fp32 normal range: products round to fp32 subnormals."""
    R, C = 256, 128
    q = random_codes((R, C), 7)
    s = random_scales((1, R), 8, log2_lo=-140.0, log2_hi=-118.0)
    assert_same(orc.requant_act_t(q, s), torch_requant(q, s))


@pytest.mark.parametrize("R,C", [(256, 256), (384, 144)])
def test_power_of_two_scales_reduce_to_bf16_transposed_quantizer(orc, R, C):
    q = random_codes((R, C), 11 + R)
    k = torch.randint(-20, 11, (cdiv(C, TILE), R), generator=torch.Generator().manual_seed(C)).numpy()
    s = np.ldexp(np.float32(1.0), k).astype(np.float32)
    dec = orc.e4m3_decode_table()[q]                                     # fp64, exact
    d = dec * np.ldexp(1.0, k.T.repeat(TILE, axis=1)[:, :C])             # exact in fp64
    xb = torch.from_numpy(d.astype(np.float32)).to(torch.bfloat16)
    assert np.array_equal(xb.double().numpy(), d)                        # 4 significant bits: exact in bf16
    assert_same(orc.requant_act_t(q, s), orc.quant_act_128x1_t(bits(xb)))


@pytest.mark.parametrize("R,C", [(256, 384), (200, 144)])
def test_unit_scales_with_full_tiles_transpose_the_codes(orc, R, C):
    q = random_codes((R, C), 17 + R)
    for i in range(cdiv(R, TILE)):
        q[i * TILE, :] = np.where(np.arange(C) % 2 == 0, 0x7E, 0xFE)       # one +-448 per column tile
    s = np.ones((cdiv(C, TILE), R), dtype=np.float32)
    qt, st = orc.requant_act_t(q, s)
    assert np.all(st == 1.0)
    assert np.array_equal(qt, q.T)


def test_invariants_zero_tiles_and_signs(orc):
    R, C = 300, 256
    q = random_codes((R, C), 23)
    q[128:256, 5] = 0x00
    q[128:256:2, 5] = 0x80                                                # a tile of +-0 only
    s = random_scales((cdiv(C, TILE), R), 24)
    qt, st = orc.requant_act_t(q, s)
    assert st[1, 5] == 1.0
    assert np.array_equal(qt[5, 128:256], q[128:256, 5])
    mag = qt & 0x7F
    assert mag.max() <= 0x7E
    nz = (q & 0x7F) != 0
    for c in range(C):
        for i in range(cdiv(R, TILE)):
            if nz[i * TILE:(i + 1) * TILE, c].any():
                assert mag[c, i * TILE:(i + 1) * TILE].max() == 0x7E, (c, i)


def test_python_loop_tiny_ragged(orc):
    R, C = 131, 144
    q = random_codes((R, C), 31)
    s = random_scales((cdiv(C, TILE), R), 32)
    qt, st = orc.requant_act_t(q, s)
    table = orc.e4m3_decode_table()
    for c in range(C):
        for i in range(cdiv(R, TILE)):
            rows = range(i * TILE, min(R, (i + 1) * TILE))
            d = [np.float32(np.float32(table[q[r, c]]) * s[c // TILE, r]) for r in rows]
            amax = max(abs(v) for v in d)
            sc = np.float32(1.0) if amax == 0 else np.float32(amax) / np.float32(448.0)
            assert st[i, c].view(np.uint32) == np.float32(sc).view(np.uint32)
            for r, v in zip(rows, d):
                want = torch.tensor([np.float32(v) / sc], dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).item()
                assert qt[c, r] == want, (r, c)


def test_two_quantizations_stay_within_error_bound(orc):
    """x -> 1x128 codes -> requantized 128x1 codes: each step moves an element by at
    most half an e4m3 spacing (2^-4 relative, or 2^-10 * scale in the subnormal range)."""
    R, C = 384, 256
    xb = random_bf16((R, C), 41)
    x = xb.double().numpy()
    q, s = orc.quant_act_1x128(bits(xb))
    qt, st = orc.requant_act_t(q, s)
    table = orc.e4m3_decode_table()
    s_el = s.T.repeat(TILE, axis=1)[:, :C].astype(np.float64)
    d = table[q] * s_el
    y = (table[qt] * st.T.repeat(TILE, axis=1)[:, :R].astype(np.float64)).T
    st_el = st.repeat(TILE, axis=0)[:R, :].astype(np.float64)
    b1 = 2.0 ** -4 * np.abs(x) + 2.0 ** -10 * s_el
    b2 = 2.0 ** -4 * np.abs(d) + 2.0 ** -10 * st_el
    slack = 1 + 1e-6
    assert np.all(np.abs(d - x) <= b1 * slack)
    assert np.all(np.abs(y - d) <= b2 * slack)
    assert np.all(np.abs(y - x) <= (b1 + b2) * slack)
