"""GPU parity of the requantizer (saved 1x128 codes -> transposed 128x1 tiles):
codes and scales bit-exact against the oracle.  The input codes are drawn at
random or made by the oracle's 1x128 quantizer; none comes from the GPU."""
import numpy as np
import pytest
import torch

from helpers import assert_codes_equal, assert_scales_equal, cdiv, to_np, TILE
from workloads import bits, make, random_bf16, random_codes, random_scales

pytestmark = pytest.mark.gpu

puro = pytest.importorskip("blockwise_fp8_gemm_act_amd")


def check(orc, q: np.ndarray, s: np.ndarray):
    qt, st = puro.requant_act_t(torch.from_numpy(q).cuda(), torch.from_numpy(s).cuda())
    torch.cuda.synchronize()
    oqt, ost = orc.requant_act_t(q, s)
    assert_codes_equal(to_np(qt), oqt, "requantized codes")
    assert_scales_equal(to_np(st), ost, "requantized scales")


def saved_codes(orc, xb):
    return orc.quant_act_1x128(bits(xb))


def special_saved_input(R, C, seed):
    """Activation with an all-zero tile, an all -0 tile, a row of tiny normal
    values (scales near 2^-70), a row of 448s and three outlier channels."""
    x = random_bf16((R, C), seed).float()
    x[:, torch.randperm(C, generator=torch.Generator().manual_seed(seed))[:3]] *= 20
    xb = bits(x.to(torch.bfloat16)).copy()
    rng = np.random.default_rng(seed)
    xb[0, :min(C, 128)] = 0
    xb[1, :min(C, 128)] = 0x8000
    xb[2, :] = rng.integers(0x0080, 0x1F00, C, dtype=np.uint16)
    xb[2, ::3] |= 0x8000
    xb[3, :] = 0x43E0
    xb[4:8, :] = 0                                             # with rows 0-1: zero-heavy column tiles
    return torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16)


@pytest.mark.parametrize("R,C", [(256, 256), (144, 80), (16, 16), (1040, 400), (2064, 1024)])
def test_random_codes_and_scales(orc, R, C):
    check(orc, random_codes((R, C), R + C), random_scales((cdiv(C, TILE), R), R * C))


@pytest.mark.parametrize("R,C", [(512, 384), (208, 144), (4096, 2048)])
def test_saved_activation_codes(orc, R, C):
    check(orc, *saved_codes(orc, random_bf16((R, C), R + 3 * C)))
    check(orc, *saved_codes(orc, special_saved_input(R, C, R + 11)))


def test_scales_at_the_bottom_of_the_normal_range(orc):
    """Scales in [2^-126, 2^-112): products and new scales fall into fp32 subnormals."""
    R, C = 512, 256
    check(orc, random_codes((R, C), 5), random_scales((cdiv(C, TILE), R), 6, log2_lo=-126.0, log2_hi=-112.0))


def test_large_scales_take_the_division_path(orc):
    """Column scales above 2^60 (saved scales of 2^64 .. 2^100) divide with IEEE division;
    the middle tile column keeps ordinary scales and takes the fast path in the same launch."""
    R, C = 256, 384
    q = random_codes((R, C), 41)
    s = random_scales((cdiv(C, TILE), R), 42, log2_lo=64.0, log2_hi=100.0)
    s[1] = random_scales((R,), 43)
    check(orc, q, s)


def test_unit_scales_every_code_round_trips(orc):
    """Unit scales and a +-448 in every 128-row column tile: the result is the
    plain transpose of the codes, for every finite code byte."""
    R, C = 1024, 512
    q = random_codes((R, C), 9)
    q[::TILE, :] = np.where(np.arange(C) % 2 == 0, 0x7E, 0xFE)
    assert len(np.unique(q)) == 254
    s = np.ones((cdiv(C, TILE), R), dtype=np.float32)
    check(orc, q, s)
    qt, st = puro.requant_act_t(torch.from_numpy(q).cuda(), torch.from_numpy(s).cuda())
    assert np.array_equal(to_np(qt), q.T) and np.all(to_np(st) == 1.0)


def test_empty_inputs_enqueue_nothing():
    q = torch.zeros((0, 128), dtype=torch.uint8, device="cuda")
    s = torch.zeros((1, 0), dtype=torch.float32, device="cuda")
    qt, st = puro.requant_act_t(q, s)
    assert qt.shape == (128, 0) and st.shape == (0, 128)
    torch.cuda.synchronize()


def test_workload_size(orc):
    """The down-projection input of the layer workload (16384 x 6144, the
    largest activation), saved as 1x128 codes, rebuilt as the wgrad operand."""
    t = make("layer", names={"x_down"})
    check(orc, *saved_codes(orc, t["x_down"]))


def test_wrong_scale_shape_is_rejected():
    q = torch.zeros((128, 256), dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):
        puro.requant_act_t(q, torch.zeros((128, 2), dtype=torch.float32, device="cuda"))
