"""GPU parity of the fused SwiGLU + quantization: h, codes and scales
bit-exact against the oracle (h = bf16 of the fp64 SwiGLU value, then the
1x128 and 128x1 rules)."""
import numpy as np
import pytest
import torch

from helpers import assert_codes_equal, assert_scales_equal, bf16_bits_np, cdiv, to_np, TILE
from workloads import bits, make

pytestmark = pytest.mark.gpu

puro = pytest.importorskip("blockwise_fp8_gemm_act_amd")


def from_bits(b: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16)


def check(orc, gub: torch.Tensor, dual: bool, write_h: bool = True):
    res = puro.swiglu_quant(gub.cuda(), dual=dual, write_h=write_h)
    torch.cuda.synchronize()
    oh, oq, os_, *ot = orc.swiglu_quant(bits(gub), dual=dual)
    if write_h:
        got_h = bf16_bits_np(res[-1])
        bad = np.argwhere(got_h != oh)
        assert bad.size == 0, "h: %d mismatches, first at %s: got 0x%04x want 0x%04x (g 0x%04x u 0x%04x)" % (
            len(bad), tuple(bad[0]), got_h[tuple(bad[0])], oh[tuple(bad[0])],
            bits(gub)[bad[0][0], bad[0][1]], bits(gub)[bad[0][0], bad[0][1] + oh.shape[1]])
    assert_codes_equal(to_np(res[0]), oq, "codes")
    assert_scales_equal(to_np(res[1]), os_, "scales")
    if dual:
        assert_codes_equal(to_np(res[2]), ot[0], "transposed codes")
        assert_scales_equal(to_np(res[3]), ot[1], "transposed scales")


def gate_up(R, I, seed, std=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn((R, 2 * I), generator=g) * std).to(torch.bfloat16)


@pytest.mark.parametrize("R,I", [(256, 256), (144, 80), (16, 16), (1040, 400), (512, 2048), (400, 4096), (16, 4112)])
@pytest.mark.parametrize("dual", [False, True])
def test_random_gate_up(orc, R, I, dual):
    check(orc, gate_up(R, I, R + I), dual)
    check(orc, gate_up(R, I, R + 2 * I, std=8.0), dual)


@pytest.mark.parametrize("R,I", [(37, 400), (1, 128), (130, 16)])
def test_rows_free_without_transposed_output(orc, R, I):
    check(orc, gate_up(R, I, 3 * R + I), dual=False)


def test_h_output_is_optional(orc):
    gub = gate_up(256, 384, 9)
    q1, s1 = puro.swiglu_quant(gub.cuda())
    q2, s2, h = puro.swiglu_quant(gub.cuda(), write_h=True)
    torch.cuda.synchronize()
    assert torch.equal(q1, q2) and torch.equal(s1, s2)


def test_every_bf16_gate_value(orc):
    """Every finite bf16 gate value (65280 of them, |g| up to 3.4e38: the fp64 path
    beyond |g| = 64), each against 16 up values of magnitude <= 1 (h stays finite)."""
    b = np.arange(0x10000, dtype=np.uint32)
    g = b[((b >> 7) & 0xFF) != 0xFF].astype(np.uint16)          # 65280 = 255 x 256
    g = g.reshape(255, 256)
    rng = np.random.default_rng(4)
    ups = np.concatenate([[0x3F80, 0xBF80, 0x0001, 0x3A80],     # 1, -1, the smallest subnormal, 2^-10
                          bits(torch.from_numpy(rng.uniform(-1, 1, 12).astype(np.float32)).to(torch.bfloat16))])
    rows = []
    for uv in ups:
        rows.append(np.concatenate([g, np.full_like(g, uv)], axis=1))
    gu = np.concatenate(rows)                                    # [16 * 255][512]
    gu = gu[: (len(gu) // 16) * 16]
    check(orc, from_bits(gu), dual=True)


def test_products_near_bf16_midpoints(orc):
    """Pairs whose product lies within a few fp32 ulps of a bf16 rounding midpoint (the
    fp64 fallback of the kernel), picked from random pairs with numpy's fp64 exp."""
    rng = np.random.default_rng(21)
    n = 1 << 22
    gb = bits(torch.from_numpy(rng.standard_normal(n).astype(np.float32) * 2).to(torch.bfloat16)).ravel()
    ub = bits(torch.from_numpy(rng.standard_normal(n).astype(np.float32)).to(torch.bfloat16)).ravel()
    gf = (gb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    uf = (ub.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    v = (gf / (1.0 + np.exp(-gf)) * uf).astype(np.float32)
    lo = v.view(np.uint32) & 0xFFFF
    near = np.flatnonzero(np.abs(lo.astype(np.int64) - 0x8000) <= 8)
    assert len(near) > 100
    I = 256
    m = (len(near) // I) * I
    sel = near[:m]
    gu = np.concatenate([gb[sel].reshape(-1, I), ub[sel].reshape(-1, I)], axis=1)
    gu = gu[: (len(gu) // 16) * 16] if len(gu) >= 16 else gu
    check(orc, from_bits(gu), dual=len(gu) % 16 == 0)


def test_workload_size(orc):
    """The MLP gate/up output at 16384 tokens (16384 x 12288) -> h 16384 x 6144, dual."""
    t = make("mlp_swiglu")
    check(orc, t["gu"], dual=True)


def test_empty_inputs_enqueue_nothing():
    gu = torch.zeros((0, 256), dtype=torch.bfloat16, device="cuda")
    q, s = puro.swiglu_quant(gu)
    assert q.shape == (0, 128) and s.shape == (1, 0)
    torch.cuda.synchronize()
