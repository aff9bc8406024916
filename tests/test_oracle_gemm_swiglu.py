"""Pins of the oracle's fused gate/up fprop + SwiGLU quantizer (the down
projection's FP8 input made from the gate/up GEMM).

The composition is gu = bf16(fprop GEMM), then the SwiGLU quantizer of gu.
Independent references:
- integer-valued operands with power-of-two scales, so that the GEMM is exact
  in any precision: the product from PyTorch's own e4m3 decoding and a
  float64 matmul, rounded to bf16 by PyTorch's cast, must be the oracle's gu
  bit for bit (this pins the GEMM step, the single rounding and which half of
  the weight rows is the gate);
- random codes and scales: gu is one rounding of the product from PyTorch's
  decoding and numpy's fp64 matmul, by the pinned fp64 -> bf16 rounding;
- rows are independent: the row-sampled form equals the full result there;
- swapping the gate and up halves of the weight swaps the halves of gu.
"""
import numpy as np
import pytest
import torch

TILE = 128


def cdiv(a, b):
    return (a + b - 1) // b


def exact_operands(orc, M, I, K, seed):
    """Codes of -2..2 and power-of-two scales: every partial sum is an exact binary fraction."""
    rng = np.random.default_rng(seed)
    codes = np.array([orc.e4m3_encode(float(v)) for v in (-2, -1, 0, 1, 2)], dtype=np.uint8)
    nk = cdiv(K, TILE)
    a = rng.choice(codes, size=(M, K)).astype(np.uint8)
    b = rng.choice(codes, size=(2 * I, K)).astype(np.uint8)
    sa = (np.float32(2.0) ** rng.integers(-6, 1, size=(nk, M))).astype(np.float32)
    sb = (np.float32(2.0) ** rng.integers(-4, 0, size=(2 * I // TILE, nk))).astype(np.float32)
    return a, sa, b, sb


def torch_exact_gu(a, sa, b, sb):
    """The exact product through PyTorch's e4m3 decoding, rounded to bf16 by PyTorch."""
    M, K = a.shape
    N = b.shape[0]
    da = torch.from_numpy(a).view(torch.float8_e4m3fn).double()
    db = torch.from_numpy(b).view(torch.float8_e4m3fn).double()
    kb = torch.arange(K) // TILE
    da = da * torch.from_numpy(sa).double().t()[:, kb]                       # sa[k/128][m]
    db = db * torch.from_numpy(sb).double()[torch.arange(N) // TILE][:, kb]  # sb[n/128][k/128]
    g = da @ db.t()
    assert torch.equal(g, g.float().double())                                # exact in fp32 too
    return g.float().to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("M,I,K", [(40, 128, 384), (17, 256, 200)])
def test_exact_gemm_step_matches_library_rounding(orc, M, I, K):
    a, sa, b, sb = exact_operands(orc, M, I, K, M + I + K)
    gu, h, q, s = orc.gemm_swiglu_quant(a, sa, b, sb)
    want = torch_exact_gu(a, sa, b, sb)
    assert np.array_equal(gu, want)
    h2, q2, s2 = orc.swiglu_quant(want)
    assert np.array_equal(h, h2) and np.array_equal(q, q2) and np.array_equal(s.view(np.uint32), s2.view(np.uint32))
    assert h.shape == (M, I) and q.shape == (M, I) and s.shape == (I // TILE, M)
    assert len(np.unique(q)) > 20                                            # not a degenerate case


def test_single_rounding_of_the_gemm_on_random_operands(orc):
    """Random codes and scales: gu is the one bf16 rounding of the exact product, here the
    product from PyTorch's e4m3 decoding and numpy's fp64 matmul (it agrees with the
    oracle's fp64 GEMM to ~1e-13 relative; a midpoint that close is not expected among
    these 262144 values), rounded by the pinned fp64 -> bf16 rounding.  A rounding through
    fp32 first would differ at about 4 of them."""
    from workloads import random_codes, random_scales
    M, I, K = 256, 512, 256
    a = random_codes((M, K), 21)
    b = random_codes((2 * I, K), 22)
    sa = random_scales((K // TILE, M), 23)
    sb = random_scales((2 * I // TILE, K // TILE), 24)
    gu, _, _, _ = orc.gemm_swiglu_quant(a, sa, b, sb)
    da = torch.from_numpy(a).view(torch.float8_e4m3fn).double().numpy()
    db = torch.from_numpy(b).view(torch.float8_e4m3fn).double().numpy()
    kb = np.arange(K) // TILE
    da = da * sa.astype(np.float64).T[:, kb]
    db = db * sb.astype(np.float64)[np.arange(2 * I) // TILE][:, kb]
    want = orc.f64_to_bf16_array(da @ db.T)
    assert np.array_equal(gu, want)


def test_rows_sampled_equal_full(orc):
    a, sa, b, sb = exact_operands(orc, 64, 128, 256, 5)
    full = orc.gemm_swiglu_quant(a, sa, b, sb)
    rows = np.array([0, 3, 31, 63])
    part = orc.gemm_swiglu_quant(a, sa, b, sb, rows=rows)
    for f, p in zip(full[:3], part[:3]):
        assert np.array_equal(f[rows], p)
    assert np.array_equal(full[3][:, rows].view(np.uint32), part[3].view(np.uint32))


def test_gate_is_the_first_half_of_the_weight_rows(orc):
    a, sa, b, sb = exact_operands(orc, 32, 128, 256, 9)
    gu, h, _, _ = orc.gemm_swiglu_quant(a, sa, b, sb)
    I = 128
    b_sw = np.concatenate([b[I:], b[:I]])
    sb_sw = np.concatenate([sb[I // TILE:], sb[:I // TILE]])
    gu_sw, h_sw, _, _ = orc.gemm_swiglu_quant(a, sa, b_sw, sb_sw)
    assert np.array_equal(gu_sw, np.concatenate([gu[:, I:], gu[:, :I]], axis=1))
    assert not np.array_equal(h, h_sw)
