"""Seeded random shapes through the GPU path, every output compared with the oracle.

The fixed-shape tests pick the edges they mean to hit; these draw shapes at random
(fixed seeds, so every run checks the same ones) to reach combinations nobody picked:
ragged M, N and K in every mode and output dtype; whole-tile shapes (M and N multiples of
256, K of 128), which run the kernels that spread each slice's copies over the first
n-block steps and have no edge code; and quantizer inputs with ragged rows and columns,
including inputs wide enough (64+ blocks) to take the banded launch order.
"""
import numpy as np
import pytest
import torch

from helpers import DGRAD, FPROP, WGRAD, check_gemm, quantized_operands
from test_gpu_quant import check_act, check_t, check_w, outlier_input
from workloads import random_bf16

pytestmark = pytest.mark.gpu

puro = pytest.importorskip("blockwise_fp8_gemm_act_amd")


def gemm_shapes(seed, n):
    rng = np.random.default_rng(seed)
    return [(int(rng.integers(1, 700)), int(rng.integers(1, 700)), 16 * int(rng.integers(1, 100))) for _ in range(n)]


def interior_shapes(seed, n):
    rng = np.random.default_rng(seed)
    return [(256 * int(rng.integers(1, 6)), 256 * int(rng.integers(1, 6)), 128 * int(rng.integers(1, 17))) for _ in range(n)]


def quant_shapes(seed, n):
    """(R, C): C a multiple of 16; R a multiple of 16 too, as the transposed outputs need."""
    rng = np.random.default_rng(seed)
    out = [(16 * int(rng.integers(1, 80)), 16 * int(rng.integers(1, 200))) for _ in range(n - 1)]
    out.append((16 * int(rng.integers(1, 40)), 16 * int(rng.integers(512, 600))))    # 64+ blocks wide
    return out


@pytest.mark.parametrize("mode", [FPROP, DGRAD, WGRAD])
@pytest.mark.parametrize("M,N,K", gemm_shapes(2026, 6))
def test_gemm_random_shapes(orc, mode, M, N, K):
    a, sa, b, sb = quantized_operands(orc, mode, M, N, K, seed=31 * M + 7 * N + K)
    dv = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    for dtype in (torch.float32, torch.bfloat16):
        out = puro.gemm_fp8_blockwise(mode, dv(a), dv(sa), dv(b), dv(sb), out_dtype=dtype)
        torch.cuda.synchronize()
        check_gemm(orc, mode, a, sa, b, sb, out, "random mode %d %dx%dx%d %s" % (mode, M, N, K, dtype))


@pytest.mark.parametrize("mode", [FPROP, DGRAD, WGRAD])
@pytest.mark.parametrize("M,N,K", interior_shapes(4096, 4) + [(512, 512, 8192)])
def test_gemm_random_interior_shapes(orc, mode, M, N, K):
    """Whole tiles only; (512, 512, 8192) gives the weight gradient a split-K plan, whose
    partials then come from the spread-copy kernel too."""
    a, sa, b, sb = quantized_operands(orc, mode, M, N, K, seed=17 * M + 5 * N + K)
    dv = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    for dtype in (torch.float32, torch.bfloat16):
        out = puro.gemm_fp8_blockwise(mode, dv(a), dv(sa), dv(b), dv(sb), out_dtype=dtype)
        torch.cuda.synchronize()
        check_gemm(orc, mode, a, sa, b, sb, out, "interior mode %d %dx%dx%d %s" % (mode, M, N, K, dtype))


@pytest.mark.parametrize("R,C", quant_shapes(77, 6))
def test_quantizers_random_shapes(orc, R, C):
    """Codes and scales of every quantizer form, bit for bit: 1x128, dual transposed (ACT and
    WEIGHT) and 128x128."""
    x = outlier_input(R, C, R + 3 * C)
    check_act(orc, x)
    check_t(orc, puro.T_ACT, x, dual=True)
    w = random_bf16((R, C), R * 5 + C, std=0.02)
    check_w(orc, w)
    check_t(orc, puro.T_WEIGHT, w, dual=True)
