"""Pins of the oracle's token-major forms: the 128x1 codes left in the input's
own layout, and the wgrad over token-major operands (WGRAD_TM).

Independent references:
- a 128x1 tile of x is a 1x128 tile of x^T: the untransposed 128x1 codes and
  scales must be the pinned 1x128 quantizer's on x^T, transposed back (ragged
  row counts included);
- integer-valued codes with power-of-two scales: WGRAD_TM equals an int64
  numpy contraction over the token axis, exactly;
- random codes and scales: WGRAD_TM agrees with numpy's fp64 matmul of the
  torch-decoded, scaled operands (relative 1e-12 of the norms' product).
"""
import numpy as np
import pytest
import torch

from workloads import bits, random_bf16, random_codes, random_scales

TILE = 128


def cdiv(a, b):
    return (a + b - 1) // b


@pytest.mark.parametrize("R,C", [(256, 256), (300, 144), (16, 128), (1000, 400)])
def test_untransposed_128x1_is_the_row_quantizer_of_the_transpose(orc, R, C):
    x = bits(random_bf16((R, C), R + C))
    qc, sc = orc.quant_act_128x1(x)
    q1, s1 = orc.quant_act_1x128(np.ascontiguousarray(x.T))
    assert qc.shape == (R, C) and sc.shape == (cdiv(R, TILE), C)
    assert np.array_equal(qc, q1.T)
    assert np.array_equal(sc.view(np.uint32), s1.view(np.uint32))


def decode(orc, q):
    return orc.e4m3_decode_table()[q]


@pytest.mark.parametrize("M,N,K", [(128, 256, 384), (48, 80, 300), (256, 128, 1024)])
def test_token_major_wgrad_integer_exact(orc, M, N, K):
    rng = np.random.default_rng(M + N + K)
    codes = np.array([orc.e4m3_encode(float(v)) for v in range(-8, 9)], dtype=np.uint8)
    nk = cdiv(K, TILE)
    a = rng.choice(codes, size=(K, M)).astype(np.uint8)          # token-major
    b = rng.choice(codes, size=(K, N)).astype(np.uint8)
    ea = rng.integers(-3, 4, size=(nk, M))
    eb = rng.integers(-3, 4, size=(nk, N))
    sa = (2.0 ** ea).astype(np.float32)
    sb = (2.0 ** eb).astype(np.float32)
    out = orc.gemm(orc.WGRAD_TM, a, sa, b, sb)
    # exact: each operand times 2^3 is an integer; contract over tokens in int64
    ia = decode(orc, a).astype(np.int64) * (2 ** (ea[np.arange(K) // TILE] + 3))   # [K][M]
    ib = decode(orc, b).astype(np.int64) * (2 ** (eb[np.arange(K) // TILE] + 3))   # [K][N]
    want = (ia.T @ ib).astype(np.float64) / 2.0 ** 6
    assert np.array_equal(out, want)


def test_token_major_wgrad_random_against_numpy(orc):
    M, N, K = 96, 160, 400
    a = random_codes((K, M), 31)
    b = random_codes((K, N), 32)
    sa = random_scales((cdiv(K, TILE), M), 33)
    sb = random_scales((cdiv(K, TILE), N), 34)
    out = orc.gemm(orc.WGRAD_TM, a, sa, b, sb)
    kb = np.arange(K) // TILE
    da = torch.from_numpy(a).view(torch.float8_e4m3fn).double().numpy() * sa.astype(np.float64)[kb]
    db = torch.from_numpy(b).view(torch.float8_e4m3fn).double().numpy() * sb.astype(np.float64)[kb]
    want = da.T @ db
    scale = np.linalg.norm(da, axis=0)[:, None] * np.linalg.norm(db, axis=0)[None, :]
    assert (np.abs(out - want) <= 1e-12 * scale).all()
    na, nb = orc.deq_row_norms(orc.WGRAD_TM, a, sa, b, sb)
    assert np.allclose(na, np.linalg.norm(da, axis=0), rtol=1e-12)
    assert np.allclose(nb, np.linalg.norm(db, axis=0), rtol=1e-12)
    ms, ns = np.array([0, 5, 95]), np.array([159, 0, 77])
    assert np.array_equal(orc.gemm_at(orc.WGRAD_TM, a, sa, b, sb, ms, ns), out[ms, ns])
