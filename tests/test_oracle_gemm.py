"""Pins of the oracle's fp64 dequantized GEMM and of its bf16 rounding.

Independent references:
- integer-valued codes with power-of-two scales: every product and partial
  sum is an integer times a power of two, so the result is exactly numpy's
  int64 matmul times the scales;
- one-hot rows select single elements;
- linearity in power-of-two scales (exact);
- numpy's fp64 matmul of operands dequantized through PyTorch's
  float8_e4m3fn -> float64 conversion (a library routine, no oracle code);
- a pure-Python triple loop on a tiny ragged case;
- bf16 rounding against PyTorch's fp32 -> bf16 cast and exact midpoints.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

FPROP, DGRAD, WGRAD = 0, 1, 2
TILE = 128


def cdiv(a, b):
    return (a + b - 1) // b


def torch_decode(q: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(q)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def expand_scales(mode, sa, sb, M, N, K):
    """Per-element scale matrices SA [M][K], SB [N][K] from the tile layouts."""
    kb = np.arange(K) // TILE
    SA = sa[kb, :].T.astype(np.float64)                       # sa [nk][M]
    if mode == WGRAD:
        SB = sb[kb, :].T.astype(np.float64)                   # sb [nk][N]
    else:
        SB = sb[np.arange(N) // TILE][:, kb].astype(np.float64)  # sb [N/128][nk]
    return SA, SB


def random_operands(rng, mode, M, N, K, codes=None):
    nk = cdiv(K, TILE)
    if codes is None:
        finite = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)
        a = rng.choice(finite, size=(M, K))
        b = rng.choice(finite, size=(N, K))
    else:
        a = rng.choice(codes, size=(M, K)).astype(np.uint8)
        b = rng.choice(codes, size=(N, K)).astype(np.uint8)
    sa = rng.uniform(0.5, 2.0, size=(nk, M)).astype(np.float32) * np.float32(2.0 ** -6)
    sb = (rng.uniform(0.5, 2.0, size=(nk, N)) if mode == WGRAD else
          rng.uniform(0.5, 2.0, size=(cdiv(N, TILE), nk))).astype(np.float32) * np.float32(2.0 ** -5)
    return a, sa, b, sb


def int_codes(orc):
    """Codes of the integers -8..8 (all exact in e4m3)."""
    return np.array([orc.e4m3_encode(float(v)) for v in range(-8, 9)], dtype=np.uint8)


@pytest.mark.parametrize("mode", [FPROP, DGRAD, WGRAD])
@pytest.mark.parametrize("M,N,K", [(64, 48, 384), (33, 130, 272)])
def test_integer_exact(orc, mode, M, N, K):
    rng = np.random.default_rng(mode * 100 + M)
    a, sa, b, sb = random_operands(rng, mode, M, N, K, codes=int_codes(orc))
    # power-of-two scales
    sa = np.float32(2.0) ** rng.integers(-4, 5, size=sa.shape).astype(np.float32)
    sb = np.float32(2.0) ** rng.integers(-4, 5, size=sb.shape).astype(np.float32)
    ref = orc.gemm(mode, a, sa, b, sb)
    ai = np.rint(torch_decode(a)).astype(np.int64)
    bi = np.rint(torch_decode(b)).astype(np.int64)
    SA, SB = expand_scales(mode, sa, sb, M, N, K)
    # exact: sum over slices of (integer dot) * 2^e, evaluated per slice in int64
    exp = np.zeros((M, N), dtype=np.float64)
    for kb in range(cdiv(K, TILE)):
        sl = slice(kb * TILE, min(K, kb * TILE + TILE))
        part = ai[:, sl] @ bi[:, sl].T
        exp += part.astype(np.float64) * SA[:, sl.start][:, None] * SB[:, sl.start][None, :]
    assert np.array_equal(ref, exp)


def test_one_hot_rows_select_elements(orc):
    M, N, K = 4, 6, 256
    rng = np.random.default_rng(3)
    a, sa, b, sb = random_operands(rng, FPROP, M, N, K)
    a[:] = 0
    picks = [(0, 5), (1, 130), (2, 255), (3, 0)]
    one = orc.e4m3_encode(1.0)
    for m, k in picks:
        a[m, k] = one
    ref = orc.gemm(FPROP, a, sa, b, sb)
    B = torch_decode(b)
    for m, k in picks:
        for n in range(N):
            want = float(sa[k // TILE, m]) * B[n, k] * float(sb[n // TILE, k // TILE])
            assert ref[m, n] == want


@pytest.mark.parametrize("mode", [FPROP, WGRAD])
def test_linear_in_power_of_two_scales(orc, mode):
    M, N, K = 40, 300, 384
    rng = np.random.default_rng(11)
    a, sa, b, sb = random_operands(rng, mode, M, N, K)
    ref = orc.gemm(mode, a, sa, b, sb)
    sa2 = sa.copy()
    sa2[:, 7] *= np.float32(8.0)
    r2 = orc.gemm(mode, a, sa2, b, sb)
    assert np.array_equal(r2[7], ref[7] * 8.0)
    assert np.array_equal(np.delete(r2, 7, 0), np.delete(ref, 7, 0))
    sb2 = sb.copy()
    if mode == WGRAD:
        sb2[:, 5] *= np.float32(0.25)
        cols = [5]
    else:
        sb2[1, :] *= np.float32(0.25)           # columns 128..255
        cols = list(range(128, 256))
    r3 = orc.gemm(mode, a, sa, b, sb2)
    assert np.array_equal(r3[:, cols], ref[:, cols] * 0.25)
    assert np.array_equal(np.delete(r3, cols, 1), np.delete(ref, cols, 1))


@pytest.mark.parametrize("mode", [FPROP, DGRAD, WGRAD])
def test_matches_library_fp64_matmul(orc, mode):
    M, N, K = 96, 200, 400
    rng = np.random.default_rng(21 + mode)
    a, sa, b, sb = random_operands(rng, mode, M, N, K)
    ref = orc.gemm(mode, a, sa, b, sb)
    SA, SB = expand_scales(mode, sa, sb, M, N, K)
    A = torch_decode(a) * SA
    B = torch_decode(b) * SB
    lib = A @ B.T
    na = np.linalg.norm(A, axis=1)
    nb = np.linalg.norm(B, axis=1)
    assert np.max(np.abs(ref - lib) / (na[:, None] * nb[None, :])) < 1e-13
    ona, onb = orc.deq_row_norms(mode, a, sa, b, sb)
    assert np.allclose(ona, na, rtol=1e-14, atol=0) and np.allclose(onb, nb, rtol=1e-14, atol=0)
    assert np.array_equal(orc.dequant_a(a, sa), A)
    assert np.array_equal(orc.dequant_b(mode, b, sb), B)


def test_sampled_elements_equal_full(orc):
    M, N, K = 50, 70, 272
    rng = np.random.default_rng(8)
    a, sa, b, sb = random_operands(rng, WGRAD, M, N, K)
    full = orc.gemm(WGRAD, a, sa, b, sb)
    ms = rng.integers(0, M, 100)
    ns = rng.integers(0, N, 100)
    assert np.array_equal(orc.gemm_at(WGRAD, a, sa, b, sb, ms, ns), full[ms, ns])


def test_python_triple_loop_tiny_ragged(orc):
    M, N, K = 3, 5, 144
    rng = np.random.default_rng(4)
    for mode in (FPROP, WGRAD):
        a, sa, b, sb = random_operands(rng, mode, M, N, K)
        table = [float(v) for v in torch_decode(np.arange(256, dtype=np.uint8))]
        ref = orc.gemm(mode, a, sa, b, sb)
        for m in range(M):
            for n in range(N):
                acc = 0.0
                for k in range(K):
                    sA = float(sa[k // TILE][m])
                    sB = float(sb[k // TILE][n]) if mode == WGRAD else float(sb[n // TILE][k // TILE])
                    acc += (table[a[m][k]] * sA) * (table[b[n][k]] * sB)
                assert acc == ref[m, n]


def test_zero_k_and_empty(orc):
    z = orc.gemm(FPROP, np.zeros((3, 0), np.uint8), np.zeros((0, 3), np.float32),
                 np.zeros((4, 0), np.uint8), np.zeros((1, 0), np.float32))
    assert z.shape == (3, 4) and np.all(z == 0)


def test_bf16_rounding_matches_torch_on_fp32_values(orc):
    rng = np.random.default_rng(2)
    u = rng.integers(0, 2 ** 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    f = u.view(np.float32)
    f = f[np.isfinite(f)]
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = orc.f64_to_bf16_array(f.astype(np.float64))
    assert np.array_equal(got, ref)


def test_bf16_rounding_single_rounding_from_fp64(orc):
    # 1 + 2^-8 is the midpoint between bf16 1 and 1 + 2^-7: ties to even (1.0)
    assert orc.f64_to_bf16(1.0 + 2.0 ** -8) == 0x3F80
    # a hair above the midpoint (not representable in fp32) must round up;
    # rounding through fp32 first would give the midpoint and then 1.0
    v = 1.0 + 2.0 ** -8 + 2.0 ** -40
    assert np.float64(np.float32(v)) == 1.0 + 2.0 ** -8
    assert orc.f64_to_bf16(v) == 0x3F81
    assert orc.f64_to_bf16(-v) == 0xBF81
    assert orc.f64_to_bf16(0.0) == 0 and orc.f64_to_bf16(-0.0) == 0x8000
    # exact value of a random bf16 code survives
    for h in (0x0001, 0x007F, 0x0080, 0x4049, 0x7F7F):
        val = float(Fraction(int(np.uint32(h << 16).view(np.float32).astype(np.float64) * 2 ** 140), 2 ** 140))
        assert orc.f64_to_bf16(val) == h


@pytest.mark.parametrize("mode", [FPROP, WGRAD])
def test_accumulate_integer_exact(orc, mode):
    """Accumulating GEMM: integer codes, power-of-two scales and an integer-valued c, so
    c + GEMM is exact in fp64 and must equal numpy's int64 arithmetic."""
    M, N, K = 40, 72, 384
    rng = np.random.default_rng(17 + mode)
    a, sa, b, sb = random_operands(rng, mode, M, N, K, codes=int_codes(orc))
    sa = np.ones_like(sa)
    sb = np.ones_like(sb)
    c = rng.integers(-1000, 1000, size=(M, N)).astype(np.float32)
    got = orc.gemm_accumulate(mode, a, sa, b, sb, c)
    ai = np.rint(torch_decode(a)).astype(np.int64)
    bi = np.rint(torch_decode(b)).astype(np.int64)
    assert np.array_equal(got, (ai @ bi.T + c.astype(np.int64)).astype(np.float64))


def test_accumulate_onto_zero_is_the_gemm(orc):
    rng = np.random.default_rng(23)
    a, sa, b, sb = random_operands(rng, DGRAD, 64, 96, 256)
    assert np.array_equal(orc.gemm_accumulate(DGRAD, a, sa, b, sb, np.zeros((64, 96), np.float32)),
                          orc.gemm(DGRAD, a, sa, b, sb))
