"""GPU parity of the fused gate/up fprop + SwiGLU quantizer
(puro_gemm_fp8_swiglu_quant) against the oracle's composition: gu = bf16 of
the fp64 GEMM, then the SwiGLU quantizer of gu.

- Integer-valued codes with power-of-two scales make the GEMM exact in fp32,
  so gu, the codes and the scales must equal the oracle bit for bit (ragged
  M and K, one to several hundred work items, fast and fp64 SwiGLU paths).
- Seeded activations and weights shaped like the layer's: gu within the bf16
  GEMM tolerance; every 1x128 tile whose 256 gate/up inputs equal the
  oracle's has the oracle's codes and scale bit for bit; every dequantized
  code lies within an error bound derived from that tolerance, SwiGLU's
  Lipschitz constant and the e4m3 step (check_against_oracle).
- The fused call gives exactly what the unfused pair (bf16 fprop, then the
  SwiGLU quantizer) gives on the GPU, up to the layer's full size, for shapes
  whose plain fprop does not split its K loop (a split sums in another order).
"""
import numpy as np
import pytest
import torch

from helpers import FPROP, bf16_bits_np, cdiv, check_gemm_values, quantized_operands, to_np, TILE
from workloads import bits, make

pytestmark = pytest.mark.gpu

puro = pytest.importorskip("blockwise_fp8_gemm_act_amd")


def cuda(*arrays):
    return [torch.from_numpy(np.ascontiguousarray(x)).cuda() for x in arrays]


def run(a, sa, b, sb, write_gu=True):
    hq, hs, gu = puro.gemm_fp8_swiglu_quant(*cuda(a, sa, b, sb), write_gu=write_gu)
    torch.cuda.synchronize()
    return to_np(hq), to_np(hs), (bf16_bits_np(gu) if gu is not None else None)


def exact_operands(orc, M, I, K, seed):
    """Codes of -2..2; row scales 2^-6 .. 1 (small ones keep |g| in the fp32 SwiGLU
    range, large ones push it past 64 into the fp64 path), block scales 2^-4 .. 2^-1.
    Every promoted partial is a multiple of 2^-10 below 2^14 in magnitude: exact."""
    rng = np.random.default_rng(seed)
    codes = np.array([orc.e4m3_encode(float(v)) for v in (-2, -1, 0, 1, 2)], dtype=np.uint8)
    nk = cdiv(K, TILE)
    a = rng.choice(codes, size=(M, K)).astype(np.uint8)
    b = rng.choice(codes, size=(2 * I, K)).astype(np.uint8)
    sa = (np.float32(2.0) ** rng.integers(-6, 1, size=(nk, M))).astype(np.float32)
    sb = (np.float32(2.0) ** rng.integers(-4, 0, size=(2 * I // TILE, nk))).astype(np.float32)
    return a, sa, b, sb


def assert_same(got, want, what):
    assert got.shape == want.shape, (what, got.shape, want.shape)
    g = got.view(np.uint32) if got.dtype == np.float32 else got
    w = want.view(np.uint32) if want.dtype == np.float32 else want
    bad = np.argwhere(g != w)
    assert bad.size == 0, "%s: %d mismatches, first at %s" % (what, len(bad), tuple(bad[0]))


@pytest.mark.parametrize("M,I,K", [(256, 128, 128), (300, 256, 2000), (16, 128, 16), (1040, 384, 640),
                                   (513, 640, 4096)])
def test_exact_operands_bit_exact(orc, M, I, K):
    a, sa, b, sb = exact_operands(orc, M, I, K, M * 7 + I + K)
    hq, hs, gu = run(a, sa, b, sb)
    ogu, _, oq, os_ = orc.gemm_swiglu_quant(a, sa, b, sb)
    assert_same(gu, ogu, "gu")
    assert_same(hq, oq, "codes")
    assert_same(hs, os_, "scales")


def test_exact_operands_many_items_per_workgroup(orc):
    """272 work items (17 x 16 tiles) on at most 256 workgroups: some compute two;
    rows sampled across every row tile, the ragged last one included."""
    M, I, K = 4300, 2048, 384
    a, sa, b, sb = exact_operands(orc, M, I, K, 11)
    hq, hs, gu = run(a, sa, b, sb)
    rows = np.unique(np.concatenate([np.arange(0, M, 97), np.arange(255, M, 256), [M - 1]]))
    ogu, _, oq, os_ = orc.gemm_swiglu_quant(a, sa, b, sb, rows=rows)
    assert_same(gu[rows], ogu, "gu")
    assert_same(hq[rows], oq, "codes")
    assert_same(hs[:, rows], os_, "scales")


def bf16_value(bits16):
    return (bits16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def e4m3_value(orc, q):
    return orc.e4m3_decode_table()[q]


def check_against_oracle(orc, a, sa, b, sb, gu, hq, hs, rows, what):
    """Parity on the given rows against the oracle's composition.

    gu: the bf16 GEMM tolerance (within 1 ulp of the oracle's rounding, or
    normalized error <= 1e-4).  A tile whose 256 gate/up inputs equal the
    oracle's has the oracle's codes and scale bit for bit.  Every element: the
    GPU's gate/up values g', u' lie within eg = 2 ulp(g) + 1e-4 ||A_m|| ||B_n||
    of the oracle's (eu likewise); SwiGLU is Lipschitz in g with constant 1.1
    (|silu'| <= 1.0999), so the exact SwiGLU values differ by at most
    1.1 eg (|u| + eu) + |silu(g)| eu, and each side's bf16 rounding adds half
    an ulp.  The GPU's dequantized code dec(q) s is within half an e4m3 step
    (at its own scale) of its h, and its scale within max(bound)/448 (+ one
    fp32 rounding) of the oracle's."""
    M = len(rows)
    I = hq.shape[1]
    nt = I // TILE
    ogu, oh, oq, os_ = orc.gemm_swiglu_quant(a, sa, b, sb, rows=rows)
    ra = np.ascontiguousarray(a[rows])
    rsa = np.ascontiguousarray(sa[:, rows])
    ref = orc.gemm(FPROP, ra, rsa, b, sb)
    na, nb = orc.deq_row_norms(FPROP, ra, rsa, b, sb)
    g16 = gu[rows]
    check_gemm_values(g16, ref, na[:, None], nb[None, :], True, orc, what + " gu")
    # tiles with exactly the oracle's inputs: bit-exact
    same = (g16.reshape(M, 2, nt, TILE) == ogu.reshape(M, 2, nt, TILE)).all(axis=(1, 3))      # [row][tile]
    q = hq[rows]
    s = hs[:, rows].T                                                                           # [row][tile]
    os_t = os_.T
    qt, oqt = q.reshape(M, nt, TILE), oq.reshape(M, nt, TILE)
    assert (qt[same] == oqt[same]).all(), what + ": codes of tiles with exact inputs"
    assert (s[same].view(np.uint32) == os_t[same].view(np.uint32)).all(), what + ": scales of tiles with exact inputs"
    # every element: the error bound of the docstring
    e = np.abs(ref) * 2.0 ** -6 + 1e-4 * na[:, None] * nb[None, :]       # 2 bf16 ulps + the GEMM tolerance
    gv, uv = bf16_value(ogu[:, :I]), bf16_value(ogu[:, I:])
    eg, eu = e[:, :I], e[:, I:]
    silu = gv / (1.0 + np.exp(-gv))
    bound = 1.1 * eg * (np.abs(uv) + eu) + np.abs(silu) * eu
    hv = bf16_value(oh)
    bound += (np.abs(hv) + bound) * 2.0 ** -8                                                    # both bf16 roundings
    sfull = np.repeat(s, TILE, axis=1)
    mag = (np.abs(hv) + bound) / sfull
    half_step = sfull * 2.0 ** (np.maximum(np.floor(np.log2(np.maximum(mag, 2.0 ** -30))), -6) - 4)
    deq = e4m3_value(orc, q) * sfull
    err = np.abs(deq - hv)
    ok = err <= bound + half_step + 1e-30
    assert ok.all(), "%s: %d elements beyond the bound; worst excess %.3g" % (
        what, int((~ok).sum()), float((err - bound - half_step).max()))
    sb_tile = bound.reshape(M, nt, TILE).max(axis=2) / 448.0 + os_t.astype(np.float64) * 2.0 ** -23
    assert (np.abs(s.astype(np.float64) - os_t) <= sb_tile).all(), what + ": scales"
    print("%s: gu equal to the oracle's rounding %.5f, tiles with exact inputs %.4f, codes equal %.5f" % (
        what, float(np.mean(g16 == ogu)), float(same.mean()), float(np.mean(q == oq))))


@pytest.mark.parametrize("M,I,K", [(512, 768, 2048), (300, 384, 1008)])
def test_layer_like_operands(orc, M, I, K):
    a, sa, b, sb = quantized_operands(orc, FPROP, M, 2 * I, K, M + I + K)
    hq, hs, gu = run(a, sa, b, sb)
    check_against_oracle(orc, a, sa, b, sb, gu, hq, hs, np.arange(M), "M=%d I=%d K=%d" % (M, I, K))


def unfused(a, sa, b, sb):
    ta, tsa, tb, tsb = cuda(a, sa, b, sb)
    gu = puro.gemm_fp8_blockwise(FPROP, ta, tsa, tb, tsb, out_dtype=torch.bfloat16)
    q, s = puro.swiglu_quant(gu)
    torch.cuda.synchronize()
    return to_np(q), to_np(s), bf16_bits_np(gu)


@pytest.mark.parametrize("M,I,K", [(1000, 256, 528), (2600, 1024, 1040), (3000, 3072, 752)])
def test_fused_equals_unfused_pair(orc, M, I, K):
    """Row-tile counts of 4, 11 and 12 (not multiples of 8) and ragged edges; 288 work
    items in the last case, so some workgroups take two.  The plain fprop of these shapes
    runs without a split of its K loop, as the fused kernel does (at 6 K slices no split
    is allowed)."""
    assert puro.puro_gemm_workspace_bytes(FPROP, M, 2 * I, K) == 0
    a, sa, b, sb = quantized_operands(orc, FPROP, M, 2 * I, K, 3 * M + I)
    for got, want, what in zip(run(a, sa, b, sb), unfused(a, sa, b, sb), ("codes", "scales", "gu")):
        assert_same(got, want, what)


def test_workload_size(orc):
    """The layer's gate/up projection at 16384 tokens (X [16384x2048], W [12288x2048]):
    the fused call against the unfused pair everywhere, and against the oracle on
    sampled rows."""
    t = make("layer", names={"x_gate_up", "w_gate_up"})
    a, sa = orc.quant_act_1x128(bits(t["x_gate_up"]))
    b, sb = orc.quant_w_128x128(bits(t["w_gate_up"]))
    hq, hs, gu = run(a, sa, b, sb)
    assert puro.puro_gemm_workspace_bytes(FPROP, 16384, 12288, 2048) == 0
    for got, want, what in zip((hq, hs, gu), unfused(a, sa, b, sb), ("codes", "scales", "gu")):
        assert_same(got, want, what)
    rows = np.unique(np.concatenate([np.arange(0, 16384, 1031), [255, 256, 8191, 16383]]))
    check_against_oracle(orc, a, sa, b, sb, gu, hq, hs, rows, "16384 tokens")


def test_without_gate_up_output(orc):
    a, sa, b, sb = exact_operands(orc, 300, 256, 512, 4)
    hq, hs, gu = run(a, sa, b, sb)
    hq2, hs2, gu2 = run(a, sa, b, sb, write_gu=False)
    assert gu2 is None
    assert_same(hq2, hq, "codes")
    assert_same(hs2, hs, "scales")


def test_k_zero_and_empty():
    a = torch.zeros((200, 0), dtype=torch.uint8, device="cuda")
    sa = torch.zeros((0, 200), dtype=torch.float32, device="cuda")
    b = torch.zeros((512, 0), dtype=torch.uint8, device="cuda")
    sb = torch.zeros((4, 0), dtype=torch.float32, device="cuda")
    hq, hs, gu = puro.gemm_fp8_swiglu_quant(a, sa, b, sb)
    torch.cuda.synchronize()
    assert (hq == 0).all() and (hs == 1.0).all() and (gu.view(torch.int16) == 0).all()
    a0 = torch.zeros((0, 256), dtype=torch.uint8, device="cuda")
    hq, hs, gu = puro.gemm_fp8_swiglu_quant(a0, torch.zeros((2, 0), dtype=torch.float32, device="cuda"),
                                            torch.zeros((256, 256), dtype=torch.uint8, device="cuda"),
                                            torch.ones((2, 2), dtype=torch.float32, device="cuda"))
    assert hq.shape == (0, 128) and hs.shape == (1, 0) and gu.shape == (0, 256)


def test_inter_must_be_a_multiple_of_128():
    a = torch.zeros((256, 256), dtype=torch.uint8, device="cuda")
    sa = torch.ones((2, 256), dtype=torch.float32, device="cuda")
    b = torch.zeros((192, 256), dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):
        puro.gemm_fp8_swiglu_quant(a, sa, b, torch.ones((2, 2), dtype=torch.float32, device="cuda"))
