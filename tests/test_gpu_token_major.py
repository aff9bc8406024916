"""GPU parity of the token-major wgrad path: the 128x1 codes written in the
input's own layout (puro_quant_act_128x1) and the wgrad that reads them
(PURO_WGRAD_TM).

- Quantizer: codes and scales bit-exact against the oracle, and its dual
  1x128 output too, on ragged shapes and the layer's largest gradient.
- GEMM: integer-valued cases bit-exact against the oracle; seeded layer-like
  operands within the fp32 GEMM tolerance; bit-exact equal to PURO_WGRAD on the
  transposed operands (the same products summed in the same order), split-K,
  edge tiles and a ragged last slice included; the accumulating form equal to
  c + the plain result.
"""
import numpy as np
import pytest
import torch

from helpers import WGRAD, assert_codes_equal, assert_scales_equal, cdiv, check_gemm_values, to_np, TILE
from workloads import bits, make, random_bf16, random_codes, random_scales

pytestmark = pytest.mark.gpu

puro = pytest.importorskip("blockwise_fp8_gemm_act_amd")
WGRAD_TM = 3


@pytest.mark.parametrize("R,C", [(256, 256), (300, 144), (16, 128), (1000, 400), (2064, 1024)])
@pytest.mark.parametrize("dual", [False, True])
def test_quant_128x1_untransposed(orc, R, C, dual):
    x = random_bf16((R, C), 3 * R + C)
    x[5, : min(C, 64)] = 0.0
    out = puro.quant_act_128x1(x.cuda(), dual=dual)
    torch.cuda.synchronize()
    qc, sc = orc.quant_act_128x1(bits(x))
    assert_codes_equal(to_np(out[0]), qc, "128x1 codes")
    assert_scales_equal(to_np(out[1]), sc, "128x1 scales")
    if dual:
        q, s = orc.quant_act_1x128(bits(x))
        assert_codes_equal(to_np(out[2]), q, "1x128 codes")
        assert_scales_equal(to_np(out[3]), s, "1x128 scales")


def test_quant_128x1_workload_gradient(orc):
    """The gate_up output gradient of the layer at 16384 tokens (16384 x 12288)."""
    dy = make("layer", names={"dy_gate_up"})["dy_gate_up"]
    qc, sc, q, s = puro.quant_act_128x1(dy.cuda(), dual=True)
    torch.cuda.synchronize()
    oqc, osc = orc.quant_act_128x1(bits(dy))
    assert_codes_equal(to_np(qc), oqc, "128x1 codes")
    assert_scales_equal(to_np(sc), osc, "128x1 scales")
    oq, os_ = orc.quant_act_1x128(bits(dy))
    assert_codes_equal(to_np(q), oq, "1x128 codes")
    assert_scales_equal(to_np(s), os_, "1x128 scales")


def run(mode, a, sa, b, sb, dtype=torch.float32):
    out = puro.gemm_fp8_blockwise(mode, *[torch.from_numpy(np.ascontiguousarray(t)).cuda() for t in (a, sa, b, sb)],
                                  out_dtype=dtype)
    torch.cuda.synchronize()
    return out


def operands(M, N, K, seed):
    nk = cdiv(K, TILE)
    return (random_codes((K, M), seed), random_scales((nk, M), seed + 1),
            random_codes((K, N), seed + 2), random_scales((nk, N), seed + 3))


@pytest.mark.parametrize("M,N,K", [(256, 256, 256), (160, 272, 400), (512, 768, 1024)])
def test_integer_valued_bit_exact(orc, M, N, K):
    rng = np.random.default_rng(M * N + K)
    codes = np.array([orc.e4m3_encode(float(v)) for v in range(-8, 9)], dtype=np.uint8)
    nk = cdiv(K, TILE)
    a = rng.choice(codes, size=(K, M)).astype(np.uint8)
    b = rng.choice(codes, size=(K, N)).astype(np.uint8)
    sa = (np.float32(2.0) ** rng.integers(-3, 4, size=(nk, M))).astype(np.float32)
    sb = (np.float32(2.0) ** rng.integers(-3, 4, size=(nk, N))).astype(np.float32)
    out = to_np(run(WGRAD_TM, a, sa, b, sb))
    ref = orc.gemm(WGRAD_TM, a, sa, b, sb)
    assert np.array_equal(out.astype(np.float64), ref)


@pytest.mark.parametrize("M,N,K", [(256, 256, 2048), (400, 272, 1040), (2048, 2048, 16384), (4096, 2048, 16384),
                                   (2048, 6144, 8192), (16, 16, 16), (2048, 6144, 1024), (2000, 6096, 1040),
                                   (4096, 2048, 2048), (2000, 1984, 8000), (9216, 2048, 16384)])
def test_equals_wgrad_on_transposed_operands(M, N, K):
    """Same products, same promotion order: the bits of PURO_WGRAD on a^T, b^T.  (2048, 6144, 1024)
    to (2000, 1984, 8000) plan 192- or 128-column tiles (whole and ragged), which both layouts
    then use.  (9216, 2048, 16384) numbers its 288 tiles in row bands (A over 128 MiB) and
    computes 256 of them whole and the other 32 split over K."""
    a, sa, b, sb = operands(M, N, K, M + 7 * N + K)
    for dtype in (torch.float32, torch.bfloat16):
        got = run(WGRAD_TM, a, sa, b, sb, dtype)
        want = run(WGRAD, a.T, sa, b.T, sb, dtype)
        assert torch.equal(got.view(torch.uint8) if dtype == torch.float32 else got.view(torch.int16),
                           want.view(torch.uint8) if dtype == torch.float32 else want.view(torch.int16)), (M, N, K, dtype)


@pytest.mark.parametrize("T,Nout,Kin", [(1024, 512, 768), (1040, 272, 400)])
def test_layer_like_operands(orc, T, Nout, Kin):
    """dY (1e-3 t4) and X (N(0,1), outlier channels) quantized 128x1 by the oracle, token-major."""
    dy = bits(random_bf16((T, Nout), T + 1, std=1e-3))
    x = bits(random_bf16((T, Kin), T + 2))
    a, sa = orc.quant_act_128x1(dy)
    b, sb = orc.quant_act_128x1(x)
    out = to_np(run(WGRAD_TM, a, sa, b, sb))
    ref = orc.gemm(WGRAD_TM, a, sa, b, sb)
    na, nb = orc.deq_row_norms(WGRAD_TM, a, sa, b, sb)
    worst, _ = check_gemm_values(out, ref, na[:, None], nb[None, :], False, orc, "wgrad token-major")
    print("token-major wgrad %dx%dx%d: max normalized error %.3g" % (Nout, Kin, T, worst))


def test_workload_size_sampled(orc):
    """The gate_up wgrad of the layer at 16384 tokens (dW 12288 x 2048) from GPU-quantized
    token-major operands, against the oracle on sampled outputs; the oracle also
    requantizes the inputs itself, so the operands are checked on the way."""
    t = make("layer", names={"dy_gate_up", "x_gate_up"})
    dy, x = t["dy_gate_up"], t["x_gate_up"]
    qa, sa = puro.quant_act_128x1(dy.cuda())
    qb, sb = puro.quant_act_128x1(x.cuda())
    out = puro.gemm_fp8_blockwise(WGRAD_TM, qa, sa, qb, sb, out_dtype=torch.float32)
    torch.cuda.synchronize()
    a, osa = orc.quant_act_128x1(bits(dy))
    b, osb = orc.quant_act_128x1(bits(x))
    assert_codes_equal(to_np(qa), a, "dY codes")
    assert_codes_equal(to_np(qb), b, "X codes")
    rng = np.random.default_rng(5)
    ms = np.concatenate([rng.integers(0, 12288, 2048), [0, 255, 256, 12287]])
    ns = np.concatenate([rng.integers(0, 2048, 2048), [2047, 0, 128, 1024]])
    ref = orc.gemm_at(WGRAD_TM, a, osa, b, osb, ms, ns)
    na, nb = orc.deq_row_norms(WGRAD_TM, a, osa, b, osb)
    check_gemm_values(to_np(out)[ms, ns], ref, na[ms], nb[ns], False, orc, "gate_up wgrad token-major")


@pytest.mark.parametrize("M,N,K", [(2048, 2048, 16384), (2048, 6144, 1024), (4096, 2048, 2048)])
def test_accumulate_equals_c_plus_plain(M, N, K):
    """Split-K plan (256 columns), then unsplit 192- and 128-column plans."""
    a, sa, b, sb = operands(M, N, K, 77)
    plain = run(WGRAD_TM, a, sa, b, sb)
    c = torch.from_numpy(np.random.default_rng(1).standard_normal((M, N)).astype(np.float32)).cuda()
    acc = c.clone()
    puro.gemm_fp8_blockwise_accumulate(WGRAD_TM, *[torch.from_numpy(np.ascontiguousarray(t)).cuda()
                                                   for t in (a, sa, b, sb)], acc)
    torch.cuda.synchronize()
    assert torch.equal((c + plain).view(torch.int32), acc.view(torch.int32))


def test_rows_must_be_multiples_of_16():
    a = torch.zeros((256, 200), dtype=torch.uint8, device="cuda")          # M = 200
    b = torch.zeros((256, 256), dtype=torch.uint8, device="cuda")
    sa = torch.ones((2, 200), dtype=torch.float32, device="cuda")
    sb = torch.ones((2, 256), dtype=torch.float32, device="cuda")
    with pytest.raises(puro.PuroError):
        puro.gemm_fp8_blockwise(WGRAD_TM, a, sa, b, sb, out_dtype=torch.float32)
