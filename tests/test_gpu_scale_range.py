"""The GEMMs on GPU-made codes of tiny inputs, near the small end of the
promotion's domain (every product sA * sB a normal fp32 value, >= 2^-126).

X, W and dY are N(0, 1) (X and dY with outlier channels x20) scaled by 2^-52,
an exact power-of-two scaling of bf16 values, so that tile maxima sit near
2^-50 and the scale products a GEMM slice forms lie between about 2^-122 and
2^-109.  The quantizers' codes and scales are bit-exact against the oracle, and
every output of fprop, dgrad and wgrad (fp32 and bf16) meets the rule of every
GEMM test against the oracle's fp64 GEMM of the same codes; the token-major
wgrad gives the bits of the wgrad.  Shapes are ragged in every dimension."""
import numpy as np
import pytest
import torch

from helpers import DGRAD, FPROP, WGRAD, assert_codes_equal, assert_scales_equal, check_gemm, to_np
from workloads import bits, random_bf16

pytestmark = pytest.mark.gpu

puro = pytest.importorskip("blockwise_fp8_gemm_act_amd")

WGRAD_TM = 3
TINY = 2.0 ** -52
T, K_IN, N_OUT = 1040, 400, 272


def tiny(shape, seed, outliers):
    x = random_bf16(shape, seed).float()
    if outliers:
        x[:, ::37] *= 20
    return (x.to(torch.bfloat16).float() * TINY).to(torch.bfloat16)


def same(want, got, what):
    for k, (w, g) in enumerate(zip(want, got)):
        g = to_np(g)
        if w.dtype == np.uint8:
            assert_codes_equal(g, w, "%s output %d" % (what, k))
        else:
            assert_scales_equal(g, w, "%s output %d" % (what, k))


def scale_products(sa, sb_of_k):
    """Smallest and largest sA * sB in fp32 over every (row scale, column scale) pair of each K slice."""
    lo, hi = np.inf, 0.0
    for kb in range(sa.shape[0]):
        a = sa[kb].astype(np.float32)
        b = np.atleast_1d(sb_of_k(kb)).astype(np.float32)
        lo = min(lo, float(a.min() * b.min()))
        hi = max(hi, float(a.max() * b.max()))
    return lo, hi


@pytest.fixture(scope="module")
def operands(orc):
    x = tiny((T, K_IN), 41, True)
    w = tiny((N_OUT, K_IN), 42, False)
    dy = tiny((T, N_OUT), 43, True)
    X, W, DY = x.cuda(), w.cuda(), dy.cuda()
    g = {}
    g["xqt"], g["xst"], g["xq"], g["xs"] = puro.quant_transpose(puro.T_ACT, X, dual=True)
    g["wqt"], g["wst"], g["wq"], g["ws"] = puro.quant_transpose(puro.T_WEIGHT, W, dual=True)
    g["dqt"], g["dst"], g["dq"], g["ds"] = puro.quant_transpose(puro.T_ACT, DY, dual=True)
    g["xqc"], g["xsc"] = puro.quant_act_128x1(X)
    g["dqc"], g["dsc"] = puro.quant_act_128x1(DY)
    torch.cuda.synchronize()
    o = {}
    o["xq"], o["xs"] = orc.quant_act_1x128(bits(x))
    o["xqt"], o["xst"] = orc.quant_act_128x1_t(bits(x))
    o["wq"], o["ws"] = orc.quant_w_128x128(bits(w))
    o["wqt"], o["wst"] = orc.quant_w_128x128_t(bits(w))
    o["dq"], o["ds"] = orc.quant_act_1x128(bits(dy))
    o["dqt"], o["dst"] = orc.quant_act_128x1_t(bits(dy))
    for pair in (("xq", "xs"), ("xqt", "xst"), ("wq", "ws"), ("wqt", "wst"), ("dq", "ds"), ("dqt", "dst")):
        same([o[k] for k in pair], [g[k] for k in pair], pair[0])
    return g, o


def test_scale_products_in_the_low_normal_range(operands):
    """The workload does sit near the domain's lower edge (and inside it)."""
    g, o = operands
    cases = {
        "fprop": scale_products(o["xs"], lambda kb: o["ws"][:, kb]),
        "dgrad": scale_products(o["ds"], lambda kb: o["wst"][:, kb]),
        "wgrad": scale_products(o["dst"], lambda kb: o["xst"][kb]),
    }
    for name, (lo, hi) in cases.items():
        assert 2.0 ** -126 <= lo and hi <= 2.0 ** -100, (name, np.log2(lo), np.log2(hi))
    assert min(lo for lo, _ in cases.values()) <= 2.0 ** -116


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_fprop_dgrad_wgrad(orc, operands, dtype):
    g, o = operands
    y = puro.gemm_fp8_blockwise(FPROP, g["xq"], g["xs"], g["wq"], g["ws"], out_dtype=dtype)
    dx = puro.gemm_fp8_blockwise(DGRAD, g["dq"], g["ds"], g["wqt"], g["wst"], out_dtype=dtype)
    dw = puro.gemm_fp8_blockwise(WGRAD, g["dqt"], g["dst"], g["xqt"], g["xst"], out_dtype=dtype)
    torch.cuda.synchronize()
    check_gemm(orc, FPROP, o["xq"], o["xs"], o["wq"], o["ws"], y, "tiny fprop")
    check_gemm(orc, DGRAD, o["dq"], o["ds"], o["wqt"], o["wst"], dx, "tiny dgrad")
    check_gemm(orc, WGRAD, o["dqt"], o["dst"], o["xqt"], o["xst"], dw, "tiny wgrad")
    # the outputs are of the inputs' scale, not flushed to zero
    assert float(y.float().abs().max()) > 2.0 ** -100


def test_token_major_wgrad_equals_wgrad(operands):
    g, _ = operands
    for dtype in (torch.float32, torch.bfloat16):
        got = puro.gemm_fp8_blockwise(WGRAD_TM, g["dqc"], g["dsc"], g["xqc"], g["xsc"], out_dtype=dtype)
        want = puro.gemm_fp8_blockwise(WGRAD, g["dqt"], g["dst"], g["xqt"], g["xst"], out_dtype=dtype)
        torch.cuda.synchronize()
        view = torch.int32 if dtype == torch.float32 else torch.int16
        assert torch.equal(got.view(view), want.view(view)), dtype
