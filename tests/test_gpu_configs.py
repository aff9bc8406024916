"""The four smaller workloads end to end on the GPU: every tensor of the workload
quantized by the GPU in the form the workload uses, codes and scales bit-exact
against the oracle, then the workload's GEMMs run on the GPU's own codes and
checked against the oracle's fp64 GEMM of the same codes (the codes are
identical) -- on every output for the tiny fprop, on 4096 sampled outputs plus
every output of the first and last rows otherwise.

  tiny fprop     X [256][256] (2 outlier channels) 1x128, W [512][256] 128x128,
                 fprop -> fp32
  QKV fprop      X [4096][2048] (1% outlier channels) 1x128, W [4096][2048]
                 128x128, fprop -> bf16
  MLP fprop      gate_up X [8192][2048] 1x128 and W [12288][2048] 128x128; down X
                 [8192][6144] (SiLU-gated values) 1x128 and W [2048][6144] 128x128;
                 both fprops -> bf16
  MLP down bwd   dY [8192][2048] (heavy-tailed) dual 1x128 + transposed 128x1,
                 W [2048][6144] dual 128x128 + transposed, X [8192][6144] transposed
                 128x1; dgrad -> bf16 [8192][6144], wgrad -> fp32 [2048][6144]

The larger layer workload's quantizations and GEMMs are covered by
test_gpu_quant.py and test_gpu_layer_gemms.py.  Outputs start poisoned (see
conftest.py), so an element no kernel writes fails."""
import numpy as np
import pytest
import torch

from helpers import DGRAD, FPROP, WGRAD, assert_codes_equal, assert_scales_equal, check_gemm, sample_positions, to_np
from workloads import bits, make

pytestmark = pytest.mark.gpu

puro = pytest.importorskip("blockwise_fp8_gemm_act_amd")


def same(orc_out, gpu_out, what):
    """Codes and scales of one quantization: oracle tuple against GPU tuple, bit for bit."""
    for k, (want, got) in enumerate(zip(orc_out, gpu_out)):
        got = to_np(got)
        if want.dtype == np.uint8:
            assert_codes_equal(got, want, "%s output %d" % (what, k))
        else:
            assert_scales_equal(got, want, "%s output %d" % (what, k))


def gemm_on(mode, a, sa, b, sb, dtype):
    out = puro.gemm_fp8_blockwise(mode, a, sa, b, sb, out_dtype=dtype)
    torch.cuda.synchronize()
    return out


def fprop_pair(orc, t, x_name, w_name):
    """GPU 1x128 codes of X and 128x128 codes of W, checked against the oracle's."""
    xq = puro.quant_act_1x128(t[x_name].cuda())
    wq = puro.quant_w_128x128(t[w_name].cuda())
    torch.cuda.synchronize()
    ox = orc.quant_act_1x128(bits(t[x_name]))
    ow = orc.quant_w_128x128(bits(t[w_name]))
    same(ox, xq, x_name)
    same(ow, wq, w_name)
    return xq, wq, ox, ow


def test_tiny_fprop(orc):
    t = make("tiny_fprop")
    xq, wq, ox, ow = fprop_pair(orc, t, "x", "w")
    out = gemm_on(FPROP, *xq, *wq, torch.float32)
    check_gemm(orc, FPROP, *ox, *ow, out, "tiny fprop")


def test_qkv_fprop(orc):
    t = make("qkv_fprop")
    xq, wq, ox, ow = fprop_pair(orc, t, "x", "w")
    out = gemm_on(FPROP, *xq, *wq, torch.bfloat16)
    ms, ns = sample_positions(4096, 4096, 4096, 21)
    check_gemm(orc, FPROP, *ox, *ow, out, "qkv fprop", ms, ns)


@pytest.mark.parametrize("lin", ["gate_up", "down"])
def test_mlp_fprop(orc, lin):
    t = make("mlp_fprop", names={"x_" + lin, "w_" + lin})
    xq, wq, ox, ow = fprop_pair(orc, t, "x_" + lin, "w_" + lin)
    out = gemm_on(FPROP, *xq, *wq, torch.bfloat16)
    M, N = out.shape
    ms, ns = sample_positions(M, N, 4096, 22 if lin == "down" else 23)
    check_gemm(orc, FPROP, *ox, *ow, out, "mlp fprop " + lin, ms, ns)


def test_mlp_down_backward(orc):
    t = make("mlp_down_bwd")
    dy, w, x = t["dy"].cuda(), t["w"].cuda(), t["x"].cuda()
    dqt, dst, dq, ds = puro.quant_transpose(puro.T_ACT, dy, dual=True)
    wqt, wst, wq, ws = puro.quant_transpose(puro.T_WEIGHT, w, dual=True)
    xqt, xst = puro.quant_transpose(puro.T_ACT, x)
    torch.cuda.synchronize()
    o_dy = orc.quant_act_128x1_t(bits(t["dy"])) + orc.quant_act_1x128(bits(t["dy"]))
    o_w = orc.quant_w_128x128_t(bits(t["w"])) + orc.quant_w_128x128(bits(t["w"]))
    o_x = orc.quant_act_128x1_t(bits(t["x"]))
    same(o_dy, (dqt, dst, dq, ds), "dy dual")
    same(o_w, (wqt, wst, wq, ws), "w dual")
    same(o_x, (xqt, xst), "x transposed")

    dx = gemm_on(DGRAD, dq, ds, wqt, wst, torch.bfloat16)             # [8192][6144]
    ms, ns = sample_positions(8192, 6144, 4096, 24)
    check_gemm(orc, DGRAD, o_dy[2], o_dy[3], o_w[0], o_w[1], dx, "mlp down dgrad", ms, ns)

    dw = gemm_on(WGRAD, dqt, dst, xqt, xst, torch.float32)            # [2048][6144], over 8192 tokens
    ms, ns = sample_positions(2048, 6144, 4096, 25)
    check_gemm(orc, WGRAD, o_dy[0], o_dy[1], o_x[0], o_x[1], dw, "mlp down wgrad", ms, ns)
