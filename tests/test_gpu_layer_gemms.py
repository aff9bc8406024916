"""Every GEMM of the benchmark's layer step (one Qwen3-1.7B-shaped layer at 16384
tokens: four linears, fprop, dgrad and wgrad each), and the two GEMMs of the MLP
forward at 8192 tokens, at their full sizes and in the launch configuration the
benchmark uses.  Operands are the oracle's quantizations of the seeded workload
tensors; each output is checked against the oracle on 2048 sampled positions
plus the first and last rows: fprop and dgrad in bf16 (1-ulp rule), wgrad in
fp32 (normalized error <= 1e-4)."""
import numpy as np
import pytest
import torch

from helpers import DGRAD, FPROP, WGRAD, check_gemm
from workloads import LINEARS, bits, make

pytestmark = pytest.mark.gpu

puro = pytest.importorskip("blockwise_fp8_gemm_act_amd")


def operands(orc, workload, names, op):
    """Codes and scales (a, sa, b, sb) of one GEMM, quantized by the oracle."""
    x_name, w_name, dy_name = names
    t = make(workload, names={n for n in names if n})
    if op == "fprop":
        return orc.quant_act_1x128(bits(t[x_name])) + orc.quant_w_128x128(bits(t[w_name]))
    if op == "dgrad":
        return orc.quant_act_1x128(bits(t[dy_name])) + orc.quant_w_128x128_t(bits(t[w_name]))
    return orc.quant_act_128x1_t(bits(t[dy_name])) + orc.quant_act_128x1_t(bits(t[x_name]))


def check(orc, mode, a, sa, b, sb, dtype, seed, what):
    dv = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    out = puro.gemm_fp8_blockwise(mode, dv(a), dv(sa), dv(b), dv(sb), out_dtype=dtype)
    torch.cuda.synchronize()
    M, N = a.shape[0], b.shape[0]
    rng = np.random.default_rng(seed)
    ms = np.concatenate([rng.integers(0, M, 2048), np.zeros(min(N, 512), np.int64), np.full(min(N, 512), M - 1)])
    ns = np.concatenate([rng.integers(0, N, 2048), np.arange(min(N, 512)), N - 1 - np.arange(min(N, 512))])
    check_gemm(orc, mode, a, sa, b, sb, out, what, ms, ns)


@pytest.mark.parametrize("op", ["fprop", "dgrad", "wgrad"])
@pytest.mark.parametrize("lin", list(LINEARS))
def test_layer_gemm(orc, lin, op):
    names = (f"x_{lin}" if op != "dgrad" else None, f"w_{lin}" if op != "wgrad" else None,
             f"dy_{lin}" if op != "fprop" else None)
    a, sa, b, sb = operands(orc, "layer", names, op)
    mode, dtype = {"fprop": (FPROP, torch.bfloat16), "dgrad": (DGRAD, torch.bfloat16),
                   "wgrad": (WGRAD, torch.float32)}[op]
    seed = 10 * list(LINEARS).index(lin) + ["fprop", "dgrad", "wgrad"].index(op)
    check(orc, mode, a, sa, b, sb, dtype, seed, "%s %s" % (lin, op))


@pytest.mark.parametrize("lin", ["gate_up", "down"])
def test_mlp_forward_8192_tokens(orc, lin):
    a, sa, b, sb = operands(orc, "mlp_fprop", (f"x_{lin}", f"w_{lin}", None), "fprop")
    assert a.shape[0] == 8192
    check(orc, FPROP, a, sa, b, sb, torch.bfloat16, 7 if lin == "down" else 8, "mlp forward %s" % lin)
