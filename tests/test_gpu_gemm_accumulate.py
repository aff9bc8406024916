"""GPU parity of the accumulating GEMM, out = fp32(out + GEMM), against the
oracle's fp64 c + GEMM.  Bound per element: the GEMM's normalized tolerance
plus the rounding of the one fp32 addition (2^-24 of the sum, with slack)."""
import numpy as np
import pytest
import torch

from helpers import DGRAD, FPROP, WGRAD, GEMM_TOL, quantized_operands, to_np
from workloads import bits, make

pytestmark = pytest.mark.gpu

puro = pytest.importorskip("blockwise_fp8_gemm_act_amd")


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def run_acc(mode, a, sa, b, sb, c):
    out = dev(c.astype(np.float32))
    puro.gemm_fp8_blockwise_accumulate(mode, dev(a), dev(sa), dev(b), dev(sb), out)
    torch.cuda.synchronize()
    return out


def check_acc(got, ref, na, nb, what):
    bound = GEMM_TOL * na * nb * (1 + 2.0 ** -23) + 2.0 ** -23 * np.abs(ref)
    err = np.abs(got.astype(np.float64) - ref)
    bad = np.argwhere(err > bound)
    assert bad.size == 0, "%s: %d elements beyond the bound, first %s: got %r want %r" % (
        what, len(bad), tuple(bad[0]), got[tuple(bad[0])], ref[tuple(bad[0])])


def start_values(M, N, seed, scale):
    return (np.random.default_rng(seed).standard_normal((M, N)) * scale).astype(np.float32)


@pytest.mark.parametrize("mode", [FPROP, DGRAD, WGRAD])
@pytest.mark.parametrize("M,N,K", [(200, 300, 144), (257, 129, 400), (512, 512, 4096)])
def test_accumulate_matches_oracle(orc, mode, M, N, K):
    """Ragged tiles, and a split-K shape (512 x 512 x 4096) where the reduction adds."""
    a, sa, b, sb = quantized_operands(orc, mode, M, N, K, seed=M * 7 + K)
    g = orc.gemm(mode, a, sa, b, sb)
    c = start_values(M, N, M + N, float(np.abs(g).mean()) + 1e-30)
    got = to_np(run_acc(mode, a, sa, b, sb, c))
    na, nb = orc.deq_row_norms(mode, a, sa, b, sb)
    check_acc(got, orc.gemm_accumulate(mode, a, sa, b, sb, c), na[:, None], nb[None, :], "mode %d" % mode)


@pytest.mark.parametrize("mode,M,N,K", [(FPROP, 300, 200, 272), (WGRAD, 512, 512, 4096)])
def test_accumulate_is_one_fp32_addition_of_the_plain_result(orc, mode, M, N, K):
    """out + GEMM with the plain GEMM's fp32 value, bit for bit; onto zeros it is the plain result."""
    a, sa, b, sb = quantized_operands(orc, mode, M, N, K, seed=5)
    plain = to_np(puro.gemm_fp8_blockwise(mode, dev(a), dev(sa), dev(b), dev(sb), out_dtype=torch.float32))
    c = start_values(M, N, 8, float(np.abs(plain).mean()))
    got = to_np(run_acc(mode, a, sa, b, sb, c))
    assert np.array_equal(got, c + plain)
    zero = to_np(run_acc(mode, a, sa, b, sb, np.zeros((M, N), np.float32)))
    assert np.array_equal(zero, plain)


def test_two_micro_batches(orc):
    """dW += dY1^T X1, then dW += dY2^T X2 (split-K shape): against c + G1 + G2 in fp64."""
    M, N, K = 512, 768, 4096
    a1, sa1, b1, sb1 = quantized_operands(orc, WGRAD, M, N, K, seed=31)
    a2, sa2, b2, sb2 = quantized_operands(orc, WGRAD, M, N, K, seed=32)
    c = start_values(M, N, 3, 1e-3)
    out = dev(c)
    for a, sa, b, sb in ((a1, sa1, b1, sb1), (a2, sa2, b2, sb2)):
        puro.gemm_fp8_blockwise_accumulate(WGRAD, dev(a), dev(sa), dev(b), dev(sb), out)
    torch.cuda.synchronize()
    ref = c.astype(np.float64) + orc.gemm(WGRAD, a1, sa1, b1, sb1) + orc.gemm(WGRAD, a2, sa2, b2, sb2)
    na1, nb1 = orc.deq_row_norms(WGRAD, a1, sa1, b1, sb1)
    na2, nb2 = orc.deq_row_norms(WGRAD, a2, sa2, b2, sb2)
    got = to_np(out).astype(np.float64)
    bound = GEMM_TOL * (na1[:, None] * nb1[None, :] + na2[:, None] * nb2[None, :]) * 1.001 + 2.0 ** -22 * np.abs(ref)
    assert np.all(np.abs(got - ref) <= bound)


def test_zero_k_leaves_out_unchanged():
    a = torch.zeros((5, 0), dtype=torch.uint8, device="cuda")
    b = torch.zeros((7, 0), dtype=torch.uint8, device="cuda")
    sa = torch.zeros((0, 5), dtype=torch.float32, device="cuda")
    sb = torch.zeros((1, 0), dtype=torch.float32, device="cuda")
    out = torch.full((5, 7), 3.0, dtype=torch.float32, device="cuda")
    puro.gemm_fp8_blockwise_accumulate(FPROP, a, sa, b, sb, out)
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)


def test_workload_size_wgrad_sampled(orc):
    """The MLP-down wgrad of the 8192-token workload (2048 x 6144, K = 8192) accumulated onto
    a nonzero fp32 gradient; 4096 sampled outputs plus edge rows."""
    t = make("mlp_down_bwd")
    a, sa = orc.quant_act_128x1_t(bits(t["dy"]))
    b, sb = orc.quant_act_128x1_t(bits(t["x"]))
    M, N = a.shape[0], b.shape[0]
    c = start_values(M, N, 11, 1e-2)
    got = to_np(run_acc(WGRAD, a, sa, b, sb, c))
    rng = np.random.default_rng(4)
    ms = np.concatenate([rng.integers(0, M, 4096), np.full(64, M - 1), np.zeros(64, np.int64)])
    ns = np.concatenate([rng.integers(0, N, 4096), rng.integers(0, N, 64), np.arange(64) % N])
    ref = c[ms, ns].astype(np.float64) + orc.gemm_at(WGRAD, a, sa, b, sb, ms, ns)
    na, nb = orc.deq_row_norms(WGRAD, a, sa, b, sb)
    check_acc(got[ms, ns], ref, na[ms], nb[ns], "mlp_down wgrad accumulate")
