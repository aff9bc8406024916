"""The C calls enqueue kernels only (no allocation, no memset, no host wait), so
a caller can capture them in a HIP graph.  One linear's forward and backward
operands, its three GEMMs (a split-K wgrad among them), the accumulating
wgrad, the requantizer, the fused SwiGLU, the gate/up fprop with the SwiGLU
epilogue and the token-major wgrad path are captured once and replayed
several times, with eager work between the replays; every replay must give
the eager results bit for bit."""
import numpy as np
import pytest
import torch

from workloads import random_bf16

pytestmark = pytest.mark.gpu

puro = pytest.importorskip("blockwise_fp8_gemm_act_amd")


def cdiv(a, b):
    return (a + b - 1) // b


class Buffers:
    """Inputs and every output of the captured sequence, allocated up front."""

    def __init__(self, T=1024, K=768, N=512, I=256):
        d = "cuda"
        self.T, self.K, self.N, self.I = T, K, N, I
        self.x = random_bf16((T, K), 1).cuda()
        self.w = random_bf16((N, K), 2, std=0.02).cuda()
        self.dy = random_bf16((T, N), 3, std=1e-3).cuda()
        self.gu = random_bf16((T, 2 * I), 4).cuda()
        u8, f32 = torch.uint8, torch.float32
        e = lambda shape, dt=u8: torch.empty(shape, dtype=dt, device=d)
        self.xq, self.xs, self.xqt, self.xst = e((T, K)), e((cdiv(K, 128), T), f32), e((K, T)), e((cdiv(T, 128), K), f32)
        self.wq, self.ws_, self.wqt, self.wst = (e((N, K)), e((cdiv(N, 128), cdiv(K, 128)), f32), e((K, N)),
                                                 e((cdiv(K, 128), cdiv(N, 128)), f32))
        self.dq, self.ds, self.dqt, self.dst = e((T, N)), e((cdiv(N, 128), T), f32), e((N, T)), e((cdiv(T, 128), N), f32)
        self.rqt, self.rst = e((K, T)), e((cdiv(T, 128), K), f32)
        self.hq, self.hs, self.hqt, self.hst = e((T, I)), e((cdiv(I, 128), T), f32), e((I, T)), e((cdiv(T, 128), I), f32)
        self.y = e((T, N), torch.bfloat16)
        self.dx = e((T, K), torch.bfloat16)
        self.dw = e((N, K), f32)
        self.dw_acc = e((N, K), f32)
        self.gu2 = e((T, N), torch.bfloat16)                  # W read as a gate/up weight of inter N / 2
        self.fq, self.fs = e((T, N // 2)), e((N // 256, T), f32)
        self.xc, self.xcs = e((T, K)), e((cdiv(T, 128), K), f32)        # token-major 128x1 codes of X and dY
        self.dc, self.dcs = e((T, N)), e((cdiv(T, 128), N), f32)
        self.dw_tm = e((N, K), f32)
        need = max(puro.puro_gemm_workspace_bytes(m, *s) for m, s in
                   ((puro.FPROP, (T, N, K)), (puro.DGRAD, (T, K, N)), (puro.WGRAD, (N, K, T))))
        self.work = e((max(need, 16),))
        self.need = need

    def outputs(self):
        return [self.xq, self.xs, self.xqt, self.xst, self.wq, self.ws_, self.wqt, self.wst, self.dq, self.ds,
                self.dqt, self.dst, self.rqt, self.rst, self.hq, self.hs, self.hqt, self.hst, self.y, self.dx,
                self.dw, self.dw_acc, self.gu2, self.fq, self.fs, self.xc, self.xcs, self.dc, self.dcs, self.dw_tm]

    def enqueue(self):
        st = torch.cuda.current_stream().cuda_stream
        T, K, N, I = self.T, self.K, self.N, self.I
        p = lambda t: t.data_ptr()
        ok = lambda rc: rc == 0 or pytest.fail(puro.puro_status_str(rc))
        ok(puro.puro_quant_transpose(puro.T_ACT, p(self.x), T, K, p(self.xqt), p(self.xst), p(self.xq), p(self.xs), st))
        ok(puro.puro_quant_transpose(puro.T_WEIGHT, p(self.w), N, K, p(self.wqt), p(self.wst), p(self.wq), p(self.ws_), st))
        ok(puro.puro_quant_transpose(puro.T_ACT, p(self.dy), T, N, p(self.dqt), p(self.dst), p(self.dq), p(self.ds), st))
        ok(puro.puro_requant_act_t(p(self.xq), p(self.xs), T, K, p(self.rqt), p(self.rst), st))
        ok(puro.puro_swiglu_quant(p(self.gu), T, I, p(self.hq), p(self.hs), p(self.hqt), p(self.hst), None, st))
        ok(puro.puro_gemm_fp8_blockwise(puro.FPROP, p(self.xq), p(self.xs), p(self.wq), p(self.ws_), p(self.y),
                                        puro.OUT_BF16, T, N, K, p(self.work), self.need, st))
        ok(puro.puro_gemm_fp8_blockwise(puro.DGRAD, p(self.dq), p(self.ds), p(self.wqt), p(self.wst), p(self.dx),
                                        puro.OUT_BF16, T, K, N, p(self.work), self.need, st))
        ok(puro.puro_gemm_fp8_blockwise(puro.WGRAD, p(self.dqt), p(self.dst), p(self.xqt), p(self.xst), p(self.dw),
                                        puro.OUT_F32, N, K, T, p(self.work), self.need, st))
        ok(puro.puro_gemm_fp8_blockwise_accumulate(puro.WGRAD, p(self.dqt), p(self.dst), p(self.rqt), p(self.rst),
                                                   p(self.dw_acc), N, K, T, p(self.work), self.need, st))
        ok(puro.puro_gemm_fp8_swiglu_quant(p(self.xq), p(self.xs), p(self.wq), p(self.ws_), T, N // 2, K,
                                           p(self.gu2), p(self.fq), p(self.fs), st))
        ok(puro.puro_quant_act_128x1(p(self.x), T, K, p(self.xc), p(self.xcs), None, None, st))
        ok(puro.puro_quant_act_128x1(p(self.dy), T, N, p(self.dc), p(self.dcs), None, None, st))
        ok(puro.puro_gemm_fp8_blockwise(puro.WGRAD_TM, p(self.dc), p(self.dcs), p(self.xc), p(self.xcs), p(self.dw_tm),
                                        puro.OUT_F32, N, K, T, p(self.work), self.need, st))


def snapshot(buf):
    return [t.clone() for t in buf.outputs()]


def same_bits(a, b):
    return torch.equal(a.view(torch.uint8), b.view(torch.uint8))


def test_captured_path_replays_bit_exact():
    buf = Buffers()
    assert buf.need > 0                                      # the wgrad takes the split-K path
    buf.dw_acc.fill_(0.25)
    buf.enqueue()
    torch.cuda.synchronize()
    eager = snapshot(buf)

    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            buf.enqueue()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    for rep in range(3):
        for t in buf.outputs():                              # eager work between replays
            t.zero_()
        buf.dw_acc.fill_(0.25)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (got, want) in enumerate(zip(buf.outputs(), eager)):
            assert same_bits(got, want), "replay %d, output %d differs from the eager run" % (rep, i)
        np.testing.assert_array_equal(buf.xq.cpu().numpy(), eager[0].cpu().numpy())
