"""Calls on explicit streams and from several host threads at once.

The binding's helpers run on the stream they are given (a torch.cuda.Stream or a
raw hipStream_t handle) and allocate their outputs and workspace there; the C
calls keep no per-call state, so calls from several host threads, each on its
own stream, give the single-threaded results bit for bit."""
import threading

import pytest
import torch

from workloads import random_bf16

pytestmark = pytest.mark.gpu

puro = pytest.importorskip("blockwise_fp8_gemm_act_amd")


def same_bits(a, b):
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


def path(x, w, dy, stream=None):
    """Quantizers, the three GEMMs of one linear (the wgrad split over K) and the fused SwiGLU quantizer."""
    xq, xs = puro.quant_act_1x128(x, stream=stream)
    xqt, xst = puro.quant_transpose(puro.T_ACT, x, stream=stream)
    wqt, wst, wq, ws = puro.quant_transpose(puro.T_WEIGHT, w, dual=True, stream=stream)
    dqt, dst, dq, ds = puro.quant_transpose(puro.T_ACT, dy, dual=True, stream=stream)
    y = puro.gemm_fp8_blockwise(puro.FPROP, xq, xs, wq, ws, stream=stream)
    dx = puro.gemm_fp8_blockwise(puro.DGRAD, dq, ds, wqt, wst, stream=stream)
    dw = puro.gemm_fp8_blockwise(puro.WGRAD, dqt, dst, xqt, xst, out_dtype=torch.float32, stream=stream)
    hq, hs = puro.swiglu_quant(y, stream=stream)
    rqt, rst = puro.requant_act_t(xq, xs, stream=stream)
    return [xq, xs, xqt, xst, wq, ws, dq, ds, y, dx, dw, hq, hs, rqt, rst]


def operands(seed):
    x = random_bf16((1024, 512), seed).cuda()
    w = random_bf16((768, 512), seed + 1, std=0.02).cuda()
    dy = random_bf16((1024, 768), seed + 2, std=1e-3).cuda()
    return x, w, dy


def test_explicit_streams_match_the_current_stream():
    x, w, dy = operands(1)
    assert puro.puro_gemm_workspace_bytes(puro.WGRAD, 768, 512, 1024) > 0     # the wgrad splits over K
    want = path(x, w, dy)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    got = path(x, w, dy, stream=side)                        # a torch.cuda.Stream
    side.synchronize()
    raw = path(x, w, dy, stream=side.cuda_stream)            # the raw handle of the same stream
    side.synchronize()
    for i, (a, b, c) in enumerate(zip(want, got, raw)):
        assert same_bits(a, b) and same_bits(a, c), "output %d" % i


def test_threads_each_on_their_own_stream():
    data = [operands(10 * t) for t in range(4)]
    want = [path(*d) for d in data]
    torch.cuda.synchronize()
    errors = []

    def worker(t):
        try:
            s = torch.cuda.Stream()
            for _ in range(3):
                with torch.cuda.stream(s):
                    got = path(*data[t])
                s.synchronize()
                for i, (a, b) in enumerate(zip(want[t], got)):
                    if not same_bits(a, b):
                        errors.append("thread %d output %d" % (t, i))
        except Exception as e:                                # reported below, on the main thread
            errors.append("thread %d: %r" % (t, e))

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(4)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not any(th.is_alive() for th in threads), "a thread did not finish"
    assert not errors, errors
