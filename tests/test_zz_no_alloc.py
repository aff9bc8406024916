"""The allocation-free GEMM entry point, puro_gemm_fp8_blockwise_noalloc, through
the C ABI: its output equals puro_gemm_fp8_blockwise's (with a caller's
workspace) bit for bit -- the same plan and kernels -- on two calls in a row,
the first filling the whole 64 MiB scratch (the layer's O-projection weight
gradient at 16384 tokens, split 4 ways), the second a smaller split shape, then
a shape with no split.  Outputs start as NaN so an element left unwritten
fails."""
import numpy as np
import pytest
import torch

from workloads import random_codes, random_scales

pytestmark = pytest.mark.gpu

puro = pytest.importorskip("blockwise_fp8_gemm_act_amd")


def operands(mode, M, N, K, seed):
    nk = (K + 127) // 128
    a = torch.from_numpy(random_codes((M, K), seed)).cuda()
    b = torch.from_numpy(random_codes((N, K), seed + 1)).cuda()
    sa = torch.from_numpy(random_scales((nk, M), seed + 2, -12, -4)).cuda()
    sbs = (nk, N) if mode == puro.WGRAD else ((N + 127) // 128, nk)
    sb = torch.from_numpy(random_scales(sbs, seed + 3, -12, -4)).cuda()
    return a, sa, b, sb


def both(mode, M, N, K, dtype, seed):
    a, sa, b, sb = operands(mode, M, N, K, seed)
    od = puro.OUT_BF16 if dtype == torch.bfloat16 else puro.OUT_F32
    stream = torch.cuda.current_stream().cuda_stream
    need = puro.puro_gemm_workspace_bytes(mode, M, N, K)
    ws = torch.full((max(need, 16),), 0xFF, dtype=torch.uint8, device="cuda")
    ref = torch.full((M, N), float("nan"), dtype=dtype, device="cuda")
    got = torch.full((M, N), float("nan"), dtype=dtype, device="cuda")
    assert puro.puro_gemm_fp8_blockwise(mode, a.data_ptr(), sa.data_ptr(), b.data_ptr(), sb.data_ptr(),
                                        ref.data_ptr(), od, M, N, K, ws.data_ptr(), need, stream) == 0
    assert puro.puro_gemm_fp8_blockwise_noalloc(mode, a.data_ptr(), sa.data_ptr(), b.data_ptr(), sb.data_ptr(),
                                                got.data_ptr(), od, M, N, K, stream) == 0
    torch.cuda.synchronize()
    iv = torch.int16 if dtype == torch.bfloat16 else torch.int32
    assert not torch.isnan(got.float()).any(), "unwritten outputs"
    assert torch.equal(got.view(iv), ref.view(iv)), "noalloc differs from the workspace entry point"
    return need


def test_noalloc_matches_workspace_entry_point():
    need = both(puro.WGRAD, 2048, 2048, 16384, torch.float32, 11)      # the whole scratch
    assert need == puro.SCRATCH_BYTES
    need2 = both(puro.WGRAD, 512, 768, 4096, torch.bfloat16, 12)       # smaller, split, after it
    assert 0 < need2 < need
    assert both(puro.FPROP, 1000, 300, 256, torch.float32, 13) == 0   # no split: no scratch


def test_noalloc_refuses_plans_beyond_the_scratch():
    a = torch.zeros(16, dtype=torch.uint8, device="cuda")
    st = puro.puro_gemm_fp8_blockwise_noalloc(puro.WGRAD, a.data_ptr(), a.data_ptr(), a.data_ptr(), a.data_ptr(),
                                              a.data_ptr() + 4096, puro.OUT_F32, 2560, 2560, 1 << 20, None)
    assert st == 10 and "64 MiB" in puro.puro_status_str(st)
