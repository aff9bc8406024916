"""The GEMM at the largest K the ABI accepts (2^23: 256 rows x K must index in 32
bits), on a full 256x256 tile so that the interior copy path with its 32-bit lane
offsets runs, split over K.  Codes of -1, 0 and 1 with unit scales keep every
partial sum an integer below 2^24 in any order, so the output is exact: it must
equal the oracle's value bit for bit on a full row, a full column and random
samples."""
import numpy as np
import pytest
import torch

from helpers import FPROP, DGRAD, to_np, TILE

pytestmark = pytest.mark.gpu

puro = pytest.importorskip("blockwise_fp8_gemm_act_amd")


@pytest.mark.parametrize("mode", [FPROP, DGRAD])
def test_maximum_k_full_tile(orc, mode):
    M = N = 256
    K = 1 << 23
    table = np.array([orc.e4m3_encode(v) for v in (-1.0, 0.0, 1.0)], dtype=np.uint8)
    g = torch.Generator()
    g.manual_seed(20 + mode)
    a = table[torch.randint(0, 3, (M, K), generator=g, dtype=torch.uint8).numpy()]
    b = table[torch.randint(0, 3, (N, K), generator=g, dtype=torch.uint8).numpy()]
    nk = K // TILE
    sa = np.ones((nk, M), dtype=np.float32)
    sb = np.ones((N // TILE, nk), dtype=np.float32)
    assert puro.puro_gemm_workspace_bytes(mode, M, N, K) > 0            # the split-K path
    out = puro.gemm_fp8_blockwise(mode, *[torch.from_numpy(t).cuda() for t in (a, sa, b, sb)],
                                  out_dtype=torch.float32)
    torch.cuda.synchronize()
    o = to_np(out)
    rng = np.random.default_rng(mode)
    ms = np.concatenate([np.zeros(N, np.int64), np.arange(M), rng.integers(0, M, 64)])
    ns = np.concatenate([np.arange(N), np.full(M, N - 1), rng.integers(0, N, 64)])
    ref = orc.gemm_at(mode, a, sa, b, sb, ms, ns)
    assert np.abs(ref).max() < 2 ** 24
    assert np.array_equal(o[ms, ns].astype(np.float64), ref)
