"""GPU parity of the blockwise-scaled FP8 GEMM against the oracle's fp64 GEMM.

Operands are made by the oracle quantizers on the host (so these tests
isolate the GEMM) except in the end-to-end test, which quantizes on the GPU.
fp32 outputs: normalized error <= 1e-4; integer-valued cases bit-exact.
bf16 outputs: within 1 ulp of the oracle's rounding, or normalized error <= 1e-4.
"""
import numpy as np
import pytest
import torch

from helpers import (DGRAD, FPROP, WGRAD, bf16_bits_np, cdiv, check_gemm,
                     quantized_operands, to_np, TILE)
from helpers import sample_positions as edge_samples
from workloads import bits, make

pytestmark = pytest.mark.gpu

puro = pytest.importorskip("blockwise_fp8_gemm_act_amd")


def run_gpu(mode, a, sa, b, sb, dtype):
    out = puro.gemm_fp8_blockwise(mode, torch.from_numpy(a).cuda(), torch.from_numpy(sa).cuda(),
                                  torch.from_numpy(b).cuda(), torch.from_numpy(sb).cuda(), out_dtype=dtype)
    torch.cuda.synchronize()
    return out


def out_np(out):
    return bf16_bits_np(out) if out.dtype == torch.bfloat16 else to_np(out)


def check_full(orc, mode, a, sa, b, sb, dtype, what):
    return check_gemm(orc, mode, a, sa, b, sb, run_gpu(mode, a, sa, b, sb, dtype), what)


def test_tiny_fprop_workload_fp32(orc):
    """256x256 activations (2 outlier channels) x 512x256 weight -> fp32, seed 0."""
    t = make("tiny_fprop")
    a, sa = orc.quant_act_1x128(bits(t["x"]))
    b, sb = orc.quant_w_128x128(bits(t["w"]))
    worst, _ = check_full(orc, FPROP, a, sa, b, sb, torch.float32, "tiny fprop")
    print("tiny fprop: max normalized error %.3g" % worst)


@pytest.mark.parametrize("mode", [FPROP, DGRAD, WGRAD])
@pytest.mark.parametrize("M,N,K", [(256, 256, 256), (300, 200, 272), (512, 768, 1024)])
def test_integer_valued_bit_exact(orc, mode, M, N, K):
    """Codes of the integers -8..8 with power-of-two scales: every partial sum
    is exact in fp32, so the fp32 output must equal the oracle bit for bit."""
    rng = np.random.default_rng(M + N + K + mode)
    codes = np.array([orc.e4m3_encode(float(v)) for v in range(-8, 9)], dtype=np.uint8)
    nk = cdiv(K, TILE)
    a = rng.choice(codes, size=(M, K)).astype(np.uint8)
    b = rng.choice(codes, size=(N, K)).astype(np.uint8)
    sa = (np.float32(2.0) ** rng.integers(-3, 4, size=(nk, M))).astype(np.float32)
    sbs = (nk, N) if mode == WGRAD else (cdiv(N, TILE), nk)
    sb = (np.float32(2.0) ** rng.integers(-3, 4, size=sbs)).astype(np.float32)
    out = to_np(run_gpu(mode, a, sa, b, sb, torch.float32))
    ref = orc.gemm(mode, a, sa, b, sb)
    assert np.array_equal(out.astype(np.float64), ref)


@pytest.mark.parametrize("mode", [FPROP, DGRAD])
@pytest.mark.parametrize("M,N,K", [(4096, 4608, 256), (4096, 4608, 384), (8192, 2304, 1024), (2048, 2048, 128),
                                   (4352, 4608, 2048)])
def test_bf16_full_tiles_several_items_bit_exact(orc, mode, M, N, K):
    """The bf16 output of full 256 x 256 tiles, with more tiles than workgroups (some
    workgroups run 2 items, so an item's stores drain while the next item's first
    slices run), K of 2 to 16 slices, and K = 128 (one slice per item).  Integer-valued codes with power-of-two scales
    in [1/4, 4]: every partial sum is a multiple of 2^-4 below 2^20 (asserted through
    the sum of |products|), exact in fp32 and fp64 in any order, so every bf16 element equals the oracle's rounding of the exact
    value, which the product of the oracle's dequantized operands gives at this size."""
    rng = np.random.default_rng(M + N + K + 10 * mode)
    codes = np.array([orc.e4m3_encode(float(v)) for v in range(-8, 9)], dtype=np.uint8)
    nk = cdiv(K, TILE)
    a = rng.choice(codes, size=(M, K)).astype(np.uint8)
    b = rng.choice(codes, size=(N, K)).astype(np.uint8)
    sa = (np.float32(2.0) ** rng.integers(-2, 3, size=(nk, M))).astype(np.float32)
    sb = (np.float32(2.0) ** rng.integers(-2, 3, size=(cdiv(N, TILE), nk))).astype(np.float32)
    out = bf16_bits_np(run_gpu(mode, a, sa, b, sb, torch.bfloat16))
    da, db = orc.dequant_a(a, sa), orc.dequant_b(mode, b, sb)
    assert (np.abs(da) @ np.abs(db).T).max() < 2.0 ** 20       # bounds every partial sum
    exact = da @ db.T
    ms, ns = edge_samples(M, N, 512, M + N)
    assert np.array_equal(exact[ms, ns], orc.gemm_at(mode, a, sa, b, sb, ms, ns))
    ref = orc.f64_to_bf16_array(exact)
    bad = np.argwhere(out != ref)
    assert len(bad) == 0, "%d of %d elements differ, first at %s" % (len(bad), out.size, bad[:4].tolist())


@pytest.mark.parametrize("mode", [FPROP, DGRAD, WGRAD])
@pytest.mark.parametrize("M,N,K", [(200, 300, 144), (1, 17, 16), (257, 129, 400), (640, 384, 2048)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_ragged_shapes(orc, mode, M, N, K, dtype):
    a, sa, b, sb = quantized_operands(orc, mode, M, N, K, seed=M * 7 + N + K)
    check_full(orc, mode, a, sa, b, sb, dtype, "mode %d %dx%dx%d" % (mode, M, N, K))


@pytest.mark.parametrize("mode", [FPROP, WGRAD])
@pytest.mark.parametrize("M,N", [(512, 512), (510, 511)])
def test_split_k_path(orc, mode, M, N):
    """Every tile split over K; the reduction reads 4 partials per thread when M * N is a
    multiple of 4, one otherwise (510 x 511)."""
    K = 4096
    assert puro.puro_gemm_workspace_bytes(mode, M, N, K) > 0
    a, sa, b, sb = quantized_operands(orc, mode, M, N, K, seed=99)
    for dtype in (torch.float32, torch.bfloat16):
        check_full(orc, mode, a, sa, b, sb, dtype, "split-K mode %d" % mode)


@pytest.mark.parametrize("mode,M,N,K", [(FPROP, 8192, 2600, 2048), (WGRAD, 1024, 768, 8192), (DGRAD, 768, 1280, 1040)])
def test_repeated_calls_bitwise_identical(orc, mode, M, N, K):
    """The slice order and split-K sums are fixed: two calls give the same bits (several work items per
    workgroup, a split-K shape, edge tiles and a ragged K)."""
    a, sa, b, sb = quantized_operands(orc, mode, M, N, K, seed=M + N + K)
    for dtype in (torch.float32, torch.bfloat16):
        r1 = run_gpu(mode, a, sa, b, sb, dtype)
        r2 = run_gpu(mode, a, sa, b, sb, dtype)
        iv = torch.int16 if dtype == torch.bfloat16 else torch.int32
        assert torch.equal(r1.view(iv), r2.view(iv)), "mode %d %dx%dx%d %s" % (mode, M, N, K, dtype)


def whole_then_split_check(orc, mode, a, sa, b, sb, out, dtype, what):
    """Every output of the split tiles (rows 1024.., columns 10752..) and samples of the rest."""
    M, N = a.shape[0], b.shape[0]
    rm, rn = np.meshgrid(np.arange(1024, M), np.arange(10752, N), indexing="ij")
    sm, sn = sample_positions(M, N, 4096, M + N)
    ms, ns = np.concatenate([rm.ravel(), sm]), np.concatenate([rn.ravel(), sn])
    check_gemm(orc, mode, a, sa, b, sb, out, what, ms, ns)


@pytest.mark.parametrize("mode", [FPROP, DGRAD])
@pytest.mark.parametrize("N", [10900, 10899])
def test_whole_tiles_then_split_remainder(orc, mode, N):
    """258 output tiles (6 x 43) at 8 K slices: tiles 0-255 fill the compute units once and run whole in a
    first launch; only the last two, ragged in rows, columns and K, are split over K by a second launch and
    summed by the tile-range reduction (4 columns per thread when N is a multiple of 4, else one).  fp32 and
    bf16 out; two calls give the same bits."""
    M, K = 1480, 1008
    assert puro.puro_gemm_workspace_bytes(mode, M, N, K) > 0
    a, sa, b, sb = quantized_operands(orc, mode, M, N, K, seed=258)
    for dtype in (torch.float32, torch.bfloat16):
        r1 = run_gpu(mode, a, sa, b, sb, dtype)
        whole_then_split_check(orc, mode, a, sa, b, sb, r1, dtype, "mode %d %s" % (mode, dtype))
        r2 = run_gpu(mode, a, sa, b, sb, dtype)
        iv = torch.int16 if dtype == torch.bfloat16 else torch.int32
        assert torch.equal(r1.view(iv), r2.view(iv))


def test_whole_tiles_then_split_remainder_accumulate(orc):
    """The same plan in accumulate mode: whole tiles add in the GEMM's epilogue, split tiles in the
    reduction; both are one fp32 addition of the plain result."""
    M, N, K = 1480, 10900, 1008
    a, sa, b, sb = quantized_operands(orc, WGRAD, M, N, K, seed=259)
    dv = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    plain = to_np(run_gpu(WGRAD, a, sa, b, sb, torch.float32))
    c = (np.random.default_rng(7).standard_normal((M, N)) * float(np.abs(plain).mean())).astype(np.float32)
    out = dv(c)
    puro.gemm_fp8_blockwise_accumulate(WGRAD, dv(a), dv(sa), dv(b), dv(sb), out)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(out), c + plain)


def test_zero_k_writes_zeros():
    for dtype in (torch.float32, torch.bfloat16):
        a = torch.zeros((5, 0), dtype=torch.uint8, device="cuda")
        b = torch.zeros((7, 0), dtype=torch.uint8, device="cuda")
        sa = torch.zeros((0, 5), dtype=torch.float32, device="cuda")
        sb = torch.zeros((1, 0), dtype=torch.float32, device="cuda")
        out = torch.full((5, 7), 3.0, dtype=dtype, device="cuda")
        puro.gemm_fp8_blockwise(FPROP, a, sa, b, sb, out=out)
        torch.cuda.synchronize()
        assert torch.all(out == 0)


def sample_positions(M, N, n, seed):
    rng = np.random.default_rng(seed)
    ms = np.concatenate([rng.integers(0, M, n), np.full(64, M - 1), np.zeros(64, np.int64)])
    ns = np.concatenate([rng.integers(0, N, n), rng.integers(0, N, 64), np.arange(64) % N])
    return ms, ns


@pytest.mark.parametrize("which", ["qkv_fprop", "mlp_down_dgrad", "mlp_down_wgrad", "gate_up_wgrad"])
def test_workload_sizes_sampled(orc, which):
    """Full-size GEMMs, in the launch configuration the benchmark uses,
    checked on 4096 sampled outputs plus the first and last rows.  The gate/up
    wgrad of the layer at 16384 tokens (384 tiles) runs its first 256 tiles
    whole and splits the other 128 over K."""
    if which == "gate_up_wgrad":
        t = make("layer", names={"x_gate_up", "dy_gate_up"})
        a, sa = orc.quant_act_128x1_t(bits(t["dy_gate_up"]))
        b, sb = orc.quant_act_128x1_t(bits(t["x_gate_up"]))
        mode, dtype = WGRAD, torch.float32
    elif which == "qkv_fprop":
        t = make("qkv_fprop")
        a, sa = orc.quant_act_1x128(bits(t["x"]))
        b, sb = orc.quant_w_128x128(bits(t["w"]))
        mode, dtype = FPROP, torch.bfloat16
    else:
        t = make("mlp_down_bwd")
        if which == "mlp_down_dgrad":
            a, sa = orc.quant_act_1x128(bits(t["dy"]))
            b, sb = orc.quant_w_128x128_t(bits(t["w"]))
            mode, dtype = DGRAD, torch.bfloat16
        else:
            a, sa = orc.quant_act_128x1_t(bits(t["dy"]))
            b, sb = orc.quant_act_128x1_t(bits(t["x"]))
            mode, dtype = WGRAD, torch.float32
    M, N = a.shape[0], b.shape[0]
    out = run_gpu(mode, a, sa, b, sb, dtype)
    ms, ns = sample_positions(M, N, 4096, {"qkv_fprop": 1, "mlp_down_dgrad": 2, "mlp_down_wgrad": 3,
                                           "gate_up_wgrad": 4}[which])
    check_gemm(orc, mode, a, sa, b, sb, out, which, ms, ns)


def test_end_to_end_gpu_quantizers(orc):
    """Quantize on the GPU, multiply on the GPU; compare with oracle quantize + oracle GEMM."""
    t = make("tiny_fprop")
    x, w = t["x"].cuda(), t["w"].cuda()
    a, sa = puro.quant_act_1x128(x)
    b, sb = puro.quant_w_128x128(w)
    out = puro.gemm_fp8_blockwise(FPROP, a, sa, b, sb, out_dtype=torch.float32)
    torch.cuda.synchronize()
    oa, osa = orc.quant_act_1x128(bits(t["x"]))
    ob, osb = orc.quant_w_128x128(bits(t["w"]))
    check_gemm(orc, FPROP, oa, osa, ob, osb, out, "end to end")


def test_mfma_slice_accumulation_precision(orc):
    """Probe of the matrix cores (v_mfma_f32_16x16x128_f8f6f4), one 128-deep
    slice with unit scales.  Measured behaviour: products are summed in groups
    of 8 consecutive k, each group aligned to its largest product with about
    14 bits kept (smaller bits are dropped); groups then combine without loss.
    So a single slice's error relative to sum|products| is bounded by roughly
    7 * 2^-13 ~ 2^-10.2 in the worst case (one large product next to seven that
    fall just under the cut), and far smaller on ordinary data.  The per-slice
    promotion cannot undo that in-group loss; it bounds the normalized GEMM
    error by the same figure (sum over slices of sum|products| <= ||A_m|| ||B_n||)."""
    rng = np.random.default_rng(2024)
    finite = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)
    M = N = 256
    K = 128
    enc = orc.e4m3_encode

    def run(a, b):
        a = np.ascontiguousarray(a, dtype=np.uint8)
        b = np.ascontiguousarray(b, dtype=np.uint8)
        sa = np.ones((1, M), np.float32)
        sb = np.ones((2, 1), np.float32)
        out = to_np(run_gpu(FPROP, a, sa, b, sb, torch.float32)).astype(np.float64)
        exact = orc.gemm(FPROP, a, sa, b, sb)
        absum = np.abs(orc.dequant_a(a, sa)) @ np.abs(orc.dequant_b(FPROP, b, sb)).T
        return out, exact, absum

    # group structure: 448 at k = 0 plus one 2^-6 (relative 2^-14.8) elsewhere, b = 1
    a = np.zeros((M, K), np.uint8)
    a[:, 0] = enc(448.0)
    for m in range(1, K):
        a[m, m] = enc(2.0 ** -6)
    b = np.full((N, K), enc(1.0), np.uint8)
    out, exact, _ = run(a, b)
    lost = [m for m in range(1, K) if out[m, 0] != exact[m, 0]]
    print("small product dropped next to a dominant one at k =", lost)
    assert all(m < 8 for m in lost)            # only within the dominant product's group of 8

    families = {
        "uniform codes": (rng.choice(finite, (M, K)), rng.choice(finite, (N, K))),
        "normal": (orc.e4m3_encode_array(rng.standard_normal((M, K)).astype(np.float32) * 50),
                   orc.e4m3_encode_array(rng.standard_normal((N, K)).astype(np.float32) * 50)),
    }
    a = orc.e4m3_encode_array(rng.uniform(-0.05, 0.05, (M, K)).astype(np.float32))
    b = orc.e4m3_encode_array(rng.uniform(-1, 1, (N, K)).astype(np.float32))
    a[:, ::8] = enc(448.0)
    b[:, ::8] = enc(1.0)
    families["one dominant per group of 8"] = (a, b)
    worst = {}
    for name, (a, b) in families.items():
        out, exact, absum = run(a, b)
        rel = np.abs(out - exact) / np.where(absum > 0, absum, 1)
        worst[name] = float(rel.max())
        print("%s: max |err| / sum|products| = %.3g (2^%.1f)" % (name, worst[name], np.log2(max(worst[name], 1e-300))))
    assert max(worst.values()) < 2.0 ** -10
    assert worst["normal"] < 2.0 ** -14


def grouped_outliers(R, K, seed, scale=20.0, per_group=4):
    """N(0,1) bf16 [R][K] whose outlier channels (x scale) sit together inside one
    8-wide k group of each 128-deep slice: channels 128j + 8g + i, g = j mod 16, i < per_group.
    The matrix cores then sum each outlier with its neighbours in one group, where
    bits below ~2^-13 of the group's largest product are lost."""
    from workloads import random_bf16
    x = random_bf16((R, K), seed).float()
    cols = [128 * j + 8 * (j % 16) + i for j in range(cdiv(K, 128)) for i in range(per_group) if
            128 * j + 8 * (j % 16) + i < K]
    x[:, cols] *= scale
    return x.to(torch.bfloat16)


@pytest.mark.parametrize("mode", [FPROP, DGRAD, WGRAD])
def test_outliers_sharing_an_mfma_group(orc, mode):
    """Worst-case-shaped layer data, quantized on the GPU: fprop with outlier channels packed
    into one k group of every slice, dgrad with Student-t (df = 2) output gradients, wgrad
    with both (K is tokens there: the heavy tails of dY share k groups; X's outlier
    channels are features).  Checked in full against the oracle: every element within the
    by-construction bound, fp32 normalized error within 1e-4 (the logged margin shows how
    close the in-group loss comes)."""
    from workloads import random_bf16, student_t
    g = torch.Generator().manual_seed(77 + mode)
    M, N, K = 1024, 768, 2048
    dv = lambda t: t.cuda()
    if mode == FPROP:
        x = grouped_outliers(M, K, 5)
        w = random_bf16((N, K), 6, std=0.02)
        a, sa = puro.quant_act_1x128(dv(x))
        b, sb = puro.quant_w_128x128(dv(w))
    elif mode == DGRAD:
        dy = student_t((M, K), g, df=2)
        w = random_bf16((K, N), 6, std=0.02)                    # W [N_out = K][K_in = N]
        a, sa = puro.quant_act_1x128(dv(dy))
        b, sb = puro.quant_transpose(puro.T_WEIGHT, dv(w))[:2]
    else:
        dy = student_t((K, M), g, df=2)                         # dY [T = K][N_out = M]
        x = grouped_outliers(K, N, 5)                           # X [T = K][K_in = N]
        a, sa = puro.quant_transpose(puro.T_ACT, dv(dy))[:2]
        b, sb = puro.quant_transpose(puro.T_ACT, dv(x))[:2]
    torch.cuda.synchronize()
    a, sa, b, sb = (to_np(t) for t in (a, sa, b, sb))
    out = run_gpu(mode, a, sa, b, sb, torch.float32)
    worst, _ = check_gemm(orc, mode, a, sa, b, sb, out, "grouped outliers mode %d" % mode)
    print("grouped outliers, mode %d: max normalized error %.3g" % (mode, worst))


def test_helpers_reject_wrong_scale_layouts(orc):
    """Scale tensors of the wrong layout for the mode are refused before the C call
    (the kernels would read past them)."""
    a, sa, b, sb = quantized_operands(orc, WGRAD, 256, 256, 256, seed=1)
    A, SA, B, SB = (torch.from_numpy(x).cuda() for x in (a, sa, b, sb))
    with pytest.raises(ValueError):
        puro.gemm_fp8_blockwise(FPROP, A, SA, B, SB)                  # row-scaled sb given to a block-scaled mode
    with pytest.raises(ValueError):
        puro.gemm_fp8_blockwise(WGRAD, A, SA[:, :128].contiguous(), B, SB)
    with pytest.raises(TypeError):
        puro.gemm_fp8_blockwise(WGRAD, A, SA.double(), B, SB)
    with pytest.raises(ValueError):
        puro.gemm_fp8_blockwise_accumulate(WGRAD, A, SA, B, SB, torch.zeros((256, 128), device="cuda"))
    out = puro.gemm_fp8_blockwise(WGRAD, A, SA, B, SB, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert out.shape == (256, 256)


@pytest.mark.parametrize("M,N,K,bn", [(2048, 6144, 1024, 192), (2000, 6100, 1040, 192), (4096, 2048, 2048, 128),
                                      (4000, 2000, 2000, 128), (2048, 2048, 8192, 128), (2000, 1990, 8000, 128)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_wgrad_narrow_tiles(orc, M, N, K, bn, dtype):
    """Weight-gradient shapes for which the plan takes 192- or 128-column tiles (whole rounds of
    256 work items): full and ragged edges, and a 128-column plan split over K (its partials summed by
    the reduction in 256 x 128 blocks).  Every output checked; two calls give the same bits."""
    a, sa, b, sb = quantized_operands(orc, WGRAD, M, N, K, seed=M + N + K + bn)
    r1 = run_gpu(WGRAD, a, sa, b, sb, dtype)
    # samples, the first and last rows, and every column of the last (ragged) tile column
    ms, ns = edge_samples(M, N, 4096, M + N)
    em, en = np.meshgrid(np.arange(0, M, 7), np.arange(N - (N % bn or bn), N), indexing="ij")
    ms, ns = np.concatenate([ms, em.ravel()]), np.concatenate([ns, en.ravel()])
    check_gemm(orc, WGRAD, a, sa, b, sb, r1, "wgrad %dx%dx%d" % (M, N, K), ms, ns)
    r2 = run_gpu(WGRAD, a, sa, b, sb, dtype)
    iv = torch.int16 if dtype == torch.bfloat16 else torch.int32
    assert torch.equal(r1.view(iv), r2.view(iv))


@pytest.mark.parametrize("M,N,K", [(2048, 6144, 1024), (4096, 2048, 2048), (2048, 2048, 8192)])
def test_wgrad_narrow_tiles_accumulate(orc, M, N, K):
    """The narrow-tile plans in accumulate mode equal c + the plain result bit for bit."""
    a, sa, b, sb = quantized_operands(orc, WGRAD, M, N, K, seed=M + N + 1)
    dv = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    plain = to_np(run_gpu(WGRAD, a, sa, b, sb, torch.float32))
    c = (np.random.default_rng(3).standard_normal((M, N)) * float(np.abs(plain).mean())).astype(np.float32)
    out = dv(c)
    puro.gemm_fp8_blockwise_accumulate(WGRAD, dv(a), dv(sa), dv(b), dv(sb), out)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(out), c + plain)


@pytest.mark.parametrize("mode", [FPROP, DGRAD])
@pytest.mark.parametrize("M,N,K", [(512, 768, 512), (4096, 4352, 256)])
def test_spread_copy_kernel_matches_edge_kernel(orc, mode, M, N, K):
    """A whole-tile shape (M and N multiples of 256, K of 128, no split) runs the bf16 kernel
    that spreads each slice's copies over the first n-block steps and has no edge code; the
    same operands with 16 more rows of A, or of B, run the kernel with edge tiles.  Every
    output's K sum runs in an order set by its row tile alone, so the outputs they share agree
    bit for bit.  (4096, 4352, 256) gives each workgroup several items, so the next item's
    first slice is copied during the current item's last one."""
    a, sa, b, sb = quantized_operands(orc, mode, M + 16, N + 16, K, seed=M + 3 * N + 7 * K)
    nb = N // TILE
    inner = run_gpu(mode, np.ascontiguousarray(a[:M]), np.ascontiguousarray(sa[:, :M]),
                    np.ascontiguousarray(b[:N]), np.ascontiguousarray(sb[:nb]), torch.bfloat16)
    more_n = run_gpu(mode, np.ascontiguousarray(a[:M]), np.ascontiguousarray(sa[:, :M]), b, sb, torch.bfloat16)
    more_m = run_gpu(mode, a, sa, np.ascontiguousarray(b[:N]), np.ascontiguousarray(sb[:nb]), torch.bfloat16)
    want = out_np(inner)
    assert np.array_equal(out_np(more_n)[:, :N], want), "16 more columns changed the shared outputs"
    assert np.array_equal(out_np(more_m)[:M], want), "16 more rows changed the shared outputs"
    # and the whole-tile result itself is within the rule (sampled at the larger shape)
    ms, ns = (None, None) if M * N <= 1 << 20 else edge_samples(M, N, 20000, seed=M + N)
    check_gemm(orc, mode, np.ascontiguousarray(a[:M]), np.ascontiguousarray(sa[:, :M]), np.ascontiguousarray(b[:N]),
               np.ascontiguousarray(sb[:nb]), inner, "spread mode %d %dx%dx%d" % (mode, M, N, K), ms, ns)


@pytest.mark.parametrize("mode", [FPROP, DGRAD])
def test_row_band_order_matches_walk(orc, mode):
    """8 column tiles, 32 row tiles and an A operand over 128 MiB: the launch takes its tiles in
    a row band of 32 row tiles x 8 column tiles.  With 16 more columns (9 column tiles) the
    same operands run in the plain walk.  Each output's K order depends on its row tile alone,
    so the shared outputs agree bit for bit (none of them is in a split tile: the 9th column
    tile holds the only tiles past the first round)."""
    M, N, K = 8192, 2048, 16512
    a, sa, b, sb = quantized_operands(orc, mode, M, N + 16, K, seed=97 + mode)
    nb = N // TILE
    band = run_gpu(mode, a, sa, np.ascontiguousarray(b[:N]), np.ascontiguousarray(sb[:nb]), torch.bfloat16)
    walk = run_gpu(mode, a, sa, b, sb, torch.bfloat16)
    assert np.array_equal(out_np(walk)[:, :N], out_np(band)), "the row band changed the sums"
    ms, ns = edge_samples(M, N, 20000, seed=M + N + mode)
    check_gemm(orc, mode, a, sa, np.ascontiguousarray(b[:N]), np.ascontiguousarray(sb[:nb]), band,
               "row band mode %d %dx%dx%d" % (mode, M, N, K), ms, ns)
