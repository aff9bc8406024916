"""GPU parity of the quantizers: codes and scales bit-exact against the oracle."""
import numpy as np
import pytest
import torch

from helpers import assert_codes_equal, assert_scales_equal, cdiv, to_np, TILE
from workloads import LINEARS, bits, make, random_bf16

pytestmark = pytest.mark.gpu

puro = pytest.importorskip("blockwise_fp8_gemm_act_amd")


def outlier_input(R, C, seed, n_out=3):
    x = random_bf16((R, C), seed).float()
    g = torch.Generator().manual_seed(seed + 1)
    cols = torch.randperm(C, generator=g)[:n_out]
    x[:, cols] *= 20
    return x.to(torch.bfloat16)


def special_input(R, C, seed):
    """Random input whose first tiles hold zeros, -0, tiny values (divide
    path), subnormal bf16 values and exact e4m3 values."""
    x = outlier_input(R, C, seed)
    xb = bits(x).copy()
    n = min(R, 8)
    xb[0, :min(C, 128)] = 0                                    # all-zero tile
    if n > 1:
        xb[1, :min(C, 128)] = 0x8000                           # all -0 tile
    if n > 2:
        xb[2, :] = np.random.default_rng(seed).integers(1, 0x0080, C, dtype=np.uint16)       # subnormal bf16
    if n > 3:
        xb[3, :] = np.random.default_rng(seed + 1).integers(0x0080, 0x1F00, C, dtype=np.uint16)  # tiny normals
        xb[3, ::2] |= 0x8000
    if n > 4:
        xb[4, :] = 0x43E0                                      # 448 everywhere
    return torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16)


def check_act(orc, xb):
    q, s = puro.quant_act_1x128(xb.cuda())
    torch.cuda.synchronize()
    oq, os_ = orc.quant_act_1x128(bits(xb))
    assert_codes_equal(to_np(q), oq, "act codes")
    assert_scales_equal(to_np(s), os_, "act scales")


def check_w(orc, wb):
    q, s = puro.quant_w_128x128(wb.cuda())
    torch.cuda.synchronize()
    oq, os_ = orc.quant_w_128x128(bits(wb))
    assert_codes_equal(to_np(q), oq, "w codes")
    assert_scales_equal(to_np(s), os_, "w scales")


def check_t(orc, kind, xb, dual):
    res = puro.quant_transpose(kind, xb.cuda(), dual=dual)
    torch.cuda.synchronize()
    if kind == puro.T_ACT:
        oqt, ost = orc.quant_act_128x1_t(bits(xb))
        orow = orc.quant_act_1x128(bits(xb))
    else:
        oqt, ost = orc.quant_w_128x128_t(bits(xb))
        orow = orc.quant_w_128x128(bits(xb))
    assert_codes_equal(to_np(res[0]), oqt, "transposed codes")
    assert_scales_equal(to_np(res[1]), ost, "transposed scales")
    if dual:
        assert_codes_equal(to_np(res[2]), orow[0], "dual row codes")
        assert_scales_equal(to_np(res[3]), orow[1], "dual row scales")


@pytest.mark.parametrize("R,C", [(256, 256), (37, 400), (130, 16), (1, 128), (64, 1040), (300, 2048), (1040, 8320)])
def test_act_1x128(orc, R, C):
    check_act(orc, outlier_input(R, C, R + C))
    check_act(orc, special_input(R, C, 3 * R + C))


@pytest.mark.parametrize("R,C", [(512, 256), (200, 336), (17, 48), (128, 128), (1000, 1024)])
def test_w_128x128(orc, R, C):
    check_w(orc, random_bf16((R, C), R * 3 + C, std=0.02))
    check_w(orc, special_input(R, C, R + 7))


@pytest.mark.parametrize("R,C", [(256, 384), (144, 80), (16, 16), (1024, 2064),
                                 (16, 4096), (144, 4112), (400, 4096), (768, 6144), (1040, 8320), (2064, 8192)])
@pytest.mark.parametrize("dual", [False, True])
def test_transpose_act(orc, R, C, dual):
    """Ragged rows and columns, from a single 16-row block to inputs 4096-8320 wide (at least
    64 blocks wide: launched in bands of 8 block rows, with a short last band)."""
    check_t(orc, puro.T_ACT, outlier_input(R, C, R + 2 * C), dual)
    check_t(orc, puro.T_ACT, special_input(R, C, R + 5), dual)


@pytest.mark.parametrize("R,C", [(256, 384), (208, 144), (2048, 512), (400, 8320)])
@pytest.mark.parametrize("dual", [False, True])
def test_transpose_w(orc, R, C, dual):
    check_t(orc, puro.T_WEIGHT, random_bf16((R, C), R + C, std=0.02), dual)
    check_t(orc, puro.T_WEIGHT, special_input(R, C, C + 9), dual)


def test_every_bf16_value_under_many_scales(orc):
    """Tiles holding every finite bf16 magnitude <= amax (both signs) behind a
    first element equal to amax, for 48 tile maxima spread over the whole
    exponent range (tiny ones take the division path): row tiles, and the same
    tiles as columns through the transposed quantizer."""
    all_bits = np.arange(0, 0x7F80, dtype=np.uint32)
    allf = (all_bits << 16).view(np.float32)
    rng = np.random.default_rng(12)
    amax_bits = np.unique(np.concatenate([rng.integers(1, 0x7F80, 40),
                                          [0x3F80, 0x43E0, 0x0001, 0x0080, 0x7F7F, 0x1F00, 0x2000, 0x1F7F]]))
    rows = []
    for ab in amax_bits:
        amax = (np.uint32(ab) << 16).view(np.float32)
        mags = all_bits[allf <= amax]
        vals = np.concatenate([mags, mags | 0x8000]).astype(np.uint16)
        nt = cdiv(len(vals), TILE - 1)
        pad = np.zeros(nt * (TILE - 1), dtype=np.uint16)
        pad[:len(vals)] = vals
        t = np.empty((nt, TILE), dtype=np.uint16)
        t[:, 0] = ab
        t[:, 1:] = pad.reshape(nt, TILE - 1)
        rows.append(t)
    tiles = np.concatenate(rows)
    tiles = tiles[: (len(tiles) // 16) * 16]                       # rows a multiple of 16
    xb = torch.from_numpy(tiles.view(np.int16)).view(torch.bfloat16)
    check_act(orc, xb)
    xt = torch.from_numpy(np.ascontiguousarray(tiles.T).view(np.int16)).view(torch.bfloat16)
    check_t(orc, puro.T_ACT, xt, dual=False)


def test_empty_inputs_enqueue_nothing():
    x = torch.zeros((0, 128), dtype=torch.bfloat16, device="cuda")
    q, s = puro.quant_act_1x128(x)
    assert q.shape == (0, 128) and s.shape == (1, 0)
    x = torch.zeros((64, 0), dtype=torch.bfloat16, device="cuda")
    q, s = puro.quant_w_128x128(x)
    assert q.shape == (64, 0)
    torch.cuda.synchronize()


@pytest.mark.parametrize("name", [f"{k}_{lin}" for lin in LINEARS for k in ("x", "w", "dy")])
def test_layer_tensors_in_bench_form(orc, name):
    """Each of the layer step's 12 quantizations at 16384 tokens, in the form the benchmark
    runs it: the dual transposed quantizer (ACT for inputs and output gradients, WEIGHT for
    weights), codes and scales of both outputs bit-exact."""
    t = make("layer", names={name})[name]
    check_t(orc, puro.T_WEIGHT if name.startswith("w_") else puro.T_ACT, t, dual=True)


def test_workload_sizes(orc):
    """Full-size tensors of the layer workload (16384 tokens): activation
    quantizer on the gate_up input, dual transposed quantizer on the gate_up
    output gradient (the largest tensor), weight quantizers on W_down."""
    t = make("layer", names={"x_gate_up", "dy_gate_up", "w_down"})
    check_act(orc, t["x_gate_up"])
    check_t(orc, puro.T_ACT, t["dy_gate_up"], dual=True)
    check_w(orc, t["w_down"])
    check_t(orc, puro.T_WEIGHT, t["w_down"], dual=True)


@pytest.mark.parametrize("outputs", ["both", "row", "transposed"])
def test_quant_weights_grouped(orc, outputs):
    """One launch over the layer's four weights plus ragged and empty ones: each entry's codes
    and scales bit-exact against the oracle's 128x128 quantizer and its transpose."""
    row, tr = outputs in ("both", "row"), outputs in ("both", "transposed")
    t = make("layer", names={"w_" + lin for lin in LINEARS})
    ws = [t["w_" + lin] for lin in LINEARS]
    ws.append(special_input(272, 400, 5))            # ragged in both directions, special tiles
    ws.append(outlier_input(0, 128, 6))               # empty
    ws.append(outlier_input(144, 16, 7))
    got = puro.quant_weights([w.cuda() for w in ws], row=row, transposed=tr)
    torch.cuda.synchronize()
    for i, (w, (q, s_, qt, st)) in enumerate(zip(ws, got)):
        if w.numel() == 0:
            continue
        if row:
            oq, os_ = orc.quant_w_128x128(bits(w))
            assert_codes_equal(to_np(q), oq, "weight %d codes" % i)
            assert_scales_equal(to_np(s_), os_, "weight %d scales" % i)
        if tr:
            oqt, ost = orc.quant_w_128x128_t(bits(w))
            assert_codes_equal(to_np(qt), oqt, "weight %d transposed codes" % i)
            assert_scales_equal(to_np(st), ost, "weight %d transposed scales" % i)
