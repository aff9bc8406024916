"""Shared helpers of the GPU parity tests (comparison rules, input builders)."""
import numpy as np
import torch

TILE = 128
FPROP, DGRAD, WGRAD = 0, 1, 2
GEMM_TOL = 1e-4          # normalized error |out - ref| / (||A_m|| ||B_n||)


def cdiv(a, b):
    return (a + b - 1) // b


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def bf16_bits_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def assert_codes_equal(got: np.ndarray, want: np.ndarray, what: str):
    assert got.shape == want.shape, (what, got.shape, want.shape)
    bad = np.argwhere(got != want)
    assert bad.size == 0, "%s: %d code mismatches, first at %s: got 0x%02x want 0x%02x" % (
        what, len(bad), tuple(bad[0]), got[tuple(bad[0])], want[tuple(bad[0])])


def assert_scales_equal(got: np.ndarray, want: np.ndarray, what: str):
    assert got.shape == want.shape, (what, got.shape, want.shape)
    g = got.view(np.uint32)
    w = want.view(np.uint32)
    bad = np.argwhere(g != w)
    assert bad.size == 0, "%s: %d scale mismatches, first at %s: got %r want %r" % (
        what, len(bad), tuple(bad[0]), got[tuple(bad[0])], want[tuple(bad[0])])


def bf16_ordered(h: np.ndarray) -> np.ndarray:
    h = h.astype(np.int64)
    mag = h & 0x7FFF
    return np.where(h & 0x8000, -mag, mag)


def check_gemm_values(out: np.ndarray, ref: np.ndarray, na: np.ndarray, nb: np.ndarray,
                      bf16: bool, orc, what: str):
    """out/ref/na/nb aligned arrays (full matrices or samples); a bf16 output is
    passed as its uint16 bit patterns.

    fp32 output: normalized error <= 1e-4 everywhere.
    bf16 output: within 1 bf16 ulp of the oracle's bf16 rounding of its fp64
    value, or (near-cancellation elements) normalized error <= 1e-4.
    Returns (max normalized error, fraction strictly within 1 ulp)."""
    denom = na * nb
    if bf16:
        assert out.dtype == np.uint16, "bf16 outputs are compared as their bit patterns"
        vals = (out.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    else:
        vals = out.astype(np.float64)
    err = np.abs(vals - ref)
    norm = np.where(denom > 0, err / np.where(denom > 0, denom, 1), np.where(err == 0, 0.0, np.inf))
    worst = float(norm.max()) if norm.size else 0.0
    strict = 1.0
    if bf16:
        ref16 = orc.f64_to_bf16_array(ref)
        ulps = np.abs(bf16_ordered(out) - bf16_ordered(ref16))
        ok = (ulps <= 1) | (norm <= GEMM_TOL)
        strict = float(np.mean(ulps <= 1)) if ulps.size else 1.0
        assert ok.all(), "%s: %d elements beyond 1 ulp and tolerance; worst norm err %.3g" % (
            what, int((~ok).sum()), worst)
        return worst, strict
    assert worst <= GEMM_TOL, "%s: normalized error %.3g > %g" % (what, worst, GEMM_TOL)
    return worst, strict


def quantized_operands(orc, mode, M, N, K, seed, outliers=True):
    """Codes and scales for a GEMM of this mode, made by the oracle quantizers
    from seeded bf16 tensors shaped like the layer's operands."""
    from workloads import bits, random_bf16
    if mode == FPROP:
        x = random_bf16((M, K), seed)
        if outliers:
            xf = x.float()
            xf[:, torch.randperm(K, generator=torch.Generator().manual_seed(seed))[:max(1, K // 100)]] *= 20
            x = xf.to(torch.bfloat16)
        w = random_bf16((N, K), seed + 1, std=0.02)
        a, sa = orc.quant_act_1x128(bits(x))
        b, sb = orc.quant_w_128x128(bits(w))
    elif mode == DGRAD:
        dy = random_bf16((M, K), seed, std=1e-3)
        w = random_bf16((K, N), seed + 1, std=0.02)            # W [N_out = K][K_in = N]
        a, sa = orc.quant_act_1x128(bits(dy))
        b, sb = orc.quant_w_128x128_t(bits(w))
    else:
        dy = random_bf16((K, M), seed, std=1e-3)               # dY [T = K][N_out = M]
        x = random_bf16((K, N), seed + 1)                      # X  [T = K][K_in = N]
        a, sa = orc.quant_act_128x1_t(bits(dy))
        b, sb = orc.quant_act_128x1_t(bits(x))
    return a, sa, b, sb
