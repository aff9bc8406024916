"""Shared helpers of the GPU parity tests (comparison rules, input builders)."""
import json
import os

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


# Error of the matrix cores, by construction.  The FP8 MFMA sums each 128-deep
# slice in groups of 8 consecutive k; inside a group every product is aligned to
# the group's largest and bits below about 2^-13 of it are dropped (measured by
# test_mfma_slice_accumulation_precision), so a group loses less than
# 7 * 2^-13 of its largest |product|, hence of its sum of |products|.  Each
# slice's promotion into the fp32 accumulator adds one fp32 rounding, at most
# 2^-24 of the running sum of |terms|.  So for every output element
#     |acc - ref| <= (7 * 2^-13 + (nk + 2) * 2^-24) * S,   S = sum_k |A[m,k] B[n,k]|,
# with nk the number of slices, whatever the data.  A bf16 output adds half an
# ulp of its own rounding.
MFMA_GROUP_REL = 7.0 * 2.0 ** -13
# A bf16 element more than 1 ulp from the oracle's rounding must be a
# near-cancellation one: beyond 1 ulp means |out - ref| > ulp(ref) / 2 >= 2^-9 |ref|,
# and the element's error is at most its own bound above, so |ref| < 2^9 * bound.
# Such elements must also stay rare: at most 1% of the compared elements (plus 4,
# for small samples).  On the workloads 0.1-0.3% take this path.
FALLBACK_MAX_FRAC = 0.01
PARITY_LOG = os.environ.get("PURO_PARITY_LOG")


def hw_error_bound(absum: np.ndarray, nk: int) -> np.ndarray:
    return (MFMA_GROUP_REL + (nk + 2) * 2.0 ** -24) * absum


def _deq_abs(orc, codes: np.ndarray, scale_of_k: np.ndarray) -> np.ndarray:
    """|dequantized values| of some operand rows: |dec(codes)| * scales, in fp32 (at
    most one rounding, 2^-24 relative: the sums below are bounds, not results)."""
    return np.abs(orc.e4m3_decode_table().astype(np.float32)[codes]) * scale_of_k.astype(np.float32)


def abs_products_at(orc, mode, a, sa, b, sb, ms, ns) -> np.ndarray:
    """S[i] = sum_k |A[ms[i], k]| * |B[ns[i], k]| of the dequantized operands (fp64):
    the scale of the rounding errors any summation of these products can make."""
    if mode == 3:                                           # token-major wgrad: a [K][M], b [K][N]
        a, b, mode = np.ascontiguousarray(a.T), np.ascontiguousarray(b.T), WGRAD
    K = a.shape[1]
    kb = np.arange(K) // TILE
    ua, ia = np.unique(ms, return_inverse=True)
    ub, ib = np.unique(ns, return_inverse=True)
    A = _deq_abs(orc, a[ua], sa[kb][:, ua].T)
    if mode == WGRAD:
        B = _deq_abs(orc, b[ub], sb[kb][:, ub].T)
    else:
        B = _deq_abs(orc, b[ub], sb[ub // TILE][:, kb])
    out = np.empty(len(ms), np.float64)
    for i0 in range(0, len(ms), 512):
        sl = slice(i0, i0 + 512)
        out[sl] = (A[ia[sl]] * B[ib[sl]]).sum(axis=1, dtype=np.float64)
    return out * (1 + 2.0 ** -20)


def abs_products_full(orc, mode, a, sa, b, sb) -> np.ndarray:
    """|A| |B|^T of the dequantized operands (fp64), the whole [M][N] matrix."""
    if mode == 3:
        a, b, mode = np.ascontiguousarray(a.T), np.ascontiguousarray(b.T), WGRAD
    K = a.shape[1]
    kb = np.arange(K) // TILE
    A = _deq_abs(orc, a, sa[kb].T).astype(np.float64)
    B = _deq_abs(orc, b, sb[kb].T if mode == WGRAD else sb[np.arange(b.shape[0]) // TILE][:, kb]).astype(np.float64)
    return (A @ B.T) * (1 + 2.0 ** -20)


def sample_positions(M, N, n, seed, edge_rows=True):
    """n random output positions, plus every position of the first and last rows."""
    rng = np.random.default_rng(seed)
    ms, ns = [rng.integers(0, M, n)], [rng.integers(0, N, n)]
    if edge_rows:
        ms += [np.zeros(N, np.int64), np.full(N, M - 1, np.int64)]
        ns += [np.arange(N), np.arange(N)]
    return np.concatenate(ms), np.concatenate(ns)


def check_gemm(orc, mode, a, sa, b, sb, out, what, ms=None, ns=None):
    """The GEMM rule on a GPU output (torch tensor, fp32 or bf16) against the oracle:
    every element when ms/ns are None, else the sampled positions (ms[i], ns[i])."""
    bf16 = out.dtype == torch.bfloat16
    o = bf16_bits_np(out) if bf16 else to_np(out)
    K = a.shape[0] if mode == 3 else a.shape[1]
    nk = cdiv(K, TILE)
    na, nb = orc.deq_row_norms(mode, a, sa, b, sb)
    if ms is None:
        ref = orc.gemm(mode, a, sa, b, sb)
        absum = abs_products_full(orc, mode, a, sa, b, sb)
        return check_gemm_values(o, ref, na[:, None], nb[None, :], bf16, orc, what, absum, nk)
    ref = orc.gemm_at(mode, a, sa, b, sb, ms, ns)
    absum = abs_products_at(orc, mode, a, sa, b, sb, ms, ns)
    return check_gemm_values(o[ms, ns], ref, na[ms], nb[ns], bf16, orc, what, absum, nk)


def check_gemm_values(out: np.ndarray, ref: np.ndarray, na: np.ndarray, nb: np.ndarray,
                      bf16: bool, orc, what: str, absum=None, nk=None):
    """out/ref/na/nb aligned arrays (full matrices or samples); a bf16 output is
    passed as its uint16 bit patterns.

    fp32 output: normalized error <= 1e-4 everywhere.
    bf16 output: within 1 bf16 ulp of the oracle's bf16 rounding of its fp64
    value, or (near-cancellation elements) normalized error <= 1e-4; such
    fallbacks at most FALLBACK_MAX_FRAC of the elements.
    With absum (sum of |products| per element) and nk: every element also within
    the matrix cores' bound hw_error_bound, and every fallback element has
    |ref| < 2^9 times that bound.
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
    stats = {"what": what, "n": int(err.size), "max_norm_err": worst, "bf16": bool(bf16)}
    bound = None
    if absum is not None:
        absum = np.broadcast_to(absum, err.shape)
        bound = hw_error_bound(absum, nk)
        if bf16:
            bound = bound + np.ldexp(np.abs(vals), -8)      # half an ulp of the output's rounding
        over = err > bound
        stats["max_err_over_abssum"] = float(np.max(np.where(absum > 0, err / np.where(absum > 0, absum, 1), 0.0)))
        assert not over.any(), "%s: %d elements beyond the matrix cores' error bound; first %s" % (
            what, int(over.sum()), tuple(np.argwhere(over)[0]))
    if bf16:
        ref16 = orc.f64_to_bf16_array(ref)
        ulps = np.abs(bf16_ordered(out) - bf16_ordered(ref16))
        ok = (ulps <= 1) | (norm <= GEMM_TOL)
        strict_mask = ulps <= 1
        strict = float(np.mean(strict_mask)) if ulps.size else 1.0
        nfb = int((~strict_mask).sum())
        stats.update(strict_frac=strict, fallbacks=nfb, max_ulps=int(ulps.max()) if ulps.size else 0)
        assert ok.all(), "%s: %d elements beyond 1 ulp and tolerance; worst norm err %.3g" % (
            what, int((~ok).sum()), worst)
        assert nfb <= FALLBACK_MAX_FRAC * ulps.size + 4, "%s: %d of %d elements beyond 1 ulp" % (what, nfb, ulps.size)
        if nfb:
            fb = ~strict_mask
            rel = np.abs(ref[fb]) / np.where(denom[fb] > 0, denom[fb], 1) if np.ndim(denom) else np.abs(ref[fb]) / denom
            stats["fallback_max_ref_over_norms"] = float(np.max(rel))
            if bound is not None:
                assert np.all(np.abs(ref[fb]) < 2.0 ** 9 * bound[fb]), "%s: a fallback element is no near-cancellation one" % what
                stats["fallback_max_ref_over_abssum"] = float(np.max(np.abs(ref[fb]) / np.where(absum[fb] > 0, absum[fb], 1)))
    else:
        assert worst <= GEMM_TOL, "%s: normalized error %.3g > %g" % (what, worst, GEMM_TOL)
    if PARITY_LOG:
        with open(PARITY_LOG, "a") as fh:
            fh.write(json.dumps(stats) + "\n")
    print("PARITY", json.dumps(stats))
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
