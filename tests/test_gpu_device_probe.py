"""Probes of device code the kernels rely on, through a test-only HIP module
(tests/csrc/device_probe.hip, built with the library).

- The quantizers' fp32 -> e4m3 pack (pack4_e4m3: the hardware round-to-nearest-
  even conversion) against the oracle's encoder on every fp32 value a quantizer
  can hand it: all bit patterns with |f| <= 448 + 2 ulps, both signs
  (x / s never exceeds 448 by more than one ulp, since s = fp32(amax / 448)).
- The 32x32x64 FP8 matrix-core instruction: its lane layout (integer-valued
  codes, exact) and its summation precision on the families the 16x16x128 probe
  in test_gpu_gemm.py uses."""
import ctypes
import os

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "csrc", "libdevprobe.so")


@pytest.fixture(scope="module")
def probe():
    if not os.path.exists(LIB):
        pytest.fail("tests/csrc/libdevprobe.so is not built (run __graft_entry__.build())")
    lib = ctypes.CDLL(LIB)
    lib.probe_pack_e4m3.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_void_p]
    lib.probe_pack_e4m3.restype = ctypes.c_int
    lib.probe_mfma32_slice.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.probe_mfma32_slice.restype = ctypes.c_int
    return lib


def test_pack_e4m3_every_value_in_range(orc, probe):
    hi = int(np.float32(448.0).view(np.uint32)) + 2                # 448 + 2 ulps
    chunk = 1 << 26
    buf = torch.empty(chunk, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    checked = 0
    for sign in (0, 0x80000000):
        start = 0
        while start <= hi:
            count = min(chunk, hi + 1 - start)
            assert probe.probe_pack_e4m3(start, count, sign, buf.data_ptr(), stream) == 0
            got = buf[:count].cpu().numpy()
            bits = np.arange(start, start + count, dtype=np.uint32) | np.uint32(sign)
            want = orc.e4m3_encode_array(bits.view(np.float32))
            bad = np.nonzero(got != want)[0]
            assert bad.size == 0, "fp32 0x%08x: device 0x%02x, oracle 0x%02x" % (bits[bad[0]], got[bad[0]], want[bad[0]])
            checked += count
            start += count
    assert checked == 2 * (hi + 1)
    print("pack4_e4m3 equals the oracle on %d fp32 values" % checked)


def mfma32(probe, a, b):
    A = torch.from_numpy(np.ascontiguousarray(a, np.uint8)).cuda()
    B = torch.from_numpy(np.ascontiguousarray(b, np.uint8)).cuda()
    out = torch.empty((32, 32), dtype=torch.float32, device="cuda")
    assert probe.probe_mfma32_slice(A.data_ptr(), B.data_ptr(), out.data_ptr(),
                                    torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def test_mfma32_layout_exact(orc, probe):
    """Codes of the integers -8..8: every sum is exact, so out = a b^T bit for bit."""
    rng = np.random.default_rng(5)
    vals = np.arange(-8, 9)
    codes = np.array([orc.e4m3_encode(float(v)) for v in vals], np.uint8)
    ia, ib = rng.integers(0, len(vals), (32, 128)), rng.integers(0, len(vals), (32, 128))
    out = mfma32(probe, codes[ia], codes[ib])
    assert np.array_equal(out, (vals[ia] @ vals[ib].T).astype(np.float64))


def test_mfma32_precision(orc, probe):
    """Summation precision of the 32x32x64 form on one slice with unit scales: the
    group structure (which small products next to a dominant one are lost) and the
    error relative to sum|products| on the 16x16x128 probe's families."""
    enc = orc.e4m3_encode
    dec = orc.e4m3_decode_table()
    a = np.zeros((32, 128), np.uint8)
    a[:, 0] = enc(448.0)
    for m in range(1, 32):
        a[m, 4 * m] = enc(2.0 ** -6)                                # 448 + 2^-6 is exact in fp32
    b = np.full((32, 128), enc(1.0), np.uint8)
    out = mfma32(probe, a, b)
    lost = [4 * m for m in range(1, 32) if out[m, 0] != 448.0 + 2.0 ** -6]
    print("32x32x64: a 2^-6 product next to 448 at k = 0 is lost at k =", lost)

    rng = np.random.default_rng(2024)
    finite = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)
    fam = {"uniform codes": (rng.choice(finite, (32, 128)), rng.choice(finite, (32, 128))),
           "normal": (orc.e4m3_encode_array(rng.standard_normal((32, 128)).astype(np.float32) * 50),
                      orc.e4m3_encode_array(rng.standard_normal((32, 128)).astype(np.float32) * 50))}
    a = orc.e4m3_encode_array(rng.uniform(-0.05, 0.05, (32, 128)).astype(np.float32))
    b = orc.e4m3_encode_array(rng.uniform(-1, 1, (32, 128)).astype(np.float32))
    a[:, ::8] = enc(448.0)
    b[:, ::8] = enc(1.0)
    fam["one dominant per group of 8"] = (a, b)
    worst = {}
    for name, (a, b) in fam.items():
        out = mfma32(probe, a, b)
        A, B = dec[a], dec[b]
        exact = A @ B.T
        absum = np.abs(A) @ np.abs(B).T
        rel = np.abs(out - exact) / np.where(absum > 0, absum, 1)
        worst[name] = float(rel.max())
        print("32x32x64 %s: max |err| / sum|products| = %.3g (2^%.1f)" % (name, worst[name], np.log2(max(worst[name], 1e-300))))
    assert max(worst.values()) < 2.0 ** -10
