"""CPU oracle for blockwise FP8 quantization and the blockwise-scaled FP8 GEMM.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(the ``blockwise_fp8_gemm_act_amd`` package and its HIP library) never calls it
and shares no code with it.

The arithmetic lives in ``oracle.c`` (plain C99, fp64 for the GEMM); this file
only builds it with gcc and marshals numpy arrays through ctypes.  What each
function computes, and the passage it follows, is stated in ``oracle.c``.

Functions: the e4m3 and bf16 scalars, the tile quantizers (1x128, 128x128,
128x1 and transposed 128x128), the requantizer of saved 1x128 codes, SwiGLU
of the gate/up output, and the fp64 GEMM (full, sampled, accumulating, and
followed by the SwiGLU quantizer).

Parity pins: every function here is pinned by ``tests/test_oracle_*.py``
(exhaustive e4m3 agreement with PyTorch's CPU cast, code round-trips, tile
invariants, hand-derived golden tiles, integer-exact GEMMs, linearity in
power-of-two scales, a library fp64 matmul cross-check, brute force on tiny
inputs, 50-digit arithmetic for SwiGLU).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

FPROP, DGRAD, WGRAD, WGRAD_TM = 0, 1, 2, 3
TILE = 128

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc into oracle/liboracle.so (no fast-math, no FP contraction)."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c99", "-O2", "-fopenmp", "-fno-fast-math", "-ffp-contract=off",
           "-fno-finite-math-only", "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.orc_bf16_to_f32.argtypes = [ctypes.c_uint16]
    lib.orc_bf16_to_f32.restype = ctypes.c_float
    lib.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.orc_e4m3_decode.restype = ctypes.c_double
    lib.orc_e4m3_encode.argtypes = [ctypes.c_float]
    lib.orc_e4m3_encode.restype = ctypes.c_uint8
    lib.orc_tile_scale.argtypes = [ctypes.c_float]
    lib.orc_tile_scale.restype = ctypes.c_float
    lib.orc_quantize_value.argtypes = [ctypes.c_float, ctypes.c_float]
    lib.orc_quantize_value.restype = ctypes.c_uint8
    lib.orc_e4m3_encode_array.argtypes = [P, I64, P]
    for name in ("orc_quant_act_1x128", "orc_quant_w_128x128",
                 "orc_quant_act_128x1_t", "orc_quant_w_128x128_t"):
        getattr(lib, name).argtypes = [P, I64, I64, P, P]
    lib.orc_requant_act_t.argtypes = [P, P, I64, I64, P, P]
    lib.orc_swiglu_value.argtypes = [ctypes.c_uint16, ctypes.c_uint16]
    lib.orc_swiglu_value.restype = ctypes.c_uint16
    lib.orc_swiglu.argtypes = [P, I64, I64, P]
    lib.orc_gemm_element.argtypes = [ctypes.c_int, P, P, P, P, I64, I64, I64, I64, I64]
    lib.orc_gemm_element.restype = ctypes.c_double
    lib.orc_gemm.argtypes = [ctypes.c_int, P, P, P, P, I64, I64, I64, P]
    lib.orc_gemm_at.argtypes = [ctypes.c_int, P, P, P, P, I64, I64, I64, P, P, I64, P]
    lib.orc_deq_row_norms.argtypes = [ctypes.c_int, P, P, P, P, I64, I64, I64, P, P]
    lib.orc_dequant_a.argtypes = [P, P, I64, I64, P]
    lib.orc_dequant_b.argtypes = [ctypes.c_int, P, P, I64, I64, P]
    lib.orc_f64_to_bf16.argtypes = [ctypes.c_double]
    lib.orc_f64_to_bf16.restype = ctypes.c_uint16
    lib.orc_f64_to_bf16_array.argtypes = [P, I64, P]
    lib.orc_num_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def _u16(x) -> np.ndarray:
    x = np.ascontiguousarray(x)
    if x.dtype != np.uint16:
        raise TypeError("bf16 inputs are passed as their uint16 bit patterns")
    return x


def _cdiv(a: int, b: int) -> int:
    return (a + b - 1) // b


def num_threads() -> int:
    return int(_load().orc_num_threads())


# ---------------------------------------------------------------- scalars
def bf16_to_f32(h: int) -> float:
    return float(_load().orc_bf16_to_f32(int(h)))


def e4m3_decode(c: int) -> float:
    return float(_load().orc_e4m3_decode(int(c)))


def e4m3_decode_table() -> np.ndarray:
    """fp64 value of each of the 256 codes (NaN for 0x7F / 0xFF)."""
    lib = _load()
    return np.array([lib.orc_e4m3_decode(c) for c in range(256)], dtype=np.float64)


def e4m3_encode(f: float) -> int:
    return int(_load().orc_e4m3_encode(float(f)))


def e4m3_encode_array(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    q = np.empty(x.shape, dtype=np.uint8)
    _load().orc_e4m3_encode_array(_ptr(x), x.size, _ptr(q))
    return q


def tile_scale(amax: float) -> float:
    return float(_load().orc_tile_scale(float(amax)))


def quantize_value(x: float, s: float) -> int:
    return int(_load().orc_quantize_value(float(x), float(s)))


def f64_to_bf16(v: float) -> int:
    return int(_load().orc_f64_to_bf16(float(v)))


def f64_to_bf16_array(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    _load().orc_f64_to_bf16_array(_ptr(v), v.size, _ptr(out))
    return out


# ---------------------------------------------------------------- quantizers
def quant_act_1x128(x: np.ndarray):
    """x: uint16 (bf16 bits) [R][C] -> (q uint8 [R][C], s float32 [ceil(C/128)][R])."""
    x = _u16(x)
    R, C = x.shape
    q = np.empty((R, C), dtype=np.uint8)
    s = np.empty((_cdiv(C, TILE), R), dtype=np.float32)
    _load().orc_quant_act_1x128(_ptr(x), R, C, _ptr(q), _ptr(s))
    return q, s


def quant_w_128x128(w: np.ndarray):
    """w: uint16 [R][C] -> (q uint8 [R][C], s float32 [ceil(R/128)][ceil(C/128)])."""
    w = _u16(w)
    R, C = w.shape
    q = np.empty((R, C), dtype=np.uint8)
    s = np.empty((_cdiv(R, TILE), _cdiv(C, TILE)), dtype=np.float32)
    _load().orc_quant_w_128x128(_ptr(w), R, C, _ptr(q), _ptr(s))
    return q, s


def quant_act_128x1_t(x: np.ndarray):
    """x: uint16 [R][C] -> (qt uint8 [C][R], st float32 [ceil(R/128)][C])."""
    x = _u16(x)
    R, C = x.shape
    qt = np.empty((C, R), dtype=np.uint8)
    st = np.empty((_cdiv(R, TILE), C), dtype=np.float32)
    _load().orc_quant_act_128x1_t(_ptr(x), R, C, _ptr(qt), _ptr(st))
    return qt, st


def quant_act_128x1(x: np.ndarray):
    """The 128x1 tiles of quant_act_128x1_t with the codes in x's own layout:
    x uint16 [R][C] -> (q uint8 [R][C], s float32 [ceil(R/128)][C]), q[r][c] = qt[c][r]."""
    qt, st = quant_act_128x1_t(x)
    return np.ascontiguousarray(qt.T), st


def quant_w_128x128_t(w: np.ndarray):
    """w: uint16 [R][C] -> (qt uint8 [C][R], st float32 [ceil(C/128)][ceil(R/128)])."""
    w = _u16(w)
    R, C = w.shape
    qt = np.empty((C, R), dtype=np.uint8)
    st = np.empty((_cdiv(C, TILE), _cdiv(R, TILE)), dtype=np.float32)
    _load().orc_quant_w_128x128_t(_ptr(w), R, C, _ptr(qt), _ptr(st))
    return qt, st


def requant_act_t(q: np.ndarray, s: np.ndarray):
    """Saved 1x128 codes q uint8 [R][C] with scales s float32 [ceil(C/128)][R]
    -> (qt uint8 [C][R], st float32 [ceil(R/128)][C]): dequantize to fp32, then
    quantize in transposed 128x1 tiles."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    s = np.ascontiguousarray(s, dtype=np.float32)
    R, C = q.shape
    if s.shape != (_cdiv(C, TILE), R):
        raise ValueError("scales must be [ceil(C/128)][R], got %s" % (s.shape,))
    qt = np.empty((C, R), dtype=np.uint8)
    st = np.empty((_cdiv(R, TILE), C), dtype=np.float32)
    _load().orc_requant_act_t(_ptr(q), _ptr(s), R, C, _ptr(qt), _ptr(st))
    return qt, st


def swiglu_value(g: int, u: int) -> int:
    """bf16 bits of bf16(silu(g) * u) for bf16 bit patterns g, u."""
    return int(_load().orc_swiglu_value(int(g), int(u)))


def swiglu(gu: np.ndarray) -> np.ndarray:
    """gu: uint16 (bf16 bits) [R][2*I], gate then up -> h uint16 [R][I] = bf16(silu(gate) * up)."""
    gu = _u16(gu)
    R, C2 = gu.shape
    if C2 % 2:
        raise ValueError("the gate/up input needs an even number of columns")
    h = np.empty((R, C2 // 2), dtype=np.uint16)
    _load().orc_swiglu(_ptr(gu), R, C2 // 2, _ptr(h))
    return h


def swiglu_quant(gu: np.ndarray, dual: bool = False):
    """SwiGLU then quantization of h: (q, s) as quant_act_1x128(h), plus (qt, st) as
    quant_act_128x1_t(h) when dual.  Returns (h, q, s) or (h, q, s, qt, st)."""
    h = swiglu(gu)
    q, s = quant_act_1x128(h)
    if not dual:
        return h, q, s
    qt, st = quant_act_128x1_t(h)
    return h, q, s, qt, st


# ---------------------------------------------------------------- GEMM
def gemm_swiglu_quant(a, sa, b, sb, rows=None):
    """Fprop of a fused gate/up projection followed by the SwiGLU quantizer: the
    down projection's FP8 input made straight from the gate/up GEMM (the pages put
    the main linears on the FP8 path: en.roboind.com article on Puro-2B, section
    "FP8 takes advantage of the RTX 5090's low precision efficiency").
      gu = bf16(gemm(FPROP, a, sa, b, sb))   one rounding of each fp64 value
      (h, q, s) = swiglu_quant(gu)           b's first half of rows is the gate
    rows: optional row indices; the result then covers a[rows] only (rows of the
    product are independent).  Returns (gu, h, q, s)."""
    a = np.ascontiguousarray(a, dtype=np.uint8)
    sa = np.ascontiguousarray(sa, dtype=np.float32)
    if rows is not None:
        rows = np.asarray(rows, dtype=np.int64)
        a = np.ascontiguousarray(a[rows])
        sa = np.ascontiguousarray(sa[:, rows])
    gu = f64_to_bf16_array(gemm(FPROP, a, sa, b, sb))
    h, q, s = swiglu_quant(gu)
    return gu, h, q, s


def _token_major(mode, a, b):
    """WGRAD_TM takes the wgrad operands token-major ([K][M], [K][N]); the sum is
    the wgrad's over the transposed arrays (a layout change only)."""
    if mode != WGRAD_TM:
        return mode, a, b
    a = np.ascontiguousarray(np.asarray(a, dtype=np.uint8).T)
    b = np.ascontiguousarray(np.asarray(b, dtype=np.uint8).T)
    return WGRAD, a, b


def _gemm_args(mode, a, sa, b, sb):
    a = np.ascontiguousarray(a, dtype=np.uint8)
    b = np.ascontiguousarray(b, dtype=np.uint8)
    sa = np.ascontiguousarray(sa, dtype=np.float32)
    sb = np.ascontiguousarray(sb, dtype=np.float32)
    M, K = a.shape
    N, Kb = b.shape
    if Kb != K:
        raise ValueError("a and b must share K")
    nk = _cdiv(K, TILE)
    if sa.shape != (nk, M):
        raise ValueError("sa must be [ceil(K/128)][M]")
    want_sb = (nk, N) if mode == WGRAD else (_cdiv(N, TILE), nk)
    if sb.shape != want_sb:
        raise ValueError("sb must be %r for this mode" % (want_sb,))
    return a, sa, b, sb, M, N, K


def gemm(mode: int, a, sa, b, sb) -> np.ndarray:
    """fp64 reference out[M][N] = sum_k deq(a)[m][k] * deq(b)[n][k]."""
    mode, a, b = _token_major(mode, a, b)
    a, sa, b, sb, M, N, K = _gemm_args(mode, a, sa, b, sb)
    out = np.empty((M, N), dtype=np.float64)
    _load().orc_gemm(mode, _ptr(a), _ptr(sa), _ptr(b), _ptr(sb), M, N, K, _ptr(out))
    return out


def gemm_accumulate(mode: int, a, sa, b, sb, c) -> np.ndarray:
    """The accumulating GEMM (micro-batched weight gradients summed into one fp32
    buffer: the en.roboind.com article on Puro-2B tunes micro-batch sizes, section
    "Unit cost, higher computing power"): c + gemm(...), both in fp64, c an fp32 [M][N]
    array.  The kernels add in fp32, so they differ from this by that addition's
    rounding (half an fp32 ulp of the sum) on top of the GEMM's own tolerance."""
    c = np.asarray(c, dtype=np.float32)
    return c.astype(np.float64) + gemm(mode, a, sa, b, sb)


def gemm_at(mode: int, a, sa, b, sb, ms, ns) -> np.ndarray:
    """fp64 reference values at positions (ms[i], ns[i])."""
    mode, a, b = _token_major(mode, a, b)
    a, sa, b, sb, M, N, K = _gemm_args(mode, a, sa, b, sb)
    ms = np.ascontiguousarray(ms, dtype=np.int64)
    ns = np.ascontiguousarray(ns, dtype=np.int64)
    if ms.shape != ns.shape:
        raise ValueError("ms and ns must have one shape")
    if ms.size and (ms.min() < 0 or ms.max() >= M or ns.min() < 0 or ns.max() >= N):
        raise IndexError("sample position out of range")
    out = np.empty(ms.shape, dtype=np.float64)
    _load().orc_gemm_at(mode, _ptr(a), _ptr(sa), _ptr(b), _ptr(sb), M, N, K,
                        _ptr(ms), _ptr(ns), ms.size, _ptr(out))
    return out


def deq_row_norms(mode: int, a, sa, b, sb):
    """(||A_m||_2 for each m, ||B_n||_2 for each n) of the dequantized operands, fp64."""
    mode, a, b = _token_major(mode, a, b)
    a, sa, b, sb, M, N, K = _gemm_args(mode, a, sa, b, sb)
    na = np.empty(M, dtype=np.float64)
    nb = np.empty(N, dtype=np.float64)
    _load().orc_deq_row_norms(mode, _ptr(a), _ptr(sa), _ptr(b), _ptr(sb), M, N, K,
                              _ptr(na), _ptr(nb))
    return na, nb


def dequant_a(a, sa) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.uint8)
    sa = np.ascontiguousarray(sa, dtype=np.float32)
    M, K = a.shape
    out = np.empty((M, K), dtype=np.float64)
    _load().orc_dequant_a(_ptr(a), _ptr(sa), M, K, _ptr(out))
    return out


def dequant_b(mode: int, b, sb) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint8)
    sb = np.ascontiguousarray(sb, dtype=np.float32)
    N, K = b.shape
    out = np.empty((N, K), dtype=np.float64)
    _load().orc_dequant_b(mode, _ptr(b), _ptr(sb), N, K, _ptr(out))
    return out
