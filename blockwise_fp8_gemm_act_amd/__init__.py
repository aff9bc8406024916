"""Python binding of libpuro.so: blockwise-FP8 quantizers and the
blockwise-scaled FP8 GEMM for MI355X (gfx950).

Argument marshalling only.  Every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/puro.h``; PyTorch is used for
device memory and streams.  There is no fallback: if the library is missing,
importing this package fails.

The raw C calls keep their C names (``puro_quant_act_1x128``,
``puro_quant_w_128x128``, ``puro_quant_transpose``, ``puro_quant_weights``, ``puro_requant_act_t``,
``puro_gemm_fp8_blockwise``, ``puro_gemm_fp8_blockwise_noalloc``,
``puro_gemm_fp8_blockwise_accumulate``,
``puro_gemm_fp8_swiglu_quant``, ...) and take integer device pointers.  The
tensor-level helpers ``quant_act_1x128``, ``quant_w_128x128``,
``quant_transpose``, ``requant_act_t``, ``swiglu_quant``,
``gemm_fp8_blockwise``, ``gemm_fp8_blockwise_accumulate`` and
``gemm_fp8_swiglu_quant`` allocate outputs with torch and call them on the
current stream.
"""
from __future__ import annotations

import ctypes
import functools
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpuro.so")

PURO_OK = 0
STATUS_NAMES = {0: "PURO_OK", 1: "PURO_ERR_NULL", 2: "PURO_ERR_SHAPE", 3: "PURO_ERR_ALIGN",
                4: "PURO_ERR_MODE", 5: "PURO_ERR_DTYPE", 6: "PURO_ERR_WORKSPACE",
                7: "PURO_ERR_DEVICE", 8: "PURO_ERR_LAUNCH", 9: "PURO_ERR_ALIAS", 10: "PURO_ERR_SCRATCH"}
SCRATCH_BYTES = 64 << 20       # device scratch of puro_gemm_fp8_blockwise_noalloc, per GPU
FPROP, DGRAD, WGRAD, WGRAD_TM = 0, 1, 2, 3
OUT_F32, OUT_BF16 = 0, 1
T_ACT, T_WEIGHT = 0, 1
TILE = 128

if not os.path.exists(LIB_PATH):
    raise ImportError("libpuro.so is not built: run `python blockwise_fp8_gemm_act_amd/build.py` "
                      "(or __graft_entry__.build())")

_lib = ctypes.CDLL(LIB_PATH)
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_lib.puro_quant_act_1x128.argtypes = [_P, _I64, _I64, _P, _P, _P]
_lib.puro_quant_act_1x128.restype = ctypes.c_int
_lib.puro_quant_w_128x128.argtypes = [_P, _I64, _I64, _P, _P, _P]
_lib.puro_quant_w_128x128.restype = ctypes.c_int
_lib.puro_quant_transpose.argtypes = [ctypes.c_int, _P, _I64, _I64, _P, _P, _P, _P, _P]
_lib.puro_quant_transpose.restype = ctypes.c_int
_lib.puro_quant_act_128x1.argtypes = [_P, _I64, _I64, _P, _P, _P, _P, _P]
_lib.puro_quant_act_128x1.restype = ctypes.c_int


class PuroWeight(ctypes.Structure):
    """puro_weight: one entry of puro_quant_weights."""
    _fields_ = [("w", _P), ("rows", _I64), ("cols", _I64), ("q", _P), ("s", _P), ("qt", _P), ("st", _P)]


_lib.puro_quant_weights.argtypes = [ctypes.c_int, ctypes.POINTER(PuroWeight), _P]
_lib.puro_quant_weights.restype = ctypes.c_int
_lib.puro_requant_act_t.argtypes = [_P, _P, _I64, _I64, _P, _P, _P]
_lib.puro_swiglu_quant.argtypes = [_P, _I64, _I64, _P, _P, _P, _P, _P, _P]
_lib.puro_swiglu_quant.restype = ctypes.c_int
_lib.puro_requant_act_t.restype = ctypes.c_int
_lib.puro_gemm_workspace_bytes.argtypes = [ctypes.c_int, _I64, _I64, _I64]
_lib.puro_gemm_workspace_bytes.restype = ctypes.c_size_t
_lib.puro_gemm_fp8_blockwise.argtypes = [ctypes.c_int, _P, _P, _P, _P, _P, ctypes.c_int,
                                         _I64, _I64, _I64, _P, ctypes.c_size_t, _P]
_lib.puro_gemm_fp8_blockwise.restype = ctypes.c_int
_lib.puro_gemm_fp8_blockwise_noalloc.argtypes = [ctypes.c_int, _P, _P, _P, _P, _P, ctypes.c_int,
                                                 _I64, _I64, _I64, _P]
_lib.puro_gemm_fp8_blockwise_noalloc.restype = ctypes.c_int
_lib.puro_gemm_fp8_blockwise_accumulate.argtypes = [ctypes.c_int, _P, _P, _P, _P, _P,
                                                    _I64, _I64, _I64, _P, ctypes.c_size_t, _P]
_lib.puro_gemm_fp8_blockwise_accumulate.restype = ctypes.c_int
_lib.puro_gemm_fp8_swiglu_quant.argtypes = [_P, _P, _P, _P, _I64, _I64, _I64, _P, _P, _P, _P]
_lib.puro_gemm_fp8_swiglu_quant.restype = ctypes.c_int
_lib.puro_status_str.argtypes = [ctypes.c_int]
_lib.puro_status_str.restype = ctypes.c_char_p
_lib.puro_abi_version.argtypes = []
_lib.puro_abi_version.restype = ctypes.c_int


def _torch_empty(shape, dtype, device):
    return torch.empty(shape, dtype=dtype, device=device)


# Allocator of every output and workspace buffer the tensor helpers create.  It is
# a module attribute so that a test harness can substitute one that fills new
# buffers with a poison value: a kernel that skips part of its output then leaves
# the poison in place instead of whatever the caching allocator's memory held.
empty = _torch_empty


class PuroError(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        super().__init__("%s failed: %s (%s)" % (call, STATUS_NAMES.get(status, status),
                                                 puro_status_str(status)))


# ---------------------------------------------------------------- raw C calls
def puro_quant_act_1x128(x, rows, cols, q, s, stream=None) -> int:
    return _lib.puro_quant_act_1x128(x, rows, cols, q, s, stream)


def puro_quant_w_128x128(w, rows, cols, q, s, stream=None) -> int:
    return _lib.puro_quant_w_128x128(w, rows, cols, q, s, stream)


def puro_quant_transpose(kind, x, rows, cols, qt, st, q_row, s_row, stream=None) -> int:
    return _lib.puro_quant_transpose(kind, x, rows, cols, qt, st, q_row, s_row, stream)


def puro_quant_act_128x1(x, rows, cols, qc, sc, q_row, s_row, stream=None) -> int:
    return _lib.puro_quant_act_128x1(x, rows, cols, qc, sc, q_row, s_row, stream)


def puro_quant_weights(weights, stream=None) -> int:
    """weights: a sequence of PuroWeight (or of 7-tuples w, rows, cols, q, s, qt, st)."""
    arr = (PuroWeight * max(len(weights), 1))(*[w if isinstance(w, PuroWeight) else PuroWeight(*w) for w in weights])
    return _lib.puro_quant_weights(len(weights), arr, stream)


def puro_requant_act_t(q, s, rows, cols, qt, st, stream=None) -> int:
    return _lib.puro_requant_act_t(q, s, rows, cols, qt, st, stream)


def puro_swiglu_quant(gu, rows, inter, q, s, qt, st, h, stream=None) -> int:
    return _lib.puro_swiglu_quant(gu, rows, inter, q, s, qt, st, h, stream)


def puro_gemm_workspace_bytes(mode, M, N, K) -> int:
    return int(_lib.puro_gemm_workspace_bytes(mode, M, N, K))


def puro_gemm_fp8_blockwise(mode, a, sa, b, sb, out, out_dtype, M, N, K, workspace, workspace_bytes,
                            stream=None) -> int:
    return _lib.puro_gemm_fp8_blockwise(mode, a, sa, b, sb, out, out_dtype, M, N, K, workspace,
                                        workspace_bytes, stream)


def puro_gemm_fp8_blockwise_noalloc(mode, a, sa, b, sb, out, out_dtype, M, N, K, stream=None) -> int:
    return _lib.puro_gemm_fp8_blockwise_noalloc(mode, a, sa, b, sb, out, out_dtype, M, N, K, stream)


def puro_gemm_fp8_blockwise_accumulate(mode, a, sa, b, sb, out, M, N, K, workspace, workspace_bytes,
                                       stream=None) -> int:
    return _lib.puro_gemm_fp8_blockwise_accumulate(mode, a, sa, b, sb, out, M, N, K, workspace,
                                                   workspace_bytes, stream)


def puro_gemm_fp8_swiglu_quant(a, sa, b, sb, M, inter, K, gu, hq, hs, stream=None) -> int:
    return _lib.puro_gemm_fp8_swiglu_quant(a, sa, b, sb, M, inter, K, gu, hq, hs, stream)


def puro_status_str(status: int) -> str:
    return _lib.puro_status_str(status).decode()


def puro_abi_version() -> int:
    return int(_lib.puro_abi_version())


# ---------------------------------------------------------------- tensor helpers
def _cdiv(a: int, b: int) -> int:
    return (a + b - 1) // b


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _on_stream(fn):
    """The helpers below allocate their outputs (and the GEMM's workspace) with torch's
    caching allocator.  Given an explicit `stream`, the helper runs with it as torch's
    current stream, so that those allocations belong to the stream the kernels are
    enqueued on: freeing one then cannot hand its memory to other work before the
    kernels that use it have finished.  `stream` is a torch.cuda.Stream or a raw
    hipStream_t handle."""
    @functools.wraps(fn)
    def run(*args, stream=None, **kw):
        if stream is None:
            return fn(*args, **kw)
        ts = stream if isinstance(stream, torch.cuda.Stream) else torch.cuda.ExternalStream(int(stream))
        with torch.cuda.stream(ts):
            return fn(*args, **kw)
    return run


def _check(status: int, call: str):
    if status != PURO_OK:
        raise PuroError(status, call)


def _bf16_input(x: torch.Tensor, name: str):
    if x.dtype != torch.bfloat16 or x.dim() != 2 or not x.is_cuda:
        raise TypeError("%s must be a 2-D bfloat16 CUDA tensor" % name)
    if not x.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _tensor(t, name: str, dtype, shape, device=None):
    """The C calls take raw pointers and cannot check sizes: every tensor handed to them
    through these helpers is checked here (CUDA, dtype, exact shape, contiguous, device)."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("%s must be a CUDA tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    return t


def _gemm_operands(mode: int, a, sa, b, sb):
    if mode not in (FPROP, DGRAD, WGRAD, WGRAD_TM):
        raise ValueError("unknown GEMM mode %r" % (mode,))
    if not isinstance(a, torch.Tensor) or a.dim() != 2 or not isinstance(b, torch.Tensor) or b.dim() != 2:
        raise TypeError("a and b must be 2-D tensors")
    if mode == WGRAD_TM:              # token-major: a [K][M], b [K][N]
        K, M = a.shape
        N = b.shape[1]
        if b.shape[0] != K:
            raise ValueError("a and b must share K (their first dimension)")
    else:
        M, K = a.shape
        N = b.shape[0]
        if b.shape[1] != K:
            raise ValueError("a and b must share K")
    dev = a.device
    nk = _cdiv(K, TILE)
    _tensor(a, "a", torch.uint8, tuple(a.shape))
    _tensor(b, "b", torch.uint8, tuple(b.shape), dev)
    _tensor(sa, "sa", torch.float32, (nk, M), dev)
    _tensor(sb, "sb", torch.float32, (nk, N) if mode in (WGRAD, WGRAD_TM) else (_cdiv(N, TILE), nk), dev)
    return M, N, K, dev


@_on_stream
def quant_act_1x128(x: torch.Tensor, q=None, s=None, stream=None):
    """1x128 tiles: returns (q uint8 [R][C], s fp32 [ceil(C/128)][R])."""
    _bf16_input(x, "x")
    R, C = x.shape
    q = empty((R, C), dtype=torch.uint8, device=x.device) if q is None else q
    s = empty((_cdiv(C, TILE), R), dtype=torch.float32, device=x.device) if s is None else s
    _tensor(q, "q", torch.uint8, (R, C), x.device)
    _tensor(s, "s", torch.float32, (_cdiv(C, TILE), R), x.device)
    _check(puro_quant_act_1x128(x.data_ptr(), R, C, q.data_ptr(), s.data_ptr(), _stream(stream)),
           "puro_quant_act_1x128")
    return q, s


@_on_stream
def quant_w_128x128(w: torch.Tensor, q=None, s=None, stream=None):
    """128x128 blocks: returns (q uint8 [R][C], s fp32 [ceil(R/128)][ceil(C/128)])."""
    _bf16_input(w, "w")
    R, C = w.shape
    q = empty((R, C), dtype=torch.uint8, device=w.device) if q is None else q
    s = empty((_cdiv(R, TILE), _cdiv(C, TILE)), dtype=torch.float32, device=w.device) if s is None else s
    _tensor(q, "q", torch.uint8, (R, C), w.device)
    _tensor(s, "s", torch.float32, (_cdiv(R, TILE), _cdiv(C, TILE)), w.device)
    _check(puro_quant_w_128x128(w.data_ptr(), R, C, q.data_ptr(), s.data_ptr(), _stream(stream)),
           "puro_quant_w_128x128")
    return q, s


@_on_stream
def quant_transpose(kind: int, x: torch.Tensor, dual: bool = False, stream=None):
    """Transposed quantization.  Returns (qt, st) or (qt, st, q_row, s_row) when dual.

    kind T_ACT:    qt [C][R], st [ceil(R/128)][C]; row outputs as quant_act_1x128
    kind T_WEIGHT: qt [C][R], st [ceil(C/128)][ceil(R/128)]; row outputs as quant_w_128x128
    """
    _bf16_input(x, "x")
    R, C = x.shape
    dev = x.device
    qt = empty((C, R), dtype=torch.uint8, device=dev)
    if kind == T_ACT:
        st = empty((_cdiv(R, TILE), C), dtype=torch.float32, device=dev)
        s_shape = (_cdiv(C, TILE), R)
    else:
        st = empty((_cdiv(C, TILE), _cdiv(R, TILE)), dtype=torch.float32, device=dev)
        s_shape = (_cdiv(R, TILE), _cdiv(C, TILE))
    q = s = None
    if dual:
        q = empty((R, C), dtype=torch.uint8, device=dev)
        s = empty(s_shape, dtype=torch.float32, device=dev)
    _check(puro_quant_transpose(kind, x.data_ptr(), R, C, qt.data_ptr(), st.data_ptr(),
                                q.data_ptr() if dual else None, s.data_ptr() if dual else None,
                                _stream(stream)), "puro_quant_transpose")
    return (qt, st, q, s) if dual else (qt, st)


@_on_stream
def quant_weights(ws, row: bool = True, transposed: bool = True, stream=None):
    """Several weights (2-D bf16 CUDA tensors, at most 8) quantized in 128x128 blocks by one
    launch.  Returns, per weight, (q, s) and/or (qt, st) as quant_w_128x128 and
    quant_transpose(T_WEIGHT) return them: a list of tuples (q, s, qt, st) with None
    for the outputs not requested."""
    if not (row or transposed):
        raise ValueError("request row-wise and/or transposed outputs")
    if len(ws) > 8:
        raise ValueError("at most 8 weights per call")
    outs, descs = [], []
    for i, w in enumerate(ws):
        _bf16_input(w, "ws[%d]" % i)
        R, C = w.shape
        dev = w.device
        q = empty((R, C), dtype=torch.uint8, device=dev) if row else None
        s = empty((_cdiv(R, TILE), _cdiv(C, TILE)), dtype=torch.float32, device=dev) if row else None
        qt = empty((C, R), dtype=torch.uint8, device=dev) if transposed else None
        st = empty((_cdiv(C, TILE), _cdiv(R, TILE)), dtype=torch.float32, device=dev) if transposed else None
        outs.append((q, s, qt, st))
        ptr = lambda t: t.data_ptr() if t is not None else None
        descs.append(PuroWeight(w.data_ptr(), R, C, ptr(q), ptr(s), ptr(qt), ptr(st)))
    _check(puro_quant_weights(descs, _stream(stream)), "puro_quant_weights")
    return outs


@_on_stream
def quant_act_128x1(x: torch.Tensor, dual: bool = False, stream=None):
    """128x1 tiles with the codes in x's own layout: returns (qc uint8 [R][C], sc fp32
    [ceil(R/128)][C]), plus (q, s) as quant_act_1x128 when dual."""
    _bf16_input(x, "x")
    R, C = x.shape
    dev = x.device
    qc = empty((R, C), dtype=torch.uint8, device=dev)
    sc = empty((_cdiv(R, TILE), C), dtype=torch.float32, device=dev)
    q = s = None
    if dual:
        q = empty((R, C), dtype=torch.uint8, device=dev)
        s = empty((_cdiv(C, TILE), R), dtype=torch.float32, device=dev)
    _check(puro_quant_act_128x1(x.data_ptr(), R, C, qc.data_ptr(), sc.data_ptr(),
                                q.data_ptr() if dual else None, s.data_ptr() if dual else None, _stream(stream)),
           "puro_quant_act_128x1")
    return (qc, sc, q, s) if dual else (qc, sc)


@_on_stream
def requant_act_t(q: torch.Tensor, s: torch.Tensor, qt=None, st=None, stream=None):
    """Saved 1x128 codes q uint8 [R][C] and scales s fp32 [ceil(C/128)][R] ->
    (qt uint8 [C][R], st fp32 [ceil(R/128)][C]) in transposed 128x1 tiles."""
    if not isinstance(q, torch.Tensor) or q.dim() != 2:
        raise TypeError("q must be a 2-D tensor")
    R, C = q.shape
    _tensor(q, "q", torch.uint8, (R, C))
    _tensor(s, "s", torch.float32, (_cdiv(C, TILE), R), q.device)
    qt = empty((C, R), dtype=torch.uint8, device=q.device) if qt is None else qt
    st = empty((_cdiv(R, TILE), C), dtype=torch.float32, device=q.device) if st is None else st
    _tensor(qt, "qt", torch.uint8, (C, R), q.device)
    _tensor(st, "st", torch.float32, (_cdiv(R, TILE), C), q.device)
    _check(puro_requant_act_t(q.data_ptr(), s.data_ptr(), R, C, qt.data_ptr(), st.data_ptr(),
                              _stream(stream)), "puro_requant_act_t")
    return qt, st


@_on_stream
def swiglu_quant(gu: torch.Tensor, dual: bool = False, write_h: bool = False, stream=None):
    """SwiGLU of a [R][2I] gate/up bf16 tensor (gate first) fused with quantization of
    h = bf16(silu(gate) * up).  Returns (q, s) [+ (qt, st) when dual] [+ h when write_h]."""
    _bf16_input(gu, "gu")
    R, C2 = gu.shape
    if C2 % 2:
        raise ValueError("gu needs an even number of columns (gate then up)")
    I = C2 // 2
    dev = gu.device
    q = empty((R, I), dtype=torch.uint8, device=dev)
    s = empty((_cdiv(I, TILE), R), dtype=torch.float32, device=dev)
    qt = st = h = None
    if dual:
        qt = empty((I, R), dtype=torch.uint8, device=dev)
        st = empty((_cdiv(R, TILE), I), dtype=torch.float32, device=dev)
    if write_h:
        h = empty((R, I), dtype=torch.bfloat16, device=dev)
    _check(puro_swiglu_quant(gu.data_ptr(), R, I, q.data_ptr(), s.data_ptr(),
                             qt.data_ptr() if dual else None, st.data_ptr() if dual else None,
                             h.data_ptr() if write_h else None, _stream(stream)), "puro_swiglu_quant")
    out = (q, s)
    if dual:
        out += (qt, st)
    if write_h:
        out += (h,)
    return out


def gemm_workspace(mode: int, M: int, N: int, K: int, device="cuda"):
    n = puro_gemm_workspace_bytes(mode, M, N, K)
    return empty((max(n, 16),), dtype=torch.uint8, device=device), n


@_on_stream
def gemm_fp8_blockwise(mode: int, a, sa, b, sb, out_dtype=torch.bfloat16, out=None, workspace=None,
                       stream=None):
    """out[m][n] = sum_k deq(a)[m][k] * deq(b)[n][k]; a [M][K], b [N][K] uint8 codes
    (WGRAD_TM: a [K][M], b [K][N], token-major).  sa [ceil(K/128)][M]; sb [ceil(N/128)][ceil(K/128)]
    (FPROP, DGRAD) or [ceil(K/128)][N] (WGRAD, WGRAD_TM)."""
    M, N, K, dev = _gemm_operands(mode, a, sa, b, sb)
    if out is None:
        out = empty((M, N), dtype=out_dtype, device=dev)
    if out.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("out must be bfloat16 or float32")
    _tensor(out, "out", out.dtype, (M, N), dev)
    od = OUT_BF16 if out.dtype == torch.bfloat16 else OUT_F32
    need = puro_gemm_workspace_bytes(mode, M, N, K)
    if workspace is None and need > 0:
        workspace = empty((need,), dtype=torch.uint8, device=dev)
    if workspace is not None and (not workspace.is_cuda or not workspace.is_contiguous() or workspace.device != dev):
        raise ValueError("workspace must be a contiguous CUDA tensor on %s" % dev)
    wptr = workspace.data_ptr() if workspace is not None else None
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(puro_gemm_fp8_blockwise(mode, a.data_ptr(), sa.data_ptr(), b.data_ptr(), sb.data_ptr(),
                                   out.data_ptr(), od, M, N, K, wptr, wbytes, _stream(stream)),
           "puro_gemm_fp8_blockwise")
    return out


@_on_stream
def gemm_fp8_blockwise_noalloc(mode: int, a, sa, b, sb, out: torch.Tensor, stream=None):
    """gemm_fp8_blockwise into a caller's `out` (bf16 or fp32 [M][N]) with no allocation at
    all: split-K partials go to the library's per-GPU device scratch.  Returns out."""
    M, N, K, dev = _gemm_operands(mode, a, sa, b, sb)
    if out.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("out must be bfloat16 or float32")
    _tensor(out, "out", out.dtype, (M, N), dev)
    od = OUT_BF16 if out.dtype == torch.bfloat16 else OUT_F32
    _check(puro_gemm_fp8_blockwise_noalloc(mode, a.data_ptr(), sa.data_ptr(), b.data_ptr(), sb.data_ptr(),
                                           out.data_ptr(), od, M, N, K, _stream(stream)),
           "puro_gemm_fp8_blockwise_noalloc")
    return out


@_on_stream
def gemm_fp8_blockwise_accumulate(mode: int, a, sa, b, sb, out: torch.Tensor, workspace=None, stream=None):
    """out (fp32 [M][N]) += the blockwise-scaled FP8 GEMM of a [M][K] and b [N][K]; returns out.
    Scale layouts as for gemm_fp8_blockwise."""
    M, N, K, dev = _gemm_operands(mode, a, sa, b, sb)
    _tensor(out, "out", torch.float32, (M, N), dev)
    need = puro_gemm_workspace_bytes(mode, M, N, K)
    if workspace is None and need > 0:
        workspace = empty((need,), dtype=torch.uint8, device=dev)
    if workspace is not None and (not workspace.is_cuda or not workspace.is_contiguous() or workspace.device != dev):
        raise ValueError("workspace must be a contiguous CUDA tensor on %s" % dev)
    wptr = workspace.data_ptr() if workspace is not None else None
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(puro_gemm_fp8_blockwise_accumulate(mode, a.data_ptr(), sa.data_ptr(), b.data_ptr(), sb.data_ptr(),
                                              out.data_ptr(), M, N, K, wptr, wbytes, _stream(stream)),
           "puro_gemm_fp8_blockwise_accumulate")
    return out


@_on_stream
def gemm_fp8_swiglu_quant(a, sa, b, sb, write_gu: bool = True, stream=None):
    """Fprop of a fused gate/up projection with the SwiGLU quantizer as its epilogue.
    a [M][K] codes, sa [ceil(K/128)][M]; b [2I][K] codes (gate rows, then up rows),
    sb [2I/128][ceil(K/128)].  Returns (hq uint8 [M][I], hs fp32 [I/128][M], gu), gu being
    the bf16 gate/up output [M][2I] (None unless write_gu)."""
    M, N, K, dev = _gemm_operands(FPROP, a, sa, b, sb)
    if N % (2 * TILE):
        raise ValueError("b must have 2*I rows with I a multiple of 128")
    I = N // 2
    hq = empty((M, I), dtype=torch.uint8, device=dev)
    hs = empty((I // TILE, M), dtype=torch.float32, device=dev)
    gu = empty((M, N), dtype=torch.bfloat16, device=dev) if write_gu else None
    _check(puro_gemm_fp8_swiglu_quant(a.data_ptr(), sa.data_ptr(), b.data_ptr(), sb.data_ptr(), M, I, K,
                                      gu.data_ptr() if write_gu else None, hq.data_ptr(), hs.data_ptr(),
                                      _stream(stream)), "puro_gemm_fp8_swiglu_quant")
    return hq, hs, gu
