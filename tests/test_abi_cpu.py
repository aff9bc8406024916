"""C-ABI checks that need no GPU: the library loads, exports every function
include/puro.h declares, and rejects invalid arguments on the host before it
touches a device (fake, never dereferenced pointers are enough for that).
On a machine without a GPU a valid call stops at the device check."""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "puro.h")

import blockwise_fp8_gemm_act_amd as puro  # noqa: E402

OK, NULL, SHAPE, ALIGN, MODE, DTYPE, WS, DEVICE, LAUNCH, ALIAS, SCRATCH = range(11)

# fake, 16-byte aligned, well separated device addresses (never dereferenced)
A0, A1, A2, A3, A4, A5, A6 = (0x7F0000000000 + i * (1 << 32) for i in range(7))


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*[\w\s\*]*?\b(puro_\w+)\s*\(", text, re.M)))


def test_header_declares_the_abi():
    names = declared_functions()
    assert names == sorted(["puro_quant_act_1x128", "puro_quant_w_128x128", "puro_quant_transpose", "puro_quant_act_128x1",
                            "puro_requant_act_t", "puro_swiglu_quant", "puro_gemm_workspace_bytes", "puro_gemm_fp8_blockwise",
                            "puro_gemm_fp8_blockwise_noalloc", "puro_quant_weights",
                            "puro_gemm_fp8_blockwise_accumulate", "puro_gemm_fp8_swiglu_quant",
                            "puro_status_str", "puro_abi_version"])


def test_library_exports_every_declared_function():
    out = subprocess.run(["nm", "-D", "--defined-only", puro.LIB_PATH], check=True,
                         capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (puro_\w+)", out))
    for name in declared_functions():
        assert name in exported, name
        assert callable(getattr(puro._lib, name))


def test_version_and_status_strings():
    assert puro.puro_abi_version() == 8
    for s in range(11):
        assert puro.puro_status_str(s) and puro.puro_status_str(s) != "unknown status"
    assert puro.puro_status_str(99) == "unknown status"


def no_gpu():
    import torch
    return not torch.cuda.is_available()


# ---------------------------------------------------------------- quantizers
def test_quant_act_validation():
    f = puro.puro_quant_act_1x128
    assert f(A0, -1, 128, A1, A2) == SHAPE
    assert f(A0, 4, 100, A1, A2) == SHAPE                 # cols not a multiple of 16
    assert f(A0, 1 << 31, 128, A1, A2) == SHAPE           # over the dimension limit
    assert f(A0, 1 << 30, 1 << 20, A1, A2) == SHAPE       # over the element limit
    assert f(None, 0, 128, None, None) == OK              # empty: nothing to do
    assert f(A0, 4, 0, A1, A2) == OK
    assert f(None, 4, 128, A1, A2) == NULL
    assert f(A0, 4, 128, None, A2) == NULL
    assert f(A0, 4, 128, A1, None) == NULL
    assert f(A0 + 8, 4, 128, A1, A2) == ALIGN
    assert f(A0, 4, 128, A1 + 4, A2) == ALIGN
    assert f(A0, 4, 128, A0 + 512, A2) == ALIAS           # q inside x
    assert f(A0, 4, 128, A1, A1 + 256) == ALIAS           # s inside q
    if no_gpu():   # valid arguments: only safe to call with fake pointers when no device exists
        assert f(A0, 4, 128, A1, A1 + 512) == DEVICE


def test_quant_w_validation():
    f = puro.puro_quant_w_128x128
    assert f(A0, 128, 120, A1, A2) == SHAPE
    assert f(A0, 128, 128, None, A2) == NULL
    assert f(A0, 128, 128, A1, A2 + 4) == ALIGN
    assert f(A0, 128, 128, A1, A1) == ALIAS


def test_quant_transpose_validation():
    f = puro.puro_quant_transpose
    assert f(2, A0, 128, 128, A1, A2, None, None) == MODE
    assert f(0, A0, 120, 128, A1, A2, None, None) == SHAPE    # rows must be a multiple of 16 here
    assert f(1, A0, 128, 8, A1, A2, None, None) == SHAPE
    assert f(0, A0, 128, 128, A1, A2, A3, None) == NULL       # q_row without s_row
    assert f(0, A0, 128, 128, None, A2, None, None) == NULL
    assert f(0, A0, 128, 128, A1, A2, A3 + 8, A4) == ALIGN
    assert f(0, A0, 128, 128, A1, A2, A1 + 1024, A4) == ALIAS  # q_row overlaps qt
    assert f(0, A0, 0, 128, None, None, None, None) == OK


def test_quant_act_128x1_validation():
    f = puro.puro_quant_act_128x1
    assert f(A0, 128, 100, A1, A2, None, None) == SHAPE                   # cols not a multiple of 16
    assert f(A0, -1, 128, A1, A2, None, None) == SHAPE
    assert f(A0, 120, 128, A1, A2, None, None) != SHAPE                   # rows free
    assert f(None, 0, 128, None, None, None, None) == OK
    assert f(A0, 128, 128, A1, A2, A3, None) == NULL                      # q_row without s_row
    assert f(A0, 128, 128, None, A2, None, None) == NULL
    assert f(A0, 128, 128, A1, None, None, None) == NULL
    assert f(A0 + 8, 128, 128, A1, A2, None, None) == ALIGN
    assert f(A0, 128, 128, A1, A2 + 4, None, None) == ALIGN
    assert f(A0, 128, 128, A1, A2, A3 + 2, A4) == ALIGN
    assert f(A0, 128, 128, A0 + 4096, A2, None, None) == ALIAS            # codes inside x
    assert f(A0, 128, 128, A1, A2, A1 + 64, A4) == ALIAS                  # row codes overlap the 128x1 codes
    if no_gpu():
        assert f(A0, 128, 128, A1, A2, A3, A4) == DEVICE


def test_requant_validation():
    f = puro.puro_requant_act_t
    assert f(A0, A1, 120, 128, A2, A3) == SHAPE               # rows must be a multiple of 16
    assert f(A0, A1, 128, 100, A2, A3) == SHAPE
    assert f(A0, A1, -16, 128, A2, A3) == SHAPE
    assert f(A0, A1, 1 << 31, 128, A2, A3) == SHAPE
    assert f(None, None, 0, 128, None, None) == OK            # empty: nothing to do
    assert f(A0, A1, 128, 0, None, None) == OK
    assert f(None, A1, 128, 128, A2, A3) == NULL
    assert f(A0, None, 128, 128, A2, A3) == NULL
    assert f(A0, A1, 128, 128, None, A3) == NULL
    assert f(A0, A1, 128, 128, A2, None) == NULL
    assert f(A0 + 8, A1, 128, 128, A2, A3) == ALIGN
    assert f(A0, A1 + 4, 128, 128, A2, A3) == ALIGN
    assert f(A0, A1, 128, 128, A2, A3 + 4) == ALIGN
    assert f(A0, A1, 128, 128, A0 + 1024, A3) == ALIAS        # qt overlaps q
    assert f(A0, A1, 128, 128, A2, A1 + 256) == ALIAS         # st overlaps s
    assert f(A0, A1, 128, 128, A2, A2 + 4096) == ALIAS        # st inside qt
    if no_gpu():
        assert f(A0, A1, 128, 128, A2, A3) == DEVICE


def test_swiglu_quant_validation():
    f = puro.puro_swiglu_quant
    assert f(A0, 128, 100, A1, A2, None, None, None) == SHAPE             # inter not a multiple of 16
    assert f(A0, 120, 128, A1, A2, A3, A4, None) == SHAPE                 # rows must be a multiple of 16 for qt
    assert f(A0, -1, 128, A1, A2, None, None, None) == SHAPE
    assert f(A0, 16, 1 << 30, A1, A2, None, None, None) == SHAPE          # 2 * inter over the dimension limit
    assert f(A0, 120, 128, A1, A2, None, None, None) != SHAPE             # rows free without qt
    assert f(None, 0, 128, None, None, None, None, None) == OK
    assert f(A0, 128, 128, A1, A2, A3, None, None) == NULL                # qt without st
    assert f(None, 128, 128, A1, A2, None, None, None) == NULL
    assert f(A0, 128, 128, None, A2, None, None, None) == NULL
    assert f(A0, 128, 128, A1, None, None, None, None) == NULL
    assert f(A0 + 8, 128, 128, A1, A2, None, None, None) == ALIGN
    assert f(A0, 128, 128, A1, A2, None, None, A5 + 2) == ALIGN           # h misaligned
    assert f(A0, 128, 128, A1, A2, A3 + 4, A4, None) == ALIGN
    assert f(A0, 128, 128, A0 + 4096, A2, None, None, None) == ALIAS      # q inside gu
    assert f(A0, 128, 128, A1, A2, None, None, A1 + 64) == ALIAS          # h overlaps q
    assert f(A0, 128, 128, A1, A2, A3, A3 + 1024, None) == ALIAS          # st inside qt
    if no_gpu():
        assert f(A0, 128, 128, A1, A2, A3, A4, A5) == DEVICE


# ---------------------------------------------------------------- GEMM
def test_gemm_validation():
    f = puro.puro_gemm_fp8_blockwise
    M, N, K = 256, 256, 256
    args = dict(a=A0, sa=A1, b=A2, sb=A3, out=A4)

    def call(mode=0, od=0, M=M, N=N, K=K, ws=None, wsb=0, **kw):
        a = dict(args, **kw)
        return f(mode, a["a"], a["sa"], a["b"], a["sb"], a["out"], od, M, N, K, ws, wsb)

    assert call(mode=4) == MODE
    assert call(mode=-1) == MODE
    assert call(od=2) == DTYPE
    assert call(mode=3, M=200) == SHAPE                   # token-major wgrad: M and N multiples of 16
    assert call(mode=3, N=8) == SHAPE
    assert call(mode=3, M=1 << 30, N=16, K=16) == SHAPE   # 4 rows of a must index in 32 bits
    assert call(K=100) == SHAPE
    assert call(M=-5) == SHAPE
    assert call(K=1 << 24) == SHAPE
    assert call(M=0) == OK and call(N=0) == OK
    assert call(out=None) == NULL
    assert call(a=None) == NULL
    assert call(sb=None) == NULL
    assert call(a=A0 + 1) == ALIGN
    assert call(out=A4 + 2) == ALIGN
    assert call(out=A0) == ALIAS
    assert call(out=A3) == ALIAS                          # out starts on sb
    if no_gpu():   # valid arguments: only safe to call with fake pointers when no device exists
        assert call() == DEVICE
        assert call(K=0, a=None, sa=None, b=None, sb=None) == DEVICE


def test_gemm_accumulate_validation():
    f = puro.puro_gemm_fp8_blockwise_accumulate
    M, N, K = 256, 256, 256
    args = dict(a=A0, sa=A1, b=A2, sb=A3, out=A4)

    def call(mode=0, M=M, N=N, K=K, ws=None, wsb=0, **kw):
        a = dict(args, **kw)
        return f(mode, a["a"], a["sa"], a["b"], a["sb"], a["out"], M, N, K, ws, wsb)

    assert call(mode=4) == MODE
    assert call(K=100) == SHAPE
    assert call(M=0) == OK
    assert call(out=None) == NULL
    assert call(b=None) == NULL
    assert call(out=A4 + 4) == ALIGN
    assert call(out=A2 + 1024) == ALIAS                   # out inside b
    assert call(mode=2, M=2048, N=2048, K=16384) == WS      # split-K plan needs a workspace
    if no_gpu():
        assert call() == DEVICE
        assert call(K=0, a=None, sa=None, b=None, sb=None) == DEVICE


def test_gemm_swiglu_quant_validation():
    f = puro.puro_gemm_fp8_swiglu_quant
    M, I, K = 256, 256, 256
    args = dict(a=A0, sa=A1, b=A2, sb=A3, gu=A4, hq=A5, hs=A6)

    def call(M=M, I=I, K=K, **kw):
        a = dict(args, **kw)
        return f(a["a"], a["sa"], a["b"], a["sb"], M, I, K, a["gu"], a["hq"], a["hs"])

    assert call(I=192) == SHAPE                            # inter must be a multiple of 128
    assert call(I=-128) == SHAPE
    assert call(K=100) == SHAPE
    assert call(M=-1) == SHAPE
    assert call(K=1 << 24) == SHAPE
    assert call(I=1 << 30, K=16) == SHAPE                  # 2 * inter over the dimension limit
    assert call(I=1 << 22, K=1024) == SHAPE                # B row offsets past 32 bits
    assert call(M=0) == OK and call(I=0) == OK
    assert call(hq=None) == NULL
    assert call(hs=None) == NULL
    assert call(a=None) == NULL
    assert call(sb=None) == NULL
    assert call(a=A0 + 1) == ALIGN
    assert call(gu=A4 + 2) == ALIGN
    assert call(hs=A6 + 4) == ALIGN
    assert call(hq=A2 + 4096) == ALIAS                     # hq inside b
    assert call(hs=A4 + 1024) == ALIAS                     # hs inside gu
    assert call(gu=A5) == ALIAS                            # gu starts on hq
    if no_gpu():   # valid arguments: only safe to call with fake pointers when no device exists
        assert call() == DEVICE
        assert call(gu=None) == DEVICE
        assert call(K=0, a=None, sa=None, b=None, sb=None) == DEVICE


def test_gemm_workspace_sizing():
    ws = puro.puro_gemm_workspace_bytes
    # invalid arguments size to 0
    assert ws(5, 256, 256, 256) == 0 and ws(0, 0, 256, 256) == 0 and ws(0, 256, 256, -1) == 0
    # plenty of output tiles: no split
    assert ws(0, 4096, 4096, 2048) == 0
    # deterministic
    for shape in [(2, 2048, 6144, 8192), (2, 2048, 2048, 16384), (0, 256, 256, 8192)]:
        assert ws(*shape) == ws(*shape)
    # a split-K shape has one 256 x 256 fp32 block per split of each split tile
    tile = 256 * 256 * 4
    n = ws(2, 2048, 2048, 16384)
    assert n > 0 and n % tile == 0
    # the layer's split wgrads at 16384 tokens: qkv (128 tiles) in 2, o (64 tiles) in 4, gate_up
    # (384 tiles: 256 whole, the other 128 in 2), down unsplit (256 tiles 192 columns wide)
    assert ws(2, 4096, 2048, 16384) == 2 * 128 * tile
    assert ws(2, 2048, 2048, 16384) == 4 * 64 * tile
    assert ws(2, 12288, 2048, 16384) == 2 * 128 * tile
    assert ws(2, 2048, 6144, 16384) == 0
    # none of them needs more than 64 MiB
    assert max(ws(2, M, N, 16384) for M, N in [(4096, 2048), (2048, 2048), (12288, 2048), (2048, 6144)]) == 64 << 20
    # 258 tiles (6 x 43) at 8 K slices: whole tiles first, the last two split in 2
    assert ws(0, 1480, 10900, 1008) == 2 * 2 * tile
    # ragged edge tiles take a whole block too
    assert ws(2, 510, 511, 4096) % tile == 0
    # weight-gradient shapes that narrower tiles fill in whole rounds need no workspace; a 128-column
    # plan split over K takes 256 x 128 blocks
    assert ws(2, 2048, 6144, 1024) == 0 and ws(2, 4096, 2048, 2048) == 0
    assert ws(2, 2048, 2048, 8192) == 2 * 128 * 256 * 128 * 4
    # the fprop and dgrad shapes of the layer never split
    for M, N, K in [(16384, 4096, 2048), (16384, 2048, 2048), (16384, 12288, 2048), (16384, 2048, 6144),
                    (16384, 2048, 4096), (16384, 2048, 12288), (16384, 6144, 2048)]:
        assert ws(0, M, N, K) == 0 and ws(1, M, N, K) == 0


def test_gemm_workspace_errors():
    f = puro.puro_gemm_fp8_blockwise
    M, N, K = 2048, 2048, 16384
    need = puro.puro_gemm_workspace_bytes(2, M, N, K)
    assert need > 0
    assert f(2, A0, A1, A2, A3, A4, 0, M, N, K, None, 0) == WS
    assert f(2, A0, A1, A2, A3, A4, 0, M, N, K, A5, need - 16) == WS
    assert f(2, A0, A1, A2, A3, A4, 0, M, N, K, A5 + 4, need) == ALIGN
    assert f(2, A0, A1, A2, A3, A4, 0, M, N, K, A4 + 16, need) == ALIAS
    if no_gpu():   # valid arguments: only safe to call with fake pointers when no device exists
        assert f(2, A0, A1, A2, A3, A4, 0, M, N, K, A5, need) == DEVICE


def test_quant_weights_validation():
    """The grouped weight quantizer checks every entry on the host before any launch."""
    f = puro.puro_quant_weights
    MB = 1 << 26
    def wt(i, R=256, C=256, row=True, tr=True):
        base = A0 + i * (1 << 32)
        return (base, R, C, base + MB if row else None, base + 2 * MB if row else None,
                base + 3 * MB if tr else None, base + 4 * MB if tr else None)
    assert f([]) == OK
    assert f([wt(i) for i in range(9)]) == SHAPE                     # at most 8
    assert f([wt(0), wt(1, C=100)]) == SHAPE                         # cols not a multiple of 16
    assert f([wt(0), wt(1, R=100)]) == SHAPE                         # transposed output needs rows % 16
    assert f([wt(0), wt(1, R=100, tr=False)]) == NULL                # rows free without qt, but outputs differ
    assert f([wt(0), wt(1, tr=False)]) == NULL                       # every entry the same outputs
    assert f([wt(0, row=False, tr=False)]) == NULL                   # no output at all
    bad = list(wt(1)); bad[4] = None
    assert f([wt(0), tuple(bad)]) == NULL                            # q without s
    bad = list(wt(1)); bad[0] = None
    assert f([wt(0), tuple(bad)]) == NULL                            # no input
    bad = list(wt(1)); bad[5] = bad[5] + 4
    assert f([wt(0), tuple(bad)]) == ALIGN
    bad = list(wt(1)); bad[3] = wt(0)[0]                             # an output over another entry's input
    assert f([wt(0), tuple(bad)]) == ALIAS
    bad = list(wt(1)); bad[5] = wt(0)[5]                             # two entries share an output
    assert f([wt(0), tuple(bad)]) == ALIAS
    assert f([(0, 0, 256, 0, 0, 0, 0), (0, 16, 0, 0, 0, 0, 0)]) == OK   # only empty entries: nothing to do
    if no_gpu():
        assert f([wt(0), wt(1, 2048, 6144), wt(2, 0, 512)]) == DEVICE
        assert f([(0, 0, 256, 0, 0, 0, 0), wt(1, tr=False)]) == DEVICE     # empty entries are not compared
        assert f([wt(i, tr=False) for i in range(8)]) == DEVICE


def test_gemm_noalloc_validation():
    """The allocation-free GEMM validates like the workspace one, without a workspace, and
    refuses shapes whose split-K plan needs more than the library's 64 MiB scratch."""
    f = puro.puro_gemm_fp8_blockwise_noalloc
    assert f(7, A0, A1, A2, A3, A4, 0, 256, 256, 256) == MODE
    assert f(0, A0, A1, A2, A3, A4, 5, 256, 256, 256) == DTYPE
    assert f(0, A0, A1, A2, A3, A4, 0, 256, 256, 100) == SHAPE
    assert f(0, None, A1, A2, A3, A4, 0, 256, 256, 256) == NULL
    assert f(0, A0 + 4, A1, A2, A3, A4, 0, 256, 256, 256) == ALIGN
    assert f(0, A0, A1, A2, A3, A0, 0, 256, 256, 256) == ALIAS
    assert puro.puro_gemm_workspace_bytes(2, 2560, 2560, 1 << 20) > puro.SCRATCH_BYTES
    assert f(2, A0, A1, A2, A3, A4, 0, 2560, 2560, 1 << 20) == SCRATCH
    assert f(0, A0, A1, A2, A3, A4, 0, 0, 256, 256) == OK           # empty output: nothing to do
    if no_gpu():
        # the layer's largest split plans fit the scratch; valid calls stop at the device check
        for M, N in [(4096, 2048), (2048, 2048), (12288, 2048)]:
            assert 0 < puro.puro_gemm_workspace_bytes(2, M, N, 16384) <= puro.SCRATCH_BYTES
            assert f(2, A0, A1, A2, A3, A4, 0, M, N, 16384) == DEVICE


def test_tensor_helpers_reject_host_tensors_and_bad_modes():
    """The tensor helpers check their tensors before any C call (they need CUDA tensors)."""
    import torch
    a = torch.zeros((16, 128), dtype=torch.uint8)
    sa = torch.zeros((1, 16), dtype=torch.float32)
    with pytest.raises(TypeError):
        puro.gemm_fp8_blockwise(puro.FPROP, a, sa, a, torch.zeros((1, 1)))
    with pytest.raises(ValueError):
        puro.gemm_fp8_blockwise(7, a, sa, a, torch.zeros((1, 1)))
    with pytest.raises(TypeError):
        puro.requant_act_t(a, sa)
    with pytest.raises(TypeError):
        puro.quant_act_1x128(torch.zeros((16, 128), dtype=torch.bfloat16))
