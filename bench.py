#!/usr/bin/env python3
"""Benchmark of the blockwise-FP8 path on one MI355X (gfx950).

One step = one pass of the whole path over one Qwen3-1.7B-shaped layer
(Puro-2B: hidden 2048, 16 query + 8 key/value heads of 128, MLP 6144) at
16384 tokens: for each of the four main linears (QKV 2048->4096, O
2048->2048, gate_up 2048->12288, down 6144->2048)
  - dual 128x1 / 1x128 quantization of the input X (one read of X),
  - dual transposed / plain 128x128 quantization of the weight W (the four
    weights in one launch at the start of the step),
  - dual 128x1 / 1x128 quantization of the output gradient dY,
  - fprop  Y  = X W^T     (bf16 out),
  - dgrad  dX = dY W      (bf16 out),
  - wgrad  dW = dY^T X    (fp32 out, contracting over the tokens).
Inputs are seeded synthetic tensors (see workloads.py) resident in HBM before
the timed region.  The reported value is GEMM TFLOP/s over the whole step
(quantizers included in the time).  The timed steps record HIP events only at
their two ends; the per-launch table (and the roofline of a workload of several
kernel kinds) comes from as many further steps with an event between
consecutive launches.

Other workloads (--workload):
  layer_fp8_saved  the same layer step when the forward pass keeps only the
                   1x128 FP8 codes of each input X: the wgrad operand X^T is
                   rebuilt from them by the requantizer (dequantize, 128x1
                   quantization of the transpose) instead of quantized from
                   the bf16 X;
  requant          the requantizer alone over the layer's four saved inputs
                   (16384 x 2048 three times, 16384 x 6144): HBM GB/s;
  layer_accum      the layer step of one micro-batch whose weight gradients are
                   added into persistent fp32 buffers (accumulating wgrad);
  swiglu_quant     the fused SwiGLU + 1x128 / 128x1 quantization of the MLP's
                   gate/up output at 16384 tokens (16384 x 12288 in, the down
                   projection's two operands out): HBM GB/s;
  qkv_fprop, mlp_fprop, mlp_down_bwd   single GEMM slices of the layer.

The default layer run also reports, in its `configs` block, the four smaller
workloads measured in the same invocation (tiny fprop, QKV fprop at 4096 tokens,
MLP fprop and MLP down backward at 8192 tokens), each with its quantizers and
GEMMs: ms per step, TFLOP/s and % of the FP8 peak, quantizer GB/s and % of HBM.
Every workload whose buffers (inputs, outputs, workspaces) come to less than
512 MB rotates over as many copies of them as it takes to exceed 512 MB, twice
the 256 MB of L2 and MALL.

Prints ONE JSON line.  Options: --steps K --warmup W (defaults 30 / 10 for the
layer workloads, 300 / 300 for the single-kernel ones), --no-configs,
--gpus N (only 1 is supported: the path is measured on one GPU),
--workload NAME, --no-cpu-baseline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP8_FLOPS = 5.0e15      # MI355X dense FP8 MFMA, published
PEAK_HBM_BPS = 8.0e12        # MI355X HBM3E, published
METRIC = "blockwise-FP8 GEMM TFLOP/s & % FP8 MFMA peak; quantizer GB/s, Puro-2B shapes"
_CSRC = os.path.join(ROOT, "blockwise_fp8_gemm_act_amd", "csrc")
# rocprofv3 counter records per kernel family: the file and the sources its figures were taken on
TRAFFIC = {
    "gemm": (os.path.join(ROOT, "profiles", "gemm_traffic.json"),
             [os.path.join(_CSRC, f) for f in ("gemm.hip", "device_common.h")]),
    "requant": (os.path.join(ROOT, "profiles", "requant_traffic.json"),
                [os.path.join(_CSRC, f) for f in ("quant.hip", "device_common.h")]),
    "swiglu_quant": (os.path.join(ROOT, "profiles", "swiglu_quant_traffic.json"),
                     [os.path.join(_CSRC, f) for f in ("quant.hip", "device_common.h")]),
}


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps (default: 30, or 300 for a single-kernel workload)")
    ap.add_argument("--warmup", type=int, default=None, help="untimed steps first (default: 10, or 300 for a single-kernel workload)")
    ap.add_argument("--workload", default="layer",
                    choices=["layer", "layer_fp8_saved", "layer_accum", "requant", "swiglu_quant", "qkv_fprop", "mlp_fprop",
                             "mlp_down_bwd", "mlp_swiglu_fprop", "mlp_swiglu_fused", "mlp_swiglu_fused_nogu", "layer_tm"])
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    ap.add_argument("--no-configs", action="store_true",
                    help="layer workload: skip the per-config lines of the smaller workloads")
    ap.add_argument("--config-steps", type=int, default=50,
                    help="warm-up and timed steps of each smaller workload in the configs block")
    args = ap.parse_args()
    # A single-kernel step lasts ~0.1 ms: a few hundred untimed steps first let the
    # clocks settle (5 of them left the fused SwiGLU kernel ~10% slower), and the
    # timed region still lasts only tens of milliseconds.
    micro = args.workload in ("requant", "swiglu_quant")
    if args.warmup is None:
        args.warmup = 300 if micro else 10
    if args.steps is None:
        args.steps = 300 if micro else 30
    return args


def cdiv(a, b):
    return (a + b - 1) // b


class Launch:
    """One kernel launch of a step: what it is and its algorithmic work."""

    def __init__(self, kind, name, fn, flops=0.0, bytes_=0.0):
        self.kind, self.name, self.fn, self.flops, self.bytes = kind, name, fn, flops, bytes_


def build_plan(workload, tensors, puro, torch):
    """Allocate every output once and return the list of launches of one step."""
    dev = "cuda"
    stream = torch.cuda.current_stream().cuda_stream
    keep = []
    launches = []

    def alloc(shape, dtype):
        t = torch.empty(shape, dtype=dtype, device=dev)
        keep.append(t)
        return t

    def check(st, what):
        if st != 0:
            raise RuntimeError("%s failed: %s" % (what, puro.puro_status_str(st)))

    def q_act_dual(x, name):
        R, C = x.shape
        qt, st = alloc((C, R), torch.uint8), alloc((cdiv(R, 128), C), torch.float32)
        q, s = alloc((R, C), torch.uint8), alloc((cdiv(C, 128), R), torch.float32)
        args = (puro.T_ACT, x.data_ptr(), R, C, qt.data_ptr(), st.data_ptr(), q.data_ptr(), s.data_ptr(), stream)
        launches.append(Launch("quant", name, lambda: check(puro.puro_quant_transpose(*args), name),
                               bytes_=R * C * (2 + 2 * (1 + 4 / 128))))
        return (q, s), (qt, st)

    def q_act_tm(x, name):
        """1x128 codes and the 128x1 codes in x's own layout (token-major wgrad operand), one read."""
        R, C = x.shape
        qc, sc = alloc((R, C), torch.uint8), alloc((cdiv(R, 128), C), torch.float32)
        q, s = alloc((R, C), torch.uint8), alloc((cdiv(C, 128), R), torch.float32)
        args = (x.data_ptr(), R, C, qc.data_ptr(), sc.data_ptr(), q.data_ptr(), s.data_ptr(), stream)
        launches.append(Launch("quant", name, lambda: check(puro.puro_quant_act_128x1(*args), name),
                               bytes_=R * C * (2 + 2 * (1 + 4 / 128))))
        return (q, s), (qc, sc)

    def q_act(x, name):
        R, C = x.shape
        q, s = alloc((R, C), torch.uint8), alloc((cdiv(C, 128), R), torch.float32)
        args = (x.data_ptr(), R, C, q.data_ptr(), s.data_ptr(), stream)
        launches.append(Launch("quant", name, lambda: check(puro.puro_quant_act_1x128(*args), name),
                               bytes_=R * C * (2 + 1 + 4 / 128)))
        return q, s

    def q_w_dual(w, name, transposed=True):
        R, C = w.shape
        q, s = alloc((R, C), torch.uint8), alloc((cdiv(R, 128), cdiv(C, 128)), torch.float32)
        if transposed:
            qt, st = alloc((C, R), torch.uint8), alloc((cdiv(C, 128), cdiv(R, 128)), torch.float32)
            args = (puro.T_WEIGHT, w.data_ptr(), R, C, qt.data_ptr(), st.data_ptr(), q.data_ptr(), s.data_ptr(), stream)
            launches.append(Launch("quant", name, lambda: check(puro.puro_quant_transpose(*args), name),
                                   bytes_=R * C * (2 + 2 * (1 + 4 / 16384))))
            return (q, s), (qt, st)
        args = (w.data_ptr(), R, C, q.data_ptr(), s.data_ptr(), stream)
        launches.append(Launch("quant", name, lambda: check(puro.puro_quant_w_128x128(*args), name),
                               bytes_=R * C * (2 + 1 + 4 / 16384)))
        return (q, s), None

    def q_weights(ws, name):
        """All of the layer's weights in one launch, dual (128x128 codes and their transpose)."""
        descs, outs, total = [], [], 0
        for w in ws:
            R, C = w.shape
            q, s = alloc((R, C), torch.uint8), alloc((cdiv(R, 128), cdiv(C, 128)), torch.float32)
            qt, st = alloc((C, R), torch.uint8), alloc((cdiv(C, 128), cdiv(R, 128)), torch.float32)
            descs.append((w.data_ptr(), R, C, q.data_ptr(), s.data_ptr(), qt.data_ptr(), st.data_ptr()))
            outs.append(((q, s), (qt, st)))
            total += R * C * (2 + 2 * (1 + 4 / 16384))
        arr = [puro.PuroWeight(*d) for d in descs]
        launches.append(Launch("quant", name, lambda: check(puro.puro_quant_weights(arr, stream), name), bytes_=total))
        return outs

    def requant(saved, name):
        q, s = saved
        R, C = q.shape
        qt, st = alloc((C, R), torch.uint8), alloc((cdiv(R, 128), C), torch.float32)
        args = (q.data_ptr(), s.data_ptr(), R, C, qt.data_ptr(), st.data_ptr(), stream)
        launches.append(Launch("requant", name, lambda: check(puro.puro_requant_act_t(*args), name),
                               bytes_=R * C * (2 + 4 / 128 + 4 / 128)))
        return qt, st

    def swiglu(gu, name, dual=True):
        R, C2 = gu.shape
        I = C2 // 2
        q, s = alloc((R, I), torch.uint8), alloc((cdiv(I, 128), R), torch.float32)
        qt = st = None
        if dual:
            qt, st = alloc((I, R), torch.uint8), alloc((cdiv(R, 128), I), torch.float32)
        args = (gu.data_ptr(), R, I, q.data_ptr(), s.data_ptr(), qt.data_ptr() if dual else None,
                st.data_ptr() if dual else None, None, stream)
        launches.append(Launch("swiglu_quant", name, lambda: check(puro.puro_swiglu_quant(*args), name),
                               bytes_=R * I * (4 + (2 if dual else 1) * (1 + 4 / 128))))
        return (q, s), (qt, st)

    def gemm_swiglu(a, b, name, write_gu=True):
        """gate_up fprop with the SwiGLU quantizer as its epilogue; writes gu (for the backward) too
        unless write_gu is false."""
        (aq, sa), (bq, sb) = a, b
        M, K = aq.shape
        N = bq.shape[0]
        I = N // 2
        gu = alloc((M, N), torch.bfloat16) if write_gu else None
        q, s = alloc((M, I), torch.uint8), alloc((I // 128, M), torch.float32)
        args = (aq.data_ptr(), sa.data_ptr(), bq.data_ptr(), sb.data_ptr(), M, I, K,
                gu.data_ptr() if write_gu else None, q.data_ptr(), s.data_ptr(), stream)
        launches.append(Launch("gemm:fprop_swiglu", name, lambda: check(puro.puro_gemm_fp8_swiglu_quant(*args), name),
                               flops=2.0 * M * N * K,
                               bytes_=M * K + N * K + 4 * (M + N // 128) * cdiv(K, 128) + (M * N * 2 if write_gu else 0)
                               + M * I * (1 + 4 / 128)))
        return q, s

    def gemm(mode, a, b, out_dtype, name, accumulate=False):
        (aq, sa), (bq, sb) = a, b
        if mode == 3:                               # token-major wgrad operands: a [K][M], b [K][N]
            K, M = aq.shape
            N = bq.shape[1]
        else:
            M, K = aq.shape
            N = bq.shape[0]
        out = alloc((M, N), out_dtype)
        if accumulate:
            out.zero_()
        need = puro.puro_gemm_workspace_bytes(mode, M, N, K)
        ws = alloc((max(need, 16),), torch.uint8)
        od = puro.OUT_BF16 if out_dtype == torch.bfloat16 else puro.OUT_F32
        flops = 2.0 * M * N * K
        kind = "gemm:" + {puro.WGRAD: "wgrad", 3: "wgrad_tm"}.get(mode, "fprop_dgrad") + ("_acc" if accumulate else "")
        if accumulate:
            args = (mode, aq.data_ptr(), sa.data_ptr(), bq.data_ptr(), sb.data_ptr(), out.data_ptr(),
                    M, N, K, ws.data_ptr(), need, stream)
            fn = lambda: check(puro.puro_gemm_fp8_blockwise_accumulate(*args), name)
        else:
            args = (mode, aq.data_ptr(), sa.data_ptr(), bq.data_ptr(), sb.data_ptr(), out.data_ptr(), od,
                    M, N, K, ws.data_ptr(), need, stream)
            fn = lambda: check(puro.puro_gemm_fp8_blockwise(*args), name)
        launches.append(Launch(kind, name, fn, flops=flops,
                               bytes_=M * K + N * K + 4 * M * cdiv(K, 128) + 4 * N * cdiv(K, 128)
                               + M * N * (8 if accumulate else (2 if od else 4))))
        return out

    if workload in ("layer", "layer_accum"):
        from workloads import LINEARS
        wq = dict(zip(LINEARS, q_weights([tensors["w_" + lin] for lin in LINEARS], "weights.quant_w")))
        for lin in LINEARS:
            x, dy = tensors["x_" + lin], tensors["dy_" + lin]
            xrow, xt = q_act_dual(x, lin + ".quant_x")
            wrow, wt = wq[lin]
            dyrow, dyt = q_act_dual(dy, lin + ".quant_dy")
            gemm(puro.FPROP, xrow, wrow, torch.bfloat16, lin + ".fprop")
            gemm(puro.DGRAD, dyrow, wt, torch.bfloat16, lin + ".dgrad")
            gemm(puro.WGRAD, dyt, xt, torch.float32, lin + ".wgrad", accumulate=workload == "layer_accum")
    elif workload == "layer_tm":
        from workloads import LINEARS
        wq = dict(zip(LINEARS, q_weights([tensors["w_" + lin] for lin in LINEARS], "weights.quant_w")))
        for lin in LINEARS:
            x, dy = tensors["x_" + lin], tensors["dy_" + lin]
            xrow, xc = q_act_tm(x, lin + ".quant_x")
            wrow, wt = wq[lin]
            dyrow, dyc = q_act_tm(dy, lin + ".quant_dy")
            gemm(puro.FPROP, xrow, wrow, torch.bfloat16, lin + ".fprop")
            gemm(puro.DGRAD, dyrow, wt, torch.bfloat16, lin + ".dgrad")
            gemm(3, dyc, xc, torch.float32, lin + ".wgrad")
    elif workload == "layer_fp8_saved":
        from workloads import LINEARS
        wq = dict(zip(LINEARS, q_weights([tensors["w_" + lin] for lin in LINEARS], "weights.quant_w")))
        for lin in LINEARS:
            x, dy = tensors["x_" + lin], tensors["dy_" + lin]
            xrow = q_act(x, lin + ".quant_x")
            wrow, wt = wq[lin]
            dyrow, dyt = q_act_dual(dy, lin + ".quant_dy")
            gemm(puro.FPROP, xrow, wrow, torch.bfloat16, lin + ".fprop")
            gemm(puro.DGRAD, dyrow, wt, torch.bfloat16, lin + ".dgrad")
            xt = requant(xrow, lin + ".requant_x")
            gemm(puro.WGRAD, dyt, xt, torch.float32, lin + ".wgrad")
    elif workload == "requant":
        # the saved codes are made once, outside the timed step
        from workloads import LINEARS
        for lin in LINEARS:
            x = tensors["x_" + lin]
            R, C = x.shape
            q, s = alloc((R, C), torch.uint8), alloc((cdiv(C, 128), R), torch.float32)
            check(puro.puro_quant_act_1x128(x.data_ptr(), R, C, q.data_ptr(), s.data_ptr(), stream), "setup")
            requant((q, s), lin + ".requant_x")
    elif workload == "swiglu_quant":
        swiglu(tensors["gu"], "down.swiglu_quant")
    elif workload == "tiny_fprop":
        xrow = q_act(tensors["x"], "quant_x")
        wrow, _ = q_w_dual(tensors["w"], "quant_w", transposed=False)
        gemm(puro.FPROP, xrow, wrow, torch.float32, "fprop")
    elif workload == "qkv_fprop":
        xrow = q_act(tensors["x"], "quant_x")
        wrow, _ = q_w_dual(tensors["w"], "quant_w", transposed=False)
        gemm(puro.FPROP, xrow, wrow, torch.bfloat16, "fprop")
    elif workload == "mlp_fprop":
        for lin in ("gate_up", "down"):
            xrow = q_act(tensors["x_" + lin], lin + ".quant_x")
            wrow, _ = q_w_dual(tensors["w_" + lin], lin + ".quant_w", transposed=False)
            gemm(puro.FPROP, xrow, wrow, torch.bfloat16, lin + ".fprop")
    elif workload in ("mlp_swiglu_fprop", "mlp_swiglu_fused", "mlp_swiglu_fused_nogu"):
        xrow = q_act(tensors["x_gate_up"], "gate_up.quant_x")
        wgu, _ = q_w_dual(tensors["w_gate_up"], "gate_up.quant_w", transposed=False)
        wdn, _ = q_w_dual(tensors["w_down"], "down.quant_w", transposed=False)
        if workload != "mlp_swiglu_fprop":
            h = gemm_swiglu(xrow, wgu, "gate_up.fprop_swiglu_quant", write_gu=workload == "mlp_swiglu_fused")
        else:
            gu = gemm(puro.FPROP, xrow, wgu, torch.bfloat16, "gate_up.fprop")
            h, _ = swiglu(gu, "down.swiglu_quant", dual=False)
        gemm(puro.FPROP, h, wdn, torch.bfloat16, "down.fprop")
    elif workload == "mlp_down_bwd":
        dyrow, dyt = q_act_dual(tensors["dy"], "quant_dy")
        _, wt = q_w_dual(tensors["w"], "quant_w")
        _, xt = q_act_dual(tensors["x"], "quant_x")
        gemm(puro.DGRAD, dyrow, wt, torch.bfloat16, "dgrad")
        gemm(puro.WGRAD, dyt, xt, torch.float32, "wgrad")
    return launches, keep


WORKLOAD_DESC = {
    "layer": ("Qwen3-1.7B-shaped layer (Puro-2B), 16384 tokens: QKV 2048->4096, O 2048->2048, "
              "gate_up 2048->12288, down 6144->2048; fprop+dgrad+wgrad and every quantize/transpose kernel"),
    "layer_accum": ("the layer step (16384 tokens) of one micro-batch: wgrad adds into persistent fp32 dW buffers"),
    "layer_tm": ("the layer step (16384 tokens) with token-major wgrad operands: X and dY quantized 1x128 and 128x1 "
                 "in one read with the 128x1 codes untransposed, wgrad reading them token-major"),
    "layer_fp8_saved": ("the layer step (16384 tokens) with FP8-saved inputs: X quantized 1x128 only, the wgrad "
                        "operand X^T requantized from those codes"),
    "requant": ("requantization of the layer's saved 1x128 input codes into transposed 128x1 tiles, 16384 tokens: "
                "X_qkv, X_o, X_gate_up [16384x2048], X_down [16384x6144]"),
    "swiglu_quant": ("fused SwiGLU of the MLP gate/up output [16384x12288] (gate first) with 1x128 and 128x1 "
                     "quantization of h [16384x6144], the down projection's fprop and wgrad operands"),
    "tiny_fprop": "tiny fprop: X[256x256] (2 outlier channels) x W[512x256]^T -> fp32, quantizers included",
    "qkv_fprop": "QKV projection fprop, 4096 tokens: X[4096x2048] x W[4096x2048]^T -> bf16",
    "mlp_fprop": "MLP fprop, 8192 tokens: gate_up X[8192x2048] x W[12288x2048]^T, down X[8192x6144] x W[2048x6144]^T",
    "mlp_down_bwd": "MLP down backward, 8192 tokens: dgrad dY[8192x2048] x W[2048x6144], wgrad dY^T x X[8192x6144]",
    "mlp_swiglu_fprop": ("MLP forward, 16384 tokens: gate_up fprop X[16384x2048] x W[12288x2048]^T -> bf16, SwiGLU "
                         "quantizer -> 1x128 codes of h [16384x6144], down fprop h x W[2048x6144]^T"),
    "mlp_swiglu_fused": ("MLP forward, 16384 tokens, as mlp_swiglu_fprop with the SwiGLU quantizer fused into the "
                         "gate_up GEMM's epilogue (the bf16 gate/up output is still written for the backward)"),
    "mlp_swiglu_fused_nogu": ("MLP forward, 16384 tokens, as mlp_swiglu_fused without writing the bf16 gate/up "
                              "output (a backward that recomputes it)"),
}


def _code_only(text: str) -> str:
    """C++ source without its comments and blank space, so that edits to comments do not
    count as kernel changes (the sources hold no comment markers inside string literals)."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_hash(family="gemm"):
    """Hash of the code (comments and spacing aside) of the kernel sources a traffic record was taken on."""
    h = hashlib.sha256()
    for p in TRAFFIC[family][1]:
        with open(p) as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def load_traffic(kernel_kind):
    """HBM traffic per launch measured with rocprofv3 counters, if taken on the current kernel source."""
    family = kernel_kind.split(":")[0]
    if family not in TRAFFIC:
        return None
    try:
        with open(TRAFFIC[family][0]) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != source_hash(family):
        return None
    ent = rec.get("kernels", {}).get(kernel_kind)
    return None if ent is None else ent.get("bytes_per_launch")


def cpu_baseline_requant(tensors, budget_s):
    """The oracle's requantizer (as it is) on the host cores over a bounded sample:
    row slabs of the 16384 x 6144 input's saved codes, growing until about
    `budget_s` seconds.  The saved codes of the sample come from the oracle's
    own 1x128 quantizer (not timed)."""
    import numpy as np
    import oracle
    from workloads import bits
    oracle.build(force=False)
    x = tensors["x_down"]
    R, C = x.shape
    qa, sa = oracle.quant_act_1x128(bits(x))          # 1x128 tiles: row slabs are independent
    rows = 256
    spent = 0.0
    done = 0.0
    while spent < budget_s:
        q, s = qa[:rows], np.ascontiguousarray(sa[:, :rows])
        t1 = time.perf_counter()
        oracle.requant_act_t(q, s)
        dt = time.perf_counter() - t1
        spent += dt
        done += rows * C * (2 + 4 / 128 + 4 / 128)
        if dt < budget_s / 8 and rows < R:
            rows = min(rows * 2, R)
    return {
        "value": round(done / spent / 1e9, 4),
        "unit": "GB/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": "oracle requantization of row slabs (256 rows and up) of the 16384x6144 input's saved codes, "
                  "%.0f MB of algorithmic traffic in %.1f s" % (done / 1e6, spent),
    }


def cpu_baseline_swiglu(tensors, budget_s):
    """The oracle's SwiGLU and quantizers (as they are) on the host cores over
    row slabs of the gate/up input, growing until about `budget_s` seconds."""
    import oracle
    from workloads import bits
    oracle.build(force=False)
    gu = bits(tensors["gu"])
    R, C2 = gu.shape
    I = C2 // 2
    rows = 128
    spent = 0.0
    done = 0.0
    while spent < budget_s:
        t1 = time.perf_counter()
        oracle.swiglu_quant(gu[:rows], dual=True)
        dt = time.perf_counter() - t1
        spent += dt
        done += rows * I * (4 + 2 * (1 + 4 / 128))
        if dt < budget_s / 8 and rows < R:
            rows = min(rows * 2, R)
    return {
        "value": round(done / spent / 1e9, 4),
        "unit": "GB/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": "oracle SwiGLU + 1x128 + 128x1 quantization of row slabs (128 rows and up) of the 16384x12288 "
                  "gate/up input, %.0f MB of algorithmic traffic in %.1f s" % (done / 1e6, spent),
    }


def cpu_baseline(tensors, workload, budget_s):
    """The oracle (as it is) on a bounded sample of the same work, on the host cores:
    quantize the gate_up (or first) linear's X and W in full, then compute a
    growing set of sampled fprop outputs until about `budget_s` seconds."""
    import numpy as np
    import oracle
    from workloads import bits
    oracle.build(force=False)
    if workload in ("layer", "layer_accum", "layer_fp8_saved", "layer_tm", "mlp_fprop", "mlp_swiglu_fprop",
                    "mlp_swiglu_fused", "mlp_swiglu_fused_nogu"):
        x, w = tensors["x_gate_up"], tensors["w_gate_up"]
    elif workload == "qkv_fprop":
        x, w = tensors["x"], tensors["w"]
    else:
        x, w = tensors["dy"], tensors["w"].T.contiguous()
    xb, wb = bits(x), bits(w)
    t0 = time.perf_counter()
    qa, sa = oracle.quant_act_1x128(xb)
    qb, sb = oracle.quant_w_128x128(wb)
    t_quant = time.perf_counter() - t0
    M, K = qa.shape
    N = qb.shape[0]
    rng = np.random.default_rng(0)
    n = 1024
    spent = 0.0
    done_flops = 0.0
    while spent < budget_s:
        ms = rng.integers(0, M, n)
        ns = rng.integers(0, N, n)
        t1 = time.perf_counter()
        oracle.gemm_at(oracle.FPROP, qa, sa, qb, sb, ms, ns)
        dt = time.perf_counter() - t1
        spent += dt
        done_flops += 2.0 * n * K
        if dt < budget_s / 8:
            n *= 2
    # scale: quantizing X and W is needed once per full GEMM; charge it in proportion
    frac = done_flops / (2.0 * M * N * K)
    total_s = spent + t_quant * frac
    return {
        "value": round(done_flops / total_s / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": ("fp64 oracle: 1x128/128x128 quantization of the %dx%d activation and %dx%d weight "
                   "(time charged pro rata) + %d sampled fprop outputs (K=%d), %.1f s" % (M, K, N, K, int(done_flops / (2 * K)), K, total_s)),
    }


def time_plans(plans, steps, warmup, torch, per_launch_steps):
    """Time `steps` steps cycling over the buffer sets in `plans` (lists of launches,
    all of the same kinds in the same order), with HIP events only at the two ends.
    Then per-launch durations from events between consecutive launches over
    `per_launch_steps` more steps.  Returns (ms per step, [(launch, avg ms, median ms)])."""
    def step(i, events=None):
        for j, l in enumerate(plans[i % len(plans)]):
            if events is not None:
                events[j].record()
            l.fn()
        if events is not None:
            events[len(plans[0])].record()

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        step(i)
    end.record()
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(end) / steps
    n = len(plans[0])
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(n + 1)] for _ in range(per_launch_steps)]
    for i in range(per_launch_steps):
        step(i, ev[i])
    torch.cuda.synchronize()
    rows = []
    for j, l in enumerate(plans[0]):
        d = sorted(ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(per_launch_steps))
        rows.append((l, sum(d) / len(d), d[len(d) // 2]))
    return ms_per_step, rows


# The smaller workloads reported beside the layer step: each timed on its own, its
# buffer sets rotated until their footprint exceeds 512 MB (twice the 256 MB of
# L2 + MALL), so that no step finds its inputs in the caches from the previous one.
CONFIGS = ["tiny_fprop", "qkv_fprop", "mlp_fprop", "mlp_down_bwd"]
ROTATE_BYTES = 512 << 20


def config_report(name, puro, torch, seed, steps, warmup):
    import workloads
    base = workloads.make(name, seed=seed, device="cuda")
    torch.cuda.synchronize()
    m0 = torch.cuda.memory_allocated()
    plans, keep = [], []
    launches, k = build_plan(name, base, puro, torch)
    plans.append(launches)
    keep.append((base, k))
    per_set = torch.cuda.memory_allocated() - m0 + sum(t.numel() * t.element_size() for t in base.values())
    sets = max(1, -(-ROTATE_BYTES // per_set) + (1 if ROTATE_BYTES % per_set == 0 else 0))
    for _ in range(sets - 1):
        t = {kk: v.clone() for kk, v in base.items()}
        launches, k = build_plan(name, t, puro, torch)
        plans.append(launches)
        keep.append((t, k))
    torch.cuda.synchronize()
    ms, rows = time_plans(plans, steps, warmup, torch, steps)
    flops = sum(l.flops for l in plans[0])
    gemm_ms = sum(a for l, a, _ in rows if l.kind.startswith("gemm"))
    q_ms = sum(a for l, a, _ in rows if l.kind == "quant")
    q_bytes = sum(l.bytes for l in plans[0] if l.kind == "quant")
    r = {
        "workload": WORKLOAD_DESC[name],
        "ms_per_step": round(ms, 4),
        "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
        "gemm_tflops": round(flops / (gemm_ms * 1e-3) / 1e12, 1),
        "gemm_pct_fp8_peak": round(100 * flops / (gemm_ms * 1e-3) / PEAK_FP8_FLOPS, 1),
        "quant_gbps": round(q_bytes / (q_ms * 1e-3) / 1e9, 1),
        "quant_pct_hbm_peak": round(100 * q_bytes / (q_ms * 1e-3) / PEAK_HBM_BPS, 1),
        "buffer_sets": sets,
        "footprint_mb": round(sets * per_set / 1e6),
        "kernels": [{"name": l.name, "ms_avg": round(a, 4),
                     **({"tflops": round(l.flops / (a * 1e-3) / 1e12, 1),
                         "pct_fp8_peak": round(100 * l.flops / (a * 1e-3) / PEAK_FP8_FLOPS, 1)} if l.flops else
                        {"gbps": round(l.bytes / (a * 1e-3) / 1e9, 1),
                         "pct_hbm_peak": round(100 * l.bytes / (a * 1e-3) / PEAK_HBM_BPS, 1)})}
                    for l, a, _ in rows],
    }
    if name == "tiny_fprop":
        r["note"] = "launch-bound (0.07 GFLOP): a parity case, not a throughput target"
    del plans, keep
    torch.cuda.empty_cache()
    return r


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures the path on one GPU only; --gpus %d is not supported "
              "(run with --gpus 1)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    import blockwise_fp8_gemm_act_amd as puro
    import workloads

    torch.cuda.set_device(0)
    if args.workload == "swiglu_quant":
        tensors = workloads.make("mlp_swiglu", seed=args.seed, device="cuda")
    elif args.workload in ("mlp_swiglu_fused", "mlp_swiglu_fused_nogu"):
        tensors = workloads.make("mlp_swiglu_fprop", seed=args.seed, device="cuda")
    elif args.workload in ("layer_fp8_saved", "layer_accum", "requant", "layer_tm"):
        names = None if args.workload != "requant" else {"x_" + lin for lin in workloads.LINEARS}
        tensors = workloads.make("layer", seed=args.seed, device="cuda", names=names)
    else:
        tensors = workloads.make(args.workload, seed=args.seed, device="cuda")
    torch.cuda.synchronize()
    m0 = torch.cuda.memory_allocated()
    launches, keep = build_plan(args.workload, tensors, puro, torch)
    # Workloads smaller than 512 MB (inputs, outputs, workspaces) rotate over as many
    # copies of their buffers as it takes to exceed it, so that a step does not find
    # its inputs in L2 or the 256 MB MALL from the step before.
    per_set = torch.cuda.memory_allocated() - m0
    if args.workload != "requant":            # the requantizer's step reads only the saved codes
        per_set += sum(t.numel() * t.element_size() for t in tensors.values())
    plans, sets_keep = [launches], [keep]
    while len(plans) * per_set <= ROTATE_BYTES:
        t = {k: v.clone() for k, v in tensors.items()}
        extra, k = build_plan(args.workload, t, puro, torch)
        plans.append(extra)
        sets_keep.append((t, k))
    torch.cuda.synchronize()

    cpu = None
    if not args.no_cpu_baseline:
        if args.workload == "requant":
            cpu = cpu_baseline_requant(tensors, args.cpu_seconds)
        elif args.workload == "swiglu_quant":
            cpu = cpu_baseline_swiglu(tensors, args.cpu_seconds)
        else:
            cpu = cpu_baseline(tensors, args.workload, args.cpu_seconds)

    counter = [0]

    def step(events=None):
        plan = plans[counter[0] % len(plans)]
        counter[0] += 1
        for i, l in enumerate(plan):
            if events is not None:
                events[i].record()
            l.fn()
        if events is not None:
            events[len(plan)].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Events between launches cost a few microseconds each on the GPU timeline
    # (about 0.08 ms over the layer step's 25).  The K timed steps therefore
    # carry events only at their two ends and give `value` and ms_per_step.
    # The per-launch durations come from events between consecutive launches:
    # over K more steps right after the timed ones for a workload of several
    # kernel kinds (its roofline uses them), over one more step for a single
    # kind (its roofline is total algorithmic work over the step time).
    single_kind = len({l.kind for l in launches}) == 1
    n_ev = 1 if single_kind else args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(launches) + 1)] for _ in range(n_ev)]
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for s in range(args.steps):
        step()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total = start.elapsed_time(end)
    ms_per_step = ms_total / args.steps
    for s in range(n_ev):
        step(ev[s])
    torch.cuda.synchronize()

    # per-launch durations (event before this launch -> event before the next)
    per = {}
    for s in range(n_ev):
        for i, l in enumerate(launches):
            d = ev[s][i].elapsed_time(ev[s][i + 1])
            per.setdefault(i, []).append(d)
    kinds = {}
    rows = []
    for i, l in enumerate(launches):
        d = sorted(per[i])
        med = d[len(d) // 2]
        avg = sum(d) / len(d)
        k = kinds.setdefault(l.kind, {"ms": 0.0, "flops": 0.0, "bytes": 0.0, "launches": 0})
        k["ms"] += avg
        k["flops"] += l.flops
        k["bytes"] += l.bytes
        k["launches"] += 1
        r = {"name": l.name, "ms_avg": round(avg, 4), "ms_med": round(med, 4)}
        if l.flops:
            r["tflops"] = round(l.flops / (avg * 1e-3) / 1e12, 1)
            r["pct_fp8_peak"] = round(100 * l.flops / (avg * 1e-3) / PEAK_FP8_FLOPS, 1)
        else:
            r["gbps"] = round(l.bytes / (avg * 1e-3) / 1e9, 1)
            r["pct_hbm_peak"] = round(100 * l.bytes / (avg * 1e-3) / PEAK_HBM_BPS, 1)
        rows.append(r)

    gemm_flops = sum(l.flops for l in launches)
    gemm_ms = sum(v["ms"] for k, v in kinds.items() if k.startswith("gemm"))
    quant = kinds.get("quant", {"ms": 0.0, "bytes": 0.0})
    if gemm_flops:
        value, unit, metric = gemm_flops / (ms_per_step * 1e-3) / 1e12, "TFLOP/s", METRIC
    else:
        step_bytes = sum(l.bytes for l in launches)
        value, unit = step_bytes / (ms_per_step * 1e-3) / 1e9, "GB/s"
        metric = {"requant": "requantizer HBM GB/s, Puro-2B layer inputs",
                  "swiglu_quant": "fused SwiGLU + quantizer HBM GB/s, Puro-2B MLP"}[args.workload]

    # dominant kernel: the launch type with the most time per step
    dom_kind, dom = max(((k, v) for k, v in kinds.items()), key=lambda kv: kv[1]["ms"])
    if single_kind:
        dom = dict(dom, ms=ms_per_step)
    if dom_kind.startswith("gemm"):
        achieved = dom["flops"] / (dom["ms"] * 1e-3)
        roof = {"bound": "mfma", "achieved": round(achieved / 1e12, 1), "peak": PEAK_FP8_FLOPS / 1e12,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP8_FLOPS, 4)}
    else:
        achieved = dom["bytes"] / (dom["ms"] * 1e-3)
        roof = {"bound": "hbm", "achieved": round(achieved / 1e9, 1), "peak": PEAK_HBM_BPS / 1e9,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_BPS, 4)}
    roof["kernel"] = dom_kind
    roof["launches_per_step"] = dom["launches"]
    roof["algorithmic_per_launch"] = (round(dom["flops"] / dom["launches"] / 1e9, 3) if dom_kind.startswith("gemm")
                                      else round(dom["bytes"] / dom["launches"] / 1e6, 3))
    roof["algorithmic_unit"] = "GFLOP" if dom_kind.startswith("gemm") else "MB"
    roof["avg_launch_ms"] = round(dom["ms"] / dom["launches"], 4)
    roof["timing"] = ("HIP events around the timed steps, no events between their launches" if single_kind
                      else "HIP events between consecutive launches over %d steps run right after the %d timed steps "
                           "(which carry no events between launches)" % (n_ev, args.steps))
    tr = load_traffic(dom_kind)
    roof["traffic"] = tr

    configs = None
    if args.workload == "layer" and not args.no_configs:
        configs = {}
        for name in CONFIGS:
            configs[name] = config_report(name, puro, torch, args.seed, args.config_steps, args.config_steps)
            print("config %s: %.4f ms per step" % (name, configs[name]["ms_per_step"]), file=sys.stderr, flush=True)
    if cpu is not None:
        cpu["cpu_model"] = cpu_model()

    out = {
        "metric": metric,
        "value": round(value, 2),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("e4m3 (fp32 accumulate)" if gemm_flops else
                  {"requant": "e4m3 -> fp32 -> e4m3", "swiglu_quant": "bf16 -> fp32 (fp64 near ties) -> e4m3"}[args.workload]),
        "data": "synthetic (seeded, Puro-2B-shaped; see workloads.py)",
        "config": {"workload": WORKLOAD_DESC[args.workload], "name": args.workload,
                   "tokens": {"qkv_fprop": 4096, "mlp_fprop": 8192, "mlp_down_bwd": 8192}.get(args.workload, 16384),
                   "hidden": 2048, "parallelism": "single GPU"},
        "pct_fp8_peak": round(100 * value * 1e12 / PEAK_FP8_FLOPS, 2) if gemm_flops else None,
        "gemm_only_tflops": round(gemm_flops / (gemm_ms * 1e-3) / 1e12, 1) if gemm_ms else None,
        "quant_gbps": round(quant["bytes"] / (quant["ms"] * 1e-3) / 1e9, 1) if quant["ms"] else None,
        "quant_pct_hbm_peak": round(100 * quant["bytes"] / (quant["ms"] * 1e-3) / PEAK_HBM_BPS, 1) if quant["ms"] else None,
        "requant_gbps": (round(kinds["requant"]["bytes"] / (kinds["requant"]["ms"] * 1e-3) / 1e9, 1)
                         if "requant" in kinds else None),
        "wall_s_timed": round(wall, 3),
        "buffer_sets": len(plans),
        "footprint_mb": round(len(plans) * per_set / 1e6),
        "roofline": roof,
        "cpu_baseline": cpu,
        "kernels": rows,
        "configs": configs,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
