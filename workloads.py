"""Seeded synthetic inputs for the Puro-2B-shaped FP8 path.

This module holds no arithmetic of the method: it only draws bf16 tensors of
the shapes and distributions of the workloads.  Both the HIP path and the CPU
oracle receive the very same tensors from here.

Model shape (ainews.surl.tw article on Puro-2B): 28 layers, hidden 2048,
4096-token context, a Qwen3-1.7B-compatible configuration.  That gives the
four main linears of one layer, with W stored [out_features][in_features]:
QKV 2048 -> 4096 (16 query + 8 key/value heads of 128), O 2048 -> 2048,
gate_up 2048 -> 12288 (2 x 6144), down 6144 -> 2048.

Distributions (N(0, s) has standard deviation s):
  activations  N(0, 1), with 1% of the input channels (floor(0.01 * K)
               columns, at least the stated count) multiplied by 20 before
               rounding to bf16 -- the outlier channels that make per-tile
               scaling matter;
  weights      N(0, 0.02);
  down input   silu(g) * u with g, u ~ N(0, 1), rescaled by one scalar to
               standard deviation 0.5 (the SiLU-gated values of the MLP);
  gradients    1e-3 * t_4 (Student-t with 4 degrees of freedom: heavy tails).
Every tensor has its own torch.Generator seeded with the CRC-32 of
"<seed>/<workload>/<tensor>", so a tensor does not depend on which others were
drawn.  Values are drawn in fp32 and rounded to bf16 (round to nearest even).
"""
from __future__ import annotations

import zlib
from dataclasses import dataclass, field

import numpy as np
import torch

HIDDEN = 2048
QKV_OUT = 4096          # (16 + 2 * 8) heads x 128
INTER = 6144
LINEARS = {             # name: (in_features, out_features)
    "qkv": (HIDDEN, QKV_OUT),
    "o": (HIDDEN, HIDDEN),
    "gate_up": (HIDDEN, 2 * INTER),
    "down": (INTER, HIDDEN),
}


def tensor_seed(seed: int, workload: str, name: str) -> int:
    return zlib.crc32(f"{seed}/{workload}/{name}".encode())


def _gen(seed: int, workload: str, name: str, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(tensor_seed(seed, workload, name))
    return g


def normal(shape, std, g, device="cpu", outlier_cols: int = 0, outlier_scale: float = 20.0):
    """N(0, std) in fp32, with `outlier_cols` random columns scaled, rounded to bf16."""
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std
    if outlier_cols:
        cols = torch.randperm(shape[-1], generator=g, device=device)[:outlier_cols]
        x[..., cols] *= outlier_scale
    return x.to(torch.bfloat16)


def silu_gated(shape, g, device="cpu", std=0.5):
    gate = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    up = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    h = torch.nn.functional.silu(gate) * up
    del gate, up
    h *= std / h.std()
    return h.to(torch.bfloat16)


def student_t(shape, g, device="cpu", df=4, scale=1e-3):
    """scale * Z / sqrt(V / df), V a chi-square with df degrees of freedom."""
    z = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    v = torch.zeros(shape, device=device, dtype=torch.float32)
    for _ in range(df):
        e = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        v.addcmul_(e, e)
    z *= torch.rsqrt(v / df)
    del v
    return (z * scale).to(torch.bfloat16)


def outlier_count(k: int, frac: float = 0.01) -> int:
    return int(np.floor(frac * k))


@dataclass
class Spec:
    """One tensor of a workload: its shape and how it is drawn."""
    name: str
    shape: tuple
    kind: str                      # "act", "weight", "silu", "grad"
    outliers: int = 0
    kwargs: dict = field(default_factory=dict)


def _act(name, rows, cols, outliers=None):
    return Spec(name, (rows, cols), "act", outlier_count(cols) if outliers is None else outliers)


def _w(name, rows, cols):
    return Spec(name, (rows, cols), "weight")


# The workloads.  Each maps to the tensors it needs.
WORKLOADS = {
    # 256x256 activations (2 outlier channels) against a 512x256 weight, fp32 out.
    "tiny_fprop": [_act("x", 256, 256, outliers=2), _w("w", 512, 256)],
    # QKV projection forward at 4096 tokens, bf16 out.
    "qkv_fprop": [_act("x", 4096, HIDDEN), _w("w", QKV_OUT, HIDDEN)],
    # MLP forward at 8192 tokens: gate_up then down (SiLU-gated input).
    "mlp_fprop": [_act("x_gate_up", 8192, HIDDEN), _w("w_gate_up", 2 * INTER, HIDDEN),
                  Spec("x_down", (8192, INTER), "silu"), _w("w_down", HIDDEN, INTER)],
    # MLP down-projection backward at 8192 tokens: dgrad and wgrad.
    "mlp_down_bwd": [Spec("dy", (8192, HIDDEN), "grad"), _w("w", HIDDEN, INTER),
                     Spec("x", (8192, INTER), "silu")],
    # The MLP's gate/up projection output at 16384 tokens (gate then up, 2 x 6144
    # columns): the input of the SwiGLU that feeds the down projection.
    "mlp_swiglu": [Spec("gu", (16384, 2 * INTER), "act", outliers=0)],
    # The MLP forward at 16384 tokens with the SwiGLU quantizer between its two
    # projections (gate_up X [16384x2048] x W [12288x2048]^T, down W [2048x6144]).
    "mlp_swiglu_fprop": [_act("x_gate_up", 16384, HIDDEN), _w("w_gate_up", 2 * INTER, HIDDEN),
                         _w("w_down", HIDDEN, INTER)],
    # One whole layer's four linears at 16384 tokens, forward and backward.
    "layer": [t for lin, (kin, kout) in LINEARS.items() for t in (
        _act(f"x_{lin}", 16384, kin), _w(f"w_{lin}", kout, kin),
        Spec(f"dy_{lin}", (16384, kout), "grad"))],
}


def draw(spec: Spec, seed: int, workload: str, device="cpu") -> torch.Tensor:
    g = _gen(seed, workload, spec.name, device)
    if spec.kind == "act":
        return normal(spec.shape, 1.0, g, device, outlier_cols=spec.outliers)
    if spec.kind == "weight":
        return normal(spec.shape, 0.02, g, device)
    if spec.kind == "silu":
        return silu_gated(spec.shape, g, device)
    if spec.kind == "grad":
        return student_t(spec.shape, g, device)
    raise ValueError(spec.kind)


def make(workload: str, seed: int = 0, device="cpu", names=None) -> dict:
    """All tensors of a workload as bf16 torch tensors on `device`."""
    out = {}
    for spec in WORKLOADS[workload]:
        if names is None or spec.name in names:
            out[spec.name] = draw(spec, seed, workload, device)
    return out


def bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> numpy uint16 bit patterns (a copy on the host)."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def random_bf16(shape, seed: int, std: float = 1.0, device="cpu") -> torch.Tensor:
    """A plain N(0, std) bf16 tensor for tests of arbitrary shapes."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return (torch.randn(shape, generator=g, device=device) * std).to(torch.bfloat16)


def random_codes(shape, seed: int) -> np.ndarray:
    """Uniformly drawn finite e4m3 code bytes (every byte except 0x7F and 0xFF)."""
    g = torch.Generator()
    g.manual_seed(seed)
    c = torch.randint(0, 254, shape, generator=g, dtype=torch.int64).numpy()
    c = c + (c >= 0x7F)                      # skip 0x7F; 0xFF is above the drawn range
    return c.astype(np.uint8)


def random_scales(shape, seed: int, log2_lo: float = -20.0, log2_hi: float = 4.0) -> np.ndarray:
    """Positive fp32 scales, log-uniform in [2^log2_lo, 2^log2_hi)."""
    g = torch.Generator()
    g.manual_seed(seed)
    e = torch.rand(shape, generator=g, dtype=torch.float64) * (log2_hi - log2_lo) + log2_lo
    return torch.exp2(e).to(torch.float32).numpy()
