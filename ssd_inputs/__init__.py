"""Seeded synthetic inputs for the Mamba-2 SSD scan and step.

This module only draws random numbers and shapes them.  It holds none of the
scan's arithmetic, so that both the CPU oracle and the GPU path can take their
inputs from it without sharing any code of the method.

The value distributions follow the synthetic workload of the SSD layer
(activations of a Mamba-2 block at the checkpoint shapes of "Compiler-First
State Space Duality and Portable O(1) Autoregressive Caching", Setup: Models):

  x        ~ N(0, 1)                         [Bt, T, H, P]
  dt       ~ 0.5 * N(0, 1)  (pre-activation)  [Bt, T, H]
  dt_bias  = log(expm1(u)), u ~ U(1e-3, 0.1)  [H]   (so softplus(dt_bias) = u)
  A        = -exp(U(0, ln 16))                [H]   (negative per-head decay)
  B, C     ~ N(0, 1) / sqrt(N)                [Bt, T, G, N]
  D        ~ N(0, 1)                          [H]

Draws are made in float32 on the CPU with a torch.Generator, in the fixed order
dt_bias, A, D, x, dt, B, C.  x, B and C are then rounded to bfloat16
(round-to-nearest-even) when the workload says so; every consumer receives the
same rounded values.

The depthwise causal convolution that precedes the scan in a Mamba-2 block
(O(1) cache section; Setup: kernel size k = 4, expand factor 2, so
D_conv = 2 d_model + 2 G N channels) takes, in draw order:

  weight   ~ U(-1/sqrt(k), 1/sqrt(k))         [D, k]
  bias     ~ U(-1/sqrt(k), 1/sqrt(k))         [D]
  x        ~ N(0, 1)                          [Bt, T, D]
  state    ~ N(0, 1)  (when asked)            [Bt, D, k-1]

(the bound is the usual initialisation scale of a depthwise kernel of fan-in
k); x and the state are rounded to bfloat16 for bfloat16 workloads.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Dict, Optional

import torch


@dataclass(frozen=True)
class Workload:
    """Shape and dtype of one synthetic SSD scan problem."""

    name: str
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    dstate: int
    ngroups: int = 1
    chunk: int = 256
    io_dtype: str = "f32"  # dtype of x, B, C and y: "f32" or "bf16"
    seed: int = 1000
    dt_min: float = 1e-4
    dt_max: float = 0.5
    note: str = ""

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five synthetic workloads of the SSD path.  Sizes follow the Mamba-2
# checkpoint shapes (state 128, head dim 64, chunk 256) named in the paper's
# setup; the tiny one is small enough for the CPU oracle to finish in seconds.
WORKLOADS: Dict[str, Workload] = {
    "tiny_f32": Workload("tiny_f32", 1, 512, 4, 16, 16, 1, 64, "f32", 1000,
                         note="tiny SSD scan, fp32"),
    "m130_f32": Workload("m130_f32", 1, 4096, 24, 64, 128, 1, 256, "f32", 1001,
                         note="Mamba-2-130M-shaped layer prefill, fp32"),
    "m2p7_bf16": Workload("m2p7_bf16", 1, 4096, 80, 64, 128, 1, 256, "bf16", 1002,
                          note="Mamba-2-2.7B-shaped layer prefill, bf16 x/B/C"),
    "m1p3_long_bf16": Workload("m1p3_long_bf16", 8, 16384, 64, 64, 128, 1, 256, "bf16", 1003,
                               note="Mamba-2-1.3B-shaped batched long prefill, bf16 x/B/C"),
    # decode: 4096-token prefill of the 2.7B shape followed by 1024 single steps
    "m2p7_decode": Workload("m2p7_decode", 1, 5120, 80, 64, 128, 1, 256, "bf16", 1004,
                            note="2.7B-shaped cached decode: 4096 prefill + 1024 steps"),
}

DECODE_PREFILL = 4096
DECODE_STEPS = 1024


def _torch_dtype(io_dtype: str) -> torch.dtype:
    if io_dtype == "f32":
        return torch.float32
    if io_dtype == "bf16":
        return torch.bfloat16
    raise ValueError(f"unknown io dtype {io_dtype!r}")


def make_inputs(w: Workload, seed: Optional[int] = None,
                with_initial_state: bool = False) -> Dict[str, torch.Tensor]:
    """Draw one problem's inputs on the CPU.

    Returns a dict with x, dt, dt_bias, A, B, C, D (CPU tensors; x/B/C in the
    workload's io dtype, the rest float32) and, when asked, a float32 initial
    state h0 ~ N(0, 1) [Bt, H, P, N] drawn after everything else.
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed if seed is None else seed)
    Bt, T, H, P, N, G = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups
    f32 = torch.float32
    u = torch.rand(H, generator=g, dtype=f32) * (0.1 - 1e-3) + 1e-3
    dt_bias = torch.log(torch.expm1(u))
    A = -torch.exp(torch.rand(H, generator=g, dtype=f32) * math.log(16.0))
    D = torch.randn(H, generator=g, dtype=f32)
    x = torch.randn(Bt, T, H, P, generator=g, dtype=f32)
    dt = torch.randn(Bt, T, H, generator=g, dtype=f32) * 0.5
    B = torch.randn(Bt, T, G, N, generator=g, dtype=f32) / math.sqrt(N)
    C = torch.randn(Bt, T, G, N, generator=g, dtype=f32) / math.sqrt(N)
    io = _torch_dtype(w.io_dtype)
    out = {
        "x": x.to(io), "dt": dt, "dt_bias": dt_bias, "A": A,
        "B": B.to(io), "C": C.to(io), "D": D,
    }
    if with_initial_state:
        out["h0"] = torch.randn(Bt, H, P, N, generator=g, dtype=f32)
    return out


@dataclass(frozen=True)
class ConvWorkload:
    """Shape and dtype of one synthetic depthwise causal convolution problem."""

    name: str
    batch: int
    seqlen: int
    channels: int
    width: int = 4
    io_dtype: str = "f32"  # dtype of x, y and the cached window
    silu: bool = True
    seed: int = 2000
    note: str = ""

    def with_(self, **kw) -> "ConvWorkload":
        return replace(self, **kw)


# D_conv = 2 d_model + 2 G N: 2 * 768 + 256 for the 130M shape (H = 24 heads of
# 64), 2 * 2560 + 256 for the 2.7B shape (H = 80 heads of 64).
CONV_WORKLOADS: Dict[str, ConvWorkload] = {
    "conv_m130_f32": ConvWorkload("conv_m130_f32", 1, 4096, 1792, 4, "f32", True, 2001,
                                  note="130M-shaped conv1d prefill, fp32"),
    "conv_m2p7_bf16": ConvWorkload("conv_m2p7_bf16", 1, 4096, 5376, 4, "bf16", True, 2002,
                                   note="2.7B-shaped conv1d prefill, bf16"),
    "conv_m2p7_decode": ConvWorkload("conv_m2p7_decode", 64, 1, 5376, 4, "bf16", True, 2004,
                                     note="2.7B-shaped conv1d decode step, bf16 window"),
}


def make_conv_inputs(w: ConvWorkload, seed: Optional[int] = None,
                     with_state: bool = False) -> Dict[str, torch.Tensor]:
    """Draw one convolution problem's inputs on the CPU: x and (when asked)
    state in the io dtype, weight and bias in float32."""
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed if seed is None else seed)
    Bt, T, Dc, K = w.batch, w.seqlen, w.channels, w.width
    f32 = torch.float32
    bound = 1.0 / math.sqrt(K)
    weight = (torch.rand(Dc, K, generator=g, dtype=f32) * 2.0 - 1.0) * bound
    bias = (torch.rand(Dc, generator=g, dtype=f32) * 2.0 - 1.0) * bound
    x = torch.randn(Bt, T, Dc, generator=g, dtype=f32)
    io = _torch_dtype(w.io_dtype)
    out = {"x": x.to(io), "weight": weight, "bias": bias}
    if with_state:
        out["state"] = torch.randn(Bt, Dc, K - 1, generator=g, dtype=f32).to(io)
    return out


def make_tiny(batch: int, seqlen: int, nheads: int, headdim: int, dstate: int,
              ngroups: int = 1, chunk: int = 32, io_dtype: str = "f32",
              seed: int = 7) -> Workload:
    """A small workload with the same value distributions, for parity sweeps."""
    return Workload(f"tiny_{batch}x{seqlen}_h{nheads}p{headdim}n{dstate}g{ngroups}"
                    f"_l{chunk}_{io_dtype}", batch, seqlen, nheads, headdim, dstate,
                    ngroups, chunk, io_dtype, seed)


def as_f32_numpy(t: torch.Tensor):
    """Exact upcast of a CPU tensor (bf16 or f32) to a contiguous float32 array."""
    return t.detach().to(torch.float32).contiguous().numpy()
