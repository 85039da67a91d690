"""Seeded synthetic inputs for the attention forward.

This module only draws random numbers and rounds them to bf16; it holds none of
the attention arithmetic. Both the HIP path (through the tests and the
benchmark) and the fp64 oracle consume exactly the tensors it returns.

Recipe (one generator per workload, seeded with the workload's seed):
  * torch.Generator('cpu').manual_seed(seed)
  * draw Q, then K, then V, each torch.randn(B, H, N, d, dtype=float32)
  * multiply Q and K by ``qk_std`` in fp32 (1.5 for the long causal workload,
    which makes the softmax peakier and exercises the running-max rescale)
  * round to bf16 (round-to-nearest-even), contiguous [B, H, N, d]
  * scale = fp32(1/sqrt(d))
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np
import torch

__all__ = ["Workload", "WORKLOADS", "workload", "make_inputs", "fp32_scale",
           "attn_flops"]


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    causal: bool
    seed: int
    qk_std: float = 1.0

    def as_dict(self):
        return {"workload": self.name, "B": self.B, "H": self.H, "N": self.N,
                "d": self.d, "causal": self.causal}


# The five workloads of the metric. The first is the tiny case the oracle
# checks in well under a second; the fourth (d=128, N=4096, non-causal) is the
# one the throughput target is quoted on.
WORKLOADS = (
    Workload("tiny_b1h1n128d64", 1, 1, 128, 64, False, seed=1),
    Workload("b4h16n1024d64", 4, 16, 1024, 64, False, seed=2),
    Workload("causal_b8h16n2048d64", 8, 16, 2048, 64, True, seed=3),
    Workload("b16h16n4096d128", 16, 16, 4096, 128, False, seed=4),
    Workload("causal_long_b1h32n16384d128", 1, 32, 16384, 128, True, seed=5,
             qk_std=1.5),
)


def workload(key):
    """Look a workload up by 1-based index or by name."""
    if isinstance(key, int):
        return WORKLOADS[key - 1]
    for w in WORKLOADS:
        if w.name == key:
            return w
    raise KeyError(key)


def fp32_scale(d):
    """The softmax scale 1/sqrt(d), rounded to fp32 and returned as a float."""
    return float(np.float32(1.0 / math.sqrt(d)))


def attn_flops(B, H, N, d, causal):
    """The metric's FLOP count: 4*B*H*N^2*d, halved when causal."""
    f = 4.0 * B * H * N * N * d
    return f / 2 if causal else f


def make_inputs(w, B=None, H=None, N=None, d=None, seed=None, qk_std=None,
                keep_fp32=False, dtype=torch.bfloat16):
    """Draw Q, K, V for workload ``w`` (sizes and seed may be overridden).

    Returns a dict with CPU tensors ``q``, ``k``, ``v`` [B,H,N,d] rounded to
    ``dtype`` (bf16 unless float16 is asked for), the fp32
    ``scale`` as a Python float, ``causal``, and with keep_fp32 the unrounded
    fp32 draws as ``q32``, ``k32``, ``v32``.
    """
    B = w.B if B is None else B
    H = w.H if H is None else H
    N = w.N if N is None else N
    d = w.d if d is None else d
    seed = w.seed if seed is None else seed
    qk_std = w.qk_std if qk_std is None else qk_std
    g = torch.Generator("cpu").manual_seed(seed)
    shape = (B, H, N, d)
    q32 = torch.randn(shape, dtype=torch.float32, generator=g)
    k32 = torch.randn(shape, dtype=torch.float32, generator=g)
    v32 = torch.randn(shape, dtype=torch.float32, generator=g)
    if qk_std != 1.0:
        q32.mul_(qk_std)
        k32.mul_(qk_std)
    out = {
        "q": q32.to(dtype).contiguous(),
        "k": k32.to(dtype).contiguous(),
        "v": v32.to(dtype).contiguous(),
        "scale": fp32_scale(d),
        "causal": w.causal,
    }
    if keep_fp32:
        out.update(q32=q32, k32=k32, v32=v32)
    return out
