"""Seeded synthetic workloads for exact attention: shapes, dtypes and inputs.

This module holds no attention arithmetic.  It defines the named workloads and
draws their inputs, the same stored values for the GPU path and for the CPU
checker.  The pages measure on ``torch.randn`` tensors (standard normal
q, k, v) in the shapes of their examples ("Flash Attention | Hermes Skill",
Quick start and Workflows 1-3); the workloads below keep that distribution.

Recipe (fixed so that a run can be reproduced anywhere):
  * ``numpy.random.default_rng(seed)``; draw q, then k, then v, each a float32
    standard normal array in the workload's layout shape (k and v with the
    workload's K/V head count, which may be smaller than q's).
  * 16-bit workloads: cast round-to-nearest-even through torch on the CPU.
  * fp8 workloads: per-tensor scale ``s = amax|x| / 448`` in float32, then
    ``x / s`` cast round-to-nearest-even to OCP float8 e4m3fn (torch CPU).  The
    kernel receives ``s`` as the tensor's descale.  |x / s| <= 448, the largest
    finite e4m3fn value, so nothing saturates.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Tuple

import numpy as np
import torch

FP8_E4M3_MAX = 448.0


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int
    seqlen: int
    headdim: int
    dtype: str            # "f16" | "bf16" | "fp8"
    layout: str           # "bshd" | "bhsd"
    causal: bool
    window_left: int = -1
    window_right: int = -1
    scale: Optional[float] = None
    seed: int = 1000
    heads_kv: Optional[int] = None   # K/V heads (fewer than `heads`: shared K/V)

    @property
    def softmax_scale(self) -> float:
        return self.scale if self.scale is not None else 1.0 / math.sqrt(self.headdim)

    @property
    def out_dtype(self) -> str:
        return "bf16" if self.dtype == "fp8" else self.dtype

    @property
    def kv_heads(self) -> int:
        return self.heads if self.heads_kv is None else self.heads_kv

    def shape(self, heads: Optional[int] = None) -> Tuple[int, int, int, int]:
        h = self.heads if heads is None else heads
        if self.layout == "bshd":
            return (self.batch, self.seqlen, h, self.headdim)
        return (self.batch, h, self.seqlen, self.headdim)


# The five workloads.  Indices match the order the targets list them in.
WORKLOADS = {
    "sdpa_b1h8n512d64_f16": Workload("sdpa_b1h8n512d64_f16", 1, 8, 512, 64, "f16", "bhsd", False,
                                     scale=1.0 / 8.0, seed=1000),
    "sdpa_b2h8n2048d64_f16": Workload("sdpa_b2h8n2048d64_f16", 2, 8, 2048, 64, "f16", "bhsd", False,
                                      scale=1.0 / 8.0, seed=1001),
    "sdpa_b2h8n2048d64_f16_causal": Workload("sdpa_b2h8n2048d64_f16_causal", 2, 8, 2048, 64, "f16", "bhsd", True,
                                             scale=1.0 / 8.0, seed=1001),
    "sdpa_b4h32n4096d128_bf16_causal": Workload("sdpa_b4h32n4096d128_bf16_causal", 4, 32, 4096, 128, "bf16", "bshd",
                                                True, scale=1.0 / math.sqrt(128.0), seed=1002),
    "swa_b1h32n16384d128_bf16_w4095": Workload("swa_b1h32n16384d128_bf16_w4095", 1, 32, 16384, 128, "bf16", "bshd",
                                               True, window_left=4095, window_right=0,
                                               scale=1.0 / math.sqrt(128.0), seed=1003),
    "fp8_b1h16n65536d128_causal": Workload("fp8_b1h16n65536d128_causal", 1, 16, 65536, 128, "fp8", "bshd", True,
                                           scale=1.0 / math.sqrt(128.0), seed=1004),
}

HEADLINE = "sdpa_b4h32n4096d128_bf16_causal"

# Beyond the five: the headline shape with K/V shared by groups of 4 query
# heads (8 K/V heads), and by all 32 (one K/V head).
WORKLOADS["gqa_b4h32kv8n4096d128_bf16_causal"] = Workload(
    "gqa_b4h32kv8n4096d128_bf16_causal", 4, 32, 4096, 128, "bf16", "bshd", True,
    scale=1.0 / math.sqrt(128.0), seed=1005, heads_kv=8)
WORKLOADS["mqa_b4h32kv1n4096d128_bf16_causal"] = Workload(
    "mqa_b4h32kv1n4096d128_bf16_causal", 4, 32, 4096, 128, "bf16", "bshd", True,
    scale=1.0 / math.sqrt(128.0), seed=1006, heads_kv=1)


@dataclasses.dataclass
class Inputs:
    """Stored input values on the CPU.

    q, k, v are torch CPU tensors of the stored dtype (float16, bfloat16 or
    float8_e4m3fn) in the workload layout.  ``descale`` holds the per-tensor
    fp8 scales (1.0 for 16-bit inputs).
    """
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    descale: Tuple[float, float, float]


_TORCH_DTYPES = {"f16": torch.float16, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}


def torch_dtype(name: str) -> torch.dtype:
    return _TORCH_DTYPES[name]


def quantize_e4m3_per_tensor(x: np.ndarray) -> Tuple[torch.Tensor, float]:
    """Per-tensor amax scaling to OCP e4m3fn, round to nearest even (torch CPU cast)."""
    xt = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    amax = float(xt.abs().max())
    s = np.float32(amax / FP8_E4M3_MAX) if amax > 0 else np.float32(1.0)
    q = (xt / torch.tensor(s, dtype=torch.float32)).to(torch.float8_e4m3fn)
    return q, float(s)


def make_inputs_shape(shape, dtype: str, seed: int, kv_shape=None) -> Inputs:
    rng = np.random.default_rng(seed)
    kv_shape = shape if kv_shape is None else kv_shape
    arrs = [rng.standard_normal(size=s, dtype=np.float32) for s in (shape, kv_shape, kv_shape)]
    if dtype == "fp8":
        qs = [quantize_e4m3_per_tensor(a) for a in arrs]
        return Inputs(qs[0][0], qs[1][0], qs[2][0], (qs[0][1], qs[1][1], qs[2][1]))
    td = _TORCH_DTYPES[dtype]
    ts = [torch.from_numpy(a).to(td) for a in arrs]
    return Inputs(ts[0], ts[1], ts[2], (1.0, 1.0, 1.0))


def make_inputs(w: Workload) -> Inputs:
    return make_inputs_shape(w.shape(), w.dtype, w.seed, w.shape(w.kv_heads))


def small_case(batch, heads, seqlen, headdim, dtype, layout, seed, heads_kv=None) -> Inputs:
    def shp(h):
        return (batch, seqlen, h, headdim) if layout == "bshd" else (batch, h, seqlen, headdim)
    return make_inputs_shape(shp(heads), dtype, seed, shp(heads if heads_kv is None else heads_kv))
