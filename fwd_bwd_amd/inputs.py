"""Seeded synthetic inputs and the workload table.

This module only draws random numbers and describes shapes; it holds none of
the method's arithmetic. Both the GPU path and the CPU oracle are fed from it.

The workloads follow the benchmark script of NATTEN issue #161 ("Backward pass
is very slow towards much tokens and large kernels"): q, k, v drawn from a
standard normal, token-major [B, (T,) H, W, heads, head_dim], and the backward
driven by loss = output.sum(), i.e. dout = ones. The two headline shapes are
the issue's 2D 1024x1024 grid with a 9x9 kernel and 3D 16x256x256 grid with a
(3, 5, 5) kernel, both with 8 heads of dimension 32 in fp32. The bf16 cases
draw dout from a standard normal as well. The same two shapes in fp16 follow
the maintainer's fp16 profile of the fused op (same script, dout = ones).

Draw order from one CPU torch.Generator seeded with `seed`: q, k, v, then dout
(when it is random), each in fp32, then cast to the workload dtype with
round-to-nearest-even.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Tuple

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    grid: Tuple[int, ...]          # (H, W) or (T, H, W)
    heads: int
    head_dim: int
    kernel: Tuple[int, ...]
    dilation: Tuple[int, ...]
    dtype: torch.dtype
    dout_ones: bool
    scale: float = field(default=None)

    @property
    def shape(self) -> Tuple[int, ...]:
        return (self.batch,) + tuple(self.grid) + (self.heads, self.head_dim)

    @property
    def ndim(self) -> int:
        return len(self.grid)

    @property
    def tokens(self) -> int:
        n = self.batch
        for g in self.grid:
            n *= g
        return n

    @property
    def window(self) -> int:
        n = 1
        for k in self.kernel:
            n *= k
        return n

    @property
    def the_scale(self) -> float:
        return self.head_dim ** -0.5 if self.scale is None else self.scale


WORKLOADS: Dict[str, Workload] = {
    "2d_16x16_k3_h2_d16_f32": Workload("2d_16x16_k3_h2_d16_f32", 1, (16, 16), 2, 16, (3, 3),
                                       (1, 1), torch.float32, True, 16 ** -0.5),
    "2d_1024x1024_k9_h8_d32_f32": Workload("2d_1024x1024_k9_h8_d32_f32", 1, (1024, 1024), 8, 32,
                                           (9, 9), (1, 1), torch.float32, True, 32 ** -0.5),
    "3d_16x256x256_k3x5x5_h8_d32_f32": Workload("3d_16x256x256_k3x5x5_h8_d32_f32", 1,
                                                (16, 256, 256), 8, 32, (3, 5, 5), (1, 1, 1),
                                                torch.float32, True, 32 ** -0.5),
    "3d_b2_8x128x128_k5x7x7_h8_d32_bf16": Workload("3d_b2_8x128x128_k5x7x7_h8_d32_bf16", 2,
                                                   (8, 128, 128), 8, 32, (5, 7, 7), (1, 1, 1),
                                                   torch.bfloat16, False, None),
    "2d_b4_512x512_k13_d2_h4_d64_bf16": Workload("2d_b4_512x512_k13_d2_h4_d64_bf16", 4,
                                                 (512, 512), 4, 64, (13, 13), (2, 2),
                                                 torch.bfloat16, False, 64 ** -0.5),
    "2d_1024x1024_k9_h8_d32_f16": Workload("2d_1024x1024_k9_h8_d32_f16", 1, (1024, 1024), 8, 32,
                                           (9, 9), (1, 1), torch.float16, True, 32 ** -0.5),
    "3d_16x256x256_k3x5x5_h8_d32_f16": Workload("3d_16x256x256_k3x5x5_h8_d32_f16", 1,
                                                (16, 256, 256), 8, 32, (3, 5, 5), (1, 1, 1),
                                                torch.float16, True, 32 ** -0.5),
}

# the configuration the benchmark's headline number is quoted on, and the 3D one beside it
HEADLINE = "2d_1024x1024_k9_h8_d32_f32"
HEADLINE_3D = "3d_16x256x256_k3x5x5_h8_d32_f32"


def make_inputs(w: Workload, seed: int = 0):
    """(q, k, v, dout) as CPU tensors of the workload's dtype."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    q = torch.randn(w.shape, generator=g, dtype=torch.float32)
    k = torch.randn(w.shape, generator=g, dtype=torch.float32)
    v = torch.randn(w.shape, generator=g, dtype=torch.float32)
    if w.dout_ones:
        dout = torch.ones(w.shape, dtype=torch.float32)
    else:
        dout = torch.randn(w.shape, generator=g, dtype=torch.float32)
    return tuple(t.to(w.dtype) for t in (q, k, v, dout))


def make_random(shape, dtype=torch.float32, seed: int = 0, dout_ones: bool = False):
    """(q, k, v, dout) for an arbitrary token-major shape, same recipe."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    q, k, v = (torch.randn(shape, generator=g, dtype=torch.float32) for _ in range(3))
    dout = torch.ones(shape) if dout_ones else torch.randn(shape, generator=g, dtype=torch.float32)
    return tuple(t.to(dtype) for t in (q, k, v, dout))
