"""Seeded synthetic inputs for the BitLinear workloads.

This module only draws random numbers and names shapes.  It holds none of the
method's arithmetic (no scales, no rounding to codes, no packing), so both the
library path and the CPU oracle can be fed from it.  Every tensor comes out as
bf16 (drawn in fp32, then rounded to bf16 by torch) on the device asked for.

Shapes come from the pages:
  * BitNet-b1.58-2B decode and prefill: hidden 2560, down_proj K = 6912
    ("BitVLA -- 1.58-bit Vision-Language-Action on Core AI", s2 on
    generalising the ternary kernel, and s3 on the M = 1 decode graph), with
    5 KV heads x 128 for k/v.
  * SigLIP-SO400M vision linears: K in {1152, 4304}, fc1 N = 4304 (same page,
    s2).  8 images x 256 patches = 2048 tokens (s3).
  * BitNet-Embeddings-0.6B: hidden 1024, 16 heads (8 KV) x head_dim 128,
    intermediate 3072 ("BitNet-Embeddings-0.6B/270M: I2_S Conversion and
    Inference Optimization Guide", s2 model details and the per-projection
    norm table of s3.1).

Seeds: weights of tensor i of config c use seed 1000*c + i, activations use
1000*c + 500 + i.  Fused tensors (q|k|v, gate|up) are drawn segment by segment,
each segment with its own tensor index, so every segment is its own source
tensor.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class Projection:
    name: str
    K: int
    N: int
    segments: tuple = ()          # rows of each source tensor; () = one tensor

    @property
    def seg_rows(self) -> tuple:
        return self.segments if self.segments else (self.N,)


@dataclass(frozen=True)
class Workload:
    index: int                    # 1-based config number, used in seeds
    name: str
    M: int
    projections: tuple
    layers: int = 1
    weight_dist: str = "normal"   # "normal" or "laplace", sigma 0.02
    act_dist: str = "normal"      # "normal", "normal_outliers", "student_t_channels"
    notes: str = ""
    extra: dict = field(default_factory=dict)

    def tensors(self):
        """(layer, projection) pairs in stream order."""
        return [(layer, p) for layer in range(self.layers) for p in self.projections]


BITNET2B_LAYER = (
    Projection("q_proj", 2560, 2560),
    Projection("k_proj", 2560, 640),
    Projection("v_proj", 2560, 640),
    Projection("o_proj", 2560, 2560),
    Projection("gate_proj", 2560, 6912),
    Projection("up_proj", 2560, 6912),
    Projection("down_proj", 6912, 2560),
)

WORKLOADS = {
    "c1": Workload(1, "bitlinear-2560x2560-m1", 1, (Projection("linear", 2560, 2560),),
                   act_dist="normal_outliers",
                   notes="one BitLinear; 1% of activations scaled x20"),
    "c2": Workload(2, "bitnet2b-decode-30-layers-m1", 1, BITNET2B_LAYER, layers=30,
                   notes="30 distinct layers of weights streamed, one token per projection"),
    "c3": Workload(3, "siglip-so400m-vit-m2048", 2048, (
        Projection("qkv", 1152, 3456, (1152, 1152, 1152)),
        Projection("o", 1152, 1152),
        Projection("fc1", 1152, 4304),
        Projection("fc2", 4304, 1152),
    )),
    "c4": Workload(4, "embedder-0.6b-prefill-m8192", 8192, (
        Projection("q_proj", 1024, 2048),
        Projection("k_proj", 1024, 1024),
        Projection("v_proj", 1024, 1024),
        Projection("o_proj", 2048, 1024),
        Projection("gate_proj", 1024, 3072),
        Projection("up_proj", 1024, 3072),
        Projection("down_proj", 3072, 1024),
    ), weight_dist="laplace",
        notes="Laplace latent weights (about 39% zero codes), the stand-in for a trained "
              "ternary model's higher zero fraction"),
    "c5": Workload(5, "bitnet2b-prefill-m4096", 4096, (
        Projection("gate_up", 2560, 13824, (6912, 6912)),
        Projection("down", 6912, 2560),
        Projection("qkv", 2560, 3840, (2560, 640, 640)),
    ), act_dist="student_t_channels",
        notes="1% of channels drawn from Student-t (nu = 3) at unit scale"),
}

WEIGHT_SIGMA = 0.02


def _generator(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def draw_weight(shape, seed: int, dist: str = "normal", sigma: float = WEIGHT_SIGMA,
                device="cpu") -> torch.Tensor:
    """bf16 latent weights with standard deviation ``sigma``."""
    g = _generator(seed, device)
    if dist == "normal":
        w = torch.randn(shape, generator=g, device=device, dtype=torch.float32) * sigma
    elif dist == "laplace":
        # Laplace(0, b) = b * (E1 - E2) with E1, E2 ~ Exp(1): finite for every draw
        b = sigma / math.sqrt(2.0)
        e = torch.empty((2, *shape), device=device, dtype=torch.float32).exponential_(generator=g)
        w = b * (e[0] - e[1])
    else:
        raise ValueError(dist)
    return w.to(torch.bfloat16)


def draw_activation(shape, seed: int, dist: str = "normal", device="cpu") -> torch.Tensor:
    """bf16 activations [M, K]."""
    g = _generator(seed, device)
    M, K = shape
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if dist == "normal_outliers":
        mask = torch.rand(shape, generator=g, device=device) < 0.01
        x = torch.where(mask, x * 20.0, x)
    elif dist == "student_t_channels":
        n_ch = max(1, round(0.01 * K))
        channels = torch.randperm(K, generator=g, device=device)[:n_ch]
        z = torch.randn((M, n_ch), generator=g, device=device)
        chi2 = torch.randn((M, n_ch, 3), generator=g, device=device).pow(2).sum(-1)
        x[:, channels] = z / torch.sqrt(chi2 / 3.0)
    elif dist != "normal":
        raise ValueError(dist)
    return x.to(torch.bfloat16)


def source_tensor_index(w: Workload, proj_index: int, layer: int = 0) -> int:
    """Index of the first source tensor of a projection, counting segments in stream order."""
    per_layer = sum(len(p.seg_rows) for p in w.projections)
    return layer * per_layer + sum(len(p.seg_rows) for p in w.projections[:proj_index])


def weight_for(w: Workload, proj_index: int, layer: int = 0, device="cpu") -> torch.Tensor:
    """The [N, K] latent weight of one projection (segments drawn separately)."""
    p = w.projections[proj_index]
    base = 1000 * w.index + source_tensor_index(w, proj_index, layer)
    parts = [draw_weight((rows, p.K), base + i, w.weight_dist, device=device)
             for i, rows in enumerate(p.seg_rows)]
    return parts[0] if len(parts) == 1 else torch.cat(parts, 0)


def activation_for(w: Workload, proj_index: int, layer: int = 0, M: int | None = None,
                   device="cpu") -> torch.Tensor:
    p = w.projections[proj_index]
    seed = 1000 * w.index + 500 + layer * len(w.projections) + proj_index
    return draw_activation((M or w.M, p.K), seed, w.act_dist, device=device)


def packed_bytes(w: Workload) -> int:
    """Algorithmic packed-weight bytes of one pass: sum of N*K/4 (unpadded K)."""
    return sum(p.N * p.K // 4 for _, p in w.tensors())


def int_ops(w: Workload) -> int:
    """Algorithmic integer operations of one pass: sum of 2*M*N*K."""
    return sum(2 * w.M * p.N * p.K for _, p in w.tensors())


def random_case(seed: int, M: int, N: int, K: int, *, w_dist="normal", x_dist="normal",
                segments=(), device="cpu"):
    """A small random (x, W) pair for fuzzed parity cases (drawn on the CPU)."""
    if segments:
        parts = [draw_weight((r, K), seed * 7 + i, w_dist, device="cpu") for i, r in enumerate(segments)]
        W = torch.cat(parts, 0)
    else:
        W = draw_weight((N, K), seed * 7, w_dist, device="cpu")
    x = draw_activation((M, K), seed * 7 + 3, x_dist, device="cpu")
    return x.to(device), W.to(device)
