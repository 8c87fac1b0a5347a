"""Seeded synthetic inputs for the W4A4 ConvRot linear.

This module is the only code that both the CPU oracle and the HIP path use. It
holds none of the method's arithmetic: it draws random numbers and converts
them to the input dtypes (bf16 activations, fp32 weights).

Recipe (the pages publish no dataset, so these draws stand in for a diffusion
transformer's hidden states and linear weights):

* activations ``x``: ``[M, K]`` standard normal, with 1 % of the K channels
  (at least one) multiplied by 20 in every row, the outlier channels that the
  Hadamard rotation exists to spread out (comfy-kitchen PR #63 "int4_tensorwise:
  W4A4 layout (+ConvRot)", Description; runcomfy ComfyUI-INT4-Fast page, "How
  ComfyUI-INT4-Fast Works"); rounded to bf16 with round-to-nearest-even;
* weights ``W``: ``[N, K]`` fp32 drawn from N(0, 0.02);
* LoRA factors (dynamic LoRA): down ``A`` ``[rank, K]`` fp32 and up ``B``
  ``[N, rank]`` rounded to bf16, both drawn from N(0, 0.02), so that the LoRA
  term is a visible fraction of the layer's output.

* codebook (grouped W4A8 with a frozen 16-entry codebook): the pages give no
  values, so the stand-in is the 16 quantiles of a standard normal at
  (u + 1/2) / 16, divided by the largest, in ascending order of index: a
  non-uniform, zero-free table that exercises everything uniform int4 codes
  do not (no deterministic draw is involved).

Draw order for one seed: outlier channel indices, then ``x``, then each weight
in turn. The same host arrays feed the oracle and the GPU, so the two sides
never need a shared RNG.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

OUTLIER_FRACTION = 0.01
OUTLIER_SCALE = 20.0
WEIGHT_STD = 0.02


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round-to-nearest-even) and return the uint16 bit patterns.

    Input preparation only: the layer's activations are bf16 tensors, and the
    generator draws them in fp32 first. NaN is not produced by the generator.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def outlier_channels(rng: np.random.Generator, k: int) -> np.ndarray:
    n_out = max(1, int(round(OUTLIER_FRACTION * k)))
    return np.sort(rng.choice(k, n_out, replace=False))


def make_activations(rng: np.random.Generator, m: int, k: int, idx: np.ndarray | None = None) -> np.ndarray:
    """bf16 bit patterns ``uint16 [m, k]``: N(0,1) with outlier channels x20."""
    if idx is None:
        idx = outlier_channels(rng, k)
    x = rng.standard_normal((m, k), dtype=np.float32)
    x[:, idx] *= np.float32(OUTLIER_SCALE)
    return f32_to_bf16_bits(x)


def make_weight(rng: np.random.Generator, n: int, k: int) -> np.ndarray:
    """fp32 ``[n, k]`` drawn from N(0, 0.02)."""
    return rng.normal(0.0, WEIGHT_STD, (n, k)).astype(np.float32)


LORA_STD = 0.02


def make_lora(rng: np.random.Generator, rank: int, k: int, n: int):
    """LoRA factors: (down fp32 ``[rank, k]``, up bf16 bit patterns ``uint16 [n, rank]``)."""
    a = rng.normal(0.0, LORA_STD, (rank, k)).astype(np.float32)
    b = f32_to_bf16_bits(rng.normal(0.0, LORA_STD, (n, rank)).astype(np.float32))
    return a, b


def make_codebook() -> np.ndarray:
    """fp32 ``[16]``: normal quantiles at (u + 1/2) / 16 scaled to max |.| = 1."""
    from statistics import NormalDist
    nd = NormalDist()
    q = np.array([nd.inv_cdf((u + 0.5) / 16.0) for u in range(16)], np.float64)
    return (q / np.abs(q).max()).astype(np.float32)


@dataclass
class Layer:
    m: int
    k: int
    n: int
    x_bf16: np.ndarray          # uint16 [m, k]
    weights: list               # list of fp32 [n, k]


def make_layer(m: int, k: int, n: int, seed: int = 0, n_weights: int = 1) -> Layer:
    """One layer's inputs in the fixed draw order: outlier indices, x, W_1..W_n."""
    rng = np.random.default_rng(seed)
    idx = outlier_channels(rng, k)
    x = make_activations(rng, m, k, idx)
    ws = [make_weight(rng, n, k) for _ in range(n_weights)]
    return Layer(m, k, n, x, ws)


# Named workloads. The first is small enough for exhaustive parity; the second
# is the headline layer (a 3072 x 3072 projection over 4608 tokens); the rest
# are the up/down projections, the shared-activation q/k/v case and the
# skinny-M decode shapes.
WORKLOADS = {
    "tiny": dict(m=64, k=256, n=256),
    "square_3072": dict(m=4608, k=3072, n=3072),
    "up_3072_12288": dict(m=4608, k=3072, n=12288),
    "qkv_3x3072": dict(m=4608, k=3072, n=3072, n_weights=3),
    "down_12288_3072": dict(m=4608, k=12288, n=3072),
}
SKINNY_M = (1, 2, 4, 8, 16, 64)
SKINNY_NK = ((12288, 3072), (5120, 5120))
