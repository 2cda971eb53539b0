"""Seeded synthetic inputs for the Wan-style video VAE decoder.

This module is the only code shared by the CPU oracle and the GPU path.  It
holds the decoder's weight inventory (names and shapes, in the canonical
order both sides index by), the initialisation law, the latent generator and
bf16 round-to-nearest-even.  It contains none of the decoder's arithmetic.

Architecture (the weight inventory below follows it): conv_in 48 -> 4c, a mid
block (ResBlock, per-frame single-head attention, ResBlock), four up stages of
widths [4c, 4c, 2c, c] with two ResBlocks each, a time_conv after stages 0 and
1, a nearest-2x + Conv2d 3x3 upsampler after stages 0, 1 and 2, and a head
(RMSNorm, SiLU, CausalConv3d c -> 12, 2x2 pixel shuffle).  The pages describe
this decoder as the Wan2.2 VAE decoder with 48 latent channels, 16x16 spatial
and 4x temporal compression ("Wan2.2 VAE decoder", introduction); the exact
layer list is the plainest reading of that description.

A deeper variant ("deep", 110 tensors) has three ResBlocks per up stage and
a 48 -> 48 1x1x1 conv applied to the latents before conv_in: the Wan2.2 page
("Use") counts 110 decoder tensors, which is the 84 above plus one more
ResBlock per stage (4 x 6) and that 1x1x1 conv (2).

Initialisation: every conv / linear weight is uniform(-1/sqrt(fan_in),
+1/sqrt(fan_in)) with fan_in = Cin*kt*kh*kw, every RMSNorm gamma is
1 + 0.1*N(0,1) and every bias 0.01*N(0,1).  Tensor i of the canonical list is
drawn from numpy's PCG64 seeded with [seed, i]; latent frame t is drawn from
PCG64 seeded with [seed, 10000 + t] so that the latents of a shorter clip are
exactly the first frames of a longer one.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, List, Sequence, Tuple

import numpy as np

LATENT_CHANNELS = 48
HEAD_CHANNELS = 12  # 3 colours x 2x2 pixel shuffle
LATENT_SEED_OFFSET = 10000


@dataclass(frozen=True)
class WeightSpec:
    name: str
    shape: Tuple[int, ...]
    kind: str  # "weight", "bias" or "gamma"
    fan_in: int = 0


def stage_widths(c: int) -> List[int]:
    """Channel widths of the four up stages: [4c, 4c, 2c, c]."""
    return [4 * c, 4 * c, 2 * c, c]


def _conv(name: str, cout: int, cin: int, k: Tuple[int, ...]) -> List[WeightSpec]:
    fan = cin
    for d in k:
        fan *= d
    return [WeightSpec(name + ".weight", (cout, cin) + tuple(k), "weight", fan),
            WeightSpec(name + ".bias", (cout,), "bias")]


def _resblock(name: str, cin: int, cout: int) -> List[WeightSpec]:
    out = [WeightSpec(name + ".norm1.gamma", (cin,), "gamma")]
    out += _conv(name + ".conv1", cout, cin, (3, 3, 3))
    out += [WeightSpec(name + ".norm2.gamma", (cout,), "gamma")]
    out += _conv(name + ".conv2", cout, cout, (3, 3, 3))
    if cin != cout:
        out += _conv(name + ".shortcut", cout, cin, (1, 1, 1))
    return out


NUM_WEIGHTS = 84
NUM_WEIGHTS_DEEP = 110


def res_per_stage(deep: bool) -> int:
    return 3 if deep else 2


def weight_specs(c: int, deep: bool = False) -> List[WeightSpec]:
    """The decoder tensors in canonical order (PyTorch layouts): 84, or 110
    for the deep variant (pre_conv first, three ResBlocks per up stage)."""
    c4 = 4 * c
    specs: List[WeightSpec] = []
    if deep:
        specs += _conv("pre_conv", LATENT_CHANNELS, LATENT_CHANNELS, (1, 1, 1))
    specs += _conv("conv_in", c4, LATENT_CHANNELS, (3, 3, 3))
    specs += _resblock("mid.res0", c4, c4)
    specs += [WeightSpec("mid.attn.norm.gamma", (c4,), "gamma")]
    specs += _conv("mid.attn.qkv", 3 * c4, c4, ())
    specs += _conv("mid.attn.proj", c4, c4, ())
    specs += _resblock("mid.res1", c4, c4)
    widths = stage_widths(c)
    prev = c4
    for s, cs in enumerate(widths):
        specs += _resblock(f"up{s}.res0", prev, cs)
        for k in range(1, res_per_stage(deep)):
            specs += _resblock(f"up{s}.res{k}", cs, cs)
        if s < 2:
            specs += _conv(f"up{s}.time_conv", 2 * cs, cs, (3, 1, 1))
        if s < 3:
            specs += _conv(f"up{s}.up_conv", cs, cs, (3, 3))
        prev = cs
    specs += [WeightSpec("head.norm.gamma", (c,), "gamma")]
    specs += _conv("head.conv", HEAD_CHANNELS, c, (3, 3, 3))
    return specs


def weight_names(c: int, deep: bool = False) -> List[str]:
    return [s.name for s in weight_specs(c, deep)]


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even).

    Returns float32 values that are exactly representable in bfloat16.
    Inputs here are always finite.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).reshape(a.shape)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of float32 values that are already bf16-exact."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    return (a.view(np.uint32) >> 16).astype(np.uint16)


def make_weights(c: int, seed: int = 0, bf16: bool = True, deep: bool = False) -> Dict[str, np.ndarray]:
    """Seeded float32 weights in canonical order (dict preserves the order).

    With bf16=True every tensor is rounded to bf16 (RNE) and that rounded
    model is the model both the oracle and the GPU evaluate.
    """
    out: Dict[str, np.ndarray] = {}
    for i, sp in enumerate(weight_specs(c, deep)):
        rng = np.random.Generator(np.random.PCG64([seed, i]))
        if sp.kind == "weight":
            bound = 1.0 / np.sqrt(sp.fan_in)
            t = rng.uniform(-bound, bound, size=sp.shape)
        elif sp.kind == "gamma":
            t = 1.0 + 0.1 * rng.standard_normal(sp.shape)
        else:
            t = 0.01 * rng.standard_normal(sp.shape)
        t = t.astype(np.float32)
        if bf16:
            t = bf16_round(t)
        out[sp.name] = t
    return out


def make_latents(T: int, h: int, w: int, seed: int = 0, bf16: bool = True) -> np.ndarray:
    """Latents z ~ N(0,1) of shape [1, 48, T, h, w], one PCG64 stream per frame."""
    z = np.empty((1, LATENT_CHANNELS, T, h, w), dtype=np.float32)
    for t in range(T):
        rng = np.random.Generator(np.random.PCG64([seed, LATENT_SEED_OFFSET + t]))
        z[0, :, t] = rng.standard_normal((LATENT_CHANNELS, h, w)).astype(np.float32)
    if bf16:
        z = bf16_round(z)
    return z


@dataclass(frozen=True)
class Config:
    """One decoder workload: base width c, latent frames T, latent h x w."""
    name: str
    c: int
    T: int
    h: int
    w: int
    passes: Tuple[int, ...]
    weights_bf16: bool = True
    deep: bool = False

    @property
    def video_shape(self) -> Tuple[int, int, int, int, int]:
        return (1, 3, 4 * self.T - 3, 16 * self.h, 16 * self.w)


# The five workloads: a tiny fp32 decoder, a c=64 decoder at 352x624, and the
# c=256 decoder at 704x1248 for 49, 193 and 481 video frames.
CONFIGS: Sequence[Config] = (
    Config("tiny_c16_T2_4x6", 16, 2, 4, 6, (1, 2), weights_bf16=False),
    Config("c64_T3_352x624", 64, 3, 22, 39, (1, 3)),
    Config("c256_T13_704x1248", 256, 13, 44, 78, (4,)),
    Config("c256_T49_704x1248", 256, 49, 44, 78, (4,)),
    Config("c256_T121_704x1248", 256, 121, 44, 78, (2, 4, 8, 16)),
)


# The deep (110-tensor) variant at the same sizes: parity cases and a bench
# line beside the five workloads.
DEEP_CONFIGS: Sequence[Config] = (
    Config("deep_tiny_c16_T2_4x6", 16, 2, 4, 6, (1, 2), weights_bf16=False, deep=True),
    Config("deep_c64_T3_352x624", 64, 3, 22, 39, (1, 3), deep=True),
    Config("deep_c256_T49_704x1248", 256, 49, 44, 78, (4,), deep=True),
)


def config_by_name(name: str) -> Config:
    for cfg in tuple(CONFIGS) + tuple(DEEP_CONFIGS):
        if cfg.name == name:
            return cfg
    raise KeyError(name)
