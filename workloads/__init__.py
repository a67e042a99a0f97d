"""Seeded synthetic workloads for the causal-conv video decoder: shapes and random draws.

This module holds no decoder arithmetic. It defines the workloads (tensor shapes, the decoder
topology as plain numbers, parameter names) and draws their inputs and weights from seeded
torch CPU generators, so that the oracle and the GPU path consume the very same values.

Draw rules (one seeded ``torch.Generator('cpu')`` per workload, draws in the order listed):
  * activations and latents: N(0, 1);
  * conv weights: Kaiming-normal with PyTorch's defaults, N(0, 2 / fan_in), fan_in = Ci*kt*kh*kw;
  * RMS-norm gains: 1 + 0.1 * N(0, 1);
  * biases: zero unless a workload says otherwise (no draw is spent on a zero bias);
  * bf16 workloads round every drawn value to bf16 (round to nearest even) and hand both
    paths the rounded values (the oracle as fp32 numbers, the GPU as bf16).
Order: the input, then any given cache, then the layers in execution order; inside a residual
block: norm1 gain, conv1 weight, norm2 gain, conv2 weight, shortcut weight.

The video geometry is the pages' 704x1248 (latents 44x78 at 16x spatial compression).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Tuple

import torch

LATENT_H, LATENT_W = 44, 78
VIDEO_H, VIDEO_W = 704, 1248


def generator(seed: int) -> torch.Generator:
    return torch.Generator("cpu").manual_seed(int(seed))


def randn(g: torch.Generator, shape) -> torch.Tensor:
    return torch.randn(tuple(shape), generator=g, dtype=torch.float32)


def kaiming(g: torch.Generator, shape) -> torch.Tensor:
    fan_in = 1
    for s in shape[1:]:
        fan_in *= int(s)
    return randn(g, shape) * math.sqrt(2.0 / fan_in)


def gain(g: torch.Generator, c: int) -> torch.Tensor:
    return 1.0 + 0.1 * randn(g, (c,))


def bf16_values(t: torch.Tensor) -> torch.Tensor:
    """The fp32 tensor holding t rounded to bf16 (round to nearest even)."""
    return t.to(torch.bfloat16).to(torch.float32)


# ----------------------------------------------------------------------------------------------
# Decoder topology
# ----------------------------------------------------------------------------------------------
@dataclass(frozen=True)
class DecoderSpec:
    """A Wan2.2-style synthetic decoder: conv_in, mid residual blocks, up stages, head."""

    z_channels: int = 48
    base_channels: int = 384
    stage_channels: Tuple[int, ...] = (384, 384, 192, 96)
    temporal: Tuple[bool, ...] = (True, True, False, False)
    mid_resblocks: int = 2
    stage_resblocks: int = 2
    out_channels: int = 3
    eps: float = 1e-6
    # Parts of the real Wan2.2 TI2V-5B decoder that the synthetic one leaves out (all off there)
    post_quant: bool = False        # a 1x1x1 conv z -> z in front of conv_in
    mid_attention: bool = False     # single-head attention per frame after the first mid block
    spatial: Tuple[bool, ...] = (True, True, True, True)  # the stage ends with nearest x2 + 3x3
    dup: Tuple[bool, ...] = (False, False, False, False)  # + DupUp3D of the stage input
    patch: int = 1                  # unpatchify: out_channels = 3 * patch^2 -> 3 colours
    clamp: bool = False             # clamp the video to [-1, 1]
    norm_l2: bool = False           # RMS norm as x / max(||x||, 1e-12) * sqrt(C) (else 1 / sqrt(mean + eps))


FULL_DECODER = DecoderSpec()

# The real topology (z_dim 48, decoder base 256, channel multipliers 1, 2, 4, 4, three residual
# blocks per up block, mid-block attention, DupUp3D shortcuts, 12-channel head + unpatchify +
# clamp). eps: the GPU kernels normalise by 1 / sqrt(mean x^2 + eps), which equals the page's
# x / max(||x||, 1e-12) * sqrt(C) for every x with ||x|| above 1e-12 up to rounding.
REAL_DECODER = DecoderSpec(base_channels=1024, stage_channels=(1024, 1024, 512, 256), stage_resblocks=3,
                           out_channels=12, eps=1e-27, post_quant=True, mid_attention=True,
                           spatial=(True, True, True, False), dup=(True, True, True, False), patch=2, clamp=True,
                           norm_l2=True)


def resblock_param_list(prefix: str, cin: int, cout: int) -> List[Tuple[str, tuple, str]]:
    out = [
        (f"{prefix}.norm1.gamma", (cin,), "gain"),
        (f"{prefix}.conv1.weight", (cout, cin, 3, 3, 3), "kaiming"),
        (f"{prefix}.conv1.bias", (cout,), "zero"),
        (f"{prefix}.norm2.gamma", (cout,), "gain"),
        (f"{prefix}.conv2.weight", (cout, cout, 3, 3, 3), "kaiming"),
        (f"{prefix}.conv2.bias", (cout,), "zero"),
    ]
    if cin != cout:
        out += [
            (f"{prefix}.shortcut.weight", (cout, cin, 1, 1, 1), "kaiming"),
            (f"{prefix}.shortcut.bias", (cout,), "zero"),
        ]
    return out


def decoder_param_list(spec: DecoderSpec) -> List[Tuple[str, tuple, str]]:
    """(name, shape, draw kind) of every decoder parameter, in execution (= draw) order."""
    p: List[Tuple[str, tuple, str]] = []
    c = spec.base_channels
    z = spec.z_channels
    if spec.post_quant:
        p += [("post_quant.weight", (z, z, 1, 1, 1), "kaiming"), ("post_quant.bias", (z,), "zero")]
    p += [("conv_in.weight", (c, z, 3, 3, 3), "kaiming"), ("conv_in.bias", (c,), "zero")]
    for i in range(spec.mid_resblocks):
        p += resblock_param_list(f"mid.{i}", c, c)
        if i == 0 and spec.mid_attention:
            p += [("mid.attn.norm.gamma", (c,), "gain"),
                  ("mid.attn.qkv.weight", (3 * c, c, 1, 1, 1), "kaiming"), ("mid.attn.qkv.bias", (3 * c,), "zero"),
                  ("mid.attn.proj.weight", (c, c, 1, 1, 1), "kaiming"), ("mid.attn.proj.bias", (c,), "zero")]
    for s, cs in enumerate(spec.stage_channels):
        for j in range(spec.stage_resblocks):
            p += resblock_param_list(f"up.{s}.res.{j}", c if j == 0 else cs, cs)
        c = cs
        if spec.temporal[s]:
            p += [(f"up.{s}.time.weight", (2 * c, c, 3, 1, 1), "kaiming"), (f"up.{s}.time.bias", (2 * c,), "zero")]
        if spec.spatial[s]:
            p += [(f"up.{s}.spatial.weight", (c, c, 3, 3), "kaiming"), (f"up.{s}.spatial.bias", (c,), "zero")]
    p += [("norm_out.gamma", (c,), "gain")]
    p += [("conv_out.weight", (spec.out_channels, c, 3, 3, 3), "kaiming"), ("conv_out.bias", (spec.out_channels,), "zero")]
    return p


def draw_params(g: torch.Generator, plist, bf16: bool) -> Dict[str, torch.Tensor]:
    out: Dict[str, torch.Tensor] = {}
    for name, shape, kind in plist:
        if kind == "kaiming":
            t = kaiming(g, shape)
        elif kind == "gain":
            t = gain(g, shape[0])
        elif kind == "zero":
            t = torch.zeros(shape, dtype=torch.float32)
        else:
            raise ValueError(kind)
        out[name] = bf16_values(t) if bf16 else t
    return out


# ----------------------------------------------------------------------------------------------
# The workloads (all batch 1; tensors are [1, C, T, H, W] fp32 holding the drawn values)
# ----------------------------------------------------------------------------------------------
def single_conv_fp32(seed: int = 1, C: int = 16, T: int = 5, H: int = 16, W: int = 16, Co: int = 16):
    """One causal 3x3x3 conv in fp32: x N(0,1), Kaiming weight, bias 0.01*N(0,1)."""
    g = generator(seed)
    x = randn(g, (1, C, T, H, W))
    w = kaiming(g, (Co, C, 3, 3, 3))
    b = 0.01 * randn(g, (Co,))
    return {"x": x, "weight": w, "bias": b}


def resblock_bf16(seed: int = 2, C: int = 384, T: int = 4, H: int = LATENT_H, W: int = LATENT_W, Cout: int = None,
                  hist_frames: int = 2):
    """A residual block in bf16 with a given 2-frame history (used before both of its convs)."""
    Cout = C if Cout is None else Cout
    g = generator(seed)
    x = bf16_values(randn(g, (1, C, T, H, W)))
    hist = bf16_values(randn(g, (1, C, hist_frames, H, W))) if hist_frames else None
    params = draw_params(g, resblock_param_list("res", C, Cout), bf16=True)
    return {"x": x, "hist": hist, "params": params, "eps": 1e-6}


def upsample_stage_bf16(seed: int = 3, C: int = 192, T: int = 4, H: int = 176, W: int = 312):
    """Nearest x2 + per-frame 3x3 conv, then the causal (3,1,1) time conv C -> 2C into 2T frames."""
    g = generator(seed)
    x = bf16_values(randn(g, (1, C, T, H, W)))
    ws = bf16_values(kaiming(g, (C, C, 3, 3)))
    wt = bf16_values(kaiming(g, (2 * C, C, 3, 1, 1)))
    return {"x": x, "spatial.weight": ws, "spatial.bias": torch.zeros(C), "time.weight": wt,
            "time.bias": torch.zeros(2 * C)}


def decoder_weights(spec: DecoderSpec = FULL_DECODER, seed: int = 4, latent_frames: int = 4,
                    latent_hw: Tuple[int, int] = (LATENT_H, LATENT_W)):
    """The decoder's latents z and its weights; seed 4 with the full spec is the one-pass decode."""
    g = generator(seed)
    z = bf16_values(randn(g, (1, spec.z_channels, latent_frames) + tuple(latent_hw)))
    params = draw_params(g, decoder_param_list(spec), bf16=True)
    return z, params


def streaming_latents(seed: int = 5, latent_frames: int = 31, spec: DecoderSpec = FULL_DECODER,
                      latent_hw: Tuple[int, int] = (LATENT_H, LATENT_W)):
    """Latents of the 5 s streaming decode (31 latent frames -> 121 video frames)."""
    g = generator(seed)
    return bf16_values(randn(g, (1, spec.z_channels, latent_frames) + tuple(latent_hw)))
