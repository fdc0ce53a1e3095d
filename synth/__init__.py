"""Seeded synthetic inputs for the MOSS-Image single-stream DiT denoising step.

This module is shared by the CPU oracle's tests and by the GPU path's tests and benchmark. It holds
none of the method's arithmetic: it only draws random numbers in a fixed, documented order and stores
them in the dtypes the path consumes.

* weights: ``standard_normal * std`` drawn in float64, rounded to float32, then to bfloat16
  (round-to-nearest-even) and returned as uint16 bit patterns, in the order of the C ABI's weight
  struct: t_w1, t_w2, x_embed_w, then per block (mod_w, qkv_w, out_w, gate_up_w, down_w), then
  final_mod_w, final_w. ``mod_scale`` multiplies the draws of mod_w and final_mod_w before rounding
  (1 = the literal N(0, 0.02) init; 50 = the diagnostic mode whose gates are large enough for a
  block's update to survive the bf16 residual).
* text states and latent noise: float32 standard normal, drawn after the weights.
* sigma: float32 uniform on [0, 1), drawn last.

The text encoder and the VAE of the pages (MOSS-Image: specs, settings, VRAM and text rendering
tested -- "Architecture and specs") are out of scope; these tensors stand in for their outputs.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np


@dataclass(frozen=True)
class Shape:
    """Model hyper-parameters (MOSS-Image: specs ... tested, "Architecture and specs")."""
    num_layers: int = 42
    hidden: int = 3072
    num_heads: int = 24
    head_dim: int = 128
    ffn_hidden: int = 8192
    latent_channels: int = 32
    patch: int = 2
    temb_dim: int = 256
    text_dim: int = 4096          # width of the text encoder's states (input of the text refiner)
    refiner_layers: int = 2

    @property
    def patch_dim(self) -> int:
        return self.latent_channels * self.patch * self.patch


FULL = Shape()
# Tiny single-stream DiT: 2 blocks, hidden 256, 2 heads x 128, FFN 704 (the 8/3 rule rounded up to a
# multiple of 64), 32 latent channels, 2x2 patches.
TINY = Shape(num_layers=2, hidden=256, num_heads=2, head_dim=128, ffn_hidden=704, text_dim=320)
# the FP8 tier works on whole 256-element k-tile groups: its tiny shape widens the FFN to 768
TINY_FP8 = Shape(num_layers=2, hidden=256, num_heads=2, head_dim=128, ffn_hidden=768, text_dim=320)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit pattern, round-to-nearest-even (NaN stays NaN)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    nan = np.isnan(x)
    out = rounded.astype(np.uint16)
    out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _bf16_normal(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    return f32_to_bf16_bits((rng.standard_normal(shape) * std).astype(np.float32))


@dataclass
class Weights:
    """bf16 bit patterns (uint16), layouts as in the C ABI: every linear is [out, in] row-major."""
    t_w1: np.ndarray
    t_w2: np.ndarray
    x_embed_w: np.ndarray
    mod_w: List[np.ndarray]
    qkv_w: List[np.ndarray]
    out_w: List[np.ndarray]
    gate_up_w: List[np.ndarray]
    down_w: List[np.ndarray]
    final_mod_w: np.ndarray
    final_w: np.ndarray


def make_weights(shape: Shape, seed: int = 0, std: float = 0.02, mod_scale: float = 1.0,
                 rng: Optional[np.random.Generator] = None) -> Weights:
    rng = rng if rng is not None else np.random.default_rng(seed)
    D, F, E = shape.hidden, shape.ffn_hidden, shape.temb_dim
    t_w1 = _bf16_normal(rng, (E, 256), std)
    t_w2 = _bf16_normal(rng, (E, E), std)
    x_embed_w = _bf16_normal(rng, (D, shape.patch_dim), std)
    mod_w, qkv_w, out_w, gate_up_w, down_w = [], [], [], [], []
    for _ in range(shape.num_layers):
        mod_w.append(_bf16_normal(rng, (6 * D, E), std * mod_scale))
        qkv_w.append(_bf16_normal(rng, (3 * D, D), std))
        out_w.append(_bf16_normal(rng, (D, D), std))
        gate_up_w.append(_bf16_normal(rng, (2 * F, D), std))
        down_w.append(_bf16_normal(rng, (D, F), std))
    final_mod_w = _bf16_normal(rng, (2 * D, E), std * mod_scale)
    final_w = _bf16_normal(rng, (shape.patch_dim, D), std)
    return Weights(t_w1, t_w2, x_embed_w, mod_w, qkv_w, out_w, gate_up_w, down_w, final_mod_w, final_w)


def normal_f32(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(shape).astype(np.float32)


def uniform_f32(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.random(shape).astype(np.float32)


def bf16_normal_bits(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    """bf16 activations ~N(0, std^2) as bit patterns (attention and single-block workloads)."""
    return _bf16_normal(rng, shape, std)


@dataclass
class SamplingInputs:
    """Latent noise and text states of a sampling run (empty negative prompt = zero text states)."""
    latents: np.ndarray          # fp32 [1, C, h, w]
    text_cond: np.ndarray        # fp32 [1, T, D]
    text_uncond: np.ndarray      # fp32 [1, T, D] (zeros)


def make_sampling_inputs(shape: Shape, latent_h: int, latent_w: int, text_len: int,
                         rng: np.random.Generator) -> SamplingInputs:
    text_cond = normal_f32(rng, (1, text_len, shape.hidden))
    latents = normal_f32(rng, (1, shape.latent_channels, latent_h, latent_w))
    return SamplingInputs(latents, text_cond, np.zeros_like(text_cond))


def tiny_workload(mod_scale: float = 1.0, seed: int = 0, shape: Shape = TINY):
    """Tiny 2-block DiT, 16x16 latent (64 image tokens) + 32 text tokens, seed 0."""
    rng = np.random.default_rng(seed)
    w = make_weights(shape, rng=rng, mod_scale=mod_scale)
    inp = make_sampling_inputs(shape, 16, 16, 32, rng)
    return w, inp


# Device-side weight draw for the 5B-parameter model: drawing ~5e9 normals on the host with numpy
# takes minutes, so the full-size workloads draw them with torch's seeded generator, layer by layer,
# in the same order as make_weights (per tensor: torch.randn(shape, generator=g) * std -> bf16).
def torch_weights(shape: Shape, seed: int, device, std: float = 0.02, mod_scale: float = 1.0,
                  ) -> Dict[str, object]:
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    D, F, E = shape.hidden, shape.ffn_hidden, shape.temb_dim

    def draw(rows, cols, s):
        t = torch.randn((rows, cols), generator=g, device=device, dtype=torch.float32)
        return (t * s).to(torch.bfloat16)

    out: Dict[str, object] = {
        "t_w1": draw(E, 256, std), "t_w2": draw(E, E, std), "x_embed_w": draw(D, shape.patch_dim, std),
        "mod_w": [], "qkv_w": [], "out_w": [], "gate_up_w": [], "down_w": [],
    }
    for _ in range(shape.num_layers):
        out["mod_w"].append(draw(6 * D, E, std * mod_scale))
        out["qkv_w"].append(draw(3 * D, D, std))
        out["out_w"].append(draw(D, D, std))
        out["gate_up_w"].append(draw(2 * F, D, std))
        out["down_w"].append(draw(D, F, std))
    out["final_mod_w"] = draw(2 * D, E, std * mod_scale)
    out["final_w"] = draw(shape.patch_dim, D, std)
    return out


# Text refiner weights (projection text_dim -> hidden and the refiner blocks), drawn from their own
# seeded stream so the DiT's weights and inputs above stay as they are: bf16 bit patterns (numpy) for
# the small shapes, bf16 tensors on the device (torch's generator) for the full size. Encoder states
# are N(0, 1) fp32 [B, T, text_dim].
def refiner_weights(shape: Shape, seed: int = 100, std: float = 0.02) -> Dict[str, object]:
    rng = np.random.default_rng(seed)
    D, F = shape.hidden, shape.ffn_hidden
    out: Dict[str, object] = {"text_proj_w": _bf16_normal(rng, (D, shape.text_dim), std),
                              "refiner_qkv_w": [], "refiner_out_w": [], "refiner_gate_up_w": [], "refiner_down_w": []}
    for _ in range(shape.refiner_layers):
        out["refiner_qkv_w"].append(_bf16_normal(rng, (3 * D, D), std))
        out["refiner_out_w"].append(_bf16_normal(rng, (D, D), std))
        out["refiner_gate_up_w"].append(_bf16_normal(rng, (2 * F, D), std))
        out["refiner_down_w"].append(_bf16_normal(rng, (D, F), std))
    return out


def torch_refiner_weights(shape: Shape, seed: int, device, std: float = 0.02) -> Dict[str, object]:
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    D, F = shape.hidden, shape.ffn_hidden

    def draw(rows, cols):
        return (torch.randn((rows, cols), generator=g, device=device, dtype=torch.float32) * std).to(torch.bfloat16)

    out: Dict[str, object] = {"text_proj_w": draw(D, shape.text_dim), "refiner_qkv_w": [], "refiner_out_w": [],
                              "refiner_gate_up_w": [], "refiner_down_w": []}
    for _ in range(shape.refiner_layers):
        out["refiner_qkv_w"].append(draw(3 * D, D))
        out["refiner_out_w"].append(draw(D, D))
        out["refiner_gate_up_w"].append(draw(2 * F, D))
        out["refiner_down_w"].append(draw(D, F))
    return out
