"""Seeded synthetic inputs for the delta-W4A4 linear layer.

This module only *draws* inputs; it holds none of the layer's arithmetic
(no cube means, no scales, no encodings), so both the HIP path and the CPU
oracle can take their inputs from it without sharing any of the method.

The pages measure on Wan2.2 / LTX-Video layers with VBench-type suites;
neither weights nor suites are available, so seeded synthetic tensors of the
same shapes stand in for them.  The activation recipe follows the motivation
of the DeltaQuant notes ("DeltaQuant: 4-bit Video Diffusion Models with
Spatiotemporal Delta Smoothing", 研究背景与动机 and 关键设计 1): neighbouring
tokens in time and space are similar, and a few channels carry large,
timestep-dependent outliers.

Recipe (the concrete constants are choices; the pages fix none of them):
  * per channel c: a smooth field  sum_{j<3} a_cj sin(wt_cj t + wh_cj h + ww_cj w + phi_cj)
    with a ~ N(0,1), each w ~ U(0, 0.5) rad/token, phi ~ U(0, 2 pi);
  * plus i.i.d. noise N(0, 0.05^2);
  * a random set of outlier channels, each multiplied (field and noise) by a
    factor drawn from U(lo, hi);
  * rounded once to the layer dtype (bf16 by round-to-nearest-even, or kept fp32).
Weights: N(0, 1/Ci) in nn.Linear layout [Co][Ci]; optionally a few output
channels (rows of [Co][Ci], i.e. columns of the pages' W in X.W) scaled up.

Token n of the flattened activation is (t, h, w) with n = (t*H + h)*W + w.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Tuple

import torch

__all__ = ["LayerConfig", "CONFIGS", "TextConfig", "TEXT_CONFIGS", "make_activation", "make_weight",
           "make_text_activation", "dyadic_activation", "to_f32_numpy"]


@dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int
    H: int
    W: int
    Ci: int
    Co: int
    dtype: str                      # "f32" or "bf16"
    cubes: Tuple[Tuple[int, int, int], ...]
    rank: int
    n_outliers: int
    outlier_lo: float
    outlier_hi: float
    x_seeds: Tuple[int, ...]
    w_seed: int
    w_outlier_rows: int = 0
    w_outlier_factor: float = 1.0

    @property
    def N(self) -> int:
        return self.T * self.H * self.W


# The five synthetic layers.  Shapes are Wan-like latent grids (21 latent
# frames, 480p/720p token grids) and Wan-1.3B / 14B-class channel counts.
CONFIGS = {
    "tiny": LayerConfig("tiny", 4, 8, 8, 256, 256, "f32", ((1, 2, 2),), 16,
                        4, 50.0, 50.0, (1000,), 1500, w_outlier_rows=2, w_outlier_factor=10.0),
    "wan1p3b_proj": LayerConfig("wan1p3b_proj", 21, 30, 52, 1536, 1536, "bf16", ((1, 2, 2),), 32,
                                8, 20.0, 100.0, (2000,), 2500),
    "attn14b_proj": LayerConfig("attn14b_proj", 20, 30, 52, 5120, 5120, "bf16", ((2, 2, 2),), 32,
                                16, 20.0, 100.0, (3000, 3001, 3002, 3003), 3500),
    "ffn_up_720p": LayerConfig("ffn_up_720p", 21, 45, 80, 5120, 13824, "bf16", ((1, 2, 2),), 32,
                               16, 20.0, 100.0, (4000,), 4500),
    "ffn_down_720p": LayerConfig("ffn_down_720p", 21, 45, 80, 13824, 5120, "bf16",
                                 ((1, 1, 1), (1, 2, 2), (2, 2, 2), (1, 4, 4), (21, 45, 80)), 32,
                                 16, 20.0, 100.0, (5000,), 5500),
}


@dataclass(frozen=True)
class TextConfig:
    """A 6-bit layer on text tokens: `prompts` contexts of `ctx` token slots
    each (N = prompts x ctx rows), Ci -> Co."""
    name: str
    prompts: int
    ctx: int
    valid: Tuple[int, ...]          # prompt tokens at the start of each context (the rest is zero padding)
    Ci: int
    Co: int
    dtype: str
    rank: int
    n_outliers: int
    x_seed: int
    w_seed: int

    @property
    def N(self) -> int:
        return self.prompts * self.ctx


# The cross-attention K and V projections of a 14B-class video DiT: two
# 512-slot text contexts (a conditional prompt of 180 tokens and an empty
# negative prompt, the pair that classifier-free guidance evaluates),
# channels 5120 -> K and V stacked (2 x 5120).
TEXT_CONFIGS = {
    "kv_text_14b": TextConfig("kv_text_14b", 2, 512, (180, 1), 5120, 10240, "bf16", 32, 8, 6000, 6500),
}


def make_text_activation(prompts: int, ctx: int, valid: Sequence[int], Ci: int, seed: int, dtype: str = "bf16",
                         n_outliers: int = 8, outlier_lo: float = 20.0, outlier_hi: float = 100.0) -> torch.Tensor:
    """Text-token activation [prompts * ctx, Ci]: in context p, tokens
    0 .. valid[p] - 1 are N(0, 1) embeddings with per-channel log-normal
    scales (sigma 0.5) and `n_outliers` channels scaled by U(lo, hi); the
    remaining slots are zero padding.  Rounded once to `dtype`."""
    g = torch.Generator().manual_seed(int(seed))
    scale = torch.exp(0.5 * torch.randn(Ci, generator=g))
    out = torch.zeros(prompts * ctx, Ci, dtype=torch.float32)
    perm = torch.randperm(Ci, generator=g)[:n_outliers]
    fac = outlier_lo + (outlier_hi - outlier_lo) * torch.rand(n_outliers, generator=g)
    for p in range(prompts):
        v = min(int(valid[p % len(valid)]), ctx)
        tok = torch.randn(v, Ci, generator=g) * scale
        tok[:, perm] *= fac
        out[p * ctx:p * ctx + v] = tok
    return out.to(_torch_dtype(dtype))


def _torch_dtype(dtype: str) -> torch.dtype:
    if dtype == "bf16":
        return torch.bfloat16
    if dtype == "f32":
        return torch.float32
    raise ValueError(f"unknown dtype {dtype!r}")


def make_activation(T: int, H: int, W: int, Ci: int, seed: int, dtype: str = "bf16",
                    n_outliers: int = 0, outlier_lo: float = 20.0, outlier_hi: float = 100.0,
                    noise_std: float = 0.05, device: str = "cpu") -> torch.Tensor:
    """Smooth-field + noise + outlier-channel activation, shape [T*H*W, Ci].

    Parameters are drawn on the CPU from `seed`; the field is evaluated on
    `device` frame by frame with sin(A + B) = sin A cos B + cos A sin B, so no
    [N, Ci, 3] temporary is ever formed.
    """
    g = torch.Generator().manual_seed(int(seed))
    amp = torch.randn(Ci, 3, generator=g, dtype=torch.float64)
    wt = torch.rand(Ci, 3, generator=g, dtype=torch.float64) * 0.5
    wh = torch.rand(Ci, 3, generator=g, dtype=torch.float64) * 0.5
    ww = torch.rand(Ci, 3, generator=g, dtype=torch.float64) * 0.5
    phi = torch.rand(Ci, 3, generator=g, dtype=torch.float64) * (2.0 * math.pi)
    perm = torch.randperm(Ci, generator=g)[:n_outliers]
    fac = outlier_lo + (outlier_hi - outlier_lo) * torch.rand(n_outliers, generator=g, dtype=torch.float64)
    noise_seed = int(torch.randint(0, 2**62, (1,), generator=g).item())

    dev = torch.device(device)
    hh = torch.arange(H, dtype=torch.float64, device=dev)[:, None, None]
    wv = torch.arange(W, dtype=torch.float64, device=dev)[:, None, None]
    amp_d, wt_d, wh_d, ww_d, phi_d = (v.to(dev) for v in (amp, wt, wh, ww, phi))
    B = wv * ww_d                                   # [W, Ci, 3]
    sinB, cosB = torch.sin(B).float(), torch.cos(B).float()
    out = torch.empty(T * H * W, Ci, dtype=torch.float32, device=dev)
    gn = torch.Generator(device=dev).manual_seed(noise_seed)
    for t in range(T):
        A = wt_d * t + hh * wh_d + phi_d            # [H, Ci, 3]
        sA = (amp_d * torch.sin(A)).float()
        cA = (amp_d * torch.cos(A)).float()
        frame = (sA[:, None] * cosB[None] + cA[:, None] * sinB[None]).sum(-1)   # [H, W, Ci]
        frame += noise_std * torch.randn(H, W, Ci, generator=gn, device=dev, dtype=torch.float32)
        out[t * H * W:(t + 1) * H * W] = frame.reshape(H * W, Ci)
    if n_outliers:
        out[:, perm.to(dev)] *= fac.float().to(dev)
    return out.to(_torch_dtype(dtype))


def make_weight(Ci: int, Co: int, seed: int, dtype: str = "bf16", outlier_rows: int = 0,
                outlier_factor: float = 10.0) -> torch.Tensor:
    """W^T in nn.Linear layout [Co][Ci], entries N(0, 1/Ci), on the CPU.

    `outlier_rows` output channels (columns of the pages' W) are scaled by
    `outlier_factor`.
    """
    g = torch.Generator().manual_seed(int(seed))
    w = torch.randn(Co, Ci, generator=g, dtype=torch.float32) / math.sqrt(Ci)
    if outlier_rows:
        rows = torch.randperm(Co, generator=g)[:outlier_rows]
        w[rows] *= outlier_factor
    return w.to(_torch_dtype(dtype))


def dyadic_activation(N: int, Ci: int, seed: int, kmax: int, dtype: str = "f32",
                      device: str = "cpu") -> torch.Tensor:
    """x = k * 2^-8 with integer |k| < kmax: sums and means of power-of-two
    counts of such values are exact in fp32, which the invariant tests use."""
    g = torch.Generator().manual_seed(int(seed))
    k = torch.randint(-kmax + 1, kmax, (N, Ci), generator=g, dtype=torch.int64)
    return (k.double() * 2.0 ** -8).to(_torch_dtype(dtype)).to(device)


def config_activation(cfg: LayerConfig, seed: Optional[int] = None, device: str = "cpu") -> torch.Tensor:
    return make_activation(cfg.T, cfg.H, cfg.W, cfg.Ci, cfg.x_seeds[0] if seed is None else seed,
                           cfg.dtype, cfg.n_outliers, cfg.outlier_lo, cfg.outlier_hi, device=device)


def config_weight(cfg: LayerConfig) -> torch.Tensor:
    return make_weight(cfg.Ci, cfg.Co, cfg.w_seed, cfg.dtype, cfg.w_outlier_rows, cfg.w_outlier_factor)


def to_f32_numpy(t: torch.Tensor):
    """Exact widening to a float32 numpy array (bf16 -> fp32 is exact)."""
    return t.detach().to("cpu").float().numpy()
