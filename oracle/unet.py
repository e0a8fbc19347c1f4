"""Plain float64 oracle of the U-Net parts around the Spatial-Transformer
block: SiLU, the 3x3 convolution, the ResnetBlock2D, classifier-free
guidance and the DDPM sampling step.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
library.  Every function follows its definition step by step in float64;
where the pages leave a step open, the reading taken is stated in the
docstring.

Pages cited:
  * "Stable Diffusion XL Inpainting 宏观架构" §4 "核心算子与任务差异" and
    "Stable Diffusion 2.1 Base 宏观架构" §4: ResnetBlock2D = GroupNorm + SiLU
    + Conv, add the time embedding, GroupNorm + Dropout + Conv, residual /
    shortcut add.
  * DDPM / SD / SDXL tutorial page (bfzx365): "（1）ResNetBlock模块" and the
    image-decoder passage on the ResNetBlock (GSC = GroupNorm + SiLU + Conv
    on the feature, added to the time embedding after SiLU + a fully
    connected layer, then a second GSC, added to the skip connection); the
    DownSample module (Conv 3x3, stride 2, padding 1) and the UpSample module
    (nearest interpolation + Conv); the DDPM reverse step
    x_{t-1} = 1/sqrt(alpha_t) (x_t - beta_t / sqrt(1 - alphabar_t) eps) +
    sqrt(beta_t) z with alpha_t = 1 - beta_t and alphabar_t the product of
    the alphas, and the linear schedule of beta from 0.0001 to 0.02 over
    1000 steps.
  * "企业官网建设流程全解析" (SD1.5 anatomy article) §1 and §5: the CFG scale
    (classifier-free guidance) applied to the U-Net's noise prediction.
"""
from __future__ import annotations

import math
from typing import Dict, Optional

import numpy as np

from .block import group_norm, linear


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def silu(x):
    """SiLU(x) = x * sigmoid(x) = x / (1 + exp(-x))."""
    x = _f64(x)
    # exp(-x) overflows for x < -709; the quotient is then 0 either way
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


def conv2d(x, w, b=None, stride: int = 1, padding: int = 1):
    """2-D convolution as the U-Net's Conv layers compute it, [B, Ci, H, W]
    -> [B, Co, Ho, Wo].

    w is [Co, Ci, kh, kw].  Output pixel (i, j) is the sum over the kernel
    taps (di, dj) and input channels of w[co, ci, di, dj] * x[ci, i*stride
    + di - padding, j*stride + dj - padding], with x taken as zero outside
    the image, plus b[co] -- a cross-correlation (the kernel is not
    flipped), which is what a Conv layer of the framework the pages quote
    computes; Ho = (H + 2 padding - kh) // stride + 1.
    """
    x = _f64(x)
    w = _f64(w)
    B, Ci, H, W = x.shape
    Co, Ci2, kh, kw = w.shape
    if Ci2 != Ci:
        raise ValueError("input channels of x and w differ")
    Ho = (H + 2 * padding - kh) // stride + 1
    Wo = (W + 2 * padding - kw) // stride + 1
    xp = np.zeros((B, Ci, H + 2 * padding, W + 2 * padding))
    xp[:, :, padding:padding + H, padding:padding + W] = x
    out = np.zeros((B, Co, Ho, Wo))
    for di in range(kh):
        for dj in range(kw):
            # the input pixels tap (di, dj) sees, one per output pixel
            patch = xp[:, :, di:di + stride * (Ho - 1) + 1:stride, dj:dj + stride * (Wo - 1) + 1:stride]
            out += np.einsum("oc,bchw->bohw", w[:, :, di, dj], patch, optimize=True)
    if b is not None:
        out += _f64(b)[None, :, None, None]
    return out


def upsample_nearest2x(x):
    """Nearest-neighbour upsampling by 2: out[.., i, j] = x[.., i // 2, j // 2]."""
    x = _f64(x)
    return np.repeat(np.repeat(x, 2, axis=2), 2, axis=3)


def resnet_block(x, temb, p: Dict, groups: int = 32, eps: float = 1e-5):
    """ResnetBlock2D, [B, Ci, H, W] and temb [B, Dt] -> [B, Co, H, W].

        h = Conv3x3(SiLU(GroupNorm1(x)))                      (conv1)
        h = h + Linear(SiLU(temb))[:, :, None, None]          (time embedding)
        h = Conv3x3(Dropout(SiLU(GroupNorm2(h))))             (conv2)
        y = shortcut(x) + h

    Readings taken: GroupNorm of 32 contiguous channel groups with
    population variance and eps = 1e-5 (the pages name only "GroupNorm");
    both convolutions 3x3, stride 1, padding 1 (shape preserving); the second
    GroupNorm is followed by SiLU as in the first (the tutorial's GSC =
    GroupNorm + SiLU + Conv for both, the architecture pages list "GroupNorm
    + Dropout + Conv"); Dropout is the identity (inference); the time
    embedding is added per (sample, channel) after conv1; shortcut(x) = x
    when Ci == Co, else a 1x1 convolution with bias (p["sc_w"] [Co, Ci],
    p["sc_b"]); no output scaling.

    p: gn1_w, gn1_b [Ci]; conv1_w [Co, Ci, 3, 3], conv1_b [Co]; temb_w
    [Co, Dt], temb_b [Co]; gn2_w, gn2_b [Co]; conv2_w [Co, Co, 3, 3],
    conv2_b [Co]; sc_w, sc_b when Ci != Co.
    """
    x = _f64(x)
    h = conv2d(silu(group_norm(x, p["gn1_w"], p["gn1_b"], groups, eps)), p["conv1_w"], p.get("conv1_b"))
    t = linear(silu(temb), p["temb_w"], p.get("temb_b"))
    h = h + t[:, :, None, None]
    h = conv2d(silu(group_norm(h, p["gn2_w"], p["gn2_b"], groups, eps)), p["conv2_w"], p.get("conv2_b"))
    if x.shape[1] != h.shape[1]:
        sc = conv2d(x, _f64(p["sc_w"])[:, :, None, None], p.get("sc_b"), padding=0)
    else:
        sc = x
    return sc + h


def cfg_combine(eps_uncond, eps_cond, scale: float):
    """Classifier-free guidance: eps = eps_u + scale * (eps_c - eps_u).

    Reading taken: the anatomy article names the CFG scale only; this is the
    guidance rule that scale belongs to, with the unconditional and the
    conditional prediction of the B = 2 pair (unconditional first)."""
    eu = _f64(eps_uncond)
    ec = _f64(eps_cond)
    return eu + float(scale) * (ec - eu)


def linear_schedule(T: int = 1000, beta_start: float = 1e-4, beta_end: float = 0.02):
    """beta_t linear from beta_start (t = 1) to beta_end (t = T), alpha_t =
    1 - beta_t, alphabar_t = alpha_1 * ... * alpha_t; arrays indexed t - 1."""
    if T < 1:
        raise ValueError("T must be >= 1")
    beta = np.linspace(beta_start, beta_end, T, dtype=np.float64) if T > 1 else np.array([beta_start])
    alpha = 1.0 - beta
    alphabar = np.cumprod(alpha)
    return beta, alpha, alphabar


def ddpm_step(x_t, eps, t: int, schedule, noise=None):
    """One DDPM reverse step (the tutorial page's sampling equation):
    x_{t-1} = 1/sqrt(alpha_t) * (x_t - beta_t / sqrt(1 - alphabar_t) * eps)
              + sqrt(beta_t) * z,  z = ``noise`` (None: 0).
    t runs from T down to 1."""
    beta, alpha, alphabar = schedule
    if not 1 <= t <= len(beta):
        raise ValueError("t out of range")
    bt, at, abt = beta[t - 1], alpha[t - 1], alphabar[t - 1]
    out = (_f64(x_t) - bt / math.sqrt(1.0 - abt) * _f64(eps)) / math.sqrt(at)
    if noise is not None:
        out = out + math.sqrt(bt) * _f64(noise)
    return out


def guided_ddpm_step(x_t, eps_pair, t: int, scale: float, schedule, noise=None):
    """Guidance on the U-Net's prediction for the pair [uncond; cond] (batch
    axis first, halves of equal size), then one DDPM step of x_t."""
    eps_pair = _f64(eps_pair)
    n = eps_pair.shape[0] // 2
    return ddpm_step(x_t, cfg_combine(eps_pair[:n], eps_pair[n:], scale), t, schedule, noise)


# ------------------------------------------------------------------ U-Net
def timestep_embedding(t, dim: int):
    """Sinusoidal embedding of the timesteps t [B] -> [B, dim] (the
    tutorial's sinusoidal embedding).  Reading taken: half = dim / 2
    frequencies f_i = 10000^(-i / half), i = 0 .. half - 1, and the cosines
    first: [cos(t f_0) .. cos(t f_{half-1}), sin(t f_0) .. sin(t f_{half-1})]."""
    t = _f64(t).reshape(-1)
    half = dim // 2
    f = np.exp(-math.log(10000.0) * np.arange(half, dtype=np.float64) / half)
    a = t[:, None] * f[None, :]
    return np.concatenate([np.cos(a), np.sin(a)], axis=1)


def unet_forward(x, t, ctx, P: Dict, cfg, add=None, record=None):
    """One denoiser timestep of the U-Net, x [B, in, H, W] -> [B, out, H, W].

    Follows the architecture pages' §3 topology (SDXL-Inpaint, SD2.1): the
    time embedding (sinusoidal, Linear -> SiLU -> Linear, plus the same MLP
    on ``add`` when the configuration has one); conv_in; per down level
    ``layers_per_block`` x (ResnetBlock2D, then a Spatial-Transformer block
    of the level's depth when it has one), each output kept as a skip, then
    a 3x3 stride-2 convolution (DownSample, tutorial) except on the last
    level, its output kept as a skip too; the middle block ResNet ->
    transformer -> ResNet; per up level, deepest first, (layers_per_block +
    1) x (concatenate the last kept skip along channels, ResnetBlock2D,
    transformer), then nearest 2x upsampling and a 3x3 convolution
    (UpSample, tutorial) except on the last; GroupNorm + SiLU + 3x3 conv_out.
    GroupNorms of the ResNets and of the output use eps 1e-5; the
    transformer blocks are oracle.block.block_forward (heads = C / 64).
    ``record`` (a list) receives (stage name, shape) of every stage output.
    """
    from .block import block_forward
    x = _f64(x)
    emb = timestep_embedding(t, cfg.temb_in)
    temb = linear(silu(linear(emb, P["time1_w"], P["time1_b"])), P["time2_w"], P["time2_b"])
    if cfg.add_in:
        temb = temb + linear(silu(linear(add, P["add1_w"], P["add1_b"])), P["add2_w"], P["add2_b"])

    def rec(name, a):
        if record is not None:
            record.append((name, tuple(a.shape)))
        return a

    def st(h, bp):
        return block_forward(h, ctx, bp, h.shape[1] // 64)

    h = rec("conv_in", conv2d(x, P["conv_in_w"], P["conv_in_b"]))
    skips = [h]
    L = len(cfg.channels)
    for lvl in range(L):
        d = P["down"][lvl]
        for r in range(cfg.layers_per_block):
            h = resnet_block(h, temb, d["res"][r])
            if cfg.depths[lvl]:
                h = st(h, d["attn"][r])
            skips.append(rec(f"down{lvl}.{r}", h))
        if lvl < L - 1:
            h = conv2d(h, d["down_w"], d["down_b"], stride=2)
            skips.append(rec(f"down{lvl}.downsample", h))
    m = P["mid"]
    h = resnet_block(h, temb, m["res"][0])
    if cfg.mid_depth:
        h = st(h, m["attn"][0])
    h = rec("mid", resnet_block(h, temb, m["res"][1]))
    for u, lvl in enumerate(reversed(range(L))):
        up = P["up"][u]
        for r in range(cfg.layers_per_block + 1):
            h = np.concatenate([h, skips.pop()], axis=1)
            h = resnet_block(h, temb, up["res"][r])
            if cfg.depths[lvl]:
                h = st(h, up["attn"][r])
        rec(f"up{u}", h)
        if lvl > 0:
            h = rec(f"up{u}.upsample", conv2d(upsample_nearest2x(h), up["up_w"], up["up_b"]))
    h = silu(group_norm(h, P["norm_out_w"], P["norm_out_b"], 32, 1e-5))
    return rec("conv_out", conv2d(h, P["conv_out_w"], P["conv_out_b"]))
