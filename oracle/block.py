"""Plain float64 oracle of the Spatial-Transformer block.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
library.  Every function takes NumPy arrays, upcasts them to float64 and
follows the block's definition step by step, with no fusion and no
reordering.  Where the pages leave a step open, the reading taken is stated in
the function's docstring.

Pages cited:
  * "Stable Diffusion XL Inpainting 宏观架构" (SDXL-Inpaint architecture page),
    §4 "核心算子与任务差异": Transformer2DModel = Norm -> self-attention
    (Q=K=V=image tokens), Norm -> cross-attention (K=V=context), Norm -> GEGLU,
    residual after every sublayer.
  * "Stable Diffusion 2.1 Base 宏观架构" (SD2.1 architecture page), §4: the
    block keeps the backbone shape and flattens H x W into a token sequence.
  * DDPM / SD / SDXL tutorial page (bfzx365): "（4）Spatial Transformer模块"
    (GroupNorm + Conv/Linear + BasicTransformer blocks + Conv/Linear, shape
    preserving, outer residual), "BasicTransformer Block" (LayerNorm +
    SelfAttention + CrossAttention + FeedForward, each residual), FeedForward =
    GeGLU + Dropout + Linear, the (C,H,W)->(C,HW)->(HW,C) reshape of the
    "Self-Attention Block" walk-through and its inverse.
  * "企业官网建设流程全解析" (SD1.5 anatomy article), §3.2 (cross-attention
    K/V projections map the 768-d context to the feature width) and §3.4
    (attention output = Softmax(Q K^T / sqrt(d)) V with per-head layout
    [batch, heads, tokens, dim]).

Precision: float64 throughout.  Parity unpinned by printed values: the pages
print no numeric example of the block, so absolute values are pinned only
through the closed forms, invariants, library cross-checks and brute-force
agreement in ``tests/test_oracle.py``.
"""
from __future__ import annotations

import math
from typing import Dict, Optional

import numpy as np
from scipy.special import erf

GN_GROUPS = 32
GN_EPS = 1e-6
LN_EPS = 1e-5
HEAD_DIM = 64


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def group_norm(x, gamma, beta, groups: int = GN_GROUPS, eps: float = GN_EPS):
    """GroupNorm over [B, C, H, W].

    Channels are split into ``groups`` contiguous groups of C/groups channels;
    each (sample, group) is normalised by its own mean and population variance
    over all of its channels and pixels, then scaled by gamma[c] and shifted by
    beta[c].  (The pages name only "GroupNorm"; 32 groups, eps = 1e-6 and the
    population variance are the reading taken.)
    """
    x = _f64(x)
    B, C, H, W = x.shape
    if C % groups:
        raise ValueError("C must be divisible by the number of groups")
    g = x.reshape(B, groups, C // groups, H, W)
    mean = g.mean(axis=(2, 3, 4), keepdims=True)
    var = ((g - mean) ** 2).mean(axis=(2, 3, 4), keepdims=True)
    xhat = ((g - mean) / np.sqrt(var + eps)).reshape(B, C, H, W)
    return xhat * _f64(gamma)[None, :, None, None] + _f64(beta)[None, :, None, None]


def to_tokens(z):
    """[B, C, H, W] -> [B, H*W, C]; token n = i*W + j holds pixel (i, j).

    Follows the tutorial page's reshape (C,H,W) -> (C,HW) -> (HW,C): the two
    spatial axes are merged in row-major order and the result is transposed.
    """
    z = _f64(z)
    B, C, H, W = z.shape
    return z.reshape(B, C, H * W).transpose(0, 2, 1)


def from_tokens(t, H: int, W: int):
    """Inverse of ``to_tokens``: [B, H*W, C] -> [B, C, H, W]."""
    t = _f64(t)
    B, N, C = t.shape
    if N != H * W:
        raise ValueError("token count does not match H*W")
    return t.transpose(0, 2, 1).reshape(B, C, H, W)


def linear(t, w, b=None):
    """y = t W^T + b with W stored (out_features, in_features).

    proj_in/proj_out: the tutorial page gives Linear for SDXL and a 1x1 Conv
    for SD; on token rows a 1x1 convolution with kernel [C_out, C_in, 1, 1] is
    exactly this product.
    """
    y = _f64(t) @ _f64(w).T
    if b is not None:
        y = y + _f64(b)
    return y


def layer_norm(h, gamma, beta, eps: float = LN_EPS):
    """LayerNorm over the last axis with population variance, eps = 1e-5."""
    h = _f64(h)
    mean = h.mean(axis=-1, keepdims=True)
    var = ((h - mean) ** 2).mean(axis=-1, keepdims=True)
    return (h - mean) / np.sqrt(var + eps) * _f64(gamma) + _f64(beta)


def attention(q, k, v, heads: int, row_block: int = 2048,
              return_probs: bool = False, rows: Optional[np.ndarray] = None,
              key_mask: Optional[np.ndarray] = None):
    """Multi-head scaled dot-product attention.

    q: [B, Nq, C], k and v: [B, Nk, C], C = heads * 64.  Head ``hd`` takes the
    contiguous channel slice [64*hd, 64*hd + 64) of each projection (the
    [batch, heads, tokens, dim] layout of the anatomy article §3.4).  Per head,
    P = softmax over keys of Q K^T / sqrt(64), O = P V; heads are
    concatenated back in channel order.  The softmax subtracts the row maximum
    before exponentiating (an identity of softmax, kept for range only).

    Query rows are processed ``row_block`` at a time so that no Nq x Nk matrix
    larger than row_block x Nk is ever held; this changes no arithmetic.
    ``rows`` restricts the computation to the listed query rows (per batch).
    ``return_probs`` also returns P as [B, heads, Nq, Nk] (small inputs only).

    ``key_mask`` ([B, Nk], nonzero = attend) excludes keys from the softmax:
    the anatomy article's §5.5 ("Cross-Attention mask") passes the
    tokenizer's attention_mask, 0 marking a padding token, so that padding
    positions take no part.  Reading taken: a masked key gets probability 0
    (the softmax runs over the unmasked keys only); a row of sample b whose
    every key is masked has no keys to average and outputs 0.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Nq, C = q.shape
    d = C // heads
    if d * heads != C:
        raise ValueError("C must equal heads * head_dim")
    scale = 1.0 / math.sqrt(d)
    qi = q if rows is None else q[:, rows, :]
    nq = qi.shape[1]
    out = np.empty((B, nq, C), dtype=np.float64)
    probs = np.empty((B, heads, nq, k.shape[1])) if return_probs else None
    for b in range(B):
        keep = None if key_mask is None else np.asarray(key_mask)[b] != 0
        for hd in range(heads):
            sl = slice(hd * d, (hd + 1) * d)
            kh, vh = k[b, :, sl], v[b, :, sl]
            for r0 in range(0, nq, row_block):
                qh = qi[b, r0:r0 + row_block, sl]
                if keep is not None and not keep.any():
                    out[b, r0:r0 + row_block, sl] = 0.0
                    if return_probs:
                        probs[b, hd, r0:r0 + row_block] = 0.0
                    continue
                s = (qh @ kh.T) * scale
                if keep is not None:
                    s = np.where(keep[None, :], s, -np.inf)
                s = s - s.max(axis=1, keepdims=True)
                e = np.exp(s)
                p = e / e.sum(axis=1, keepdims=True)
                out[b, r0:r0 + row_block, sl] = p @ vh
                if return_probs:
                    probs[b, hd, r0:r0 + row_block] = p
    return (out, probs) if return_probs else out


def gelu_erf(g):
    """GELU in its exact form g * Phi(g) = g/2 * (1 + erf(g / sqrt 2))."""
    g = _f64(g)
    return 0.5 * g * (1.0 + erf(g / math.sqrt(2.0)))


def geglu(z, F: int):
    """GEGLU on the 2F-wide first feed-forward projection.

    Reading taken: the first F features are the value, the last F the gate;
    out = value * GELU(gate).  ("GeGLU" is all the tutorial page names.)
    """
    z = _f64(z)
    if z.shape[-1] != 2 * F:
        raise ValueError("GEGLU input must be 2F wide")
    return z[..., :F] * gelu_erf(z[..., F:])


def self_attention_sublayer(h, lw, heads):
    """h + Attn(LN1(h)) with Q, K, V all projected from the image tokens."""
    u = layer_norm(h, lw["ln1_w"], lw["ln1_b"])
    q = linear(u, lw["q1_w"], lw.get("q1_b"))
    k = linear(u, lw["k1_w"], lw.get("k1_b"))
    v = linear(u, lw["v1_w"], lw.get("v1_b"))
    o = attention(q, k, v, heads)
    return h + linear(o, lw["o1_w"], lw.get("o1_b"))


def cross_attention_sublayer(h, ctx, lw, heads, ctx_mask=None):
    """h + Attn(Q = LN2(h) Wq, K = ctx Wk, V = ctx Wv); ctx is not normalised.

    ``ctx_mask`` ([B, 77], nonzero = a real token): the context's key
    padding mask (see ``attention``)."""
    u = layer_norm(h, lw["ln2_w"], lw["ln2_b"])
    q = linear(u, lw["q2_w"], lw.get("q2_b"))
    k = linear(ctx, lw["k2_w"], lw.get("k2_b"))
    v = linear(ctx, lw["v2_w"], lw.get("v2_b"))
    o = attention(q, k, v, heads) if ctx_mask is None else attention(q, k, v, heads, key_mask=ctx_mask)
    return h + linear(o, lw["o2_w"], lw.get("o2_b"))


def feed_forward_sublayer(h, lw):
    """h + Linear2(GEGLU(Linear1(LN3(h)))); dropout is the identity."""
    u = layer_norm(h, lw["ln3_w"], lw["ln3_b"])
    z = linear(u, lw["ff1_w"], lw.get("ff1_b"))
    F = z.shape[-1] // 2
    return h + linear(geglu(z, F), lw["ff2_w"], lw.get("ff2_b"))


def block_forward(x, ctx, params: Dict, heads: int,
                  intermediates: bool = False, ctx_mask=None):
    """The whole Spatial-Transformer block, [B, C, H, W] -> [B, C, H, W].

    GroupNorm -> flatten to tokens -> proj_in -> depth x (self-attention,
    cross-attention, GEGLU feed-forward; pre-norm, residual after each) ->
    proj_out -> back to [B, C, H, W] -> + x (outer residual).

    With ``intermediates`` the function also returns a dict holding the
    fp64 residual stream after proj_in ("h0") and after each sublayer
    ("l{i}_sa", "l{i}_ca", "l{i}_ff").  ``ctx_mask`` ([B, 77]) masks padding
    tokens of the context out of every cross-attention.
    """
    x = _f64(x)
    ctx = _f64(ctx)
    B, C, H, W = x.shape
    z = group_norm(x, params["gn_w"], params["gn_b"])
    h = linear(to_tokens(z), params["proj_in_w"], params.get("proj_in_b"))
    inter = {"h0": h}
    for i, lw in enumerate(params["layers"]):
        h = self_attention_sublayer(h, lw, heads)
        inter[f"l{i}_sa"] = h
        h = cross_attention_sublayer(h, ctx, lw, heads, ctx_mask)
        inter[f"l{i}_ca"] = h
        h = feed_forward_sublayer(h, lw)
        inter[f"l{i}_ff"] = h
    out = linear(h, params["proj_out_w"], params.get("proj_out_b"))
    y = from_tokens(out, H, W) + x
    return (y, inter) if intermediates else y
