"""Seeded synthetic inputs for the Spatial-Transformer block.

This module draws numbers and nothing else: it holds none of the block's
arithmetic, so both the fp64 oracle (``oracle/``) and the HIP path consume the
very same arrays without sharing any computation.

Workload (the pages' own run is random-init BF16, batch 1: SDXL Inpainting
architecture page §1 and §5 "run boundary"; SD2.1-base architecture page §5):

* x   [B, C, H, W] ~ N(0, 1)        latent feature map entering the block
* ctx [B, 77, D_ctx] ~ N(0, 1)      text context (77 tokens: SD tutorial page,
                                    section on the CLIP 77-token limit)
* every Linear weight ~ N(0, std^2) with std = 0.02
* every bias = 0, every norm gamma = 1, beta = 0 (standard initialisation)

Draw order with ``numpy.random.default_rng(seed)``: x, ctx, proj_in_w, then for
each layer the weights in the order of ``LAYER_WEIGHTS``, then proj_out_w.
Optional stress draws (biases, gammas, betas) come after, from a second
generator seeded ``seed + 7919`` so that the headline draws never shift.

Values are drawn in float32.  For bf16 configurations they are rounded to
bfloat16 with round-to-nearest-even; the rounded values are kept as float32
arrays (every bf16 value is exactly representable in float32 and float64), so
the oracle's float64 upcast and the device's bf16 copy hold the same numbers.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

CTX_LEN = 77

# Per-layer Linear weights, in draw order.  Shapes as (out, in).
LAYER_WEIGHTS = ("q1_w", "k1_w", "v1_w", "o1_w", "q2_w", "k2_w", "v2_w",
                 "o2_w", "ff1_w", "ff2_w")
LAYER_BIASES = ("q1_b", "k1_b", "v1_b", "o1_b", "q2_b", "k2_b", "v2_b",
                "o2_b", "ff1_b", "ff2_b")
LAYER_NORMS = ("ln1", "ln2", "ln3")


@dataclasses.dataclass(frozen=True)
class BlockConfig:
    """Shape of one Spatial-Transformer block invocation."""
    name: str
    B: int
    C: int
    H: int
    W: int
    heads: int
    D_ctx: int
    depth: int
    dtype: str  # "f32" or "bf16": storage type of inputs, weights and output

    @property
    def N(self) -> int:
        return self.H * self.W

    @property
    def T(self) -> int:
        return self.B * self.H * self.W

    @property
    def F(self) -> int:
        """GEGLU inner width (value half of the 2F-wide first FF projection)."""
        return 4 * self.C


# The five workloads: stage shapes from the SD2.1-base and SDXL topology
# diagrams (SD2.1-base architecture page §3; SDXL Inpainting architecture page
# §3), transformer depth 2 and 10 from the SD tutorial page's SDXL stage
# description, B=2 for a classifier-free-guidance pair.
CONFIGS: List[BlockConfig] = [
    BlockConfig("tiny_f32_c320_16x16_d1", 1, 320, 16, 16, 5, 768, 1, "f32"),
    BlockConfig("sd21_down0_c320_96x96_d1", 2, 320, 96, 96, 5, 1024, 1, "bf16"),
    BlockConfig("sd21_down2_c1280_24x24_d1", 2, 1280, 24, 24, 20, 1024, 1, "bf16"),
    BlockConfig("sdxl_down1_c640_64x64_d2", 2, 640, 64, 64, 10, 2048, 2, "bf16"),
    BlockConfig("sdxl_down2mid_c1280_32x32_d10", 2, 1280, 32, 32, 20, 2048, 10, "bf16"),
]


def config_seed(index: int) -> int:
    """Seed of the workload at position ``index`` of ``CONFIGS``."""
    return 1000 + index


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even).

    Returns float32 arrays holding exactly representable bf16 values.  NaN is
    kept as a quiet NaN; +-inf stay infinite.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    out = r.astype(np.uint32)
    nan = np.isnan(a)
    if nan.any():
        out = np.where(nan, np.uint32(0x7FC00000), out)
    return out.view(np.float32).reshape(a.shape)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bf16-representable."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    return (a.view(np.uint32) >> 16).astype(np.uint16)


def make_inputs(cfg: BlockConfig, seed: int, *, weight_std: float = 0.02,
                bias_std: float = 0.0, norm_std: float = 0.0,
                x_std: float = 1.0, qk_std: Optional[float] = None) -> Dict:
    """Draw x, ctx and every parameter of the block.

    ``bias_std`` > 0 draws every bias ~ N(0, bias_std^2); ``norm_std`` > 0 draws
    gammas ~ N(1, norm_std^2) and betas ~ N(0, norm_std^2).  ``qk_std`` scales
    the query and key weights of both attentions (q1, k1, q2, k2) instead of
    ``weight_std`` -- the same standard-normal draws, so only the sharpness
    of the softmax changes: with unit-variance normalised tokens the logits
    have standard deviation about qk_std^2 * C.  All three are stress
    options; the headline workloads keep the defaults.
    """
    rng = np.random.default_rng(seed)
    f32 = np.float32
    B, C, H, W, D, F = cfg.B, cfg.C, cfg.H, cfg.W, cfg.D_ctx, cfg.F

    def normal(shape, std):
        return (rng.standard_normal(size=shape, dtype=f32) * f32(std)).astype(f32)

    x = normal((B, C, H, W), x_std)
    ctx = normal((B, CTX_LEN, D), 1.0)
    proj_in_w = normal((C, C), weight_std)
    shapes = {"q1_w": (C, C), "k1_w": (C, C), "v1_w": (C, C), "o1_w": (C, C),
              "q2_w": (C, C), "k2_w": (C, D), "v2_w": (C, D), "o2_w": (C, C),
              "ff1_w": (2 * F, C), "ff2_w": (C, F)}
    qk = ("q1_w", "k1_w", "q2_w", "k2_w")
    layers = []
    for _ in range(cfg.depth):
        layers.append({k: normal(shapes[k], qk_std if (qk_std is not None and k in qk) else weight_std)
                       for k in LAYER_WEIGHTS})
    proj_out_w = normal((C, C), weight_std)

    rng2 = np.random.default_rng(seed + 7919)

    def bias(n):
        if bias_std > 0:
            return (rng2.standard_normal(size=n, dtype=f32) * f32(bias_std)).astype(f32)
        return np.zeros(n, f32)

    def gamma(n):
        if norm_std > 0:
            return (1.0 + rng2.standard_normal(size=n, dtype=f32) * f32(norm_std)).astype(f32)
        return np.ones(n, f32)

    def beta(n):
        if norm_std > 0:
            return (rng2.standard_normal(size=n, dtype=f32) * f32(norm_std)).astype(f32)
        return np.zeros(n, f32)

    bias_sizes = {"q1_b": C, "k1_b": C, "v1_b": C, "o1_b": C, "q2_b": C,
                  "k2_b": C, "v2_b": C, "o2_b": C, "ff1_b": 2 * F, "ff2_b": C}
    params = {"gn_w": gamma(C), "gn_b": beta(C), "proj_in_w": proj_in_w,
              "proj_in_b": bias(C), "proj_out_w": proj_out_w,
              "proj_out_b": bias(C), "layers": layers}
    for lw in layers:
        for k in LAYER_BIASES:
            lw[k] = bias(bias_sizes[k])
        for n in LAYER_NORMS:
            lw[n + "_w"] = gamma(C)
            lw[n + "_b"] = beta(C)

    if cfg.dtype == "bf16":
        x = round_bf16(x)
        ctx = round_bf16(ctx)
        params = map_params(params, round_bf16)
    return {"x": x, "ctx": ctx, "params": params}


def map_params(params: Dict, fn) -> Dict:
    """Apply ``fn`` to every array of a parameter tree, returning a new tree."""
    out = {k: fn(v) for k, v in params.items() if k != "layers"}
    out["layers"] = [{k: fn(v) for k, v in lw.items()} for lw in params["layers"]]
    return out


def small_config(name: str = "small", *, B=2, C=128, H=15, W=15, heads=None,
                 D_ctx=128, depth=2, dtype="bf16") -> BlockConfig:
    """A parity-test configuration the oracle finishes in well under a second."""
    return BlockConfig(name, B, C, H, W, heads if heads is not None else C // 64,
                       D_ctx, depth, dtype)


# ------------------------------------------------------------ ResnetBlock2D
@dataclasses.dataclass(frozen=True)
class ResnetConfig:
    """Shape of one ResnetBlock2D invocation (x [B, Cin, H, W], temb [B, Dt])."""
    name: str
    B: int
    Cin: int
    Cout: int
    H: int
    W: int
    Dt: int = 1280  # time-embedding width of the SD / SDXL U-Nets (4 x 320)


RESNET_WEIGHTS = ("conv1_w", "temb_w", "conv2_w", "sc_w")


def make_resnet_inputs(cfg: ResnetConfig, seed: int, *, weight_std: float = 0.02,
                       bias_std: float = 0.0, norm_std: float = 0.0) -> Dict:
    """Draw x, temb and every ResnetBlock2D parameter, rounded to bf16.

    Draw order with ``numpy.random.default_rng(seed)``: x, temb, conv1_w,
    temb_w, conv2_w, then sc_w when Cin != Cout; weights N(0, weight_std^2),
    x and temb N(0, 1).  Stress draws (biases, GroupNorm gammas/betas) come
    from a second generator seeded ``seed + 7919``; by default biases are 0,
    gammas 1, betas 0.
    """
    rng = np.random.default_rng(seed)
    f32 = np.float32
    B, Ci, Co, H, W, Dt = cfg.B, cfg.Cin, cfg.Cout, cfg.H, cfg.W, cfg.Dt

    def normal(shape, std):
        return (rng.standard_normal(size=shape, dtype=f32) * f32(std)).astype(f32)

    x = normal((B, Ci, H, W), 1.0)
    temb = normal((B, Dt), 1.0)
    p = {"conv1_w": normal((Co, Ci, 3, 3), weight_std), "temb_w": normal((Co, Dt), weight_std),
         "conv2_w": normal((Co, Co, 3, 3), weight_std)}
    if Ci != Co:
        p["sc_w"] = normal((Co, Ci), weight_std)
    rng2 = np.random.default_rng(seed + 7919)

    def extra(n, mean, std):
        if std > 0:
            return (mean + rng2.standard_normal(size=n, dtype=f32) * f32(std)).astype(f32)
        return np.full(n, mean, f32)

    p["gn1_w"], p["gn1_b"] = extra(Ci, 1.0, norm_std), extra(Ci, 0.0, norm_std)
    p["conv1_b"], p["temb_b"] = extra(Co, 0.0, bias_std), extra(Co, 0.0, bias_std)
    p["gn2_w"], p["gn2_b"] = extra(Co, 1.0, norm_std), extra(Co, 0.0, norm_std)
    p["conv2_b"] = extra(Co, 0.0, bias_std)
    if Ci != Co:
        p["sc_b"] = extra(Co, 0.0, bias_std)
    return {"x": round_bf16(x), "temb": round_bf16(temb),
            "params": {k: round_bf16(v) for k, v in p.items()}}


# ------------------------------------------------------------------ U-Net
@dataclasses.dataclass(frozen=True)
class UNetConfig:
    """Topology of a U-Net denoiser (the pages' §3 diagrams).

    ``channels`` and ``depths`` per resolution level (depth 0 = ResNet only,
    no Spatial-Transformer), ``mid_depth`` for the middle block,
    ``layers_per_block`` ResNets per down level (up levels take one more),
    ``ctx_dim`` the context width, ``add_in`` the width of an extra
    embedding added to the time embedding (SDXL: pooled text + size and crop
    conditions, 2816), 0 = none.  The time embedding is sinusoidal of width
    channels[0], then Linear -> SiLU -> Linear to 4 channels[0].
    """
    name: str
    in_channels: int
    out_channels: int
    channels: tuple
    depths: tuple
    mid_depth: int
    layers_per_block: int
    ctx_dim: int
    add_in: int = 0

    @property
    def temb_in(self) -> int:
        return self.channels[0]

    @property
    def temb_dim(self) -> int:
        return 4 * self.channels[0]


UNET_CONFIGS = {
    # SD2.1-base architecture page §3: Down 0-2 with cross-attention, Down 3
    # and Up 0 ResNet only, 4 -> 4 channels, context [1, 77, 1024]
    "sd21": UNetConfig("sd21_base", 4, 4, (320, 640, 1280, 1280), (1, 1, 1, 0), 1, 2, 1024),
    # SDXL-Inpaint architecture page §3: Down 0 ResNet only, Down 1 / Down 2
    # with cross-attention (depth 2 and 10, tutorial), 9 -> 4 channels,
    # context [1, 77, 2048]; the time embedding also takes the pooled text
    # and size/crop conditions (tutorial)
    "sdxl_inpaint": UNetConfig("sdxl_inpaint", 9, 4, (320, 640, 1280), (0, 2, 10), 10, 2, 2048, 2816),
}


def unet_skip_channels(cfg: UNetConfig) -> List[int]:
    """Channels of the skip connections in the order the down path stores
    them: conv_in's output, every down-level ResNet (+ transformer) output,
    every downsampler's output."""
    sk = [cfg.channels[0]]
    for lvl, c in enumerate(cfg.channels):
        sk += [c] * cfg.layers_per_block
        if lvl < len(cfg.channels) - 1:
            sk.append(c)
    return sk


def unet_param_shapes(cfg: UNetConfig) -> Dict:
    """Nested dict of parameter shapes (no values): the module structure of
    the U-Net, in the order the draws are taken."""
    C0, Td = cfg.channels[0], cfg.temb_dim
    P = {"time1_w": (Td, cfg.temb_in), "time1_b": (Td,), "time2_w": (Td, Td), "time2_b": (Td,)}
    if cfg.add_in:
        P.update({"add1_w": (Td, cfg.add_in), "add1_b": (Td,), "add2_w": (Td, Td), "add2_b": (Td,)})
    P["conv_in_w"] = (C0, cfg.in_channels, 3, 3)
    P["conv_in_b"] = (C0,)

    def resnet(ci, co):
        r = {"gn1_w": (ci,), "gn1_b": (ci,), "conv1_w": (co, ci, 3, 3), "conv1_b": (co,),
             "temb_w": (co, Td), "temb_b": (co,), "gn2_w": (co,), "gn2_b": (co,),
             "conv2_w": (co, co, 3, 3), "conv2_b": (co,)}
        if ci != co:
            r["sc_w"] = (co, ci)
            r["sc_b"] = (co,)
        return r

    def block(c, depth):
        D, F = cfg.ctx_dim, 4 * c
        lay = {"ln1_w": (c,), "ln1_b": (c,), "q1_w": (c, c), "k1_w": (c, c), "v1_w": (c, c),
               "o1_w": (c, c), "o1_b": (c,), "ln2_w": (c,), "ln2_b": (c,), "q2_w": (c, c),
               "k2_w": (c, D), "v2_w": (c, D), "o2_w": (c, c), "o2_b": (c,), "ln3_w": (c,),
               "ln3_b": (c,), "ff1_w": (2 * F, c), "ff1_b": (2 * F,), "ff2_w": (c, F),
               "ff2_b": (c,)}
        return {"gn_w": (c,), "gn_b": (c,), "proj_in_w": (c, c), "proj_in_b": (c,),
                "proj_out_w": (c, c), "proj_out_b": (c,), "layers": [dict(lay) for _ in range(depth)]}

    down, h = [], C0
    for lvl, c in enumerate(cfg.channels):
        d = {"res": [], "attn": []}
        for _ in range(cfg.layers_per_block):
            d["res"].append(resnet(h, c))
            h = c
            if cfg.depths[lvl]:
                d["attn"].append(block(c, cfg.depths[lvl]))
        if lvl < len(cfg.channels) - 1:
            d["down_w"], d["down_b"] = (c, c, 3, 3), (c,)
        down.append(d)
    P["down"] = down
    P["mid"] = {"res": [resnet(h, h), resnet(h, h)],
                "attn": [block(h, cfg.mid_depth)] if cfg.mid_depth else []}
    skips = unet_skip_channels(cfg)
    up = []
    for lvl in reversed(range(len(cfg.channels))):
        c = cfg.channels[lvl]
        u = {"res": [], "attn": []}
        for _ in range(cfg.layers_per_block + 1):
            u["res"].append(resnet(h + skips.pop(), c))
            h = c
            if cfg.depths[lvl]:
                u["attn"].append(block(c, cfg.depths[lvl]))
        if lvl > 0:
            u["up_w"], u["up_b"] = (c, c, 3, 3), (c,)
        up.append(u)
    P["up"] = up
    P["norm_out_w"], P["norm_out_b"] = (C0,), (C0,)
    P["conv_out_w"], P["conv_out_b"] = (cfg.out_channels, C0, 3, 3), (cfg.out_channels,)
    return P


def _walk(tree, fn, path=()):
    """Map ``fn(path, leaf)`` over a nested dict / list tree, in key order
    as written (dicts keep insertion order)."""
    if isinstance(tree, dict):
        return {k: _walk(v, fn, path + (k,)) for k, v in tree.items()}
    if isinstance(tree, list):
        return [_walk(v, fn, path + (i,)) for i, v in enumerate(tree)]
    return fn(path, tree)


def unet_param_count(cfg: UNetConfig) -> int:
    n = [0]

    def f(path, shape):
        n[0] += int(np.prod(shape))
        return shape
    _walk(unet_param_shapes(cfg), f)
    return n[0]


def make_unet_inputs(cfg: UNetConfig, seed: int, B: int, H: int, W: int, *,
                     weight_std: float = 0.02, t=(999.0,)) -> Dict:
    """Draw x [B, in, H, W], ctx [B, 77, D], add [B, add_in] (N(0, 1)), the
    timesteps (``t`` repeated to B values) and every U-Net parameter: weights
    (names ending in ``_w`` except norm gammas) N(0, weight_std^2) in
    ``unet_param_shapes`` order, biases 0, norm gammas 1, betas 0.  All
    rounded to bf16."""
    rng = np.random.default_rng(seed)
    f32 = np.float32
    x = rng.standard_normal((B, cfg.in_channels, H, W), dtype=f32)
    ctx = rng.standard_normal((B, CTX_LEN, cfg.ctx_dim), dtype=f32)
    add = rng.standard_normal((B, cfg.add_in), dtype=f32) if cfg.add_in else None
    norm_w = ("gn1_w", "gn2_w", "gn_w", "norm_out_w", "ln1_w", "ln2_w", "ln3_w")

    def draw(path, shape):
        name = path[-1]
        if name in norm_w:
            return np.ones(shape, f32)
        if name.endswith("_w"):
            return round_bf16((rng.standard_normal(size=shape, dtype=f32) * f32(weight_std)).astype(f32))
        return np.zeros(shape, f32)

    params = _walk(unet_param_shapes(cfg), draw)
    tt = np.array([t[i % len(t)] for i in range(B)], np.float32)
    return {"x": round_bf16(x), "ctx": round_bf16(ctx),
            "add": round_bf16(add) if add is not None else None, "t": tt, "params": params}
