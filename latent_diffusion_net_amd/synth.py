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
                x_std: float = 1.0) -> Dict:
    """Draw x, ctx and every parameter of the block.

    ``bias_std`` > 0 draws every bias ~ N(0, bias_std^2); ``norm_std`` > 0 draws
    gammas ~ N(1, norm_std^2) and betas ~ N(0, norm_std^2).  Both are stress
    options; the headline workloads keep them at 0.
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
    layers = []
    for _ in range(cfg.depth):
        layers.append({k: normal(shapes[k], weight_std) for k in LAYER_WEIGHTS})
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
